"""The unfused two-kernel path vs the float64 oracle: mq_linear on a handle
packed without residual (rho = 0) from the same W, then mq_residual_add with
the handle that has the residual, must give X W~^T within the same per-output
tolerance as the fused kernels (|Y - Y64| <= 2e-3 * sum|x||w~| + 1e-5)."""
import numpy as np
import pytest

import oracle
from bit_gemm_amd import synth
from tests.gpu_util import check_linear, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    return require_gpu()


def _layer(N, K, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, 3, replace=False)] *= 20
    return W.astype(np.float16)


def _unfused(mq, X16, p0, p):
    import torch
    Y = mq.mq_linear(to_dev(X16), p0)
    mq.mq_residual_add(to_dev(X16), p, Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


CASES = [(16, 128, 128, 0.05), (17, 96, 32, 0.1), (100, 640, 64, 0.02), (257, 1024, 128, 0.01),
         (130, 4224, 128, 0.004), (48, 4096, 128, 0.05), (5, 65536, 128, 0.002)]


@pytest.mark.parametrize("N,K,G,rho", CASES)
def test_unfused_matches_oracle(mq, N, K, G, rho):
    W = _layer(N, K, seed=N * 7 + K)
    p0, p = mq.mq_pack(to_dev(W), G, 0.0), mq.mq_pack(to_dev(W), G, rho)
    Wt = oracle.dequant(oracle.pack(W, G, rho))
    for M in (1, 3, 16, 17, 64, 65):
        print(f"[unfused parity] N={N} K={K} G={G} rho={rho} M={M}", flush=True)
        X = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
        check_linear(_unfused(mq, X, p0, p), X, Wt, f"unfused N={N} K={K} rho={rho} M={M}")


def test_unfused_decode_layer(mq):
    layer = synth.WORKLOADS["decode-11008x4096"].layers[0]
    W = layer.W()
    p0, p = mq.mq_pack(to_dev(W), layer.group, 0.0), mq.mq_pack(to_dev(W), layer.group, layer.rho)
    Wt = oracle.dequant(oracle.pack(W, layer.group, layer.rho))
    for M in (1, 4, 16):
        print(f"[unfused parity] decode-11008x4096 M={M}", flush=True)
        X = layer.X(M)
        check_linear(_unfused(mq, X, p0, p), X, Wt, f"unfused decode M={M}")


def test_residual_add_touches_only_rows_with_entries(mq):
    import torch
    N, K = 64, 256
    W = _layer(N, K, seed=3)
    W[:, :] = np.float16(0.01)          # identical groups: no base error anywhere ...
    W[5, 17] = np.float16(0.3)          # ... except in rows 5 and 40
    W[40, 200] = np.float16(-0.2)
    p = mq.mq_pack(to_dev(W), 128, 0.001)   # nnz = floor(0.001 * 64 * 256) = 16
    c = oracle.pack(W, 128, 0.001)
    rows = set(int(r) for r in np.repeat(np.arange(N), np.diff(c["row_ptr"])))
    X = np.random.default_rng(0).standard_normal((3, K)).astype(np.float16)
    Y0 = np.random.default_rng(1).standard_normal((3, N)).astype(np.float16)
    Y = to_dev(Y0)
    mq.mq_residual_add(to_dev(X), p, Y)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    untouched = [i for i in range(N) if i not in rows]
    assert np.array_equal(Y[:, untouched].view(np.uint16), Y0[:, untouched].view(np.uint16))
    # a handle without residual enqueues nothing
    p0 = mq.mq_pack(to_dev(W), 128, 0.0)
    Y = to_dev(Y0)
    mq.mq_residual_add(to_dev(X), p0, Y)
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy().view(np.uint16), Y0.view(np.uint16))


def test_residual_add_argument_errors(mq):
    import torch
    W = _layer(16, 128, seed=1)
    p = mq.mq_pack(to_dev(W), 128, 0.1)
    X = torch.zeros((2, 128), dtype=torch.float16, device="cuda")
    Y = torch.zeros((2, 16), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        mq.mq_residual_add(X[:, :64], p, Y)
    with pytest.raises(ValueError):
        mq.mq_residual_add(X, p, Y[:1])
    assert mq.lib.mq_residual_add(None, 2, p.handle, Y.data_ptr(), None) == -1   # MQ_ERR_INVALID_ARG
    assert mq.lib.mq_residual_add(X.data_ptr(), 0, p.handle, Y.data_ptr(), None) == -1   # MQ_ERR_INVALID_ARG
