"""Fused linear (decode GEMV and prefill GEMM kernels) vs the float64 oracle on
the identical dequantised weights: |Y - Y64| <= 2e-3 * sum|x||w~| + 1e-5."""
import numpy as np
import pytest

import oracle
from bit_gemm_amd import synth
from tests.gpu_util import check_linear, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    return require_gpu()


def _layer(N, K, seed, outlier_cols=3):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, outlier_cols, replace=False)] *= 20
    return W.astype(np.float16)


def _x(M, K, seed):
    return np.random.default_rng(seed).standard_normal((M, K)).astype(np.float16)


SHAPES = [(16, 128, 128, 0.05), (17, 96, 32, 0.1), (100, 640, 64, 0.02), (257, 1024, 128, 0.01),
          (130, 4224, 128, 0.004), (40, 4160, 64, 0.01), (24, 8256, 32, 0.02), (70, 12288, 128, 0.003)]
BATCH = [1, 3, 16, 17, 33, 64, 65, 130]


@pytest.mark.parametrize("N,K,G,rho", SHAPES)
def test_linear_small_layers_both_kernels(mq, N, K, G, rho):
    W = _layer(N, K, seed=N + K)
    p = mq.mq_pack(to_dev(W), G, rho)
    Wt = oracle.dequant(oracle.pack(W, G, rho))
    for M in BATCH:
        X = _x(M, K, seed=M)
        Xd = to_dev(X)
        kernels = [mq.KERNEL_GEMM] + ([mq.KERNEL_GEMV] if M <= mq.GEMV_MAX_M else [])
        for kern in kernels:
            print(f"[linear parity] N={N} K={K} G={G} rho={rho} M={M} kernel={kern}", flush=True)
            Y = mq.mq_linear_with(Xd, p, kern).cpu().numpy()
            check_linear(Y, X, Wt, f"N={N} K={K} M={M} kernel={kern}")


def test_one_hot_rows_reproduce_the_dequantised_weights(mq):
    """P9: X rows = unit vectors e_j give Y[:, i] = W~[i, j] (to fp16), for
    every position of a tile, so any index mistake in either kernel shows."""
    N, K, G, rho = 48, 256, 64, 0.08
    W = _layer(N, K, seed=5)
    p = mq.mq_pack(to_dev(W), G, rho)
    Wt = oracle.dequant(oracle.pack(W, G, rho))
    for j0 in range(0, K, 64):
        X = np.zeros((64, K), np.float16)
        X[np.arange(64), j0 + np.arange(64)] = 1.0
        Xd = to_dev(X)
        for kern in (mq.KERNEL_GEMV, mq.KERNEL_GEMM):
            print(f"[one-hot] j0={j0} kernel={kern}", flush=True)
            Y = mq.mq_linear_with(Xd, p, kern).cpu().numpy().astype(np.float64)
            ref = Wt[:, j0:j0 + 64].T
            assert np.all(np.abs(Y - ref) <= 2 ** -10 * np.abs(ref) + 2 ** -24), (j0, kern)


# K = 4096 decode shapes: the up-to-4-token kernel (X slices in LDS) and the
# several-row-blocks-per-workgroup kernel (1, 2 or 3 row blocks, the last
# workgroup partly past the end), ragged N, no residual, and residual
# densities whose chunks overflow the two prefetched per wave
K4096 = [(40, 128, 0.3), (16, 128, 0.0), (4100, 64, 0.01), (8210, 32, 0.002), (1000, 128, 0.02)]


@pytest.mark.parametrize("N,G,rho", K4096)
def test_linear_k4096_decode_paths(mq, N, G, rho):
    K = 4096
    W = _layer(N, K, seed=N + G)
    p = mq.mq_pack(to_dev(W), G, rho)
    Wt = oracle.dequant(oracle.pack(W, G, rho))
    for M in (1, 2, 3, 4, 5, 8, 9, 16):
        X = _x(M, K, seed=100 + M)
        for kern in (mq.KERNEL_GEMV, mq.KERNEL_GEMM):
            print(f"[linear parity] K=4096 N={N} G={G} rho={rho} M={M} kernel={kern}", flush=True)
            Y = mq.mq_linear_with(to_dev(X), p, kern).cpu().numpy()
            check_linear(Y, X, Wt, f"K=4096 N={N} G={G} rho={rho} M={M} kernel={kern}")


@pytest.mark.parametrize("name", ["tiny-1024x1024", "decode-11008x4096"])
def test_linear_workload_layers(mq, name):
    wl = synth.WORKLOADS[name]
    layer = wl.layers[0]
    W = layer.W()
    p = mq.mq_pack(to_dev(W), layer.group, layer.rho)
    Wt = oracle.dequant(oracle.pack(W, layer.group, layer.rho))
    for M in wl.batch + (64,):
        X = layer.X(M)
        for kern in (mq.KERNEL_GEMV, mq.KERNEL_GEMM):
            print(f"[linear parity] {name} M={M} kernel={kern}", flush=True)
            Y = mq.mq_linear_with(to_dev(X), p, kern).cpu().numpy()
            check_linear(Y, X, Wt, f"{name} M={M} kernel={kern}")


def test_linear_is_deterministic(mq):
    layer = synth.WORKLOADS["tiny-1024x1024"].layers[0]
    p = mq.mq_pack(to_dev(layer.W()), 128, 0.05)
    for M, kern in ((4, mq.KERNEL_GEMV), (200, mq.KERNEL_GEMM)):
        Xd = to_dev(layer.X(M))
        a = mq.mq_linear_with(Xd, p, kern).cpu().numpy()
        b = mq.mq_linear_with(Xd, p, kern).cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_linear_argument_errors(mq):
    import torch
    layer = synth.WORKLOADS["tiny-1024x1024"].layers[0]
    p = mq.mq_pack(to_dev(layer.W()), 128, 0.01)
    X = to_dev(layer.X(70))
    with pytest.raises(mq.MQError) as ei:
        mq.mq_linear_with(X, p, mq.KERNEL_GEMV)          # M > 64 on the decode kernel
    assert ei.value.code == -2
    p.free()
    with pytest.raises(mq.MQError):
        mq.mq_linear(X[:1], p)
    assert torch.cuda.is_available()


@pytest.mark.parametrize("M,kern", [(4, 1), (16, 1), (64, 2), (130, 2), (600, 2)])
def test_linear_in_graph_replays_match_eager(mq, M, kern):
    """The kernels captured in a graph (the split-K GEMM included: its
    workspace becomes a graph allocation) give the eager result on every
    replay, with other work and synchronisations between the replays."""
    import torch
    N, K = 1536, 1024
    W = _layer(N, K, seed=11)
    p = mq.mq_pack(to_dev(W), 128, 0.01)
    Xd = to_dev(_x(M, K, seed=M))
    ref = mq.mq_linear_with(Xd, p, kern).cpu().numpy()
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mq.mq_linear_with(Xd, p, kern, Y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.mq_linear_with(Xd, p, kern, Y)
    for rep in range(3):
        Y.fill_(1.0)
        junk = mq.mq_linear_with(Xd, p, kern)        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph replay] M={M} kernel={kern} replay={rep}", flush=True)
        assert np.array_equal(Y.cpu().numpy().view(np.uint16), ref.view(np.uint16))
        assert np.array_equal(junk.cpu().numpy().view(np.uint16), ref.view(np.uint16))
