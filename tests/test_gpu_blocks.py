"""Block-wise residual packing (mq_pack_blocks) against the CPU oracle
(oracle/blocks.py): the packed arrays bit-exact (base codes and scales, the
selected blocks, their scales and codes), and the fused linear on those
handles within |Y - Y64| <= 2e-3 * sum|x||w~| + 1e-5 of the float64 oracle on
the identical dequantised weights, for both kernels. h is computed here from
synthetic calibration activations, as a caller would, and handed to both."""
import ctypes

import numpy as np
import pytest

from oracle import blocks as ob
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


def _h(K, seed, hot=4):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((32, K)).astype(np.float16)
    X[:, rng.choice(K, hot, replace=False)] *= 50
    return ob.hessian_diag(X)


def _pack_both(mq, W, G, beta, h):
    p = mq.mq_pack_blocks(to_dev(W), G, beta, to_dev(h))
    got = mq.export_blocks(p)
    base = {k: v.cpu().numpy() for k, v in mq.mq_export_canonical(p, residual=False).items()}
    ref = ob.pack_blocks(W, G, beta, h)
    return p, got, base, ref


def _assert_blocks_equal(got, base, ref):
    assert np.array_equal(base["codes"], ref["codes"]), "base codes differ"
    assert np.array_equal(base["scales"].view(np.uint16), ref["scales"].view(np.uint16)), "base scales differ"
    assert np.array_equal(got["blk"], ref["blk"]), "selected blocks differ"
    assert np.array_equal(got["rscale"].view(np.uint32), ref["rscale"].view(np.uint32)), "block scales differ"
    assert np.array_equal(got["rcodes"], ref["rcodes"]), "block codes differ"


# K = 4096 runs the decode kernels that carry the blocks as code tiles
# (4200 rows: several row blocks per workgroup at M > 4; 12400 rows: 775 row
# blocks, so 4 row blocks per workgroup)
SHAPES = [(16, 128, 128, 0.5), (48, 256, 128, 0.25), (37, 384, 64, 0.3), (130, 4224, 128, 0.1),
          (20, 96, 32, 1.0), (64, 1024, 128, 0.0), (257, 2048, 32, 0.07), (40, 4096, 128, 0.2),
          (24, 4096, 32, 0.3), (90, 4096, 64, 1.0), (4200, 4096, 128, 0.05), (12400, 4096, 128, 0.03),
          (12400, 4096, 64, 0.02)]


@pytest.mark.parametrize("N,K,G,beta", SHAPES)
def test_block_packing_bit_exact_and_linear(mq, N, K, G, beta):
    W = _layer(N, K, N * 3 + K)
    h = _h(K, N + 1)
    print(f"[block pack] N={N} K={K} G={G} beta={beta}", flush=True)
    p, got, base, ref = _pack_both(mq, W, G, beta, h)
    assert p.nblk == ref["blk"].size == ob.block_budget(beta, ob.block_grid(N, K)[0] * ob.block_grid(N, K)[1])
    _assert_blocks_equal(got, base, ref)
    Wt = ob.dequant_blocks(ref)
    assert p.nnz == int(np.count_nonzero(ref["qr"].reshape(-1, 16, 128)[ref["blk"]]))
    for M in (1, 5, 16, 33, 130):
        X = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
        kernels = [mq.KERNEL_GEMM] + ([mq.KERNEL_GEMV] if M <= mq.GEMV_MAX_M else [])
        for kern in kernels:
            print(f"[block linear] N={N} K={K} beta={beta} M={M} kernel={kern}", flush=True)
            Y = mq.mq_linear_with(to_dev(X), p, kern).cpu().numpy()
            check_linear(Y, X, Wt, f"blocks N={N} K={K} beta={beta} M={M} kernel={kern}")


def test_ties_and_zero_scores(mq):
    # an exactly representable matrix: every base error is 0, so every score
    # is 0 and the selection is the lowest block indices
    N, K, G = 48, 512, 128
    rng = np.random.default_rng(5)
    C = rng.integers(-7, 8, size=(N, K)).astype(np.float64)
    C[:, ::128] = 7
    W = (C * 2.0 ** -5).astype(np.float16)
    h = np.ones(K, dtype=np.float32)
    p, got, base, ref = _pack_both(mq, W, G, 0.5, h)
    assert np.array_equal(ref["blk"], np.arange(6))
    _assert_blocks_equal(got, base, ref)
    assert p.nnz == 0


def test_decode_layer_block_budget(mq):
    # the 11008 x 4096 decode layer with 10 % of its 22016 blocks
    from bit_gemm_amd import synth
    layer = synth.WORKLOADS["decode-11008x4096"].layers[0]
    W = layer.W()
    rng = np.random.default_rng(11)
    Xcal = rng.standard_normal((64, layer.K)).astype(np.float16)
    Xcal[:, rng.choice(layer.K, 4, replace=False)] *= 50
    h = ob.hessian_diag(Xcal)
    print("[block pack] decode-11008x4096 beta=0.1", flush=True)
    p, got, base, ref = _pack_both(mq, W, layer.group, 0.1, h)
    assert p.nblk == 2201
    _assert_blocks_equal(got, base, ref)
    # the handle holds the base and the blocks as code tiles, nothing else of
    # the residual: within 1.12 x the device bytes of the plain 4-bit handle
    plain = mq.mq_pack(to_dev(W), layer.group, 0.0)
    ratio = p.device_bytes / plain.device_bytes
    print(f"[block bytes] {p.device_bytes} vs plain {plain.device_bytes}: {ratio:.4f}", flush=True)
    assert ratio <= 1.12, ratio
    plain.free()
    Wt = ob.dequant_blocks(ref)
    for M in (1, 16):
        X = layer.X(M)
        print(f"[block linear] decode-11008x4096 M={M}", flush=True)
        Y = mq.mq_linear(to_dev(X), p).cpu().numpy()
        check_linear(Y, X, Wt, f"decode layer blocks M={M}")


def test_block_handle_errors(mq):
    import torch
    W = _layer(32, 256, 1)
    h = _h(256, 2)
    hbad = h.copy()
    hbad[7] = -1.0
    with pytest.raises(mq.MQError) as ei:
        mq.mq_pack_blocks(to_dev(W), 128, 0.5, to_dev(hbad))
    assert ei.value.code == -1
    hnan = h.copy()
    hnan[3] = np.nan
    with pytest.raises(mq.MQError):
        mq.mq_pack_blocks(to_dev(W), 128, 0.5, to_dev(hnan))
    p = mq.mq_pack_blocks(to_dev(W), 128, 0.5, to_dev(h))
    X = torch.zeros((2, 256), dtype=torch.float16, device="cuda")
    Y = torch.zeros((2, 32), dtype=torch.float16, device="cuda")
    assert mq.lib.mq_residual_add(X.data_ptr(), 2, p.handle, Y.data_ptr(), None) == -2
    rp = torch.zeros(33, dtype=torch.int32, device="cuda")
    assert mq.lib.mq_export_canonical(p.handle, None, None, ctypes.c_void_p(rp.data_ptr()), None, None, None,
                                      None) == -2
    # no element-wise residual stream in a block handle
    assert mq.lib.mq_export_tiled(p.handle, None, ctypes.c_void_p(rp.data_ptr()), None, None) == -2
    q = mq.mq_pack(to_dev(W), 128, 0.01)
    assert mq.lib.mq_export_blocks(q.handle, None, None, None, None) == -2
    n = ctypes.c_int64()
    assert mq.lib.mq_block_count(q.handle, ctypes.byref(n)) == 0 and n.value == -1


@pytest.mark.parametrize("M", [4, 16, 64, 300])
def test_block_handles_in_graph_replays(mq, M):
    """The block-residual kernels captured in a graph give the eager result on
    every replay (other work and synchronisations between the replays)."""
    import torch
    N, K = 512, 4096
    W = _layer(N, K, 21)
    p = mq.mq_pack_blocks(to_dev(W), 128, 0.1, to_dev(_h(K, 22)))
    Xd = to_dev(np.random.default_rng(M).standard_normal((M, K)).astype(np.float16))
    ref = mq.mq_linear(Xd, p).cpu().numpy()
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mq.mq_linear(Xd, p, Y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.mq_linear(Xd, p, Y)
    for rep in range(3):
        Y.fill_(0.5)
        other = mq.mq_linear(Xd, p)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[block graph] M={M} replay={rep}", flush=True)
        assert np.array_equal(Y.cpu().numpy().view(np.uint16), ref.view(np.uint16))
        assert np.array_equal(other.cpu().numpy().view(np.uint16), ref.view(np.uint16))


@pytest.mark.timeout(600)
def test_prefill_layer_blocks_sampled(mq):
    # the 28672 x 8192 layer with 10 % of its blocks, GEMM at M = 512 on sampled outputs
    from bit_gemm_amd import synth
    from tests.test_gpu_fullsize import _sampled_check
    layer = synth.WORKLOADS["prefill-28672x8192"].layers[0]
    W = layer.W()
    h = ob.hessian_diag(layer.calibration(128, 4))
    print("[block pack] prefill-28672x8192 beta=0.1", flush=True)
    p = mq.mq_pack_blocks(to_dev(W), layer.group, 0.1, to_dev(h))
    got = mq.export_blocks(p)
    ref = ob.pack_blocks(W, layer.group, 0.1, h)
    del W
    assert np.array_equal(got["blk"], ref["blk"])
    assert np.array_equal(got["rcodes"], ref["rcodes"])
    Wt = ob.dequant_blocks(ref)
    del ref
    print("[block linear] prefill-28672x8192 M=512", flush=True)
    _sampled_check(mq, p, layer.X(512), Wt, mq.KERNEL_GEMM, "prefill blocks M=512", seed=512)
    p.free()
