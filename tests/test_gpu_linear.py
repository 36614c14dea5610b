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


def test_linear_k65536_with_residual_in_every_window(mq):
    """K = 65536: the residual stream's columns are stored mod 4096, so each
    of the 16 column windows of a row block has its own segment; residual in
    every window, both kernels, decode and GEMM batch sizes."""
    N, K, G, rho = 40, 65536, 64, 0.004
    W = _layer(N, K, seed=65536, outlier_cols=3)
    p = mq.mq_pack(to_dev(W), G, rho)
    ref = oracle.pack(W, G, rho)
    assert np.unique(ref["col"].astype(np.int64) // 4096).size == 16, "every window holds residual entries"
    Wt = oracle.dequant(ref)
    for M in (1, 5, 16, 17, 64):
        X = _x(M, K, seed=7 + M)
        for kern in (mq.KERNEL_GEMV, mq.KERNEL_GEMM):
            print(f"[linear parity] K=65536 rho={rho} M={M} kernel={kern}", flush=True)
            Y = mq.mq_linear_with(to_dev(X), p, kern).cpu().numpy()
            check_linear(Y, X, Wt, f"K=65536 M={M} kernel={kern}")


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
# several-row-blocks-per-workgroup kernel (1, 2, 3 or 4 row blocks, the last
# workgroup partly past the end), ragged N, no residual, and residual
# densities whose chunks overflow the two prefetched per wave
K4096 = [(40, 128, 0.3), (16, 128, 0.0), (4100, 64, 0.01), (8210, 32, 0.002), (1000, 128, 0.02),
         (11008, 128, 0.005), (14336, 128, 0.005), (12300, 64, 0.01)]


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


def _longest_segment(ref, N, K):
    """Entries in the longest (row block, code tile) segment of the patch
    stream, from the oracle's CSR: per-tile counts, each row block padded to
    whole 32-entry chunks in its last tile."""
    rp, col = ref["row_ptr"].astype(np.int64), ref["col"].astype(np.int64)
    Nb, Kt = -(-N // 16), -(-K // 128)
    rows = np.repeat(np.arange(N), np.diff(rp))
    cnt = np.bincount((rows // 16) * Kt + col // 128, minlength=Nb * Kt).reshape(Nb, Kt)
    cnt[:, -1] += (-cnt.sum(1)) % 32
    return int(cnt.max())


def _longest_row_block(ref, N):
    """Entries in the longest row-block segment of the residual stream (each
    row block padded to whole 32-entry chunks), from the oracle's CSR."""
    rp = ref["row_ptr"].astype(np.int64)
    Nb = -(-N // 16)
    per_row = np.zeros(Nb * 16, dtype=np.int64)
    per_row[:N] = np.diff(rp)
    blk = per_row.reshape(Nb, 16).sum(1)
    return int((blk + (-blk) % 32).max())


@pytest.mark.parametrize("N,G", [(17000, 128), (17000, 64), (22016, 128)])
def test_decode_wide_layers(mq, N, G):
    """Layers of more than 16384 rows at K = 4096 and 5..16 tokens: the decode
    kernel takes 5 (G = 128) or 3 (G = 64) row blocks per workgroup on 1063
    row blocks (the last workgroup part-filled, the last row block ragged),
    and 3 on 1376 (two rounds of workgroups), from its rounds model."""
    K, rho = 4096, 0.005
    rng = np.random.default_rng(N + G)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, 8, replace=False)] *= 20
    W = W.astype(np.float16)
    ref = oracle.pack(W, G, rho)
    p = mq.mq_pack(to_dev(W), G, rho)
    Wt = oracle.dequant(ref)
    for M in (5, 16):
        X = _x(M, K, seed=300 + M)
        print(f"[wide decode] N={N} G={G} M={M}", flush=True)
        Y = mq.mq_linear(to_dev(X), p).cpu().numpy()
        check_linear(Y, X, Wt, f"wide decode N={N} G={G} M={M}")
    p.free()


@pytest.mark.parametrize("N,rows,nnz,staged",
                         [(64, (20,), 2400, 64), (64, (20, 40, 41, 42), 16000, 256), (1088, (), 68 * 3277, 256)])
def test_decode_dense_row_blocks(mq, N, rows, nnz, staged):
    """Outliers in whole rows make a few row blocks far denser than the rest;
    the up-to-4-token decode kernel then copies a row block's chunks past the
    16 it holds in registers into LDS, 64 or 256 of them sized to the densest
    row block, takes any further ones through registers again, and starts the
    dense row blocks first when there are at most 64 of them. The densities
    put the densest row block at 75 and 364 chunks; the last case makes all
    68 row blocks dense (about 100 chunks each), too many to list."""
    K, G = 4096, 128
    rng = np.random.default_rng(61)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[list(rows)] *= 20
    W = W.astype(np.float16)
    rho = nnz / (N * K)   # exact: a multiple of 2^-16
    ref = oracle.pack(W, G, rho)
    chunks = _longest_row_block(ref, N) // 32
    assert chunks > 16 and (16 + 64 >= chunks) == (staged == 64), chunks
    assert staged == 64 or chunks > 16 + 256 or not rows, chunks
    p = mq.mq_pack(to_dev(W), G, rho)
    assert p.nnz == nnz
    Wt = oracle.dequant(ref)
    for M in (1, 2, 3, 4, 16):
        X = _x(M, K, seed=200 + M)
        print(f"[dense row blocks] N={N} chunks={chunks} M={M}", flush=True)
        Y = mq.mq_linear_with(to_dev(X), p, mq.KERNEL_GEMV).cpu().numpy()
        check_linear(Y, X, Wt, f"dense row block {chunks} chunks M={M}")
        Y2 = mq.mq_linear_with(to_dev(X), p, mq.KERNEL_GEMV).cpu().numpy()
        assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16))


@pytest.mark.parametrize("nnz,bucket", [(200, 1), (440, 2), (640, 3), (1100, 4)])
def test_mid_kernel_patch_segment_lengths(mq, nnz, bucket):
    """The mid-size kernel applies a tile's element-wise patches branch-free
    when no segment exceeds 64, 128 or 192 entries (1, 2 or 3 per lane) and in
    a loop of 64-entry rounds beyond. Outliers in 16 columns of one code tile
    inflate its group scales, so most selected entries fall in that tile; the
    densities put the longest segment (56, 120, 165, 283 entries) in each
    case."""
    N, K, G = 64, 1024, 128
    rng = np.random.default_rng(16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, 256 + np.arange(16) * 5] *= 40
    W = W.astype(np.float16)
    rho = nnz / (N * K)   # exact: N K is a power of two
    ref = oracle.pack(W, G, rho)
    seg = _longest_segment(ref, N, K)
    assert min(-(-seg // 64), 4) == bucket, seg
    p = mq.mq_pack(to_dev(W), G, rho)
    assert p.nnz == nnz
    Wt = oracle.dequant(ref)
    for M in (5, 16, 33, 64):
        X = _x(M, K, seed=100 + M)
        print(f"[mid patch segments] longest={seg} M={M}", flush=True)
        Y = mq.mq_linear_with(to_dev(X), p, mq.KERNEL_GEMM).cpu().numpy()
        check_linear(Y, X, Wt, f"longest segment {seg} M={M}")


def test_automatic_choice_follows_the_documented_rule(mq):
    """mq_linear picks the GEMV kernels up to 16 tokens when K <= 4096 and up
    to 3 tokens for larger K, else the GEMM path: its output is bit-identical
    to that kernel's, and within the oracle bound."""
    for N, K, G, rho in ((300, 4096, 128, 0.01), (260, 8320, 64, 0.01), (40, 640, 32, 0.05)):
        W = _layer(N, K, seed=K + 1)
        p = mq.mq_pack(to_dev(W), G, rho)
        Wt = oracle.dequant(oracle.pack(W, G, rho))
        for M in (1, 3, 4, 8, 16, 17, 64, 65):
            X = _x(M, K, seed=M + 11)
            Xd = to_dev(X)
            want = mq.KERNEL_GEMV if M <= (16 if K <= 4096 else 3) else mq.KERNEL_GEMM
            print(f"[auto] N={N} K={K} M={M} expect kernel={want}", flush=True)
            Ya = mq.mq_linear(Xd, p).cpu().numpy()
            Yk = mq.mq_linear_with(Xd, p, want).cpu().numpy()
            assert np.array_equal(Ya.view(np.uint16), Yk.view(np.uint16)), (N, K, M)
            check_linear(Ya, X, Wt, f"auto N={N} K={K} M={M}")


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


def test_free_during_graph_capture_is_deferred(mq):
    """Releasing a handle while the stream is being captured (as the garbage
    collector may do) must not free device memory then, which would
    invalidate the capture: the binding defers it to the next release."""
    import torch
    K, N, G = 4096, 64, 128
    keep = mq.mq_pack(to_dev(_layer(N, K, seed=5)), G, 0.01)
    gone = mq.mq_pack(to_dev(_layer(N, K, seed=6)), G, 0.01)
    X = to_dev(_x(4, K, seed=7))
    Y = torch.empty((4, N), dtype=torch.float16, device="cuda")
    eager = mq.mq_linear(X, keep).cpu().numpy()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.mq_linear(X, keep, Y, stream=torch.cuda.current_stream())
        gone.free()
    assert len(mq._deferred) == 1
    for _ in range(3):
        Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().view(np.uint16), eager.view(np.uint16))
    keep.free()   # outside the capture: frees the deferred handle too
    assert not mq._deferred
