"""mq_linear_group: several layers, each with its own input, in one call. Every
output must equal that layer's own mq_linear bit for bit, whether the layers
share one launch (K = 4096, 1..16 tokens, one group size, no block residual;
from 5 tokens on 1 to 5 row blocks per workgroup, by the group's rows and
group size; up to 4 tokens one row block per workgroup, for layers whose row
blocks hold at most 80 residual chunks, staging those past 16 in LDS when
any layer has such a row block) or fall back to launches of their own; one small group is also checked against the float64 oracle of the
dequantised weights."""
import ctypes

import numpy as np
import pytest

import oracle
from tests.gpu_util import check_linear, require_gpu, to_dev

pytestmark = pytest.mark.gpu
INVALID_ARG, BAD_HANDLE = -1, -6   # mq_status codes of include/mosaicq.h


@pytest.fixture(scope="module")
def mq():
    return require_gpu()


def _layer(N, K, seed, rows=()):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, 3, replace=False)] *= 20
    W[list(rows)] *= 20   # whole outlier rows: long residual segments
    return W.astype(np.float16)


def _packs(mq, spec, K, G, seed):
    """spec: (rows, residual density, outlier rows) per layer."""
    Ws = [_layer(N, K, seed + i, rows) for i, (N, _, rows) in enumerate(spec)]
    return Ws, [mq.mq_pack(to_dev(W), G, rho) for W, (_, rho, _) in zip(Ws, spec)]


def _inputs(M, Ks, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((M, K)).astype(np.float16) for K in Ks]


def _check_equal_to_single(mq, packs, Xs_host, what):
    import torch
    Xs = [to_dev(x) for x in Xs_host]
    print(f"[group] {what}: N={[p.N for p in packs]} K={[p.K for p in packs]} M={Xs_host[0].shape[0]}", flush=True)
    Ys = mq.mq_linear_group(Xs, packs)
    torch.cuda.synchronize()
    for i, (X, p, Y) in enumerate(zip(Xs, packs, Ys)):
        want = mq.mq_linear(X, p).cpu().numpy()
        got = Y.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"{what}: layer {i} differs from mq_linear"
    return Ys


# the seven linears of a 4096-hidden block but the down projection (K = 11008):
# 2400 row blocks, five per workgroup (two rounds of 240 workgroups); one
# layer without residual, one with dense outlier rows
BLOCK = [(4096, 0.005, ()), (4096, 0.005, ()), (4096, 0.0, ()), (4096, 0.005, (7, 8, 100)),
         (11008, 0.005, ()), (11008, 0.005, ())]


def _densest_row_block_chunks(mq, p):
    """Residual chunks (32 entries, each row block padded) of the densest row
    block of a handle, from its canonical CSR."""
    rp = mq.mq_export_canonical(p)["row_ptr"].cpu().numpy().astype(np.int64)
    per_row = np.zeros(-(-p.N // 16) * 16, dtype=np.int64)
    per_row[:p.N] = np.diff(rp)
    blk = per_row.reshape(-1, 16).sum(1)
    return int(((blk + 31) // 32).max())


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 16])
def test_block_group_equals_single_launches(mq, M):
    """The block's layers as above (the one with outlier rows has row blocks
    of more than 80 residual chunks, so up to 4 tokens it takes a launch of
    its own after the others' shared one), and at a residual density of
    0.2 % without the outlier rows (at most 16 chunks per row block: one
    launch at any M, nothing staged)."""
    for spec, what in ((BLOCK, "block"), ([(N, 0.002, ()) for N, _, _ in BLOCK], "block, rho 0.2 %")):
        _, ps = _packs(mq, spec, 4096, 128, seed=11)
        dense = max(_densest_row_block_chunks(mq, p) for p in ps)
        assert (dense > 80) == (spec is BLOCK) and (dense <= 16) == (spec is not BLOCK), dense
        _check_equal_to_single(mq, ps, _inputs(M, [4096] * len(ps), seed=M), what)
        for p in ps:
            p.free()


# (spec, group size) and the row blocks per workgroup the launcher picks:
# 194 row blocks (1; ragged layers), 319 (2), 831 at G = 64 (4) and at
# G = 32 (2, the most that G = 32 takes), one layer of 688 row blocks (3)
FOUR = [(4096, 0.005, ()), (4096, 0.003, ()), (4096, 0.0, ()), (1000, 0.01, (999,))]


@pytest.mark.parametrize("spec,G", [
    ([(2048, 0.01, ()), (1000, 0.004, (3,)), (40, 0.02, ())], 128),
    ([(4096, 0.005, ()), (1000, 0.0, ())], 64),
    (FOUR, 64),
    (FOUR, 32),
    ([(11008, 0.005, (11000,))], 128),
])
@pytest.mark.parametrize("M", [2, 6, 13])
def test_group_shapes_equal_single_launches(mq, spec, G, M):
    _, ps = _packs(mq, spec, 4096, G, seed=23)
    _check_equal_to_single(mq, ps, _inputs(M, [4096] * len(ps), seed=100 + M), f"G={G}")
    for p in ps:
        p.free()


@pytest.mark.parametrize("M", [1, 2, 4])
def test_small_batch_group_with_staged_chunks(mq, M):
    """Up to 4 tokens, a layer whose densest row block holds 17..80 residual
    chunks makes the shared launch stage the chunks past 16 in LDS; the
    layers with at most 16 per row block stage none there, and every output
    still equals the layer's own launch (which picks its variant alone)."""
    spec = [(4096, 0.006, ()), (2048, 0.002, ()), (1000, 0.0, ()), (520, 0.001, ())]
    _, ps = _packs(mq, spec, 4096, 128, seed=51)
    chunks = [_densest_row_block_chunks(mq, p) for p in ps]
    assert 16 < chunks[0] <= 80 and max(chunks[1:]) <= 16, chunks
    _check_equal_to_single(mq, ps, _inputs(M, [4096] * len(ps), seed=70 + M), "staged")
    for p in ps:
        p.free()


@pytest.mark.parametrize("M", [1, 16])
def test_group_matches_the_oracle(mq, M):
    spec = [(1000, 0.002, ()), (272, 0.001, ()), (40, 0.0, ())]   # at most 16 chunks per row block
    Ws, ps = _packs(mq, spec, 4096, 128, seed=41)
    assert max(_densest_row_block_chunks(mq, p) for p in ps) <= 16   # one launch at M = 1 too
    Xs = _inputs(M, [4096] * 3, seed=5)
    Ys = _check_equal_to_single(mq, ps, Xs, "oracle")
    for W, (N, rho, _), X, Y in zip(Ws, spec, Xs, Ys):
        Wt = oracle.dequant(oracle.pack(W, 128, rho))
        check_linear(Y.cpu().numpy(), X, Wt, f"group N={N} M={M}")
    for p in ps:
        p.free()


def test_more_than_eight_layers_and_a_shared_input(mq):
    spec = [(256 * (i % 4 + 1) + 16 * i, 0.005 * (i % 3), ()) for i in range(11)]
    _, ps = _packs(mq, spec, 4096, 128, seed=61)
    X = _inputs(12, [4096], seed=3)[0]
    _check_equal_to_single(mq, ps, [X] * len(ps), "11 layers, one input")
    for p in ps:
        p.free()


def test_layers_that_cannot_share_a_launch(mq):
    import torch
    # another K, then too many tokens for the grouped kernels
    _, ps = _packs(mq, [(512, 0.01, ()), (300, 0.01, ())], 4096, 128, seed=71)
    _, qs = _packs(mq, [(256, 0.01, ())], 1024, 128, seed=72)
    _check_equal_to_single(mq, ps + qs, _inputs(16, [4096, 4096, 1024], seed=9), "mixed K")
    for M in (20, 64):
        _check_equal_to_single(mq, ps, _inputs(M, [4096, 4096], seed=M), "M above 16")
    # one group size per launch, and a block residual
    _, gs = _packs(mq, [(256, 0.01, ())], 4096, 64, seed=73)
    _check_equal_to_single(mq, ps + gs, _inputs(8, [4096] * 3, seed=4), "two group sizes")
    W = torch.from_numpy(_layer(256, 4096, 74)).cuda()
    blk = mq.mq_pack_blocks(W, 128, 0.1, torch.ones(4096, dtype=torch.float32, device="cuda"))
    _check_equal_to_single(mq, ps + [blk], _inputs(8, [4096] * 3, seed=5), "block residual")
    for p in ps + qs + gs + [blk]:
        p.free()


def test_group_argument_errors(mq):
    import torch
    _, ps = _packs(mq, [(64, 0.01, ()), (64, 0.01, ())], 4096, 128, seed=81)
    X = torch.zeros((8, 4096), dtype=torch.float16, device="cuda")
    Y = torch.zeros((8, 64), dtype=torch.float16, device="cuda")
    xs = (ctypes.c_void_p * 2)(X.data_ptr(), X.data_ptr())
    ys = (ctypes.c_void_p * 2)(Y.data_ptr(), Y.data_ptr() + 2)   # second output misaligned
    hs = (ctypes.c_void_p * 2)(ps[0].handle, ps[1].handle)
    before = Y.clone()
    assert mq.lib.mq_linear_group(xs, 8, hs, ys, 2, None) == INVALID_ARG
    torch.cuda.synchronize()
    assert torch.equal(Y, before), "nothing is launched when an argument is bad"
    ps[1].free()
    ys = (ctypes.c_void_p * 2)(Y.data_ptr(), Y.data_ptr())
    assert mq.lib.mq_linear_group(xs, 8, hs, ys, 2, None) == BAD_HANDLE
    with pytest.raises(ValueError):
        mq.mq_linear_group([X, X[:4].contiguous()], [ps[0], ps[0]])
    ps[0].free()


@pytest.mark.parametrize("M", [1, 16])
def test_group_graph_replay(mq, M):
    import torch
    spec = [(1024, 0.005, ()), (2048, 0.01, ()), (512, 0.0, ())]
    _, ps = _packs(mq, spec, 4096, 128, seed=91)
    Xs = [to_dev(x) for x in _inputs(M, [4096] * 3, seed=2)]
    Ys = [torch.empty((M, p.N), dtype=torch.float16, device="cuda") for p in ps]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mq.mq_linear_group(Xs, ps, Ys, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.mq_linear_group(Xs, ps, Ys, stream=torch.cuda.current_stream())
    rng = np.random.default_rng(17)
    for rep in range(3):
        for X in Xs:   # fresh inputs between replays
            X.copy_(torch.from_numpy(rng.standard_normal(tuple(X.shape)).astype(np.float16)).cuda())
        g.replay()
        torch.cuda.synchronize()
        for i, (X, p, Y) in enumerate(zip(Xs, ps, Ys)):
            want = mq.mq_linear(X, p).cpu().numpy()
            assert np.array_equal(Y.cpu().numpy().view(np.uint16), want.view(np.uint16)), f"replay {rep} layer {i}"
    del g
    for p in ps:
        p.free()
