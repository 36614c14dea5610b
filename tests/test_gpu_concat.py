"""mq_concat: several separately packed layers that read the same input as one
handle, their rows stacked. The canonical export of the result must be the
parts' canonical arrays joined row-wise (bit-exact, residual entries
renumbered), and its linear must match the float64 oracle of the stacked
dequantised weights on every kernel."""
import ctypes

import numpy as np
import pytest

import oracle
from tests.gpu_util import check_linear, require_gpu, to_dev

pytestmark = pytest.mark.gpu
INVALID_ARG, UNSUPPORTED = -1, -2   # mq_status codes of include/mosaicq.h


@pytest.fixture(scope="module")
def mq():
    return require_gpu()


def _layer(N, K, seed, rows=()):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, 3, replace=False)] *= 20
    W[list(rows)] *= 20   # whole outlier rows: a few dense row blocks
    return W.astype(np.float16)


def _joined_reference(refs):
    """The parts' canonical arrays joined row-wise (host numpy only)."""
    codes = np.concatenate([r["codes"] for r in refs])
    scales = np.concatenate([r["scales"] for r in refs])
    rp, off = [np.zeros(1, np.int64)], 0
    for r in refs:
        rp.append(r["row_ptr"][1:].astype(np.int64) + off)
        off += int(r["row_ptr"][-1])
    col = np.concatenate([r["col"] for r in refs])
    rscale = np.concatenate([r["rscale"] for r in refs])
    return codes, scales, np.concatenate(rp), col, rscale


def _unpack_nibbles(b, n):
    u = np.empty(2 * b.size, np.uint8)
    u[0::2], u[1::2] = b & 0xF, b >> 4
    return u[:n]


# (rows, residual density, outlier rows) of each part, K = 4096 (the decode
# kernels): odd residual counts shift the nibble position of the next part's
# residual codes; one part has no residual; the third has dense row blocks
# (whole outlier rows), which the joined handle lists shifted by the rows and
# residual entries before it; the last is ragged
PARTS_K4096 = [(1024, 0.00501, ()), (512, 0.0, ()), (512, 0.0031, (5, 6, 7, 40)), (520, 0.01, ())]


def test_concat_export_is_the_parts_joined(mq):
    K, G = 4096, 128
    Ws = [_layer(N, K, seed=7 + i, rows=rows) for i, (N, _, rows) in enumerate(PARTS_K4096)]
    ps = [mq.mq_pack(to_dev(W), G, rho) for W, (_, rho, _) in zip(Ws, PARTS_K4096)]
    assert sum(p.nnz % 2 for p in ps) >= 1, "an odd residual count shifts the following codes"
    c = mq.mq_concat(ps)
    got = {k: v.cpu().numpy() for k, v in mq.mq_export_canonical(c).items()}
    parts = [{k: v.cpu().numpy() for k, v in mq.mq_export_canonical(p).items()} for p in ps]
    codes, scales, row_ptr, col, rscale = _joined_reference(parts)
    assert c.N == sum(p.N for p in ps) and c.nnz == sum(p.nnz for p in ps)
    assert np.array_equal(got["codes"], codes)
    assert np.array_equal(got["scales"].view(np.uint16), scales.view(np.uint16))
    assert np.array_equal(got["row_ptr"].astype(np.int64), row_ptr)
    assert np.array_equal(got["col"].view(np.uint16), col.view(np.uint16))
    want_u = np.concatenate([_unpack_nibbles(pp["rcodes"], p.nnz) for pp, p in zip(parts, ps)])
    assert np.array_equal(_unpack_nibbles(got["rcodes"], c.nnz), want_u)
    assert np.array_equal(got["rscale"].view(np.uint32), rscale.view(np.uint32))
    # and the parts are the oracle's packs of their layers
    for W, (N, rho, _), pp in zip(Ws, PARTS_K4096, parts):
        ref = oracle.pack(W, G, rho)
        assert np.array_equal(pp["codes"], ref["codes"]) and np.array_equal(pp["col"].view(np.uint16), ref["col"])
    for p in ps:
        p.free()
    c.free()


@pytest.mark.parametrize("K,G,parts", [(4096, 128, PARTS_K4096),
                                       (1024, 64, [(256, 0.02, ()), (48, 0.013, (3,)), (100, 0.0, ())]),
                                       (8320, 32, [(64, 0.004, ()), (80, 0.007, ())])])
def test_concat_linear_matches_the_oracle(mq, K, G, parts):
    Ws = [_layer(N, K, seed=31 + i, rows=rows) for i, (N, _, rows) in enumerate(parts)]
    ps = [mq.mq_pack(to_dev(W), G, rho) for W, (_, rho, _) in zip(Ws, parts)]
    c = mq.mq_concat(ps)
    for p in ps:   # the result owns its memory
        p.free()
    Wt = np.concatenate([oracle.dequant(oracle.pack(W, G, rho)) for W, (_, rho, _) in zip(Ws, parts)])
    for M in (1, 4, 16, 40, 100):
        X = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
        kernels = [mq.KERNEL_GEMM] + ([mq.KERNEL_GEMV] if M <= mq.GEMV_MAX_M else [])
        for kern in kernels:
            print(f"[concat linear] K={K} G={G} M={M} kernel={kern}", flush=True)
            Y = mq.mq_linear_with(to_dev(X), c, kern).cpu().numpy()
            check_linear(Y, X, Wt, f"concat K={K} M={M} kernel={kern}")
    c.free()


def test_concat_errors(mq):
    import torch
    W = torch.from_numpy(_layer(40, 256, 3)).cuda()
    a = mq.mq_pack(W, 128, 0.01)          # 40 rows: not whole row blocks
    b = mq.mq_pack(W[:32].contiguous(), 128, 0.01)
    d = mq.mq_pack(torch.from_numpy(_layer(32, 512, 4)).cuda(), 128, 0.01)
    h = torch.ones(256, dtype=torch.float32, device="cuda")
    blk = mq.mq_pack_blocks(W[:32].contiguous(), 128, 0.5, h)

    def status(*parts):
        arr = (ctypes.c_void_p * len(parts))(*[p.handle for p in parts])
        out = ctypes.c_void_p()
        return mq.lib.mq_concat(arr, len(parts), None, ctypes.byref(out)), out

    assert status(a, b)[0] == INVALID_ARG     # ragged part before the last
    assert status(b, d)[0] == INVALID_ARG     # K differs
    assert status(b, blk)[0] == UNSUPPORTED   # block residual
    rc, out = status(b, a)                    # a ragged last part is fine
    assert rc == mq.MQ_OK
    mq.lib.mq_free(out)
    one = mq.mq_concat([a])                     # one part: a copy of it
    g1 = {k: v.cpu().numpy() for k, v in mq.mq_export_canonical(one).items()}
    g0 = {k: v.cpu().numpy() for k, v in mq.mq_export_canonical(a).items()}
    assert all(np.array_equal(g1[k], g0[k]) for k in g0)
    one.free()
    for p in (a, b, d, blk):
        p.free()
