"""Helpers of the GPU parity tests: run the HIP path through the C ABI binding
and compare with the CPU oracle (expected values come only from oracle/)."""
import numpy as np

import oracle


def require_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X; none is visible"
    from bit_gemm_amd import mosaicq   # raises if the HIP library is missing
    return mosaicq


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_canonical(mq, W16, G, rho):
    p = mq.mq_pack(to_dev(W16), G, rho)
    c = mq.mq_export_canonical(p)
    return p, {k: v.cpu().numpy() for k, v in c.items()}


def assert_canonical_equal(got: dict, ref: dict):
    """Bit-exact comparison of the canonical packed arrays."""
    assert np.array_equal(got["codes"], ref["codes"]), "base codes differ"
    assert np.array_equal(got["scales"].view(np.uint16), ref["scales"].view(np.uint16)), "scales differ"
    assert np.array_equal(got["row_ptr"], ref["row_ptr"]), "row_ptr differs"
    assert np.array_equal(got["col"].view(np.uint16), ref["col"]), "residual columns differ"
    assert np.array_equal(got["rcodes"], ref["rcodes"]), "residual codes differ"
    assert np.array_equal(got["rscale"].view(np.uint32), ref["rscale"].view(np.uint32)), "residual scales differ"


def check_linear(Y_gpu, X16, Wt, what=""):
    """Per-output tolerance |Y - Y64| <= 2e-3 * sum|x||w~| + 1e-5 against the
    float64 oracle on the identical dequantised weights."""
    Y64, B = oracle.linear(X16, Wt)
    Y = Y_gpu.astype(np.float64)
    ok = oracle.within_tolerance(Y, Y64, B)
    if not ok.all():
        bad = np.argwhere(~ok)
        m, n = bad[0]
        raise AssertionError(f"{what}: {bad.shape[0]} of {ok.size} outputs out of tolerance; first "
                             f"[{m},{n}] gpu={Y[m, n]!r} ref={Y64[m, n]!r} bound={2e-3 * B[m, n] + 1e-5!r}")
    return np.max(np.abs(Y - Y64) / (B + 1e-30))
