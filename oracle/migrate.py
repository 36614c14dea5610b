"""Plain CPU oracle for moving activation outliers into the weights before packing.

TEST INFRASTRUCTURE ONLY, like mosaic.py: only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may use it. It shares no code with
the HIP library.

Source: MosaicQuant explainer (gist.science), Technical Summary, Methodology
section 1 "Inlier-Outlier Disaggregation" [MQ-M1]: before the decomposition
the activation outliers are migrated into the weight matrix with an
equivalent transformation (SmoothQuant or QuaRot are named), and the
migrated matrix W^ is what is split into base and residual.

Readings taken where the pages are silent:
  * the SmoothQuant form with migration strength 1/2: input channel j is
    scaled by s_j ~ sqrt(max|X_j| / max|W_j|), W^_:j = W_:j s_j and
    X^_:j = X_:j / s_j, so X^ W^^T = X W^T;
  * s_j is a power of two, 2^e_j, so both scalings are exact in fp16 except
    where a value falls below the normal range (then one round-half-even
    rounding): e_j = floor((E_x - E_w) / 2) with E = floor(log2(max)) taken
    from the floating-point exponent (integer arithmetic only); e_j = 0 for
    a channel whose two maxima are not both positive; e_j is clamped so that
    neither max|W^_j| nor max|X^_j| can exceed the fp16 range (exponent
    <= 15), and to [-24, 24];
  * max|X_j| comes from calibration activations and is supplied by the
    caller (float32, >= 0); max|W_j| is taken from W itself.
"""
from __future__ import annotations

import numpy as np

E_CLAMP = 24
FP16_MAX_EXP = 15   # 2^15 <= 65504 < 2^16


def floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for a > 0 from the exponent of the float (exact); 0 elsewhere."""
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(a)          # a = m 2^ex, 0.5 <= m < 1
    return np.where(a > 0, ex - 1, 0).astype(np.int64)


def smooth_exponents(W16: np.ndarray, amax_x32: np.ndarray) -> np.ndarray:
    """[MQ-M1 outlier migration, SmoothQuant with strength 1/2] e_j per input
    channel (int32 [K]) as described in the module docstring."""
    aw = np.abs(np.asarray(W16).astype(np.float64)).max(axis=0)
    ax = np.asarray(amax_x32, dtype=np.float32).astype(np.float64)
    Ew, Ex = floor_log2(aw), floor_log2(ax)
    live = (aw > 0) & (ax > 0)
    e = np.floor_divide(Ex - Ew, 2)
    hi = np.minimum(FP16_MAX_EXP - Ew, E_CLAMP)       # max|W^_j| < 2^16
    lo = np.maximum(Ex - FP16_MAX_EXP, -E_CLAMP)      # max|X^_j| < 2^16
    e = np.minimum(np.maximum(e, lo), hi)
    return np.where(live, e, 0).astype(np.int32)


def scale_columns(A16: np.ndarray, e: np.ndarray) -> np.ndarray:
    """fp16_RNE(A_ij * 2^e_j) (exact unless the result is fp16-subnormal)."""
    A = np.asarray(A16).astype(np.float64)
    return (A * np.exp2(np.asarray(e, dtype=np.float64))[None, :]).astype(np.float16)


def migrate(W16: np.ndarray, amax_x32: np.ndarray):
    """Returns (W^ fp16 [N, K], e int32 [K]): W^_:j = W_:j 2^e_j."""
    e = smooth_exponents(W16, amax_x32)
    return scale_columns(W16, e), e


def smooth_activations(X16: np.ndarray, e: np.ndarray) -> np.ndarray:
    """X^_:j = X_:j 2^-e_j, the activations that go with W^."""
    return scale_columns(X16, -np.asarray(e, dtype=np.int64))
