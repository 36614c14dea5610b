"""Plain CPU oracle for the 4-bit-activation (W4A4) form of the fused linear.

TEST INFRASTRUCTURE ONLY, like mosaic.py: only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may use it. It shares no code with
the HIP library.

Sources:
  [MQ-R]  MosaicQuant explainer (gist.science), Experimental Results, Accuracy:
          the method is evaluated with both weights and activations in 4 bits.
  [MQ-M3] same page, Methodology section 3 (ZipperEngine): quantization is one
          of the stages of the overlapped pipeline, next to the dense compute,
          the sparse compensation and the reduction-add.

The pages do not say how activations are quantized. Readings taken:
  * the same symmetric absmax quantizer as the base weights, per token and per
    group of G consecutive input columns (G is the weight handle's group
    size): sx[m, g] = fp16_RNE(max_{j in g} |x_mj| / 7),
    qx = clamp(rint(x / sx), -7, 7), qx = 0 where sx == 0;
  * the layer then computes Y = X^ W~^T with X^ = sx * qx and W~ the
    dequantized weight (base plus residual); here exactly, in float64.
"""
from __future__ import annotations

import numpy as np

from .mosaic import base_codes, base_scales, OracleInputError, SUPPORTED_GROUPS


def quantize_activations(X16: np.ndarray, G: int):
    """[MQ-R, MQ-M3 quantization stage] (qx int8 [M, K], sx float16 [M, K/G]):
    the base weight quantizer (O1, O2) applied to the rows of X."""
    X16 = np.asarray(X16)
    if X16.dtype != np.float16 or X16.ndim != 2:
        raise OracleInputError("X must be a 2-D float16 array")
    M, K = X16.shape
    if G not in SUPPORTED_GROUPS or K % G != 0:
        raise OracleInputError("need G in (32, 64, 128) and K % G == 0")
    if not np.all(np.isfinite(X16)):
        raise OracleInputError("X has non-finite entries")
    sx = base_scales(X16, G)
    return base_codes(X16, sx, G), sx


def dequant_activations(qx: np.ndarray, sx: np.ndarray, G: int) -> np.ndarray:
    """X^ = sx * qx in float64 [M, K] (exact: at most 14 significant bits)."""
    return np.repeat(np.asarray(sx).astype(np.float64), G, axis=1) * np.asarray(qx).astype(np.float64)


def code_sums(qx: np.ndarray, G: int) -> np.ndarray:
    """Sum of the codes of each (token, group), int32 [M, K/G]."""
    M, K = qx.shape
    return qx.astype(np.int32).reshape(M, K // G, G).sum(axis=2).astype(np.int32)


def linear_a4(X16: np.ndarray, Wt: np.ndarray, G: int):
    """[MQ-M3] Y = X^ W~^T in float64 with X^ the 4-bit activations, and the
    error scale B = |X^| |W~|^T. Returns (Y64 [M, N], B [M, N])."""
    qx, sx = quantize_activations(X16, G)
    Xh = dequant_activations(qx, sx, G)
    return Xh @ Wt.T, np.abs(Xh) @ np.abs(Wt).T
