"""Plain CPU oracle for block-wise residual allocation with a Hessian-guided score.

TEST INFRASTRUCTURE ONLY, like mosaic.py: only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may use it. It shares no code with
the HIP library.

Source: MosaicQuant explainer (gist.science), Technical Summary, Methodology
section 2 "Block-Wise Residual Allocation" [MQ-M2]. The pages state that the
residual budget goes to blocks rather than channels; that a Delta-score,
built from the residual error weighted by the diagonal Hessian estimate of
the input channels, approximates each block's marginal reduction of the
output distortion; that the top-K blocks by that score receive a 4-bit
residual; and that 10 % of the blocks recover more than half of the output
distortion.

Readings taken where the pages are silent (each marked where it is used):
  * distortion of a linear layer on calibration activations X: ||X (W - W~)^T||^2,
    whose diagonal-Hessian estimate is sum_ij h_j (W - W~)_ij^2 with
    h_j = sum_m X_mj^2 (the caller supplies h, float32);
  * a block is BR rows x BC input columns, aligned (16 x 128 here: one code
    tile of the base), partial at the right and bottom edges;
  * the block residual quantises the base error e of every entry of the
    block: per block row, sr = fp32(max |e| / 7), qr = clamp(rint(e / sr), -7, 7)
    with a float64 division (the same quantiser as the element-wise residual,
    scoped to one block row);
  * Delta_b = sum over the block, rows then columns in ascending order, of
    h_j * (r * (2 e - r)) with r = sr * qr, every operation one float64
    rounding and the sum taken left to right from +0.0. This equals
    sum h_j (e^2 - (e - r)^2), the drop in the estimated distortion; the
    order is fixed so that a GPU that follows it reaches the same score bits
    and so the same selection;
  * budget: floor(beta * number of blocks) blocks, ranked by (Delta
    descending, block index rb * Kt + kt ascending).

Arithmetic is float64 (numpy); the base quantiser comes from mosaic.py.
"""
from __future__ import annotations

import numpy as np

from .mosaic import QMAX, base_codes, base_error, base_scales, check_inputs, to_fp32_rne

BLOCK_ROWS = 16
BLOCK_COLS = 128


def hessian_diag(X16: np.ndarray) -> np.ndarray:
    """[MQ-M2, diagonal Hessian estimate of the input channels]: h_j = sum_m x_mj^2
    over calibration activations, summed in float64, rounded once to float32."""
    X = np.asarray(X16).astype(np.float64)
    return to_fp32_rne((X * X).sum(axis=0))


def block_grid(N: int, K: int, br: int = BLOCK_ROWS, bc: int = BLOCK_COLS):
    """Number of block rows and block columns (partial edge blocks included)."""
    return -(-N // br), -(-K // bc)


def _blocked(a: np.ndarray, br: int, bc: int) -> np.ndarray:
    """[N, K] -> [nrb, nkt, br, bc], zero padded past the edges."""
    N, K = a.shape
    nrb, nkt = block_grid(N, K, br, bc)
    p = np.zeros((nrb * br, nkt * bc), dtype=a.dtype)
    p[:N, :K] = a
    return p.reshape(nrb, br, nkt, bc).transpose(0, 2, 1, 3)


def block_residual(e: np.ndarray, br: int = BLOCK_ROWS, bc: int = BLOCK_COLS):
    """Residual of every block [MQ-M1 sparse 4-bit residual, scoped to a block
    row by the reading above]: sr = fp32_RNE(max_{j in block} |e_ij| / 7) per
    block row, qr = clamp(rint(e / sr), -7, 7) (float64 division), 0 where
    sr == 0. Returns (sr float32 [nrb, nkt, br], qr int8 [nrb, nkt, br, bc]);
    rows and columns past the matrix hold qr = 0 and do not enter the max."""
    eb = _blocked(e, br, bc)
    sr = to_fp32_rne(np.abs(eb).max(axis=3) / QMAX)
    s = sr.astype(np.float64)[..., None]
    safe = np.where(s == 0.0, 1.0, s)
    qr = np.clip(np.rint(eb / safe), -QMAX, QMAX)
    qr = np.where(s == 0.0, 0.0, qr)
    return sr, qr.astype(np.int8)


def block_scores(e: np.ndarray, sr: np.ndarray, qr: np.ndarray, h32: np.ndarray,
                 br: int = BLOCK_ROWS, bc: int = BLOCK_COLS) -> np.ndarray:
    """Delta-score of every block [MQ-M2]: the drop of the diagonal-Hessian
    distortion sum h_j (e^2 - (e - r)^2) if the block gets its residual,
    evaluated as h_j * (r * (2 e - r)) per entry and summed left to right over
    the block's rows, then columns (np.cumsum is a sequential running sum).
    Padding entries contribute +0.0. Returns float64 [nrb * nkt], indexed
    rb * nkt + kt."""
    N, K = e.shape
    nrb, nkt = block_grid(N, K, br, bc)
    eb = _blocked(e, br, bc)
    r = sr.astype(np.float64)[..., None] * qr.astype(np.float64)      # exact: 24-bit x 3-bit
    hp = np.zeros(nkt * bc, dtype=np.float64)
    hp[:K] = np.asarray(h32, dtype=np.float32).astype(np.float64)
    hb = hp.reshape(nkt, bc)[None, :, None, :]
    t = hb * (r * (2.0 * eb - r))
    return np.cumsum(t.reshape(nrb * nkt, br * bc), axis=1)[:, -1]


def block_budget(beta: float, nblocks: int) -> int:
    """Number of residual blocks: floor(beta * nblocks) in float64 (like the
    element budget of mosaic.budget)."""
    return min(int(np.floor(np.float64(beta) * np.float64(nblocks))), nblocks)


def select_blocks(delta: np.ndarray, k: int) -> np.ndarray:
    """[MQ-M2 top-K blocks]: the k blocks first in the order (Delta descending,
    index ascending), as ascending indices (int64); threshold form as in
    mosaic.select_topk."""
    n = delta.size
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    if k >= n:
        return np.arange(n, dtype=np.int64)
    T = np.partition(delta, n - k)[n - k]
    above = np.flatnonzero(delta > T)
    ties = np.flatnonzero(delta == T)[: k - above.size]
    return np.sort(np.concatenate([above, ties])).astype(np.int64)


def pack_blocks(W16: np.ndarray, G: int, beta: float, h32: np.ndarray,
                br: int = BLOCK_ROWS, bc: int = BLOCK_COLS) -> dict:
    """The block-wise disaggregation [MQ-M1 Eq. (1) with MQ-M2's allocation].

    Canonical arrays:
      codes  uint8 [N, K/2]        base codes (as mosaic.pack)
      scales fp16  [N, K/G]        base scales
      blk    int32 [nsel]          selected block indices rb * Kt + kt, ascending
      rscale float32 [nsel, br]    residual scale of each block row
      rcodes uint8 [nsel, br, bc/2] residual code u = qr + 8, even column in the
                                    low nibble; rows/columns past the matrix hold 8
    plus the intermediates (s, q, e, sr, qr of every block, delta)."""
    check_inputs(W16, G, 0.0)
    if not (0.0 <= float(beta) <= 1.0):
        raise ValueError("beta must lie in [0, 1]")
    h32 = np.asarray(h32, dtype=np.float32)
    N, K = W16.shape
    if h32.shape != (K,) or not np.all(np.isfinite(h32)) or np.any(h32 < 0):
        raise ValueError("h must be K finite non-negative float32 values")
    s = base_scales(W16, G)
    q = base_codes(W16, s, G)
    e = base_error(W16, s, q, G)
    nrb, nkt = block_grid(N, K, br, bc)
    sr, qr = block_residual(e, br, bc)
    delta = block_scores(e, sr, qr, h32, br, bc)
    blk = select_blocks(delta, block_budget(beta, nrb * nkt))
    u_base = (q.astype(np.int16) + 8).astype(np.uint8)
    srf = sr.reshape(nrb * nkt, br)
    ub = (qr.reshape(nrb * nkt, br, bc).astype(np.int16) + 8).astype(np.uint8)
    return {
        "N": N, "K": K, "G": G, "beta": float(beta), "br": br, "bc": bc, "nkt": nkt,
        "s": s, "q": q, "e": e, "sr": sr, "qr": qr, "delta": delta,
        "codes": (u_base[:, 0::2] | (u_base[:, 1::2] << 4)).astype(np.uint8),
        "scales": s,
        "blk": blk.astype(np.int32),
        "rscale": srf[blk],
        "rcodes": (ub[blk][:, :, 0::2] | (ub[blk][:, :, 1::2] << 4)).astype(np.uint8),
    }


def dequant_blocks(canon: dict) -> np.ndarray:
    """W~ = s*q + sum over the selected blocks of sr * qr, from the canonical
    arrays, in float64. Returns float64 [N, K]."""
    N, K, G, br, bc, nkt = canon["N"], canon["K"], canon["G"], canon["br"], canon["bc"], canon["nkt"]
    codes = np.asarray(canon["codes"], dtype=np.uint8).reshape(N, K // 2)
    u = np.empty((N, K), dtype=np.int16)
    u[:, 0::2] = codes & 0xF
    u[:, 1::2] = codes >> 4
    s = np.repeat(np.asarray(canon["scales"]).astype(np.float64).reshape(N, K // G), G, axis=1)
    Wt = s * (u - 8).astype(np.float64)
    blk = np.asarray(canon["blk"], dtype=np.int64)
    if blk.size:
        rc = np.asarray(canon["rcodes"], dtype=np.uint8).reshape(blk.size, br, bc // 2)
        ur = np.empty((blk.size, br, bc), dtype=np.int16)
        ur[:, :, 0::2] = rc & 0xF
        ur[:, :, 1::2] = rc >> 4
        r = np.asarray(canon["rscale"]).astype(np.float64).reshape(blk.size, br)[:, :, None] * (ur - 8)
        for n, b in enumerate(blk):
            rb, kt = divmod(int(b), nkt)
            i0, j0 = rb * br, kt * bc
            i1, j1 = min(N, i0 + br), min(K, j0 + bc)
            Wt[i0:i1, j0:j1] += r[n, : i1 - i0, : j1 - j0]
    return Wt


def distortion(W16: np.ndarray, Wt: np.ndarray, h32: np.ndarray) -> float:
    """Diagonal-Hessian estimate of the output distortion: sum_ij h_j (W - W~)_ij^2 (float64)."""
    d = np.asarray(W16).astype(np.float64) - Wt
    return float((d * d * np.asarray(h32, dtype=np.float32).astype(np.float64)[None, :]).sum())
