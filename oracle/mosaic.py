"""Plain CPU oracle for the fused "dense 4-bit base + sparse 4-bit residual" linear.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module:
only the test suite, the smoke check and the CPU-baseline leg of the benchmark
use it. It shares no code with the HIP library and imports nothing from it.

Sources (the pages this follows):
  [MQ-M1]  MosaicQuant explainer (gist.science), Technical Summary, Methodology
           section 1 "Inlier-Outlier Disaggregation", Eq. (1): the weight is split
           into a dense 4-bit base Q(W) plus a sparse 4-bit residual R that
           compensates the base's quantisation error.
  [MQ-M2]  same page, Methodology section 2 "Block-Wise Residual Allocation":
           the residual budget goes to the highest-scoring units (top-K).
  [MQ-M3]  same page, Methodology section 3 "ZipperEngine": the residual is
           computed together with the dense 4-bit GEMM; mathematically the layer
           is Y = X (Q(W) + R)^T.
  [MQ-Abs] MosaicQuant arXiv abstract (OpenAlex record): the base quantises the
           full matrix; the residual targets the most error-critical entries.

The pages leave the quantiser's details open. This file takes the readings
listed below (each marked in the function that uses it):
  * base: symmetric round-to-nearest INT4 per (row, group of G input columns),
    scale = fp16(absmax / 7), codes clamped to [-7, 7];
  * the residual's unit is a single entry, ranked by the size of the base error
    |e| (the Hessian-weighted score with an identity Hessian and 1x1 blocks),
    taken globally over the matrix, ties broken by ascending row-major index;
  * budget k = floor(rho * N * K);
  * residual scale per row = fp32(max selected |e| / 7), codes clamped [-7, 7];
  * every rounding is round-half-to-even.

Arithmetic is float64 (numpy). Parity status of each step is stated in the
function's docstring; every step here is pinned by the oracle self-tests.
"""
from __future__ import annotations

import numpy as np

QMAX = 7                       # symmetric 4-bit range used for both components
SUPPORTED_GROUPS = (32, 64, 128)
MAX_K = 65536                  # column index is stored as uint16


class OracleInputError(ValueError):
    pass


# ----------------------------------------------------------------- roundings
def to_fp16_rne(x64: np.ndarray) -> np.ndarray:
    """float64 -> float16, round-half-to-even, overflow to inf.

    numpy converts doubles to halves directly from the double's bits with RNE
    (no intermediate float32), which the self-tests check against exact
    rational rounding for every value this oracle feeds it.
    """
    return np.asarray(x64, dtype=np.float64).astype(np.float16)


def to_fp32_rne(x64: np.ndarray) -> np.ndarray:
    """float64 -> float32, round-half-to-even."""
    return np.asarray(x64, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------- validation
def check_inputs(W16: np.ndarray, G: int, rho: float) -> None:
    if W16.dtype != np.float16 or W16.ndim != 2:
        raise OracleInputError("W must be a 2-D float16 array")
    N, K = W16.shape
    if G not in SUPPORTED_GROUPS:
        raise OracleInputError(f"group size {G} not in {SUPPORTED_GROUPS}")
    if N <= 0 or K <= 0 or K % G != 0:
        raise OracleInputError("need N > 0, K > 0 and K % G == 0")
    if K > MAX_K:
        raise OracleInputError("K must be <= 65536")
    if not (0.0 <= float(rho) <= 1.0):          # also rejects NaN
        raise OracleInputError("rho must lie in [0, 1]")
    if not np.all(np.isfinite(W16)):
        raise OracleInputError("W has non-finite entries")


# ------------------------------------------------------------ O1: base scales
def base_scales(W16: np.ndarray, G: int) -> np.ndarray:
    """O1 [MQ-M1, dense 4-bit base]: s[i, g] = fp16_RNE(max_{j in g} |W_ij| / 7).

    Reading: symmetric absmax quantiser per row and per group of G columns
    along the input dimension, scale held in fp16. Returns float16 [N, K/G].
    """
    N, K = W16.shape
    a = np.abs(W16.astype(np.float64)).reshape(N, K // G, G).max(axis=2)
    return to_fp16_rne(a / QMAX)


# ------------------------------------------------------------- O2: base codes
def base_codes(W16: np.ndarray, s16: np.ndarray, G: int) -> np.ndarray:
    """O2 [MQ-M1]: q = clamp(rint(W / s), -7, 7); q = 0 where s == 0.

    rint is round-half-to-even; the division is float64. Returns int8 [N, K].
    """
    N, K = W16.shape
    w = W16.astype(np.float64).reshape(N, K // G, G)
    s = s16.astype(np.float64)[:, :, None]
    safe = np.where(s == 0.0, 1.0, s)
    q = np.clip(np.rint(w / safe), -QMAX, QMAX)
    q = np.where(s == 0.0, 0.0, q)
    return q.reshape(N, K).astype(np.int8)


# ---------------------------------------------------------- O3: base error
def base_error(W16: np.ndarray, s16: np.ndarray, q: np.ndarray, G: int) -> np.ndarray:
    """O3 [MQ-M1, the error R compensates]: e = W - s*q in float64.

    Exact: s*q has at most 14 significant bits and both W and s*q are
    multiples of 2^-24 below 2^20, so the difference is representable.
    Returns float64 [N, K].
    """
    N, K = W16.shape
    s = np.repeat(s16.astype(np.float64), G, axis=1)
    return W16.astype(np.float64) - s * q.astype(np.float64)


# ------------------------------------------------------------- O4: budget
def budget(rho: float, N: int, K: int) -> int:
    """O4 [MQ-M2, the residual budget]: k = min(floor(rho * N * K), N * K).

    rho * (N*K) is one float64 product (N*K is exact in float64).
    """
    nk = int(N) * int(K)
    return min(int(np.floor(np.float64(rho) * np.float64(nk))), nk)


# ---------------------------------------------------------- O5: selection
def select_topk(e: np.ndarray, k: int) -> np.ndarray:
    """O5 [MQ-M2 top-K; MQ-Abs]: the k entries that come first in the order
    (|e| descending, row-major index ascending).

    Written as the equivalent threshold form: T is the k-th largest |e|;
    every entry with |e| > T is taken, then the entries with |e| == T in
    ascending index order until k are chosen. (A full sort of all N*K keys
    gives the same set and is what the brute-force pin compares against; the
    threshold form needs only a partition, which keeps layers of 10^8
    weights within seconds.) Returns the selected row-major indices,
    ascending (int64).
    """
    flat = np.abs(e).ravel()
    n = flat.size
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    if k >= n:
        return np.arange(n, dtype=np.int64)
    T = np.partition(flat, n - k)[n - k]          # the k-th largest |e|
    above = np.flatnonzero(flat > T)
    ties = np.flatnonzero(flat == T)[: k - above.size]
    return np.sort(np.concatenate([above, ties])).astype(np.int64)


# --------------------------------------------------- O6/O7: residual encode
def residual_scales(e: np.ndarray, sel_idx: np.ndarray) -> np.ndarray:
    """O6 [MQ-M1 sparse 4-bit residual]: sr_i = fp32_RNE(max_{j in S_i} |e_ij| / 7).

    Rows with no selected entry get 0. Returns float32 [N].
    """
    N, K = e.shape
    rows = sel_idx // K
    mx = np.zeros(N, dtype=np.float64)
    if sel_idx.size:
        np.maximum.at(mx, rows, np.abs(e.ravel()[sel_idx]))
    return to_fp32_rne(mx / QMAX)


def residual_codes(e: np.ndarray, sel_idx: np.ndarray, sr32: np.ndarray) -> np.ndarray:
    """O7: qr = clamp(rint(e / sr), -7, 7) with a float64 division; 0 if sr == 0.

    One code per selected index, in the order of sel_idx. Returns int8.
    """
    N, K = e.shape
    rows = sel_idx // K
    ev = e.ravel()[sel_idx]
    sr = sr32.astype(np.float64)[rows]
    safe = np.where(sr == 0.0, 1.0, sr)
    qr = np.clip(np.rint(ev / safe), -QMAX, QMAX)
    qr = np.where(sr == 0.0, 0.0, qr)
    return qr.astype(np.int8)


# ------------------------------------------------------ O8: canonical layout
def pack_nibbles(u: np.ndarray) -> np.ndarray:
    """Two 4-bit values per byte: element 2t in the low nibble, 2t+1 in the high
    nibble; an odd tail leaves the last high nibble 0."""
    u = np.asarray(u, dtype=np.uint8).ravel()
    if u.size % 2:
        u = np.concatenate([u, np.zeros(1, np.uint8)])
    return (u[0::2] | (u[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray, count: int) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8).ravel()
    out = np.empty(b.size * 2, dtype=np.uint8)
    out[0::2] = b & 0xF
    out[1::2] = b >> 4
    return out[:count]


def pack(W16: np.ndarray, G: int, rho: float) -> dict:
    """Steps O1-O8: the whole disaggregation [MQ-M1 Eq. (1), MQ-M2].

    Returns a dict with the intermediate values (s, q, e, sel, sr, qr) and the
    canonical arrays:
      codes  uint8 [N, K/2]   base code u = q + 8, even column in the low nibble
      scales fp16  [N, K/G]   base scales
      row_ptr int32 [N+1]     CSR row pointer of the residual
      col    uint16 [nnz]     column of each residual entry, ascending per row
      rcodes uint8 [ceil(nnz/2)] residual code u = qr + 8, two per byte
      rscale float32 [N]      residual row scale
    Zero residual codes are kept, so nnz == k exactly.
    """
    check_inputs(W16, G, rho)
    N, K = W16.shape
    s = base_scales(W16, G)
    q = base_codes(W16, s, G)
    e = base_error(W16, s, q, G)
    k = budget(rho, N, K)
    sel = select_topk(e, k)
    sr = residual_scales(e, sel)
    qr = residual_codes(e, sel, sr)
    rows = sel // K
    cols = sel % K
    counts = np.bincount(rows, minlength=N) if sel.size else np.zeros(N, np.int64)
    row_ptr = np.zeros(N + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    u_base = (q.astype(np.int16) + 8).astype(np.uint8)
    return {
        "N": N, "K": K, "G": G, "rho": float(rho), "nnz": int(k),
        "s": s, "q": q, "e": e, "sel": sel, "sr": sr, "qr": qr,
        "codes": (u_base[:, 0::2] | (u_base[:, 1::2] << 4)).astype(np.uint8),
        "scales": s,
        "row_ptr": row_ptr.astype(np.int32),
        "col": cols.astype(np.uint16),
        "rcodes": pack_nibbles((qr.astype(np.int16) + 8).astype(np.uint8)),
        "rscale": sr,
    }


# ----------------------------------------------------------- O9: dequant
def dequant(canon: dict) -> np.ndarray:
    """O9 [MQ-M1 Eq. (1)]: W~ = s*q + [j in S_i] * sr_i * qr_ij, read back from
    the canonical arrays, in float64. Returns float64 [N, K]."""
    N, K, G = canon["N"], canon["K"], canon["G"]
    codes = np.asarray(canon["codes"], dtype=np.uint8).reshape(N, K // 2)
    u = np.empty((N, K), dtype=np.int16)
    u[:, 0::2] = codes & 0xF
    u[:, 1::2] = codes >> 4
    q = (u - 8).astype(np.float64)
    s = np.repeat(np.asarray(canon["scales"]).astype(np.float64).reshape(N, K // G), G, axis=1)
    Wt = s * q
    row_ptr = np.asarray(canon["row_ptr"], dtype=np.int64)
    nnz = int(row_ptr[-1])
    if nnz:
        rows = np.repeat(np.arange(N), np.diff(row_ptr))
        cols = np.asarray(canon["col"], dtype=np.int64)[:nnz]
        qr = unpack_nibbles(canon["rcodes"], nnz).astype(np.int16) - 8
        sr = np.asarray(canon["rscale"]).astype(np.float64)[rows]
        np.add.at(Wt, (rows, cols), sr * qr.astype(np.float64))
    return Wt


# ------------------------------------------------------------ O10: linear
def linear(X16: np.ndarray, Wt: np.ndarray):
    """O10 [MQ-M3]: Y = X W~^T in float64, and the error scale B = |X| |W~|^T.

    Returns (Y64 [M, N], B [M, N]).
    """
    X = np.asarray(X16).astype(np.float64)
    return X @ Wt.T, np.abs(X) @ np.abs(Wt).T


TOL_REL = 2e-3
TOL_ABS = 1e-5


def within_tolerance(Y, Y64, B) -> np.ndarray:
    """Per-output acceptance: |Y - Y64| <= 2e-3 * B + 1e-5 (elementwise bool)."""
    Y = np.asarray(Y).astype(np.float64)
    return np.abs(Y - Y64) <= TOL_REL * B + TOL_ABS
