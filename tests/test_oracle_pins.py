"""Pins for the CPU oracle: checks against the definitions, closed forms,
invariants and brute force -- never against the oracle itself.

The pages print no worked numbers for this method, so each step is pinned by
mathematics instead (exact rational rounding, hand-derived small cases,
brute-force sorts, and the invariants the construction implies).
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from tests._exact import all_finite_fp16, fp16_exact, fp32_exact, round_half_even


def _frac(x) -> Fraction:
    return Fraction(float(x))


# --------------------------------------------------------------- roundings
def test_fp16_scale_rounding_matches_ieee_definition_for_every_absmax():
    """O1's fp16 rounding of absmax/7, for every positive finite fp16 absmax."""
    vals = all_finite_fp16()
    pos = vals[vals > 0].astype(np.float64)
    got = oracle.to_fp16_rne(pos / 7.0)
    for a, s in zip(pos.tolist(), got.tolist()):
        assert _frac(s) == fp16_exact(Fraction(a) / 7), a


def test_fp16_rounding_midpoints_and_overflow():
    # exact midpoints between fp16 neighbours must go to the even significand
    one = 1.0
    ulp = 2.0 ** -10
    assert float(oracle.to_fp16_rne(np.array([one + ulp / 2]))[0]) == one
    assert float(oracle.to_fp16_rne(np.array([one + 1.5 * ulp]))[0]) == one + 2 * ulp
    # subnormal midpoint 0.5 * 2^-24 rounds to 0, 1.5 * 2^-24 to 2 * 2^-24
    assert float(oracle.to_fp16_rne(np.array([2.0 ** -25]))[0]) == 0.0
    assert float(oracle.to_fp16_rne(np.array([3 * 2.0 ** -25]))[0]) == 2 * 2.0 ** -24
    assert math.isinf(float(oracle.to_fp16_rne(np.array([65520.0]))[0]))
    assert float(oracle.to_fp16_rne(np.array([65519.99]))[0]) == 65504.0


def test_fp32_residual_scale_rounding_matches_ieee_definition():
    """O6's fp32 rounding of max|e|/7 over the values max|e| can take
    (multiples of 2^-24 below 2^17)."""
    rng = np.random.default_rng(7)
    m = np.concatenate([np.arange(1, 5000), rng.integers(1, 2 ** 41, 20000)])
    x = m.astype(np.float64) * 2.0 ** -24
    got = oracle.to_fp32_rne(x / 7.0)
    for mi, s in zip(m.tolist(), got.tolist()):
        assert _frac(s) == fp32_exact(Fraction(mi, 7) * Fraction(1, 2 ** 24)), mi


# -------------------------------------------------- P1: base quantiser sweep
def _groups_for_absmax(a: float, G: int):
    """Rows of G values whose absmax is exactly a: a, then every finite fp16
    with |w| <= a (both signs), padded with zeros."""
    vals = all_finite_fp16()
    inside = vals[np.abs(vals.astype(np.float64)) <= a]
    per = G - 1
    n = -(-inside.size // per)
    body = np.zeros(n * per, dtype=np.float16)
    body[: inside.size] = inside
    rows = np.concatenate([np.full((n, 1), a, dtype=np.float16), body.reshape(n, per)], axis=1)
    return rows


@pytest.mark.parametrize("a_bits", [0x0001, 0x0003, 0x0004, 0x002D, 0x0200, 0x03FF,
                                    0x0400, 0x0C00, 0x1400, 0x2E66, 0x3800, 0x3C00,
                                    0x4700, 0x5A00, 0x7000, 0x7BFF])
def test_base_quantiser_sweep_every_fp16_in_range(a_bits):
    """P1: for groups with absmax a, every finite fp16 w with |w| <= a:
    |q| <= 7, e == w - s*q exactly, q is the exact RNE of w/s (clamped), and
    |e| <= s/2 when s is normal; absmax itself maps to +-7 once a > 2.7e-6."""
    a = float(np.array([a_bits], dtype=np.uint16).view(np.float16)[0])
    G = 128
    W = _groups_for_absmax(a, G)
    s = oracle.base_scales(W, G)
    assert np.all(s.astype(np.float64) == float(oracle.to_fp16_rne(np.array([a / 7.0]))[0]))
    q = oracle.base_codes(W, s, G)
    e = oracle.base_error(W, s, q, G)
    assert np.all(np.abs(q) <= 7)
    sv = float(s[0, 0])
    w64 = W.astype(np.float64)
    if sv == 0.0:
        assert np.all(q == 0) and np.all(e == w64)
        return
    # exact check of every (w, q, e) triple against rational arithmetic on a
    # subsample, and the half-step bound on all of them
    S = Fraction(sv)
    flat_w = w64.ravel()
    flat_q = q.ravel().astype(np.int64)
    flat_e = e.ravel()
    idx = np.unique(np.linspace(0, flat_w.size - 1, 3000).astype(np.int64))
    for t in idx.tolist():
        W_ = Fraction(flat_w[t])
        qq = max(-7, min(7, round_half_even(W_ / S)))
        assert flat_q[t] == qq
        assert Fraction(flat_e[t]) == W_ - S * qq
    if sv >= 2.0 ** -14:
        assert np.all(np.abs(e) <= sv / 2)
    if a > 2.7e-6:
        assert q[0, 0] == 7


def test_base_codes_are_rne_not_floor_or_half_up():
    # s = 1: w = 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 0.5 -> 0, 1.5 -> 2
    w = np.zeros((1, 32), dtype=np.float16)
    w[0, :6] = [7.0, 2.5, 3.5, -2.5, 0.5, 1.5]
    s = oracle.base_scales(w, 32)
    assert float(s[0, 0]) == 1.0
    q = oracle.base_codes(w, s, 32)
    assert q[0, :6].tolist() == [7, 2, 4, -2, 0, 2]


# ------------------------------------------------------ P2: closed form
def test_exactly_representable_groups_have_zero_error():
    """P2: w = s*c with c in [-7, 7] and a +-7 in every group gives q = c and
    e = 0; every selected residual code is then 0 and W~ == W."""
    rng = np.random.default_rng(3)
    N, K, G = 8, 256, 64
    mant = rng.integers(1, 256, size=(N, K // G)).astype(np.float64)   # <= 8 bits
    sc = mant * 2.0 ** rng.integers(-12, 0, size=(N, K // G))
    c = rng.integers(-7, 8, size=(N, K))
    c[:, ::G] = 7 * rng.choice([-1, 1], size=(N, K // G))
    W = (np.repeat(sc, G, axis=1) * c).astype(np.float16)
    assert np.all(W.astype(np.float64) == np.repeat(sc, G, axis=1) * c)
    p = oracle.pack(W, G, 0.25)
    assert np.all(p["s"].astype(np.float64) == sc)
    assert np.all(p["q"] == c)
    assert np.all(p["e"] == 0)
    assert p["nnz"] == int(0.25 * N * K)
    assert np.all(p["qr"] == 0) and np.all(p["sr"] == 0)
    assert np.all(oracle.dequant(p) == W.astype(np.float64))


# --------------------------------------------- hand-derived worked example
def test_hand_worked_example():
    """A 2x64 matrix, G = 32, budget 5 entries, derived by hand:

    row 0, group 0: absmax 7 -> s = 1; -3.5 -> -4 (tie to even), e = 0.5;
        2.5 -> 2, e = 0.5; 1.25 -> 1, e = 0.25; 0.5 -> 0, e = 0.5.
    row 0, group 1: absmax 14 -> s = 2; 3 -> 2 (1.5 ties up to even 2), e = -1;
        5 -> 2, e = 1; 0.75 -> 0, e = 0.75; -14 -> -7.
    row 1, group 0: absmax 0.5 -> s = fp16(0.5/7) = 1170 * 2^-14;
        0.5 -> 7, e = 2^-13; 0.25 -> 4 (3.5009), e = -0.03564453125.
    row 1, group 1: all zero -> s = 0.
    Order by (|e| desc, index asc): 33, 34, 35, 1, 2 | 4, 3, 65, 64, ...
    The tie at |e| = 0.5 between indices 1, 2, 4 is cut after index 2.
    Row 0 residual scale: fp32(1/7) = 9586981 * 2^-26; codes rint(e/sr):
        0.5 -> 3 (3.4999998), -1 -> -7, 1 -> 7, 0.75 -> 5.
    """
    W = np.zeros((2, 64), dtype=np.float16)
    W[0, :5] = [7.0, -3.5, 2.5, 1.25, 0.5]
    W[0, 32:36] = [-14.0, 3.0, 5.0, 0.75]
    W[1, :2] = [0.5, 0.25]
    rho = 5 / 128
    p = oracle.pack(W, 32, rho)
    s1 = 1170 * 2.0 ** -14
    assert p["scales"].astype(np.float64).tolist() == [[1.0, 2.0], [s1, 0.0]]
    assert p["nnz"] == 5
    assert p["sel"].tolist() == [1, 2, 33, 34, 35]
    assert p["row_ptr"].tolist() == [0, 5, 5]
    assert p["col"].tolist() == [1, 2, 33, 34, 35]
    assert _frac(p["rscale"][0]) == Fraction(9586981, 2 ** 26)
    assert float(p["rscale"][1]) == 0.0
    assert p["qr"].tolist() == [3, 3, -7, 7, 5]
    assert p["rcodes"].tolist() == [0xBB, 0xF1, 0x0D]
    assert p["codes"][0, :3].tolist() == [0x4F, 0x9A, 0x88]
    assert p["codes"][0, 16:18].tolist() == [0xA1, 0x8A]
    assert p["codes"][1, :2].tolist() == [0xCF, 0x88]
    assert np.all(p["codes"][1, 16:] == 0x88)
    e = p["e"]
    assert e[1, 0] == 2.0 ** -13 and e[1, 1] == -0.03564453125
    Wt = oracle.dequant(p)
    sr = Fraction(9586981, 2 ** 26)
    assert Fraction(Wt[0, 1]) == -4 + 3 * sr
    assert Fraction(Wt[0, 33]) == 4 - 7 * sr
    assert Fraction(Wt[0, 4]) == 0          # index 4 lost the tie
    assert Fraction(Wt[1, 0]) == 7 * Fraction(s1)


# ---------------------------------------------------- P3: brute-force top-k
def _brute_select(e: np.ndarray, k: int):
    flat = [abs(float(v)) for v in e.ravel()]
    order = sorted(range(len(flat)), key=lambda t: (-flat[t], t))
    return sorted(order[:k])


@pytest.mark.parametrize("seed", range(40))
def test_topk_matches_brute_force_sort(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 5))
    K = 32 * int(rng.integers(1, 9))
    kind = seed % 4
    if kind == 0:
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    elif kind == 1:       # heavy ties: few distinct values
        W = rng.choice(np.array([0.0, 0.25, -0.25, 0.3, 0.31, 1.0]), size=(N, K)).astype(np.float16)
    elif kind == 2:       # constant rows
        W = np.repeat(rng.standard_normal((N, 1)), K, axis=1).astype(np.float16)
    else:                 # outliers on a coarse grid
        W = (rng.integers(-40, 41, size=(N, K)) / 16.0).astype(np.float16)
        W[:, 3] *= 8
    G = 32
    s = oracle.base_scales(W, G)
    q = oracle.base_codes(W, s, G)
    e = oracle.base_error(W, s, q, G)
    for rho in (0.0, 0.01, 0.1, 0.37, 0.5, 1.0):
        k = oracle.budget(rho, N, K)
        assert oracle.select_topk(e, k).tolist() == _brute_select(e, k)


# ------------------------------------------------- P4: rho = 0 is plain W4
def test_rho_zero_is_plain_rtn_w4_and_linear_matches_loops():
    rng = np.random.default_rng(11)
    N, K, M, G = 5, 64, 3, 32
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    p = oracle.pack(W, G, 0.0)
    assert p["nnz"] == 0 and p["row_ptr"].tolist() == [0] * (N + 1)
    assert np.all(p["sr"] == 0) and p["col"].size == 0
    Wt = oracle.dequant(p)
    Y, B = oracle.linear(X, Wt)
    for m in range(M):
        for i in range(N):
            terms = [float(X[m, j]) * float(p["s"][i, j // G]) * int(p["q"][i, j]) for j in range(K)]
            assert abs(Y[m, i] - math.fsum(terms)) <= 1e-12 * (1 + math.fsum(abs(t) for t in terms))
            assert abs(B[m, i] - math.fsum(abs(t) for t in terms)) <= 1e-12 * (1 + B[m, i])


# ---------------------------------------- P5/P6: error invariants
@pytest.mark.parametrize("seed,rho", [(0, 0.01), (1, 0.05), (2, 0.3), (3, 1.0), (4, 0.002)])
def test_residual_never_increases_error(seed, rho):
    """P5: |w - W~| <= |e| for every entry (a nonzero residual code has
    |e| >= sr/2 >= |e - sr*qr|)."""
    rng = np.random.default_rng(seed)
    N, K = 16, 256
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[:, rng.choice(K, 3, replace=False)] *= 20
    p = oracle.pack(W, 128, rho)
    err = np.abs(W.astype(np.float64) - oracle.dequant(p))
    assert np.all(err <= np.abs(p["e"]))
    assert np.linalg.norm(err) <= np.linalg.norm(p["e"])
    if rho >= 0.01:
        assert np.linalg.norm(err) < np.linalg.norm(p["e"])


@pytest.mark.parametrize("seed", range(4))
def test_density_one_bounds_error_by_half_residual_step(seed):
    """P6: at rho = 1 every entry is selected and |e - sr*qr| <= sr/2."""
    rng = np.random.default_rng(100 + seed)
    N, K = 12, 128
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
    W[rng.integers(0, N), :] *= 30
    p = oracle.pack(W, 64, 1.0)
    assert p["nnz"] == N * K
    sr = p["sr"].astype(np.float64)[:, None]
    res = np.abs(W.astype(np.float64) - oracle.dequant(p))
    assert np.all(res <= sr / 2)
    assert np.all(np.abs(p["qr"]) <= 7)


def test_empty_rows_get_zero_residual_scale():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((6, 128)) * 0.02).astype(np.float16)
    W[2, 5] = 3.0       # the only large error sits in row 2 (group of one outlier)
    W[2, 6] = 1.4
    p = oracle.pack(W, 128, 2 / (6 * 128))
    assert p["nnz"] == 2
    counts = np.diff(p["row_ptr"])
    assert np.all(p["sr"][counts == 0] == 0)
    assert np.all(p["sr"][counts > 0] > 0)


# ------------------------------------------- P7/P8: nesting and threshold
def test_selection_nesting_and_threshold():
    rng = np.random.default_rng(9)
    N, K = 20, 256
    W = (rng.integers(-60, 61, size=(N, K)) / 64.0).astype(np.float16)     # many ties
    W[:, :3] *= 16
    prev = set()
    for rho in (0.0, 0.001, 0.01, 0.05, 0.2, 0.5, 0.9, 1.0):
        p = oracle.pack(W, 128, rho)
        S = set(p["sel"].tolist())
        assert prev <= S
        prev = S
        a = np.abs(p["e"]).ravel()
        mask = np.zeros(a.size, bool)
        mask[p["sel"]] = True
        if mask.any() and (~mask).any():
            T = a[mask].min()
            assert T >= a[~mask].max()
            tied_in = np.flatnonzero(mask & (a == T))
            tied_out = np.flatnonzero(~mask & (a == T))
            if tied_in.size and tied_out.size:
                assert tied_in.max() < tied_out.min()


# ----------------------------------------------------- canonical layout
def test_canonical_layout_roundtrip():
    rng = np.random.default_rng(21)
    N, K, G = 9, 192, 64
    W = (rng.standard_normal((N, K)) * 0.1).astype(np.float16)
    W[rng.integers(0, N, 5), rng.integers(0, K, 5)] = 4.0
    p = oracle.pack(W, G, 0.03)
    u = np.empty((N, K), np.int16)
    u[:, 0::2] = p["codes"] & 0xF
    u[:, 1::2] = p["codes"] >> 4
    assert np.all(u - 8 == p["q"])
    assert np.all((u >= 1) & (u <= 15))
    rp = p["row_ptr"].astype(np.int64)
    assert rp[0] == 0 and rp[-1] == p["nnz"] and np.all(np.diff(rp) >= 0)
    for i in range(N):
        c = p["col"][rp[i]:rp[i + 1]].astype(np.int64)
        assert np.all(np.diff(c) > 0)
        assert np.all(np.isin(i * K + c, p["sel"]))
    qr = oracle.unpack_nibbles(p["rcodes"], p["nnz"]).astype(np.int16) - 8
    assert np.all(qr == p["qr"])
    assert p["rcodes"].size == (p["nnz"] + 1) // 2
    if p["nnz"] % 2:
        assert p["rcodes"][-1] >> 4 == 0


def test_budget_rounding():
    assert oracle.budget(0.0, 11008, 4096) == 0
    assert oracle.budget(1.0, 11008, 4096) == 11008 * 4096
    assert oracle.budget(0.005, 11008, 4096) == 225443
    assert oracle.budget(0.01, 28672, 8192) == 2348810
    assert oracle.budget(0.01, 1024, 1024) == 10485
    assert [oracle.budget(r, 14336, 4096) for r in (0.001, 0.005, 0.02, 0.05)] == \
        [58720, 293601, 1174405, 2936012]


def test_residual_codes_exact_near_half_steps():
    """O7 must divide in float64: codes are the exact RNE of e/sr (clamped),
    checked on errors placed within a few units of 2^-24 of (n + 1/2) * sr,
    where a float32 division rounds onto the half step and picks the wrong code."""
    rng = np.random.default_rng(31)
    sr32 = (rng.uniform(1e-4, 2.0, size=400)).astype(np.float32)
    rows, es = [], []
    for i, s in enumerate(sr32.astype(np.float64).tolist()):
        for n in range(0, 7):
            centre = round((n + 0.5) * s * 2 ** 24)
            for d in (-2, -1, 0, 1, 2):
                rows.append(i)
                es.append((centre + d) * 2.0 ** -24 * (1 if (n + d) % 2 else -1))
    rows = np.array(rows)
    N = sr32.size
    per = np.bincount(rows, minlength=N).max()
    e = np.zeros((N, per))
    cols = np.zeros(rows.size, np.int64)
    fill = np.zeros(N, np.int64)
    for t, (i, v) in enumerate(zip(rows.tolist(), es)):
        e[i, fill[i]] = v
        cols[t] = fill[i]
        fill[i] += 1
    sel = rows * per + cols
    order = np.argsort(sel)
    qr = oracle.residual_codes(e, sel[order], sr32)
    for t, code in zip(order.tolist(), qr.tolist()):
        ex = Fraction(es[t]) / Fraction(float(sr32[rows[t]]))
        assert code == max(-7, min(7, round_half_even(ex))), (t, es[t], float(sr32[rows[t]]))


# ------------------------------------------------------------ validation
def test_invalid_inputs_rejected():
    W = np.zeros((4, 64), np.float16)
    with pytest.raises(oracle.OracleInputError):
        oracle.pack(W, 48, 0.1)
    with pytest.raises(oracle.OracleInputError):
        oracle.pack(np.zeros((4, 96), np.float16), 64, 0.1)
    with pytest.raises(oracle.OracleInputError):
        oracle.pack(W, 32, 1.5)
    with pytest.raises(oracle.OracleInputError):
        oracle.pack(W, 32, float("nan"))
    bad = W.copy()
    bad[1, 2] = np.inf
    with pytest.raises(oracle.OracleInputError):
        oracle.pack(bad, 32, 0.1)


# ------------------------------------------------------- P10: linear
def test_linear_matches_exact_sums_on_tiny_inputs():
    rng = np.random.default_rng(17)
    M, N, K = 3, 4, 64
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.3).astype(np.float16)
    p = oracle.pack(W, 32, 0.2)
    Wt = oracle.dequant(p)
    Y, B = oracle.linear(X, Wt)
    assert Y.shape == (M, N)
    for m in range(M):
        for i in range(N):
            ex = sum(Fraction(float(X[m, j])) * Fraction(Wt[i, j]) for j in range(K))
            assert abs(Fraction(Y[m, i]) - ex) <= Fraction(1, 2 ** 40)
            exb = sum(abs(Fraction(float(X[m, j])) * Fraction(Wt[i, j])) for j in range(K))
            assert abs(Fraction(B[m, i]) - exb) <= Fraction(1, 2 ** 40)
    ok = oracle.within_tolerance(Y.astype(np.float16), Y, B)
    assert ok.all()
    assert not oracle.within_tolerance(Y + 0.01 * B + 1e-3, Y, B).any()


# ------------------------------------------------ golden fixtures (by hand)
def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as fh:
        return json.load(fh)


def golden_matrix(g):
    W = np.zeros((g["N"], g["K"]), dtype=np.float16)
    for i, j, v in g["W_nonzero"]:
        W[i, j] = v
    return W


def test_oracle_reproduces_the_hand_derived_fixture():
    """tests/golden/hand_2x64_g32.json holds a packing derived by hand from the
    rules (its `derivation` lines); the oracle must give every array of it."""
    g = _golden("hand_2x64_g32.json")
    p = oracle.pack(golden_matrix(g), g["G"], g["rho_num"] / g["rho_den"])
    ex = g["expected"]
    assert p["scales"].view(np.uint16).tolist() == ex["scales_fp16_bits"]
    assert [bytes(r).hex() for r in p["codes"]] == ex["codes_hex"]
    assert p["nnz"] == ex["nnz"]
    assert p["row_ptr"].tolist() == ex["row_ptr"]
    assert p["col"].tolist() == ex["col"]
    assert p["rscale"].view(np.uint32).tolist() == ex["rscale_fp32_bits"]
    assert p["qr"].tolist() == ex["qr"]
    assert p["rcodes"].tolist() == ex["rcodes"]
