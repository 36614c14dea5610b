"""Pins of the block-wise residual oracle (oracle/blocks.py) against what the
mathematics fixes, independent of its own arithmetic:

* beta = 0 is the plain W4 base (the element-wise oracle at rho = 0);
* every score is >= 0 and every selected block can only shrink each entry's
  error (|e - r| <= |e| because r is the 4-bit rounding of e);
* scores equal the exactly rounded sums of h_j (e^2 - (e - r)^2), with r
  rebuilt from scratch in plain Python (round-half-even division), on many
  small blocks, and the selection equals a full sort by (score desc, index);
* a block whose only base error is one entry e scores h_j e^2 (to the fp32
  rounding of the block scale);
* beta = 1 leaves every entry within half a residual step;
* selections are nested in beta and the estimated distortion never grows.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import blocks as ob


def _layer(N, K, seed, outlier_cols=3):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, outlier_cols, replace=False)] *= 20
    return W.astype(np.float16)


def _h(K, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((24, K)).astype(np.float16)
    X[:, rng.choice(K, 2, replace=False)] *= 50
    return ob.hessian_diag(X)


def test_beta_zero_is_plain_w4():
    W = _layer(48, 256, 1)
    c = ob.pack_blocks(W, 128, 0.0, _h(256, 2))
    assert c["blk"].size == 0
    assert np.array_equal(ob.dequant_blocks(c), oracle.dequant(oracle.pack(W, 128, 0.0)))
    assert np.array_equal(c["codes"], oracle.pack(W, 128, 0.0)["codes"])


@pytest.mark.parametrize("N,K,G,beta", [(48, 256, 128, 0.3), (37, 384, 64, 0.5), (20, 96, 32, 0.7)])
def test_scores_nonnegative_and_errors_never_grow(N, K, G, beta):
    W = _layer(N, K, N + K)
    h = _h(K, N)
    c = ob.pack_blocks(W, G, beta, h)
    assert np.all(c["delta"] >= 0.0)
    Wt = ob.dequant_blocks(c)
    err = np.abs(W.astype(np.float64) - Wt)
    assert np.all(err <= np.abs(c["e"]))
    base = oracle.dequant(oracle.pack(W, G, 0.0))
    assert ob.distortion(W, Wt, h) <= ob.distortion(W, base, h)


def _rne_div(a, b):
    """round-half-even of a / b for floats, via exact rationals."""
    x = Fraction(a) / Fraction(b)
    f = math.floor(x)
    d = x - f
    if d > Fraction(1, 2) or (d == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


@pytest.mark.parametrize("seed", range(6))
def test_scores_match_exact_sums_and_full_sort(seed):
    br, bc, N, K, G = 2, 4, 7, 32, 32        # 4 x 8 = 32 blocks, the last block row partial
    W = _layer(N, K, 100 + seed, outlier_cols=4)
    h = _h(K, 200 + seed)
    c = ob.pack_blocks(W, G, 0.25, h, br=br, bc=bc)
    e = c["e"]
    nrb, nkt = ob.block_grid(N, K, br, bc)
    exact = []
    for rb in range(nrb):
        for kt in range(nkt):
            terms = []
            for i in range(rb * br, min(N, rb * br + br)):
                cols = range(kt * bc, min(K, kt * bc + bc))
                m = max(abs(Fraction(float(e[i, j]))) for j in cols)
                sr = float(np.float32(float(m / 7)))           # fp32 of the exact max / 7
                for j in cols:
                    qr = 0 if sr == 0.0 else max(-7, min(7, _rne_div(float(e[i, j]), sr)))
                    r = Fraction(sr) * qr
                    ev = Fraction(float(e[i, j]))
                    terms.append(Fraction(float(h[j])) * (ev * ev - (ev - r) ** 2))
            exact.append(sum(terms, Fraction(0)))
    exact = np.array([float(x) for x in exact])
    scale = np.maximum(np.abs(exact), 1e-300)
    assert np.all(np.abs(c["delta"] - exact) <= 1e-12 * scale + 1e-300)
    order = sorted(range(exact.size), key=lambda b: (-exact[b], b))
    gaps = np.diff(np.sort(np.unique(exact)))
    assert gaps.size == 0 or gaps.min() > 1e-9 * np.abs(exact).max()   # no near-ties in these seeds
    for k in range(exact.size + 1):
        assert np.array_equal(ob.select_blocks(c["delta"], k), np.sort(order[:k]))


def test_single_error_block_scores_h_e_squared():
    # exact base: every group holds multiples of s0 = 2^-4 and one entry 7 s0,
    # so s = s0 and e = 0, except for planted entries w = c s0 + delta
    N, K, G = 32, 256, 128
    s0 = 2.0 ** -4
    rng = np.random.default_rng(7)
    C = rng.integers(-6, 7, size=(N, K)).astype(np.float64)
    C[:, 0] = 7
    C[:, 128] = -7
    W = (C * s0).astype(np.float16)
    planted = {(3, 40): 3 * 2.0 ** -10, (20, 200): -5 * 2.0 ** -10, (17, 130): 2 * 2.0 ** -10}
    for (i, j), d in planted.items():
        W[i, j] = np.float16(C[i, j] * s0 + d)
    h = np.ones(K, dtype=np.float32)
    h[40], h[200], h[130] = 2.0, 0.5, 9.0
    c = ob.pack_blocks(W, G, 0.5, h)
    nkt = c["nkt"]
    want = np.zeros(4)
    for (i, j), d in planted.items():
        want[(i // 16) * nkt + j // 128] += float(h[j]) * d * d
    assert np.all(c["delta"][want == 0] == 0.0)
    nz = want > 0
    assert np.allclose(c["delta"][nz], want[nz], rtol=1e-5, atol=0)
    # beta = 0.5 of 4 blocks: the two with the largest h e^2 (blocks 3 and 0)
    top2 = np.sort(np.argsort(-want, kind="stable")[:2])
    assert np.array_equal(top2, [0, 3])
    assert np.array_equal(c["blk"], top2)


def test_beta_one_within_half_a_step():
    W = _layer(40, 384, 5)
    c = ob.pack_blocks(W, 64, 1.0, _h(384, 6))
    assert c["blk"].size == c["delta"].size
    sr = c["sr"].astype(np.float64)[..., None]
    r = sr * c["qr"].astype(np.float64)
    eb = ob._blocked(c["e"], 16, 128)
    assert np.all(np.abs(eb - r) <= sr / 2)


def test_selection_nested_and_distortion_monotone():
    W = _layer(64, 512, 9)
    h = _h(512, 10)
    prev_set, prev_d = set(), math.inf
    for beta in (0.0, 0.1, 0.25, 0.5, 0.75, 1.0):
        c = ob.pack_blocks(W, 128, beta, h)
        cur = set(c["blk"].tolist())
        assert prev_set <= cur
        d = ob.distortion(W, ob.dequant_blocks(c), h)
        assert d <= prev_d
        prev_set, prev_d = cur, d


def test_hessian_weight_decides_between_equal_errors():
    # two blocks with the same errors; the one whose columns carry larger h wins
    N, K = 16, 256
    W = _layer(N, K, 11, outlier_cols=0)
    W[:, 128:] = W[:, :128]
    h = np.ones(K, dtype=np.float32)
    h[128:] = 3.0
    c = ob.pack_blocks(W, 128, 0.5, h)
    assert c["delta"][1] > c["delta"][0]
    assert np.array_equal(c["blk"], [1])


def test_block_budget_and_inputs():
    assert ob.block_budget(0.1, 22016) == 2201
    assert ob.block_budget(1.0, 7) == 7 and ob.block_budget(0.0, 7) == 0
    W = _layer(16, 128, 3)
    with pytest.raises(ValueError):
        ob.pack_blocks(W, 128, 1.5, np.ones(128, np.float32))
    with pytest.raises(ValueError):
        ob.pack_blocks(W, 128, 0.1, -np.ones(128, np.float32))


def test_hessian_diag_closed_form():
    X = np.full((5, 64), 0.5, dtype=np.float16)
    X[:, 3] = -2.0
    h = ob.hessian_diag(X)
    assert h.dtype == np.float32
    assert np.all(h[np.arange(64) != 3] == 1.25) and h[3] == 20.0
