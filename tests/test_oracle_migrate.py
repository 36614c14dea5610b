"""Pins of the outlier-migration oracle (oracle/migrate.py): the power-of-two
scaling is exact (W^ 2^-e == W and X^ 2^e == X entry by entry, hence
X^ W^^T == X W^T) away from the fp16 subnormal range; the exponent rule on
hand-computed cases (including zero channels and the fp16 range clamps); and
the balance SmoothQuant aims for: after migration the two per-channel maxima
are within a factor of 4 of each other."""
import numpy as np

from oracle import migrate as om


def _wx(K=256, seed=0):
    # magnitudes kept >= 2^-8 so that no scaled value leaves fp16's normal range
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((64, K)) * 0.02).astype(np.float32)
    W = np.where(np.abs(W) < 2.0 ** -8, np.copysign(2.0 ** -8, W), W)
    W[:, rng.choice(K, 3, replace=False)] *= 20
    X = rng.standard_normal((32, K)).astype(np.float32)
    X = np.where(np.abs(X) < 2.0 ** -4, np.copysign(2.0 ** -4, X), X)
    X[:, rng.choice(K, 4, replace=False)] *= 50
    return W.astype(np.float16), X.astype(np.float16)


def test_scaling_is_exact_and_preserves_the_product():
    W, X = _wx()
    amax = np.abs(X.astype(np.float32)).max(axis=0)
    Wh, e = om.migrate(W, amax)
    Xh = om.smooth_activations(X, e)
    assert np.any(e != 0)
    # no value of these inputs lands in the subnormal range after scaling
    assert np.abs(Wh[W != 0]).min() >= 2.0 ** -14 and np.abs(Xh[X != 0]).min() >= 2.0 ** -14
    assert np.array_equal(Wh.astype(np.float64) * np.exp2(-e.astype(np.float64)), W.astype(np.float64))
    assert np.array_equal(Xh.astype(np.float64) * np.exp2(e.astype(np.float64)), X.astype(np.float64))
    P = X.astype(np.float64)[:, None, :] * W.astype(np.float64)[None, :, :]
    Ph = Xh.astype(np.float64)[:, None, :] * Wh.astype(np.float64)[None, :, :]
    assert np.array_equal(P, Ph)


def test_exponent_rule_hand_cases():
    K = 6
    W = np.zeros((2, K), dtype=np.float16)
    W[0] = [2.0 ** -4, 8.0, 1.0, 0.0, 2.0 ** 14, 0.75]
    W[1] = [-2.0 ** -5, 1.0, 0.5, 0.0, 1.0, -0.5]
    ax = np.array([64.0, 1.0, 0.0, 5.0, 2.0 ** 15, 3.0], dtype=np.float32)
    e = om.smooth_exponents(W, ax)
    # col 0: E_x 6, E_w -4 -> 5; col 1: E_x 0, E_w 3 -> floor(-1.5) = -2;
    # col 2: no activation -> 0; col 3: zero weights -> 0;
    # col 4: E_x 15, E_w 14 -> floor(0.5) = 0, and at most 15 - 14 = 1 anyway;
    # col 5: E_x 1 (3 = 1.5 * 2), E_w -1 (0.75) -> 1
    assert e.tolist() == [5, -2, 0, 0, 0, 1]
    # the clamp toward fp16's range: a huge activation next to a huge weight
    W2 = np.array([[2.0 ** 12]], dtype=np.float16)
    e2 = om.smooth_exponents(W2, np.array([2.0 ** 15], dtype=np.float32))
    assert e2.tolist() == [1]                           # floor(3 / 2) = 1 <= 15 - 12
    W3 = np.array([[2.0 ** 15]], dtype=np.float16)
    e3 = om.smooth_exponents(W3, np.array([2.0 ** 15 * 1.5], dtype=np.float32))
    assert e3.tolist() == [0]                           # 15 - 15 = 0 caps it


def test_channel_maxima_balanced_after_migration():
    W, X = _wx(K=512, seed=3)
    ax = np.abs(X.astype(np.float32)).max(axis=0)
    Wh, e = om.migrate(W, ax)
    Xh = om.smooth_activations(X, e)
    mw = np.abs(Wh.astype(np.float64)).max(axis=0)
    mx = np.abs(Xh.astype(np.float64)).max(axis=0)
    d = om.floor_log2(mx) - om.floor_log2(mw)
    assert np.all((d == 0) | (d == 1))
    r = mx / mw
    assert np.all((r >= 0.5) & (r < 4.0))


def test_subnormal_results_round_half_even():
    W = np.array([[2.0 ** -14, 3 * 2.0 ** -24, 2.0 ** -13]], dtype=np.float16)
    Wh = om.scale_columns(W, np.array([-2, -1, -12]))
    # 2^-16 is exact (subnormal, 4 quanta); 3 * 2^-25 is a tie between 1 and 2
    # quanta of 2^-24 -> 2 (even); 2^-25 is half a quantum -> 0 (even)
    assert Wh.astype(np.float64).tolist() == [[2.0 ** -16, 2 * 2.0 ** -24, 0.0]]
