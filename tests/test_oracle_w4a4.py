"""Pins of the 4-bit activation oracle (oracle/w4a4.py).

Each pin fixes the result by something other than the oracle's own formula:
  * a hand-worked group (scale, ties rounded to even, clamping, zero group);
  * the error bound of round-to-nearest: |x - x^| <= sx / 2 inside the range,
    and the largest entry of each group maps to code +-7;
  * exact round trips: activations that are already 4-bit values (a power-of-
    two scale times codes with a +-7 in every group) come back unchanged, and
    then the W4A4 product equals the plain W4A16 product of the weight oracle;
  * scaling X by 2^k scales sx by 2^k and leaves the codes unchanged;
  * a transposed or shifted group layout (a plausible indexing mistake) fails
    the hand case.
"""
import numpy as np
import pytest

import oracle
from oracle import w4a4 as oa


def test_hand_group():
    G = 32
    x = np.zeros((2, G), dtype=np.float32)
    # max |x| = 7 -> sx = 1 exactly; -3.5 and 2.5 are ties (to even: -4, 2)
    x[0, :6] = [7.0, -3.5, 2.5, 0.5, 1.4990234375, -6.75]
    qx, sx = oa.quantize_activations(x.astype(np.float16), G)
    assert sx.dtype == np.float16 and sx.tolist() == [[1.0], [0.0]]
    assert qx[0, :6].tolist() == [7, -4, 2, 0, 1, -7]
    assert not qx[0, 6:].any() and not qx[1].any()      # zero group -> scale 0, codes 0
    assert oa.code_sums(qx, G).tolist() == [[7 - 4 + 2 + 1 - 7], [0]]


def test_hand_scale_rounding():
    # max |x| = 1 -> 1/7 rounds to the fp16 0.142822265625 (below 1/7), so
    # 1 / sx = 7.0017... rounds to 7 and the clamp is not needed
    x = np.zeros((1, 64), dtype=np.float16)
    x[0, 3] = -1.0
    x[0, 40] = 0.5
    qx, sx = oa.quantize_activations(x, 64)
    assert float(sx[0, 0]) == 0.142822265625
    assert qx[0, 3] == -7 and qx[0, 40] == 4              # 0.5 / sx = 3.5008... -> 4


@pytest.mark.parametrize("G", [32, 64, 128])
def test_rounding_error_bound(G):
    rng = np.random.default_rng(G)
    X = (rng.standard_normal((17, 4 * G)) * np.exp2(rng.integers(-6, 6, (17, 1)))).astype(np.float16)
    X[:, rng.choice(4 * G, 3, replace=False)] *= 40
    qx, sx = oa.quantize_activations(X, G)
    Xh = oa.dequant_activations(qx, sx, G)
    s = np.repeat(sx.astype(np.float64), G, axis=1)
    x = X.astype(np.float64)
    inside = np.abs(x) <= 7 * s
    assert np.all(np.abs(x - Xh)[inside] <= s[inside] / 2)
    assert np.all(np.abs(qx) <= 7)
    # the largest entry of every group lands on +-7
    amax_code = np.abs(qx.astype(np.int64)).reshape(17, 4, G).max(axis=2)
    assert np.all(amax_code == 7)


def _exact_acts(M, K, G, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-7, 8, (M, K))
    q.reshape(M, K // G, G)[:, :, 0] = rng.choice([-7, 7], (M, K // G))
    e = rng.integers(-8, 3, (M, K // G))
    return (q * np.repeat(np.exp2(e), G, axis=1)).astype(np.float16), q, np.exp2(e)


@pytest.mark.parametrize("G", [32, 128])
def test_exact_round_trip_and_w4a16_equivalence(G):
    M, N, K = 5, 24, 256
    X, q, s = _exact_acts(M, K, G, 7)
    qx, sx = oa.quantize_activations(X, G)
    assert np.array_equal(qx, q) and np.array_equal(sx.astype(np.float64), s)
    W = (np.random.default_rng(1).standard_normal((N, K)) * 0.05).astype(np.float16)
    Wt = oracle.dequant(oracle.pack(W, G, 0.02))
    Y4, B4 = oa.linear_a4(X, Wt, G)
    Y16, B16 = oracle.linear(X, Wt)
    assert np.array_equal(Y4, Y16) and np.array_equal(B4, B16)


def test_power_of_two_scaling():
    G = 64
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((9, 192)) * 0.3).astype(np.float16)
    qx, sx = oa.quantize_activations(X, G)
    for k in (-3, 4):
        qk, sk = oa.quantize_activations((X.astype(np.float64) * 2.0 ** k).astype(np.float16), G)
        assert np.array_equal(qk, qx)
        assert np.array_equal(sk.astype(np.float64), sx.astype(np.float64) * 2.0 ** k)


def test_rejects_bad_inputs():
    with pytest.raises(oracle.OracleInputError):
        oa.quantize_activations(np.zeros((2, 96), np.float16), 64)
    with pytest.raises(oracle.OracleInputError):
        oa.quantize_activations(np.full((1, 32), np.inf, np.float16), 32)
    with pytest.raises(oracle.OracleInputError):
        oa.quantize_activations(np.zeros((2, 64), np.float32), 32)
