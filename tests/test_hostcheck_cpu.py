"""The packer's exact integer arithmetic (quant_exact.h), built for the host,
checked against exact rational arithmetic and the pinned oracle. The GPU
packer compiles the same header, so this catches arithmetic mistakes before
any GPU run."""
import ctypes
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._exact import all_finite_fp16, fp16_exact, fp32_exact, round_half_even

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HC = os.path.join(ROOT, "bit_gemm_amd", "libmq_hostcheck.so")
U = 2 ** 24   # one unit = 2^-24


@pytest.fixture(scope="module")
def hc():
    assert os.path.exists(HC), "libmq_hostcheck.so is not built"
    h = ctypes.CDLL(HC)
    u64, i64 = ctypes.c_uint64, ctypes.c_int64
    h.mqh_fp16_units.argtypes = [ctypes.c_uint32]
    h.mqh_fp16_units.restype = i64
    h.mqh_fp16_div7.argtypes = [u64, ctypes.POINTER(u64)]
    h.mqh_fp16_div7.restype = ctypes.c_uint32
    h.mqh_fp16_round_units.argtypes = [u64, ctypes.POINTER(u64)]
    h.mqh_fp16_round_units.restype = ctypes.c_uint32
    h.mqh_fp32_div7.argtypes = [u64, ctypes.POINTER(u64), ctypes.POINTER(ctypes.c_int)]
    h.mqh_fp32_div7.restype = ctypes.c_uint32
    h.mqh_quant7.argtypes = [i64, u64]
    h.mqh_quant7.restype = ctypes.c_int
    h.mqh_quant7_scaled.argtypes = [i64, u64, ctypes.c_int]
    h.mqh_quant7_scaled.restype = ctypes.c_int
    h.mqh_err_key.argtypes = [u64]
    h.mqh_err_key.restype = u64
    h.mqh_fp16_div7_h.argtypes = [ctypes.c_uint32]
    h.mqh_fp16_div7_h.restype = ctypes.c_uint32
    h.mqh_quant7_f.argtypes = [ctypes.c_float, ctypes.c_float]
    h.mqh_quant7_f.restype = ctypes.c_int
    return h


def _bits16(x):
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def test_fp16_units_exact_for_every_finite_fp16(hc):
    for v in all_finite_fp16().tolist():
        assert Fraction(hc.mqh_fp16_units(_bits16(v)), U) == Fraction(v)


def test_fp16_div7_matches_oracle_and_definition_for_every_absmax(hc):
    vals = all_finite_fp16()
    pos = vals[vals >= 0]
    ref = oracle.to_fp16_rne(pos.astype(np.float64) / 7.0)
    S = ctypes.c_uint64()
    for a, r in zip(pos.tolist(), ref.tolist()):
        A = hc.mqh_fp16_units(_bits16(a))
        bits = hc.mqh_fp16_div7(A, ctypes.byref(S))
        assert bits == _bits16(r), a
        assert Fraction(S.value, U) == fp16_exact(Fraction(a) / 7)


def test_fp16_round_units(hc):
    rng = np.random.default_rng(1)
    R = ctypes.c_uint64()
    # domain: the finite fp16 range (the packer rejects scales with 7 s > 65504)
    for V in list(range(0, 5000)) + rng.integers(0, 65504 * U + 1, 20000).tolist():
        bits = hc.mqh_fp16_round_units(V, ctypes.byref(R))
        ex = fp16_exact(Fraction(V, U))
        assert Fraction(R.value, U) == ex
        assert bits == _bits16(float(ex))


def test_fp32_div7_matches_oracle_and_definition(hc):
    rng = np.random.default_rng(2)
    m, Q = ctypes.c_uint64(), ctypes.c_int()
    Ms = list(range(0, 3000)) + rng.integers(1, 2 ** 41, 20000).tolist()
    ref = oracle.to_fp32_rne(np.array(Ms, dtype=np.float64) * 2.0 ** -24 / 7.0)
    for Mx, r in zip(Ms, ref.tolist()):
        bits = hc.mqh_fp32_div7(Mx, ctypes.byref(m), ctypes.byref(Q))
        assert bits == int(np.array([r], np.float32).view(np.uint32)[0]), Mx
        val = Fraction(m.value) * Fraction(2) ** Q.value / U
        assert val == fp32_exact(Fraction(Mx, 7 * U))


def test_quant7_is_clamped_rne(hc):
    rng = np.random.default_rng(3)
    for _ in range(20000):
        S = int(rng.integers(1, 2 ** 38))
        a = int(rng.integers(-8 * S, 8 * S + 1))
        assert hc.mqh_quant7(a, S) == max(-7, min(7, round_half_even(Fraction(a, S))))
    # exact half steps: (n + 1/2) S
    for S in (2, 6, 1000, 2 ** 37 + 2):
        for n in range(-8, 8):
            a2 = (2 * n + 1) * S
            if a2 % 2:
                continue
            assert hc.mqh_quant7(a2 // 2, S) == max(-7, min(7, round_half_even(Fraction(a2, 2 * S))))
    assert hc.mqh_quant7(12345, 0) == 0


def test_quant7_scaled_matches_oracle_residual_codes(hc):
    """Residual codes from the integer route equal the oracle's float64 codes."""
    rng = np.random.default_rng(4)
    m, Q = ctypes.c_uint64(), ctypes.c_int()
    for _ in range(300):
        Mx = int(rng.integers(1, 2 ** 40))
        es = rng.integers(-Mx, Mx + 1, 40)
        hc.mqh_fp32_div7(Mx, ctypes.byref(m), ctypes.byref(Q))
        sr = oracle.to_fp32_rne(np.array([Mx * 2.0 ** -24 / 7.0]))
        e = (es.astype(np.float64) * 2.0 ** -24)[None, :]
        ref = oracle.residual_codes(e, np.arange(es.size), np.repeat(sr, 1))
        got = [hc.mqh_quant7_scaled(int(v), m.value, Q.value) for v in es.tolist()]
        assert got == ref.tolist()


def test_err_key_preserves_order(hc):
    rng = np.random.default_rng(5)
    v = np.unique(np.concatenate([np.arange(0, 100), rng.integers(0, 2 ** 41, 5000)]))
    keys = [hc.mqh_err_key(int(x)) for x in v.tolist()]
    assert keys == sorted(keys)
    assert all((k & 0xFFF) == 0 for k in keys)


def test_fp16_div7_h_matches_the_oracle_scale_for_every_fp16(hc):
    # the activation quantizer's 32-bit scale rule, for every finite fp16
    # magnitude, against the oracle's fp16(a / 7) and exact rational rounding
    mags = all_finite_fp16()
    mags = np.unique(np.abs(mags))
    want = oracle.to_fp16_rne(mags.astype(np.float64) / 7).view(np.uint16)
    bits = mags.astype(np.float16).view(np.uint16)
    got = np.array([hc.mqh_fp16_div7_h(int(b)) for b in bits.tolist()], dtype=np.uint16)
    assert np.array_equal(got, want)
    for v in mags[::97].tolist():
        assert Fraction(float(np.uint16(hc.mqh_fp16_div7_h(_bits16(v))).view(np.float16))) == \
            fp16_exact(Fraction(v) / 7)


def test_quant7_f_matches_the_oracle_codes(hc):
    # random fp16 pairs over the whole range, every scale's ties (x = (n + 1/2) s)
    # and values just beside them, against clamp(rint(x / s)) in float64
    rng = np.random.default_rng(5)
    s = np.abs(rng.standard_normal(4000) * np.exp2(rng.integers(-26, 14, 4000))).astype(np.float16)
    s = s[(s > 0) & np.isfinite(s)]
    xs, ss = [], []
    ties = 0
    for sv in s[:600].tolist():
        for n in range(8):
            t = np.float64(sv) * (n + 0.5)
            h = np.float16(t)
            if not np.isfinite(h):
                continue
            cands = [np.nextafter(h, np.float16(np.inf)), np.nextafter(h, np.float16(0))]
            if np.float64(h) == t:                      # the midpoint itself is an fp16 value: a tie
                cands.append(h)
                ties += 1
            for x in cands:
                if np.isfinite(x):
                    xs.append(x); ss.append(sv)
    assert ties > 300
    x = np.concatenate([np.array(xs, dtype=np.float16),
                        (rng.standard_normal(20000) * 7 * np.repeat(s[:200], 100)[:20000]).astype(np.float16)])
    sv = np.concatenate([np.array(ss, dtype=np.float16), np.repeat(s[:200], 100)[:20000]])
    ok = np.isfinite(x)
    x, sv = x[ok], sv[ok]
    x = np.where(np.random.default_rng(1).random(x.size) < 0.5, -x, x).astype(np.float16)
    want = np.clip(np.rint(x.astype(np.float64) / sv.astype(np.float64)), -7, 7).astype(int)
    got = np.array([hc.mqh_quant7_f(float(a), float(b)) for a, b in zip(x.tolist(), sv.tolist())])
    assert np.array_equal(got, want)
    assert hc.mqh_quant7_f(3.0, 0.0) == 0
