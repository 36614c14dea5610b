// Exact integer arithmetic of the 4-bit quantiser (device code; also builds for the host).
//
// Every fp16 value is an integer multiple of 2^-24, so the packer works in
// "units" of 2^-24 held in 64-bit integers: weights, scales, products s*q and
// base errors e = w - s*q are all exact there (|w| * 2^24 < 2^41). Roundings to
// fp16 / fp32 are done on those integers by the IEEE-754 definition (nearest,
// ties to even), so no floating-point division is involved anywhere.
//
// Readings of the pages (MosaicQuant explainer, Methodology sections 1-2):
// symmetric absmax INT4 with codes in [-7, 7]; fp16 base scale per group,
// fp32 residual scale per row; round-half-to-even everywhere.
#pragma once
#include <cstdint>

#if defined(__HIPCC__)
#define MQ_HD __host__ __device__ __forceinline__
#else
#define MQ_HD inline   // host-only build of the same arithmetic, used by CPU tests
#endif

namespace mq {

// fp16 bit pattern -> value * 2^24 (exact). Inf/NaN patterns are reported by
// the caller; their result here is meaningless.
MQ_HD int64_t fp16_units(uint32_t h) {
  const uint32_t e = (h >> 10) & 31u;
  const uint32_t m = h & 1023u;
  const int64_t mag = (e == 0) ? (int64_t)m : ((int64_t)(1024u + m) << (e - 1));
  return (h & 0x8000u) ? -mag : mag;
}

MQ_HD bool fp16_is_finite(uint32_t h) { return (h & 0x7C00u) != 0x7C00u; }

// Encode a value of V units that is exactly representable in fp16.
MQ_HD uint32_t fp16_encode_exact(uint64_t V) {
  if (V < 1024u) return (uint32_t)V;                     // subnormal: quantum 1 unit
  const int b = 63 - __builtin_clzll(V);              // 2^b <= V < 2^(b+1)
  const uint32_t expf = (uint32_t)(b - 9);               // biased exponent
  if (expf >= 31u) return 0x7C00u;
  const uint32_t mant = (uint32_t)(V >> (b - 10)) - 1024u;
  return (expf << 10) | mant;
}

// Round V units (0 <= V <= 65504 * 2^24) to the nearest fp16, ties to even.
// Returns the fp16 bits; *rounded receives the rounded value in units.
MQ_HD uint32_t fp16_round_units(uint64_t V, uint64_t* rounded) {
  if (V < 2048u) { *rounded = V; return fp16_encode_exact(V); }   // quantum is 1 unit below 2^-13
  const int b = 63 - __builtin_clzll(V);
  const int sh = b - 10;                                 // quantum 2^sh units
  uint64_t m = V >> sh;
  const uint64_t rem = V & ((1ull << sh) - 1ull);
  const uint64_t half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (m & 1ull))) ++m;
  const uint64_t R = m << sh;
  *rounded = R;
  return fp16_encode_exact(R);
}

// fp16 nearest to A/7 units (A >= 0), ties to even. *S receives it in units.
MQ_HD uint32_t fp16_div7(uint64_t A, uint64_t* S) {
  const uint64_t t = A / 7u;
  int Q = 0;                                            // quantum 2^Q units
  if (t >= 2048u) Q = (63 - __builtin_clzll(t)) - 10;
  const uint64_t den = 7ull << Q;
  uint64_t m = (A >> Q) / 7u;                           // floor(A / (7 * 2^Q))
  const uint64_t rem = A - m * den;
  if (2u * rem > den || (2u * rem == den && (m & 1ull))) ++m;
  const uint64_t V = m << Q;
  *S = V;
  return fp16_encode_exact(V);
}

// fp32 nearest to Mx/7 units (Mx >= 0), ties to even. Returns fp32 bits and
// the value as m * 2^Q units (m = 0 for zero).
MQ_HD uint32_t fp32_div7(uint64_t Mx, uint64_t* m_out, int* Q_out) {
  if (Mx == 0) { *m_out = 0; *Q_out = 0; return 0u; }
  const int b = 63 - __builtin_clzll(Mx);
  int L = b - 2;                                        // floor(log2(Mx/7)) is b-2 or b-3
  const bool ge = (b >= 2) ? (Mx >= (7ull << (b - 2))) : ((Mx << (2 - b)) >= 7u);
  if (!ge) L = b - 3;
  int Q = L - 23;
  uint64_t m, rem, den;
  if (Q >= 0) {
    den = 7ull << Q;
    m = (Mx >> Q) / 7u;
    rem = Mx - m * den;
  } else {
    const uint64_t num = Mx << (-Q);                    // < 7 * 2^24
    den = 7u;
    m = num / 7u;
    rem = num - 7u * m;
  }
  if (2u * rem > den || (2u * rem == den && (m & 1ull))) ++m;
  if (m == (1ull << 24)) { m = 1ull << 23; ++Q; }
  *m_out = m;
  *Q_out = Q;
  return ((uint32_t)(Q + 126) << 23) | (uint32_t)(m - (1ull << 23));
}

// fp32 bits of a positive normal value -> m * 2^Q units.
MQ_HD void fp32_units(uint32_t bits, uint64_t* m, int* Q) {
  if (bits == 0u) { *m = 0; *Q = 0; return; }
  *m = (1ull << 23) | (bits & 0x7FFFFFu);
  *Q = (int)((bits >> 23) & 0xFFu) - 126;
}

// clamp(rne(a / S), -7, 7) for a signed numerator and a positive denominator,
// both integers; 0 when S == 0. Compares 2|a| with (2n+1) S, n = 0..6.
MQ_HD int quant7(int64_t a, uint64_t S) {
  if (S == 0u) return 0;
  const uint64_t two_a = 2u * (uint64_t)(a < 0 ? -a : a);
  uint64_t t = S;
  int cnt = 0;
  bool tie = false;
#pragma unroll
  for (int n = 0; n < 7; ++n) {
    cnt += (two_a > t) ? 1 : 0;
    tie |= (two_a == t);
    t += 2u * S;
  }
  const int qm = cnt + ((tie && (cnt & 1)) ? 1 : 0);
  return a < 0 ? -qm : qm;
}

// Residual code: clamp(rne(e / sr), -7, 7) with sr = m * 2^Q units.
MQ_HD int quant7_scaled(int64_t e, uint64_t m, int Q) {
  if (m == 0u) return 0;
  if (Q >= 0) return quant7(e, m << Q);
  return quant7(e * (int64_t)(1ull << (-Q)), m);
}

// fp16 bits of fp16_rne(a / 7) for a finite fp16 magnitude a given by its
// bit pattern h (sign clear), in 32-bit integers (the activation quantizer's
// form of fp16_div7). a = m 2^E with m the significand; m 2^16 / 7 = t +
// rem / 7 holds 14..27 bits, rounded to 11 significant bits, or to the 2^-24
// quantum below the normal range, with rem as the sticky part.
MQ_HD uint32_t fp16_div7_h(uint32_t h) {
  if (h == 0u) return 0u;
  const uint32_t e5 = h >> 10, m10 = h & 1023u;
  const uint32_t m = e5 ? (1024u | m10) : m10;
  const int E = (int)(e5 ? e5 : 1u) - 25;
  const uint32_t n = m << 16;
  const uint32_t t = n / 7u, rem = n - 7u * t;
  const int L = 32 - __builtin_clz(t);
  int sh = L - 11;
  if (-8 - E > sh) sh = -8 - E;          // keeps the result's quantum >= 2^-24 (sh <= 16)
  uint32_t r = t >> sh;
  const uint32_t low = t & ((1u << sh) - 1u), half = 1u << (sh - 1);
  if (low > half || (low == half && (rem != 0u || (r & 1u)))) ++r;
  int F = sh + E - 16;                    // result = r 2^F
  if (r == 2048u) {
    r = 1024u;
    ++F;
  }
  return r >= 1024u ? (((uint32_t)(F + 25) << 10) | (r - 1024u)) : r;   // normal, or subnormal at F = -24
}

// clamp(rne(x / s), -7, 7) for fp16 values held as floats, s >= 0 (0 when
// s == 0). The estimate |x| (1 / s) is within one of the answer; the
// decision itself compares 2 |x| with (2 n +- 1) s, products of at most 15
// significant bits and so exact in fp32 (ties go to the even code).
MQ_HD int quant7_f(float x, float s) {
  if (!(s > 0.0f)) return 0;
  const float ax = x < 0.0f ? -x : x;
  const float a2 = 2.0f * ax;
  int n = (int)(ax * (1.0f / s) + 0.5f);
  if (n > 7) n = 7;
  if (n > 0) {
    const float b = (float)(2 * n - 1) * s;
    if (a2 < b || (a2 == b && (n & 1))) --n;
  }
  if (n < 7) {
    const float b = (float)(2 * n + 1) * s;
    if (a2 > b || (a2 == b && (n & 1))) ++n;
  }
  return x < 0.0f ? -n : n;
}

// Order-preserving 64-bit key of |e| (|e| in units, < 2^41): the bits of the
// exact double. The low 12 bits are always zero.
MQ_HD uint64_t err_key(uint64_t abs_e) {
  return __builtin_bit_cast(uint64_t, (double)abs_e);
}

}  // namespace mq
