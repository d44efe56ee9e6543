// Scalar numerics of the PACE quantiser, usable on host and device so that the CPU
// test suite can check them against exact arithmetic.
//
// Quantiser (PACE summary, "How it differs": channel-aligned key-axis groups with a bf16
// scale, symmetric for PACE-4, integer zero points for PACE-4/8):
//   scale   = bf16 value rounded toward +inf of range / levels,
//   code    = round-half-to-even(x / scale), decided exactly for fp32 x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

namespace pace {

__host__ __device__ inline uint32_t f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u;
}
__host__ __device__ inline float bits_f32(uint32_t u) {
  float x;
  memcpy(&x, &u, 4);
  return x;
}
__host__ __device__ inline uint64_t f64_bits(double x) {
  uint64_t u;
  memcpy(&u, &x, 8);
  return u;
}
__host__ __device__ inline double bits_f64(uint64_t u) {
  double x;
  memcpy(&x, &u, 8);
  return x;
}

// bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern.
__host__ __device__ inline float bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__host__ __device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = f32_bits(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Smallest bf16 value >= d for 0 <= d (finite, below bf16 max).  Exact: the double is
// first rounded up to fp32 (exactly representable results stay put), then the fp32
// pattern is rounded up to its upper 16 bits.
__host__ __device__ inline float bf16_ceil_from_f64(double d) {
  if (!(d > 0.0)) return 0.0f;
  float f = (float)d;                 // round to nearest
  if ((double)f < d) f = bits_f32(f32_bits(f) + 1u);   // next fp32 up (d > 0)
  uint32_t u = f32_bits(f);
  if (u & 0xFFFFu) u = (u + 0x10000u) & 0xFFFF0000u;
  return bits_f32(u);
}

// Correctly rounded m / k from the correctly rounded reciprocal rk = fl(1 / k), in three
// operations (Markstein's correction: q = fl(m rk) is within an ulp of m / k, the
// residual m - q k is exact in one fused multiply-add, and fl(q + residual * rk) is the
// correctly rounded quotient).  Used with the integer divisors 7, 15, 127 and 255, for
// which it agrees with IEEE division on every positive fp32 m.
__host__ __device__ inline float div_rn(float m, float k, float rk) {
  const float q = m * rk;
  const float e = fmaf(-q, k, m);
  return fmaf(e, rk, q);
}

// Smallest bf16 value >= m / k for fp32 m >= 0 and a divisor k in {7, 15, 127, 255}
// (rk = fl(1 / k)), without leaving fp32: q = fl(m / k) is correctly rounded; if q * k < m
// (decided exactly by one fused multiply-add, whose product q * k needs at most 24 + 8
// bits) the quotient was rounded down and q is moved one fp32 ulp up; the result is then
// rounded up to bf16.  Exact because bf16 values are fp32 values.
__host__ __device__ inline float bf16_ceil_div(float m, float k, float rk) {
  if (!(m > 0.0f)) return 0.0f;
  float q = div_rn(m, k, rk);
  if (fmaf(q, k, -m) < 0.0f) q = bits_f32(f32_bits(q) + 1u);
  uint32_t u = f32_bits(q);
  if (u & 0xFFFFu) u = (u + 0x10000u) & 0xFFFF0000u;
  return bits_f32(u);
}

// Correctly rounded 1 / s for a bf16-valued s >= 2^-126 from any estimate r0 within an
// fp32 ulp of it: the residual 1 - r0 s is exact in one fused multiply-add, and one
// Newton step in fma form then rounds correctly for each of the 128 bf16 significands
// (checked exhaustively with exact rationals, for every start within an ulp).
__host__ __device__ inline float rcp_fix(float s, float r0) {
  const float e = fmaf(-r0, s, 1.0f);
  return fmaf(e, r0, r0);
}

// 1 / s, correctly rounded, for a bf16-valued scale 2^-126 <= s <= 2^126 (on the device:
// the hardware reciprocal, within an ulp, and one correction).  Scales below 2^-126 (a
// group whose values all lie under 2^-123 in magnitude) take 1 / 2^-126 instead, which
// keeps x / s bounded by the code range, so their codes stay valid.
__host__ __device__ inline float rcp_bf16(float s) {
  const float c = fmaxf(s, 0x1p-126f);
#if defined(__HIP_DEVICE_COMPILE__)
  return rcp_fix(c, __builtin_amdgcn_rcpf(c));
#else
  return 1.0f / c;
#endif
}

// round-half-to-even(x / s) for fp32 x and a bf16-valued scale s > 0, exactly.
// r = 1/s (any fp32 approximation).  A first guess n = rne(x * r) is within one of the
// answer; the residual e = x - n*s is exact in fp32 (s has 8 significant bits and
// |e| < 2s), so comparing 2e with +-s settles the rounding, ties going to even.
__host__ __device__ inline float rne_quotient(float x, float s, float r) {
  float n = rintf(x * r);
  float e = fmaf(-n, s, x);
  float e2 = 2.0f * e;
  if (e2 > s) {
    n += 1.0f;
    e2 -= 2.0f * s;
  } else if (e2 < -s) {
    n -= 1.0f;
    e2 += 2.0f * s;
  }
  // now |x/s - n| <= 1/2; resolve exact ties to even (n is an integer below 2^24)
  if (e2 == s || e2 == -s) {
    float alt = n + (e2 > 0 ? 1.0f : -1.0f);
    if ((int)n & 1) n = alt;
  }
  return n;
}

// Group parameters of the quantiser from the group's min and max (fp32 pre-rounding
// values).  Symmetric: s = bf16_ceil(max|x| / (2^(b-1)-1)), z = 2^(b-1).  Asymmetric:
// lo = min(0, min), hi = max(0, max), s = bf16_ceil((hi - lo) / (2^b - 1)),
// z = clip(rne(-lo / s), 0, 2^b - 1) decided exactly.  s = 0 gives z = 0 (asym).
struct GroupQuant {
  float s, r;   // scale and its correctly rounded reciprocal (0 when s = 0)
  int z;        // zero point / stored offset
};

__host__ __device__ inline GroupQuant group_quant(float mn, float mx, bool asym, int bits) {
  GroupQuant q;
  const int levels = (1 << bits) - 1, zsym = 1 << (bits - 1);
  if (!asym) {
    const float M = fmaxf(fabsf(mx), fabsf(mn));
    q.s = bf16_ceil_div(M, (float)(zsym - 1), bits == 8 ? 1.0f / 127.0f : 1.0f / 7.0f);
    q.z = zsym;
  } else {
    const float lo = fminf(mn, 0.f), hi = fmaxf(mx, 0.f);
    // hi - lo rounded up to fp32 keeps the ceiling exact: the scale only moves up when
    // the exact range lies above its fp32 rounding.  hi >= 0 >= lo, so with a = the
    // larger and b = the smaller of hi and -lo, the rounding error of a + b is
    // b - (range - a), exactly (Dekker's fast two-sum).
    const float a = fmaxf(hi, -lo), b = fminf(hi, -lo);
    float range = a + b;
    if (b - (range - a) > 0.f) range = bits_f32(f32_bits(range) + 1u);
    q.s = bf16_ceil_div(range, (float)levels, bits == 8 ? 1.0f / 255.0f : 1.0f / 15.0f);
  }
  q.r = q.s > 0.f ? rcp_bf16(q.s) : 0.f;
  if (asym) q.z = q.s > 0.f ? (int)fminf(fmaxf(rne_quotient(-fminf(mn, 0.f), q.s, q.r), 0.f), (float)levels) : 0;
  return q;
}

// Stored code of x: round-half-even(x * r) + z, clipped to [lo, hi] (symmetric:
// [1, 2^b - 1], asymmetric: [0, 2^b - 1]).  One fused multiply-add against the
// constant 1.5 * 2^23 + z leaves the integer in the low mantissa bits (the product
// x * r is exact inside the fma, so the only rounding is the final one); a clamp on the
// bit pattern and a mask finish it.  Versus round-half-even(x / s) this can differ only
// where x / s lies within a few fp32 ulps of a half-integer.
__host__ __device__ inline int code_of(float x, float r, float magic, float lo, float hi) {
  const float f = fminf(fmaxf(fmaf(x, r, magic), lo), hi);
  return (int)(f32_bits(f) & 0xFFu);
}

struct CodeRange {
  float magic, lo, hi;   // 1.5 * 2^23 + z and the clamp bounds in the same domain
};

__host__ __device__ inline CodeRange code_range(int z, bool asym, int bits) {
  CodeRange c;
  const float base = 12582912.0f;       // 1.5 * 2^23: bit pattern 0x4B400000
  c.magic = base + (float)z;
  c.lo = base + (asym ? 0.f : 1.f);
  c.hi = base + (float)((1 << bits) - 1);
  return c;
}

}  // namespace pace
