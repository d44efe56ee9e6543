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
  // now |x/s - n| <= 1/2; resolve exact ties to even
  if (e2 == s || e2 == -s) {
    float alt = n + (e2 > 0 ? 1.0f : -1.0f);
    if (fmodf(n, 2.0f) != 0.0f) n = alt;
  }
  return n;
}

}  // namespace pace
