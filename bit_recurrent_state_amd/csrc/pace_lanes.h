// Exchanges between the four 16-lane rows of a wave64 on the vector ALU (gfx950's lane
// swaps), in place of LDS permutes on the rounding paths.
//
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with the even
// rows of its second; v_permlane32_swap does the same with 32-lane halves.  Given the same
// value x as both operands, a lane of row r (0..3) therefore receives
//   pair16(x) = { x of row r & ~1, x of row r | 1 },
//   pair32(x) = { x of row r & 1,  x of row r | 2 }   (rows 0/1 and 2/3 of the lower / upper half).
// Every lane of the wave must be active.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pace {

struct LanePair {
  uint32_t lo, hi;   // value of the lower / upper row of the pair
};

__device__ inline LanePair pair16(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return {r[0], r[1]};
}

__device__ inline LanePair pair32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return {r[0], r[1]};
}

// Maximum / minimum over the four rows; every lane of a 16-lane column ends with it.
__device__ inline float rows_max(float x) {
  const LanePair a = pair16(__float_as_uint(x));
  x = fmaxf(__uint_as_float(a.lo), __uint_as_float(a.hi));
  const LanePair b = pair32(__float_as_uint(x));
  return fmaxf(__uint_as_float(b.lo), __uint_as_float(b.hi));
}

__device__ inline float rows_min(float x) {
  const LanePair a = pair16(__float_as_uint(x));
  x = fminf(__uint_as_float(a.lo), __uint_as_float(a.hi));
  const LanePair b = pair32(__float_as_uint(x));
  return fminf(__uint_as_float(b.lo), __uint_as_float(b.hi));
}

// Reduce-scatter over the four rows for NG groups at once (NG = 1, 2 or 4): x[g] is the
// lane's own value of group g; the lane of row r returns the reduction (op = max or min)
// of group r mod NG over the four rows of its column.  The first swap pairs rows r and
// r ^ 1 and leaves each even row group 0 (2) and each odd row group 1 (3) of the pair;
// the second pairs rows r and r ^ 2.  Three swaps for four groups, instead of two per group.
template <int NG, bool MAX>
__device__ inline float rows_reduce_own(const float (&x)[4]) {
  auto op = [](float u, float v) { return MAX ? fmaxf(u, v) : fminf(u, v); };
  auto f = [](uint32_t u) { return __uint_as_float(u); };
  if constexpr (NG == 1) {
    const LanePair a = pair16(__float_as_uint(x[0]));
    const float y = op(f(a.lo), f(a.hi));
    const LanePair b = pair32(__float_as_uint(y));
    return op(f(b.lo), f(b.hi));
  } else {
    // even rows keep group 0, odd rows group 1 (of this pair of rows)
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[0]), __float_as_uint(x[1]), false, false);
    const float p = op(f(a[0]), f(a[1]));
    if constexpr (NG == 2) {
      const LanePair b = pair32(__float_as_uint(p));
      return op(f(b.lo), f(b.hi));
    } else {
      // even rows keep group 2, odd rows group 3
      const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[2]), __float_as_uint(x[3]), false, false);
      const float q = op(f(c[0]), f(c[1]));
      // lower rows keep p (groups 0 / 1), upper rows q (groups 2 / 3)
      const auto d = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(q), false, false);
      return op(f(d[0]), f(d[1]));
    }
  }
}

// Value of row g of the lane's column, for every g < ng (ng = 1, 2 or 4, uniform across
// the wave), where row r holds the value of g = r mod ng: out[g].
__device__ inline void rows_gather(uint32_t x, int ng, uint32_t (&out)[4]) {
  out[0] = out[1] = out[2] = out[3] = x;
  if (ng == 2) {
    const LanePair a = pair16(x);
    out[0] = a.lo;
    out[1] = a.hi;
  } else if (ng == 4) {
    const LanePair a = pair16(x);
    const LanePair e = pair32(a.lo), o = pair32(a.hi);
    out[0] = e.lo;
    out[1] = o.lo;
    out[2] = e.hi;
    out[3] = o.hi;
  }
}

}  // namespace pace
