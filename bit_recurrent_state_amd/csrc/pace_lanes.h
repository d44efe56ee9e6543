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
