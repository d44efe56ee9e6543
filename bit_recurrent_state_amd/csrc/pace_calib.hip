// Offline calibration of the head ranking inputs (PACE summary, onedev.kr "How it
// differs": the 8-bit heads are those with the largest retained error
// E_h = e_h / (1 - a_h^(2 dP)), e_h being the error energy one rounding leaves and a_h the
// head's decay; review, "3. Method & Key Results": head-level precision allocation).
//
// For every value head h: run the exact gated-delta recurrence (review, "1. Key Terms &
// Definitions") from S = 0 over T tokens of each of the B calibration sequences, and at
// every dP-th token add the squared Frobenius error of one rounding of S by the layer's
// 4-bit quantiser (channel-aligned key groups of g, bf16 scales rounded up, symmetric or
// asymmetric as configured).  e_h = mean of those energies over all rounding points of all
// sequences; a_h = mean of a_t over all tokens and sequences.
//
// One workgroup (4 wave64s) per head, sequences one after another, so the means need no
// cross-workgroup reduction.  D/8 lanes share a value column, each holding 8 consecutive
// keys of it in fp32 registers.
#include <hip/hip_runtime.h>

#include "pace_internal.h"
#include "pace_numerics.h"

namespace pace {
namespace {

constexpr int kThreads = 256;

template <int W>
__device__ inline float seg_sum(float x) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <bool BF16>
__device__ inline float ld(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  else return ((const float*)p)[i];
}

// Squared error of rounding the lane's 8 keys of one column with the group quantiser; the
// group spans `width` consecutive lanes (g / 8), all of which call this together.
__device__ inline float group_error2(const float x[8], int width, bool asym) {
  float mx = x[0], mn = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) { mx = fmaxf(mx, x[e]); mn = fminf(mn, x[e]); }
  for (int o = width / 2; o > 0; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    mn = fminf(mn, __shfl_xor(mn, o));
  }
  const GroupQuant gq = group_quant(mn, mx, asym, 4);
  const CodeRange cr = code_range(gq.z, asym, 4);
  float e2 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = code_of(x[e], gq.r, cr.magic, cr.lo, cr.hi);
    const float d = gq.s * (float)(c - gq.z) - x[e];
    e2 = fmaf(d, d, e2);
  }
  return e2;
}

template <int D, int IO>
__global__ __launch_bounds__(kThreads) void calib_kernel(CalibParams p) {
  constexpr int LPC = D / 8;                     // lanes per value column
  constexpr int CPB = kThreads / LPC;            // columns per pass
  constexpr int PASSES = D / CPB;
  constexpr bool kBf16 = IO == 1;
  __shared__ double red[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int h = blockIdx.x, kh = h / p.gamma;
  const int m = lane % LPC;                      // keys 8m .. 8m+7
  const int width = p.group / 8;
  const bool asym = p.asym != 0;

  double e_acc = 0.0, a_acc = 0.0;
  int points = 0;
  for (int b = 0; b < p.B; ++b) {
    float S[PASSES][8];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
      for (int e = 0; e < 8; ++e) S[ps][e] = 0.f;
    for (int t = 0; t < p.T; ++t) {
      float kk[8];
      const size_t kb = (((size_t)b * p.T + t) * p.Hk + kh) * D + 8 * m;
#pragma unroll
      for (int e = 0; e < 8; ++e) kk[e] = ld<kBf16>(p.k, kb + e);
      const size_t gi = ((size_t)b * p.T + t) * p.Hv + h;
      const float a = p.a[gi], beta = p.beta[gi];
      if (tid == 0) a_acc += (double)a;
      const bool round_now = (t + 1) % p.dP == 0;
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        const int j = ps * CPB + tid / LPC;
        float sk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sk = fmaf(S[ps][e], kk[e], sk);
        sk = seg_sum<LPC>(sk);
        const float u = beta * (ld<kBf16>(p.v, gi * D + j) - a * sk);
#pragma unroll
        for (int e = 0; e < 8; ++e) S[ps][e] = fmaf(a, S[ps][e], kk[e] * u);
        if (round_now) e_acc += (double)group_error2(S[ps], width, asym);
      }
      if (round_now) ++points;
    }
  }
  // block sum of the error energies
  for (int o = 32; o > 0; o >>= 1) e_acc += __shfl_xor(e_acc, o);
  if (lane == 0) red[wave] = e_acc;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
    p.e_h[h] = points ? tot / points : 0.0;
    p.a_h[h] = a_acc / ((double)p.B * p.T);
  }
}

}  // namespace

hipError_t launch_calib(const CalibParams& p, int dk, int io_bf16, hipStream_t stream) {
  if (dk == 128) {
    if (io_bf16) hipLaunchKernelGGL((calib_kernel<128, 1>), dim3(p.Hv), dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((calib_kernel<128, 0>), dim3(p.Hv), dim3(kThreads), 0, stream, p);
  } else {
    if (io_bf16) hipLaunchKernelGGL((calib_kernel<64, 1>), dim3(p.Hv), dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((calib_kernel<64, 0>), dim3(p.Hv), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pace
