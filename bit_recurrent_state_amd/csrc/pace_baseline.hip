// Per-token bf16-state gated-delta decode: the comparator of the PACE throughput study
// (PACE summary, onedev.kr "Assumptions and limits": periodic INT4 decode is timed
// against per-token bf16 decode, which reads and writes the bf16 state every token).
//
// State layout: bf16 [B][Hv][dv][dk], value-column-major.  One workgroup (4 waves) per
// (sequence, head); D/8 lanes share a column, each holding 8 consecutive keys, so every
// wave instruction moves contiguous 1 KB.  Per token:
//   u = beta (v - a S^T k);  S' = a S + k u^T;  o = S'^T q;  S <- bf16_rne(S').
#include <hip/hip_runtime.h>

#include "pace_internal.h"
#include "pace_numerics.h"

namespace pace {
namespace {

typedef unsigned v4u32 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <int LPC>
__device__ inline float seg_sum(float x) {
#pragma unroll
  for (int o = LPC / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// NTS: the state is read and written non-temporally (chosen by state size, as for the
// int4 kernel).
template <int D, int IO, bool NTS>
__global__ __launch_bounds__(kThreads) void bf16_decode_kernel(Bf16Params p) {
  constexpr int LPC = D / 8;                 // lanes per column
  constexpr int CPW = 64 / LPC;              // columns per wave per pass
  constexpr int CPB = CPW * (kThreads / 64); // columns per workgroup per pass
  constexpr int PASSES = D / CPB;
  constexpr bool kBf16 = IO == 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int b = blockIdx.x / p.Hv, h = blockIdx.x % p.Hv, kh = h / p.gamma;
  const int m = lane % LPC;                  // keys 8m .. 8m+7
  float kk[8], qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const size_t i = ((size_t)b * p.Hk + kh) * D + 8 * m + e;
    kk[e] = kBf16 ? bf16_to_f32(((const uint16_t*)p.k)[i]) : ((const float*)p.k)[i];
    qv[e] = kBf16 ? bf16_to_f32(((const uint16_t*)p.q)[i]) : ((const float*)p.q)[i];
  }
  const float a = p.a[(size_t)b * p.Hv + h], beta = p.beta[(size_t)b * p.Hv + h];
  uint16_t* tile = p.state + ((size_t)b * p.Hv + h) * D * D;
#pragma unroll 2
  for (int pass = 0; pass < PASSES; ++pass) {
    const int j = pass * CPB + wave * CPW + lane / LPC;
    uint4* src = (uint4*)(tile + (size_t)j * D + 8 * m);
    // the state is a stream (read and written once per launch); when it is large,
    // non-temporal accesses keep it from displacing reused data, as in the int4 kernel
    uint4 raw;
    if constexpr (NTS) {
      const v4u32 rv = __builtin_nontemporal_load((const v4u32*)src);
      raw = make_uint4(rv.x, rv.y, rv.z, rv.w);
    } else {
      raw = *src;
    }
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float s[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[2 * e] = bits_f32(w[e] << 16);
      s[2 * e + 1] = bits_f32(w[e] & 0xFFFF0000u);
    }
    float dk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dk += s[e] * kk[e];
    dk = seg_sum<LPC>(dk);
    const size_t vi = ((size_t)b * p.Hv + h) * D + j;
    const float vj = kBf16 ? bf16_to_f32(((const uint16_t*)p.v)[vi]) : ((const float*)p.v)[vi];
    const float u = beta * (vj - a * dk);
    float oq = 0.f;
    uint32_t outw[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[e] = a * s[e] + kk[e] * u;
      oq += s[e] * qv[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      outw[e] = (uint32_t)f32_to_bf16_rne(s[2 * e]) | ((uint32_t)f32_to_bf16_rne(s[2 * e + 1]) << 16);
    if constexpr (NTS) __builtin_nontemporal_store(v4u32{outw[0], outw[1], outw[2], outw[3]}, (v4u32*)src);
    else *src = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    oq = seg_sum<LPC>(oq);
    if (m == 0) {
      if (kBf16) ((uint16_t*)p.o)[vi] = f32_to_bf16_rne(oq);
      else ((float*)p.o)[vi] = oq;
    }
  }
}

}  // namespace

hipError_t launch_bf16_decode(const Bf16Params& p, int dk, int dv, int io_bf16,
                              hipStream_t stream) {
  (void)dv;
  const unsigned grid = (unsigned)p.B * (unsigned)p.Hv;
  // the same rule as the int4 kernel: stream the state once a layer's state reaches 8 MiB
  const bool nts = (uint64_t)p.B * p.Hv * dk * dk * 2 >= (8ull << 20);
  if (dk == 128) {
    if (io_bf16) {
      if (nts) hipLaunchKernelGGL((bf16_decode_kernel<128, 1, true>), dim3(grid), dim3(kThreads), 0, stream, p);
      else hipLaunchKernelGGL((bf16_decode_kernel<128, 1, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    } else {
      if (nts) hipLaunchKernelGGL((bf16_decode_kernel<128, 0, true>), dim3(grid), dim3(kThreads), 0, stream, p);
      else hipLaunchKernelGGL((bf16_decode_kernel<128, 0, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    }
  } else {
    if (io_bf16) {
      if (nts) hipLaunchKernelGGL((bf16_decode_kernel<64, 1, true>), dim3(grid), dim3(kThreads), 0, stream, p);
      else hipLaunchKernelGGL((bf16_decode_kernel<64, 1, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    } else {
      if (nts) hipLaunchKernelGGL((bf16_decode_kernel<64, 0, true>), dim3(grid), dim3(kThreads), 0, stream, p);
      else hipLaunchKernelGGL((bf16_decode_kernel<64, 0, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    }
  }
  return hipGetLastError();
}

}  // namespace pace
