// Chunked prefill with one rounding per chunk (PACE summary, onedev.kr "How it works":
// the prefill rounding period equals the chunk kernel's chunk length, 256 tokens; news
// item "Two observations": chunked prefill writes the state once per chunk).
//
// This kernel runs the exact recurrence token by token inside each chunk with the
// unrounded fp32 state held in registers, emits o_t from the post-update state, and
// requantises the state into the packed record after every `chunk` tokens and after the
// last token.  One workgroup (4 waves) per (sequence, value head); D/8 lanes share a
// value column, each holding 8 consecutive keys.
#include <hip/hip_runtime.h>

#include "pace_internal.h"
#include "pace_numerics.h"

namespace pace {
namespace {

constexpr int kThreads = 256;

template <int LPC>
__device__ inline float seg_sum(float x) {
#pragma unroll
  for (int o = LPC / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ inline float seg_max(float x, int width) {
  for (int o = width / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float seg_min(float x, int width) {
  for (int o = width / 2; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o));
  return x;
}

template <bool BF16>
__device__ inline float ld(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  else return ((const float*)p)[i];
}

struct Rec {
  uint8_t* base;
  uint16_t* scales;
  uint8_t* zeros;
  int bits, NG, group, asym;
};

// Packed-record position of the 8 keys 8m..8m+7 of column j: the unit u whose base key
// is 8m, i.e. u = (m mod 4) * (D/32) + m / 4.
template <int D>
__device__ inline uint8_t* unit_ptr(const Rec& r, int j, int m) {
  const int KB = D / 32;
  const int u = (m & 3) * KB + (m >> 2);
  return r.base + (size_t)j * (D * r.bits / 8) + u * r.bits;
}

template <int D>
__device__ inline void dequant_unit(const Rec& r, int j, int m, float x[8]) {
  const uint8_t* up = unit_ptr<D>(r, j, m);
  const int G = (8 * m) / r.group;
  const float s = bf16_to_f32(r.scales[j * r.NG + G]);
  int z;
  if (r.asym) {
    const int e = j * r.NG + G;
    z = r.bits == 8 ? (int)r.zeros[e] : (int)((r.zeros[e >> 1] >> (4 * (e & 1))) & 15);
  } else {
    z = 1 << (r.bits - 1);
  }
  if (r.bits == 4) {
    const uint32_t d = *(const uint32_t*)up;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s * (float)((int)((d >> (8 * (e & 3) + 4 * (e >> 2))) & 15) - z);
  } else {
    const uint2 d = *(const uint2*)up;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = e < 4 ? d.x : d.y;
      x[e] = s * (float)((int)((w >> (8 * (e & 3))) & 255) - z);
    }
  }
}

// Requantise the lane's 8 keys of column j (group of g/8 lanes), write codes, scale and
// zero point, and replace x by its dequantised value.
template <int D>
__device__ inline void requant_unit(const Rec& r, int j, int m, float x[8]) {
  const int width = r.group / 8;       // lanes per group
  float mx = x[0], mn = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) { mx = fmaxf(mx, x[e]); mn = fminf(mn, x[e]); }
  mx = seg_max(mx, width);
  mn = seg_min(mn, width);
  const int levels = (1 << r.bits) - 1, zsym = 1 << (r.bits - 1);
  const float qmax = (float)(zsym - 1);
  float sn;
  int z;
  if (!r.asym) {
    sn = bf16_ceil_from_f64((double)fmaxf(fabsf(mx), fabsf(mn)) / (double)qmax);
    z = zsym;
  } else {
    const float lo = fminf(mn, 0.f), hi = fmaxf(mx, 0.f);
    sn = bf16_ceil_from_f64(((double)hi - (double)lo) / (double)levels);
    z = sn > 0.f ? (int)fminf(fmaxf(rne_quotient(-lo, sn, 1.f / sn), 0.f), (float)levels) : 0;
  }
  const float rcp = sn > 0.f ? 1.f / sn : 0.f;
  int code[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (sn == 0.f) code[e] = r.asym ? 0 : zsym;
    else if (!r.asym) code[e] = (int)fminf(fmaxf(rne_quotient(x[e], sn, rcp), -qmax), qmax) + zsym;
    else code[e] = (int)fminf(fmaxf(rne_quotient(x[e], sn, rcp) + (float)z, 0.f), (float)levels);
    x[e] = sn * (float)(code[e] - z);
  }
  uint8_t* up = unit_ptr<D>(r, j, m);
  if (r.bits == 4) {
    uint32_t d = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) d |= (uint32_t)code[e] << (8 * (e & 3) + 4 * (e >> 2));
    *(uint32_t*)up = d;
  } else {
    uint32_t d0 = 0, d1 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) { d0 |= (uint32_t)code[e] << (8 * e); d1 |= (uint32_t)code[e + 4] << (8 * e); }
    *(uint2*)up = make_uint2(d0, d1);
  }
  const int G = (8 * m) / r.group;
  const int zn = __shfl_down(z, width, 64);     // zero point of group G+1 (next lanes)
  if (m % width == 0) {
    r.scales[j * r.NG + G] = (uint16_t)(f32_bits(sn) >> 16);
    if (r.asym) {
      const int e = j * r.NG + G;
      if (r.bits == 8) r.zeros[e] = (uint8_t)z;
      else if ((e & 1) == 0) r.zeros[e >> 1] = (uint8_t)(z | (zn << 4));
    }
  }
}

template <int D, int IO>
__global__ __launch_bounds__(kThreads) void prefill_seq_kernel(PrefillParams p) {
  constexpr int LPC = D / 8;
  constexpr int CPW = 64 / LPC;
  constexpr int CPB = CPW * (kThreads / 64);
  constexpr int PASSES = D / CPB;
  constexpr bool kBf16 = IO == 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.Hv, h = blockIdx.x % p.Hv, kh = h / p.gamma;
  const int m = lane % LPC;

  const bool is8 = (p.mask8 >> h) & 1ull;
  const uint64_t below = h ? (p.mask8 & ((1ull << h) - 1ull)) : 0ull;
  const uint64_t n8 = (uint64_t)__popcll(below);
  Rec r;
  r.base = p.state + (uint64_t)b * p.seq_stride + (uint64_t)h * p.rec4 + n8 * (p.rec8 - p.rec4);
  r.scales = (uint16_t*)(r.base + (is8 ? p.scales_off8 : p.scales_off4));
  r.zeros = r.base + (is8 ? p.zeros_off8 : p.zeros_off4);
  r.bits = is8 ? 8 : 4;
  r.NG = D / p.group;
  r.group = p.group;
  r.asym = p.asym;

  float S[PASSES][8];
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int j = pass * CPB + wave * CPW + lane / LPC;
    dequant_unit<D>(r, j, m, S[pass]);
  }
  for (int t = 0; t < p.T; ++t) {
    float kk[8], qv[8];
    const size_t kbase = (((size_t)b * p.T + t) * p.Hk + kh) * D + 8 * m;
#pragma unroll
    for (int e = 0; e < 8; ++e) { kk[e] = ld<kBf16>(p.k, kbase + e); qv[e] = ld<kBf16>(p.q, kbase + e); }
    const size_t gi = ((size_t)b * p.T + t) * p.Hv + h;
    const float a = p.a[gi], beta = p.beta[gi];
    const bool round_now = ((t + 1) % p.chunk == 0) || (t == p.T - 1);
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int j = pass * CPB + wave * CPW + lane / LPC;
      float dk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dk += S[pass][e] * kk[e];
      dk = seg_sum<LPC>(dk);
      const size_t vi = gi * D + j;
      const float u = beta * (ld<kBf16>(p.v, vi) - a * dk);
      float oq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        S[pass][e] = a * S[pass][e] + kk[e] * u;
        oq += S[pass][e] * qv[e];
      }
      oq = seg_sum<LPC>(oq);
      if (m == 0) {
        if (kBf16) ((uint16_t*)p.o)[vi] = f32_to_bf16_rne(oq);
        else ((float*)p.o)[vi] = oq;
      }
      if (round_now) requant_unit<D>(r, j, m, S[pass]);
    }
  }
}

}  // namespace

size_t prefill_workspace_bytes(int B, int Hv, int dk, int dv, int T, int chunk) {
  (void)B; (void)Hv; (void)dk; (void)dv; (void)T; (void)chunk;
  return 0;
}

hipError_t launch_prefill(const PrefillParams& p, int dk, int dv, int io_bf16, hipStream_t stream) {
  (void)dv;
  const unsigned grid = (unsigned)p.B * (unsigned)p.Hv;
  if (dk == 128) {
    if (io_bf16) hipLaunchKernelGGL((prefill_seq_kernel<128, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((prefill_seq_kernel<128, 0>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else {
    if (io_bf16) hipLaunchKernelGGL((prefill_seq_kernel<64, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((prefill_seq_kernel<64, 0>), dim3(grid), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pace
