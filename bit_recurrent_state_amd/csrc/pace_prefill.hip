// Chunked prefill with one rounding per chunk (PACE summary, onedev.kr "How it works":
// the prefill rounding period equals the chunk kernel's chunk length, 256 tokens; news
// item "Two observations": chunked prefill writes the state once per chunk).
//
// WY form of the gated delta rule (review, "1. Key Terms & Definitions": u_t =
// beta_t (v_t - a_t S^T k_t), S_t = a_t S + k_t u_t^T), applied to sub-blocks of 64
// tokens with the state kept unrounded in fp32 between sub-blocks and rounded only at
// chunk boundaries and after the call's last token.  For a sub-block with cumulative
// log-decays g_t (Gamma_t = e^{g_t}) and starting state S:
//   A = strictly lower [beta_t e^{g_t - g_i} k_t . k_i]
//   (I + A) U = diag(beta) V - diag(beta Gamma) K S                   (forward solve)
// The solve is blocked by 16 tokens: the four 16x16 unit-lower diagonal blocks are
// inverted by substitution, and U_i = (I + A_ii)^{-1} (R_i - sum_{j<i} A_ij U_j) runs on
// MFMA with U kept in accumulators.
//   O = diag(Gamma) Q S + (lower-incl [e^{g_t - g_i} q_t . k_i]) U
//   S' = Gamma_end S + K^T diag(e^{g_end - g}) U
// which is the token loop's result exactly in real arithmetic.  The state must stay
// accurate to ~1e-5 relative for the rounding decisions at the chunk end, so every
// contraction is fp32-accurate: with bf16 inputs, K K^T and Q K^T are single bf16 MFMA
// passes (exact products), K S, Q S and K^T (decayed U) take the fp32 operand as three
// bf16 pieces (v_mfma_f32_16x16x32_bf16), and the small P U and solve products use
// v_mfma_f32_16x16x4_f32; with fp32 inputs everything uses the fp32 MFMA.
//
// One workgroup (4 wave64s) per (sequence, value head) and block of D/CS value columns:
// the recurrence is independent per value column (keys and gates are shared, the
// rounding groups run along the keys of one column), so when twice the (sequence, head)
// pairs still fit the CUs in one round, CS = 2 splits each one over two workgroups that
// repeat only the key-side work (Gram, query-key tiles, the triangular solve).  The
// state S lives in the MFMA accumulators for the whole call: wave w owns its block's
// value columns [w DC/4, (w+1) DC/4) (DC = D/CS), all keys;
// lane l of a 16x16 accumulator tile holds rows 4(l/16)+r, column l%16.  Contractions over
// keys use those accumulators directly as the B operand, pairing them with an A operand
// read in the matching (permuted) key order.  The next sub-block's inputs are prefetched
// into registers while the current one is computed.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pace_internal.h"
#include "pace_lanes.h"
#include "pace_numerics.h"

namespace pace {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kSB = 64;              // tokens per sub-block

__device__ inline v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct Rec {
  uint8_t* base;
  uint16_t* scales;
  uint8_t* zeros;
  int bits, NG, asym;
};

// Packed-record position of the 8 keys 8m..8m+7 of column j: the unit u whose base key
// is 8m, i.e. u = (m mod 4) * (D/32) + m / 4.
template <int D>
__device__ inline uint8_t* unit_ptr(const Rec& r, int j, int m) {
  constexpr int KB = D / 32;
  const int u = (m & 3) * KB + (m >> 2);
  return r.base + (uint32_t)(j * (D * r.bits / 8) + u * r.bits);   // (a 32-bit per-lane offset)
}

template <int D>
__device__ inline void store_codes4(const Rec& r, int j, int kt, int qd, uint32_t c4) {
  uint8_t* up = unit_ptr<D>(r, j, 2 * kt + (qd >> 1));
  if (r.bits == 4) {
    const uint32_t hi = pair16(c4).hi;               // keys 8m + 4 .. 8m + 7 (lane group qd | 1)
    if ((qd & 1) == 0) *(uint32_t*)up = c4 | (hi << 4);
  } else {
    *(uint32_t*)(up + 4 * (qd & 1)) = c4;
  }
}

// Round the accumulator state of one column tile to the packed record (and replace it by
// its dequantised value), groups of GS keys.  Column j of this lane; lane group qd.
template <int D, int GS>
__device__ inline void requant_tile(v4f (&S)[D / 16], const Rec& r, int j, int qd) {
  constexpr int KPG = GS / 16;         // key tiles per group
  constexpr int NG = D / GS;
  int zprev = 0;
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    float mx = S[G * KPG][0], mn = S[G * KPG][0];
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) { mx = fmaxf(mx, S[G * KPG + kk][i]); mn = fminf(mn, S[G * KPG + kk][i]); }
    mx = rows_max(mx);
    mn = rows_min(mn);
    const GroupQuant gq = group_quant(mn, mx, r.asym != 0, r.bits);
    const CodeRange cr = code_range(gq.z, r.asym != 0, r.bits);
    const float fz = (float)gq.z;
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      const int kt = G * KPG + kk;
      uint32_t c4 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // symmetric codes need no clamp: |x| / s <= 2^(b-1) - 1 up to one rounding
        const int c = r.asym ? code_of(S[kt][i], gq.r, cr.magic, cr.lo, cr.hi)
                             : (int)(f32_bits(fmaf(S[kt][i], gq.r, cr.magic)) & 0xFFu);
        c4 |= (uint32_t)c << (8 * i);
        S[kt][i] = gq.s * ((float)c - fz);
      }
      store_codes4<D>(r, j, kt, qd, c4);
    }
    if (qd == 0) {
      const int e = j * NG + G;
      r.scales[e] = (uint16_t)(f32_bits(gq.s) >> 16);
      if (r.asym) {
        if (r.bits == 8) r.zeros[e] = (uint8_t)gq.z;
        else if (G & 1) r.zeros[e >> 1] = (uint8_t)(zprev | (gq.z << 4));
      }
    }
    zprev = gq.z;
  }
}

template <int D, int IO>
struct Inputs {
  // raw 16-byte vectors of one sub-block: K, Q rows of the key head, V rows of the head
  static constexpr int ES = IO == 1 ? 2 : 4;                 // element bytes
  static constexpr int VPR = D * ES / 16;                    // vectors per row
  static constexpr int NV = kSB * VPR / kThreads;            // vectors per thread per tensor
  uint4 k[NV], q[NV], v[NV];
  float a, beta;
};

template <int D, int IO>
__device__ inline void load_inputs(Inputs<D, IO>& in, const PrefillParams& p, int b, int h, int kh,
                                   int t0, int nt, int tid) {
  using I = Inputs<D, IO>;
#pragma unroll
  for (int it = 0; it < I::NV; ++it) {
    const int i = tid + it * kThreads;
    const int t = i / I::VPR, c = i % I::VPR;
    if (t < nt) {
      const size_t kq = (((size_t)b * p.T + t0 + t) * p.Hk + kh) * (size_t)(D * I::ES) + 16 * c;
      const size_t vo = (((size_t)b * p.T + t0 + t) * p.Hv + h) * (size_t)(D * I::ES) + 16 * c;
      in.k[it] = *(const uint4*)((const uint8_t*)p.k + kq);
      in.q[it] = *(const uint4*)((const uint8_t*)p.q + kq);
      in.v[it] = *(const uint4*)((const uint8_t*)p.v + vo);
    } else {
      in.k[it] = in.q[it] = in.v[it] = make_uint4(0, 0, 0, 0);
    }
  }
  if (tid < kSB) {
    const bool ok = tid < nt;
    const size_t gi = ((size_t)b * p.T + t0 + (ok ? tid : 0)) * p.Hv + h;
    in.a = ok ? p.a[gi] : 1.f;           // padding tokens: no decay, no write
    in.beta = ok ? p.beta[gi] : 0.f;
  }
}

template <int IO>
__device__ inline void put8(float* dst, uint4 w) {
  if constexpr (IO == 1) {
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) { f[2 * e] = bits_f32(x[e] << 16); f[2 * e + 1] = bits_f32(x[e] & 0xFFFF0000u); }
    *(float4*)dst = make_float4(f[0], f[1], f[2], f[3]);
    *(float4*)(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
  } else {
    *(float4*)dst = make_float4(bits_f32(w.x), bits_f32(w.y), bits_f32(w.z), bits_f32(w.w));
  }
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v8f __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf16_t __attribute__((ext_vector_type(4)));

__device__ inline v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight fp32 values as three bf16 pieces whose sum is the value to ~2^-24 relative
// (each piece rounds the remainder of the previous ones to nearest).
__device__ inline void split3(v8f x, v8bf& p0, v8bf& p1, v8bf& p2) {
  p0 = __builtin_convertvector(x, v8bf);
  x -= __builtin_convertvector(p0, v8f);
  p1 = __builtin_convertvector(x, v8bf);
  x -= __builtin_convertvector(p1, v8f);
  p2 = __builtin_convertvector(x, v8bf);
}

// Two groups of four consecutive bf16 (8 bytes each) as one MFMA operand.
__device__ inline v8bf load_2x4(const uint16_t* lo, const uint16_t* hi) {
  const uint2 a = *(const uint2*)lo, b = *(const uint2*)hi;
  const uint4 w = make_uint4(a.x, a.y, b.x, b.y);
  v8bf r;
  __builtin_memcpy(&r, &w, 16);
  return r;
}

// Two transposing LDS reads (ds_read_b64_tr_b16) as one MFMA operand: within each group
// of 16 lanes, lane i receives element i % 4 of the 4-element pieces addressed by lanes
// i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12 of its group.
typedef short v4s16 __attribute__((ext_vector_type(4)));
__device__ inline v8bf load_tr16_2x4(const uint16_t* lo, const uint16_t* hi) {
  typedef __attribute__((address_space(3))) v4s16* lds_v4s16;
  const v4s16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16)lo);
  const v4s16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16)hi);
  const v8bf r = __builtin_shufflevector(__builtin_bit_cast(v4bf16_t, a), __builtin_bit_cast(v4bf16_t, b), 0, 1, 2, 3, 4, 5, 6, 7);
  return r;
}

__device__ inline v8bf load_8(const uint16_t* p) {
  const uint4 w = *(const uint4*)p;
  v8bf r;
  __builtin_memcpy(&r, &w, 16);
  return r;
}

// Operand tiles of one sub-block: fp32 (fp32 inputs, fp32 MFMA) or the bf16 inputs as
// they are, plus the keys transposed (bf16 MFMA).
template <int D, int IO>
struct Operands;

template <int D>
struct Operands<D, 0> {
  static constexpr int LD = D + 4;
  float K[kSB][LD];
  float Q[kSB][LD];
  float V[kSB][LD];
};

template <int D>
struct Operands<D, 1> {
  static constexpr int LD = D + 8;     // bf16 row stride: 16-byte aligned rows
  static constexpr int LT = kSB + 8;
  uint16_t K[kSB][LD];
  uint16_t Q[kSB][LD];
  uint16_t V[kSB][LD];
  uint16_t Kt[D][LT];                  // keys, [key][token]
};

template <int D, int IO>
struct Smem {
  static constexpr int LA = kSB + 4;
  Operands<D, IO> x;
  float A[kSB][LA];                    // beta_t e^{g_t-g_i} k_t.k_i, strictly lower
  float Ti[kSB / 16][16][20];          // inverses of the diagonal blocks (I + A_ii)
  float P[kSB][LA];                    // e^{g_t-g_i} q_t.k_i, lower incl. diagonal
  alignas(16) float g[kSB];            // cumulative log decay
  alignas(16) float beta[kSB];
  alignas(16) float gam[kSB];          // e^{g_t}
  alignas(16) float wend[kSB];         // e^{g_end - g_t}
};

template <int D, int IO, int CS>
__global__ __launch_bounds__(kThreads) void prefill_wy_kernel(PrefillParams p) {
  constexpr int KT = D / 16;           // key tiles
  constexpr int CT = D / (64 * CS);    // column tiles per wave
  static_assert(CT >= 1, "a wave owns at least one 16-column tile");
  constexpr int TT = kSB / 16;         // token tiles
  constexpr int VS = IO == 1 ? 8 : 4;  // elements per 16-byte input vector
  using I = Inputs<D, IO>;
  __shared__ Smem<D, IO> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches and addresses
  const int l16 = lane & 15, qd = lane >> 4;
  const int tile = blockIdx.x / CS, cb = (blockIdx.x % CS) * (D / CS);   // first column
  const int b = tile / p.Hv, h = tile % p.Hv, kh = h / p.gamma;

  const bool is8 = (p.mask8 >> h) & 1ull;
  const uint64_t below = h ? (p.mask8 & ((1ull << h) - 1ull)) : 0ull;
  const uint64_t n8 = (uint64_t)__popcll(below);
  Rec rec;
  rec.base = p.state + (uint64_t)b * p.seq_stride + (uint64_t)h * p.rec4 + n8 * (p.rec8 - p.rec4);
  rec.scales = (uint16_t*)(rec.base + (is8 ? p.scales_off8 : p.scales_off4));
  rec.zeros = rec.base + (is8 ? p.zeros_off8 : p.zeros_off4);
  rec.bits = is8 ? 8 : 4;
  rec.NG = D / p.group;
  rec.asym = p.asym;

  // ---- initial state: dequantise this lane's accumulator entries (all loads first,
  // branch-free: symmetric records read their scales in place of zero points)
  v4f S[CT][KT];
  {
    uint32_t c4[CT][KT];
    uint16_t sc[CT][KT];
    uint8_t zb[CT][KT];
    const int ub = rec.bits;                         // bytes per 8-key unit
    const int sel8 = is8 ? 4 * (qd & 1) : 0;
    const uint8_t* zsrc = p.asym ? rec.zeros : (const uint8_t*)rec.scales;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int j = cb + 16 * (wave * CT + c) + l16;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int m = 2 * kt + (qd >> 1);
        const int u = (m & 3) * (D / 32) + (m >> 2);
        c4[c][kt] = *(const uint32_t*)(rec.base + (size_t)j * (D * ub / 8) + u * ub + sel8);
        const int e = j * rec.NG + (16 * kt) / p.group;
        sc[c][kt] = rec.scales[e];
        zb[c][kt] = p.asym ? zsrc[is8 ? e : (e >> 1)] : 0;
      }
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int j = cb + 16 * (wave * CT + c) + l16;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int e = j * rec.NG + (16 * kt) / p.group;
        const float s = bf16_to_f32(sc[c][kt]);
        int z = 1 << (rec.bits - 1);
        if (p.asym) z = is8 ? (int)zb[c][kt] : (int)((zb[c][kt] >> (4 * (e & 1))) & 15);
        const uint32_t w = is8 ? c4[c][kt] : ((c4[c][kt] >> (4 * (qd & 1))) & 0x0F0F0F0Fu);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[c][kt][i] = s * ((float)((w >> (8 * i)) & 0xFFu) - (float)z);
      }
    }
  }

  const int nsb = (p.T + kSB - 1) / kSB;
  I in;
  load_inputs<D, IO>(in, p, b, h, kh, 0, min(kSB, p.T), tid);

  for (int sb = 0; sb < nsb; ++sb) {
    const int t0 = sb * kSB;
    const int nt = min(kSB, p.T - t0);
    // ---------------------------------------------------------------- inputs -> LDS
#pragma unroll
    for (int it = 0; it < I::NV; ++it) {
      const int i = tid + it * kThreads;
      const int t = i / I::VPR, c = (i % I::VPR) * VS;
      if constexpr (IO == 1) {
        *(uint4*)&sm.x.K[t][c] = in.k[it];
        *(uint4*)&sm.x.Q[t][c] = in.q[it];
        *(uint4*)&sm.x.V[t][c] = in.v[it];
      } else {
        put8<IO>(&sm.x.K[t][c], in.k[it]);
        put8<IO>(&sm.x.Q[t][c], in.q[it]);
        put8<IO>(&sm.x.V[t][c], in.v[it]);
      }
    }
    if (wave == 0) {
      // inclusive scan of log a over the 64 tokens (a = 0 is clamped to e^-80)
      float x = fmaxf(logf(in.a), -80.f);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      const float gend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
      sm.g[lane] = x * 1.4426950408889634f;   // log2 units: decays are exp2 of differences
      sm.beta[lane] = in.beta;
      sm.gam[lane] = expf(x);
      sm.wend[lane] = expf(gend - x);
    }
    __syncthreads();

    // ------------------------------------------- Gram and query-key tiles (lower)
    // 20 jobs (10 lower-triangular token-tile pairs for K K^T and for Q K^T), five per
    // wave, all issued together; job j of wave w is pair (j / 2) * 4 + w ... in the fixed
    // order below.
    {
      constexpr int NJ = TT * (TT + 1);          // 20
      constexpr int JPW = NJ / 4;                // 5 per wave
      v4f acc[JPW];
      int tis[JPW], tjs[JPW];
      bool isqs[JPW];
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int job = wave + 4 * jj;
        const bool isq = job >= NJ / 2;
        int pr = isq ? job - NJ / 2 : job;
        int ti = 0;
        while (pr > ti) { pr -= ti + 1; ++ti; }
        tis[jj] = ti; tjs[jj] = pr; isqs[jj] = isq;
        acc[jj] = v4f{0.f, 0.f, 0.f, 0.f};
      }
      if constexpr (IO == 1) {         // exact bf16 inputs: one pass
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) {
          v8bf xa[JPW], xb[JPW];
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj) {
            const uint16_t* X = isqs[jj] ? &sm.x.Q[16 * tis[jj] + l16][0] : &sm.x.K[16 * tis[jj] + l16][0];
            xa[jj] = load_8(X + 32 * kb + 8 * qd);
            xb[jj] = load_8(&sm.x.K[16 * tjs[jj] + l16][32 * kb + 8 * qd]);
          }
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj) acc[jj] = mfma_bf16(xa[jj], xb[jj], acc[jj]);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          const float* X = isqs[jj] ? &sm.x.Q[16 * tis[jj] + l16][0] : &sm.x.K[16 * tis[jj] + l16][0];
#pragma unroll
          for (int v = 0; v < D / 16; ++v) {
            const float4 xa = *(const float4*)(X + 16 * v + 4 * qd);
            const float4 xb = *(const float4*)&sm.x.K[16 * tjs[jj] + l16][16 * v + 4 * qd];
            acc[jj] = mfma4(xa.x, xb.x, acc[jj]);
            acc[jj] = mfma4(xa.y, xb.y, acc[jj]);
            acc[jj] = mfma4(xa.z, xb.z, acc[jj]);
            acc[jj] = mfma4(xa.w, xb.w, acc[jj]);
          }
        }
      }
      // decays and betas of every job's rows and column, read as vectors and all issued
      // before any is used (one LDS round trip instead of one per element)
      float4 g4[JPW], b4[JPW];
      float gi[JPW];
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        g4[jj] = *(const float4*)&sm.g[16 * tis[jj] + 4 * qd];
        b4[jj] = *(const float4*)&sm.beta[16 * tis[jj] + 4 * qd];
        gi[jj] = sm.g[16 * tjs[jj] + l16];
      }
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int i = 16 * tjs[jj] + l16;
        const float gt[4] = {g4[jj].x, g4[jj].y, g4[jj].z, g4[jj].w};
        const float bt[4] = {b4[jj].x, b4[jj].y, b4[jj].z, b4[jj].w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * tis[jj] + 4 * qd + r;
          // (the hardware exp2: decays under 2^-126 read as 0, far below any fp32 sum)
          const float dec = __builtin_amdgcn_exp2f(fminf(gt[r] - gi[jj], 0.f));
          if (isqs[jj]) sm.P[t][i] = t >= i ? dec * acc[jj][r] : 0.f;
          else sm.A[t][i] = t > i ? bt[r] * dec * acc[jj][r] : 0.f;
        }
      }
    }
    // prefetch the next sub-block while the rest of this one is computed
    if (sb + 1 < nsb) load_inputs<D, IO>(in, p, b, h, kh, t0 + kSB, min(kSB, p.T - t0 - kSB), tid);
    if constexpr (IO == 1) {
      // keys transposed for the state update: thread -> (key, 8-token block); column
      // reads and one 16-byte row write per pair, both free of bank conflicts
#pragma unroll
      for (int it = 0; it < D * (kSB / 8) / kThreads; ++it) {
        const int pidx = tid + it * kThreads;
        const int key = pidx % D, blk = pidx / D;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)sm.x.K[8 * blk + 2 * e][key] | ((uint32_t)sm.x.K[8 * blk + 2 * e + 1][key] << 16);
        *(uint4*)&sm.x.Kt[key][8 * blk] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }

    // ------ K S and Q S of the sub-block's starting state (own columns, accumulators)
    v4f KS[CT][TT], QS[CT][TT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) KS[c][tt] = QS[c][tt] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (IO == 1) {
      // 32-key blocks: lane group qd feeds keys 32 kb + 4 qd + (0..3) and 32 kb + 16 +
      // 4 qd + (0..3), i.e. its accumulator entries of key tiles 2 kb and 2 kb + 1; the
      // state enters as three bf16 pieces, K and Q as they are
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int kb = 0; kb < KT / 2; ++kb) {
          const v4f s0 = S[c][2 * kb], s1 = S[c][2 * kb + 1];
          v8bf p0, p1, p2;
          split3(v8f{s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]}, p0, p1, p2);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const int row = 16 * tt + l16;
            const v8bf ak = load_2x4(&sm.x.K[row][32 * kb + 4 * qd], &sm.x.K[row][32 * kb + 16 + 4 * qd]);
            const v8bf aq = load_2x4(&sm.x.Q[row][32 * kb + 4 * qd], &sm.x.Q[row][32 * kb + 16 + 4 * qd]);
            KS[c][tt] = mfma_bf16(ak, p0, KS[c][tt]);
            KS[c][tt] = mfma_bf16(ak, p1, KS[c][tt]);
            KS[c][tt] = mfma_bf16(ak, p2, KS[c][tt]);
            QS[c][tt] = mfma_bf16(aq, p0, QS[c][tt]);
            QS[c][tt] = mfma_bf16(aq, p1, QS[c][tt]);
            QS[c][tt] = mfma_bf16(aq, p2, QS[c][tt]);
          }
        }
    } else {                           // fp32: K S here, Q S with the outputs
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int row = 16 * tt + l16;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const float4 kx = *(const float4*)&sm.x.K[row][16 * kt + 4 * qd];
          const float kv[4] = {kx.x, kx.y, kx.z, kx.w};
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < CT; ++c) KS[c][tt] = mfma4(kv[r], S[c][kt][r], KS[c][tt]);
        }
      }
    }
    // right-hand sides R = diag(beta) V - diag(beta Gamma) K S
    v4f R[CT][TT];
    float4 bet4[TT], gam4[TT];               // this lane's rows, read as vectors up front
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      bet4[tt] = *(const float4*)&sm.beta[16 * tt + 4 * qd];
      gam4[tt] = *(const float4*)&sm.gam[16 * tt + 4 * qd];
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int j = cb + 16 * (wave * CT + c) + l16;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const float bt[4] = {bet4[tt].x, bet4[tt].y, bet4[tt].z, bet4[tt].w};
        const float gt[4] = {gam4[tt].x, gam4[tt].y, gam4[tt].z, gam4[tt].w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * tt + 4 * qd + r;
          float vv;
          if constexpr (IO == 1) vv = bf16_to_f32(sm.x.V[t][j]);
          else vv = sm.x.V[t][j];
          R[c][tt][r] = bt[r] * fmaf(-gt[r], KS[c][tt][r], vv);
        }
      }
    }
    __syncthreads();     // A and P complete

    // ------------- inverse of diagonal block `wave`: lanes 0..15 = columns of (I + A_ww)^-1
    {
      const int cc = lane & 15, base = 16 * wave;
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float acc = t == cc ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < t; ++i) acc = fmaf(-sm.A[base + t][base + i], x[i], acc);
        x[t] = acc;
      }
      if (lane < 16) {
#pragma unroll
        for (int t = 0; t < 16; ++t) sm.Ti[wave][t][cc] = x[t];
      }
    }
    __syncthreads();

    // --------- blocked forward solve: U_i = Ti_i (R_i - sum_{j<i} A_ij U_j), accumulators
    v4f U[CT][TT];
#pragma unroll
    for (int ib = 0; ib < TT; ++ib) {
      v4f acc[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[c] = R[c][ib];
#pragma unroll
      for (int jb = 0; jb < ib; ++jb) {
        const float4 av = *(const float4*)&sm.A[16 * ib + l16][16 * jb + 4 * qd];
        const float na[4] = {-av.x, -av.y, -av.z, -av.w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int c = 0; c < CT; ++c) acc[c] = mfma4(na[r], U[c][jb][r], acc[c]);
      }
      const float4 tv = *(const float4*)&sm.Ti[ib][l16][4 * qd];
      const float ti[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        U[c][ib] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) U[c][ib] = mfma4(ti[r], acc[c][r], U[c][ib]);
      }
    }

    // ----------------------------- outputs O = diag(Gamma) Q S + P U, own columns
    auto store_out = [&](int tt, const v4f (&O)[CT]) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int j = cb + 16 * (wave * CT + c) + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * tt + 4 * qd + r;
          if (t < nt) {
            const size_t oi = (((size_t)b * p.T + t0 + t) * p.Hv + h) * D + j;
            if constexpr (IO == 1) ((uint16_t*)p.o)[oi] = f32_to_bf16_rne(O[c][r]);
            else ((float*)p.o)[oi] = O[c][r];
          }
        }
      }
    };
    if constexpr (IO == 1) {
      // all four token tiles at once, so that consecutive MFMAs feed different
      // accumulators (the chains of P U overlap instead of running one after another)
      v4f O[TT][CT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gr = r == 0 ? gam4[tt].x : r == 1 ? gam4[tt].y : r == 2 ? gam4[tt].z : gam4[tt].w;
            O[tt][c][r] = gr * QS[c][tt][r];
          }
#pragma unroll
      for (int ib = 0; ib < TT; ++ib) {
        float4 px[TT];
#pragma unroll
        for (int tt = ib; tt < TT; ++tt) px[tt] = *(const float4*)&sm.P[16 * tt + l16][16 * ib + 4 * qd];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int tt = ib; tt < TT; ++tt) {
            const float pv = s == 0 ? px[tt].x : s == 1 ? px[tt].y : s == 2 ? px[tt].z : px[tt].w;
#pragma unroll
            for (int c = 0; c < CT; ++c) O[tt][c] = mfma4(pv, U[c][ib][s], O[tt][c]);
          }
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) store_out(tt, O[tt]);
    } else {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int tr = 16 * tt + l16;
        v4f O[CT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const float4 qx = *(const float4*)&sm.x.Q[tr][16 * kt + 4 * qd];
          const float qv[4] = {qx.x, qx.y, qx.z, qx.w};
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < CT; ++c) QS[c][tt] = mfma4(qv[r], S[c][kt][r], QS[c][tt]);
        }
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gr = r == 0 ? gam4[tt].x : r == 1 ? gam4[tt].y : r == 2 ? gam4[tt].z : gam4[tt].w;
            O[c][r] = gr * QS[c][tt][r];
          }
#pragma unroll
        for (int ib = 0; ib <= tt; ++ib) {
          const float4 px = *(const float4*)&sm.P[tr][16 * ib + 4 * qd];
          const float pv[4] = {px.x, px.y, px.z, px.w};
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < CT; ++c)
              O[c] = mfma4(pv[s], U[c][ib][s], O[c]);
        }
        store_out(tt, O);
      }
    }

    // --------------------------- state S' = Gamma_end S + K^T diag(e^{g_end - g}) U
    {
      const float ge = sm.gam[kSB - 1];
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) S[c][kt] *= ge;
      if constexpr (IO == 1) {
        // 32-token blocks: lane group qd feeds tokens 32 tb + 4 qd + (0..3) and 32 tb +
        // 16 + 4 qd + (0..3) (its accumulator entries of token tiles 2 tb and 2 tb + 1);
        // the decayed U enters as three bf16 pieces, the transposed keys as they are
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int tb = 0; tb < TT / 2; ++tb) {
            const float4 w0 = *(const float4*)&sm.wend[32 * tb + 4 * qd];
            const float4 w1 = *(const float4*)&sm.wend[32 * tb + 16 + 4 * qd];
            const v4f u0 = U[c][2 * tb], u1 = U[c][2 * tb + 1];
            v8bf p0, p1, p2;
            split3(v8f{u0[0] * w0.x, u0[1] * w0.y, u0[2] * w0.z, u0[3] * w0.w,
                       u1[0] * w1.x, u1[1] * w1.y, u1[2] * w1.z, u1[3] * w1.w}, p0, p1, p2);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
              const uint16_t* kr = &sm.x.Kt[16 * kt + l16][0];
              const v8bf ak = load_2x4(kr + 32 * tb + 4 * qd, kr + 32 * tb + 16 + 4 * qd);
              S[c][kt] = mfma_bf16(ak, p0, S[c][kt]);
              S[c][kt] = mfma_bf16(ak, p1, S[c][kt]);
              S[c][kt] = mfma_bf16(ak, p2, S[c][kt]);
            }
          }
      } else {
#pragma unroll
        for (int tb = 0; tb < TT; ++tb) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int tok = 16 * tb + 4 * qd + s;
            const float w = sm.wend[tok];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
              const float kv = sm.x.K[tok][16 * kt + l16] * w;
#pragma unroll
              for (int c = 0; c < CT; ++c) S[c][kt] = mfma4(kv, U[c][tb][s], S[c][kt]);
            }
          }
        }
      }
    }

    // ---------------------------------- rounding at chunk ends and after the last token
    const int done = t0 + nt;
    if (done % p.chunk == 0 || done == p.T) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int j = cb + 16 * (wave * CT + c) + l16;
        if (p.group == 64) requant_tile<D, 64>(S[c], rec, j, qd);
        else requant_tile<D, 32>(S[c], rec, j, qd);
      }
    }
    __syncthreads();     // the next sub-block overwrites K, Q, V, A, P
  }
}

// ------------------------------------------------------------------------------------
// Warp-specialised variant for bf16 I/O with the column split (two workgroups per
// (sequence, head)), eight waves.  Waves 0-3 (consumers) own this block's state columns
// and run the state-dependent chain of each sub-block: K S and Q S, with the query-key
// tiles P from the same operands, right-hand sides; then the solve and the outputs; then
// the state update, whose K^T operand is read transposed straight from the row-major key
// tile (ds_read_b64_tr_b16); then the rounding.  Waves 4-7 (producers) run beside them:
// during the consumers' first stage they form the sub-block's Gram tiles with their
// decays (A) and the inverses of the diagonal blocks, and request the next sub-block's
// inputs; during the
// rest (which no longer reads Q or V, and reads the keys of the other parity) they store
// those inputs and the next gates into LDS.  Two workgroup barriers per sub-block (and one before the loops), passed by every
// wave; neither role leaves its loop early, so the barriers always pair up.
constexpr int kWsThreads = 512;

template <int D>
struct SmemWS {
  static constexpr int LA = kSB + 4;
  static constexpr int LD = D + 8;     // bf16 row stride: 16-byte aligned rows
  uint16_t K[2][kSB][LD];              // keys by sub-block parity (the state update of one
                                       // sub-block reads them while the next ones arrive)
  uint16_t Q[kSB][LD];                 // queries and values of the current sub-block
  uint16_t V[kSB][LD];
  float A[kSB][LA];                    // beta_t e^{g_t-g_i} k_t.k_i, strictly lower
  float Ti[kSB / 16][16][20];          // inverses of the diagonal blocks (I + A_ii)
  float P[kSB][LA];                    // e^{g_t-g_i} q_t.k_i, lower incl. diagonal
  alignas(16) float g[2][kSB];         // gates by sub-block parity: cumulative log2 decay,
  alignas(16) float beta[2][kSB];      // beta, e^{g_t}, e^{g_end - g_t}
  alignas(16) float gam[2][kSB];
  alignas(16) float wend[2][kSB];
};

// Token-tile pairs (row tile, column tile) of the lower triangle, split over the waves:
// the producers form the Gram tiles A (wave w's first pair is the diagonal (w, w), whose
// inverse it then forms from its own LDS writes); the consumers form the query-key tiles
// P from the key and query tiles they already hold for K S and Q S.  -1: no job.
constexpr int kKkJobs[4][3][2] = {{{0, 0}, {3, 0}, {3, 1}}, {{1, 1}, {1, 0}, {2, 0}},
                                  {{2, 2}, {2, 1}, {3, 2}}, {{3, 3}, {-1, -1}, {-1, -1}}};
constexpr int kKkCount[4] = {3, 3, 3, 1};
constexpr int kQkJobs[4][3][2] = {{{0, 0}, {1, 0}, {1, 1}}, {{2, 0}, {2, 1}, {2, 2}},
                                  {{3, 0}, {3, 1}, {-1, -1}}, {{3, 2}, {3, 3}, {-1, -1}}};
constexpr int kQkCount[4] = {3, 3, 2, 2};

template <int D>
__global__ __launch_bounds__(kWsThreads) void prefill_ws_kernel(PrefillParams p) {
  constexpr int KT = D / 16;           // key tiles
  constexpr int CT = D / 128;          // column tiles per consumer wave (D / 2 columns)
  constexpr int TT = kSB / 16;         // token tiles
  using I = Inputs<D, 1>;
  __shared__ SmemWS<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  const int tid = threadIdx.x & (kThreads - 1);                         // index within the role
  const int l16 = lane & 15, qd = lane >> 4;
  const int tile = blockIdx.x / 2, cb = (blockIdx.x % 2) * (D / 2);   // first column
  const int b = tile / p.Hv, h = tile % p.Hv, kh = h / p.gamma;
  const int nsb = (p.T + kSB - 1) / kSB;

  if (wave < 4) {
    // ===================================================================== consumers
    const bool is8 = (p.mask8 >> h) & 1ull;
    const uint64_t below = h ? (p.mask8 & ((1ull << h) - 1ull)) : 0ull;
    const uint64_t n8 = (uint64_t)__popcll(below);
    Rec rec;
    rec.base = p.state + (uint64_t)b * p.seq_stride + (uint64_t)h * p.rec4 + n8 * (p.rec8 - p.rec4);
    rec.scales = (uint16_t*)(rec.base + (is8 ? p.scales_off8 : p.scales_off4));
    rec.zeros = rec.base + (is8 ? p.zeros_off8 : p.zeros_off4);
    rec.bits = is8 ? 8 : 4;
    rec.NG = D / p.group;
    rec.asym = p.asym;

    // initial state: dequantise this lane's accumulator entries (all loads first)
    v4f S[CT][KT];
    {
      uint32_t c4[CT][KT];
      uint16_t sc[CT][KT];
      uint8_t zb[CT][KT];
      const int ub = rec.bits;
      const int sel8 = is8 ? 4 * (qd & 1) : 0;
      const uint8_t* zsrc = p.asym ? rec.zeros : (const uint8_t*)rec.scales;
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int j = cb + 16 * (wave * CT + c) + l16;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int m = 2 * kt + (qd >> 1);
          const int u = (m & 3) * (D / 32) + (m >> 2);
          c4[c][kt] = *(const uint32_t*)(rec.base + (size_t)j * (D * ub / 8) + u * ub + sel8);
          const int e = j * rec.NG + (16 * kt) / p.group;
          sc[c][kt] = rec.scales[e];
          zb[c][kt] = p.asym ? zsrc[is8 ? e : (e >> 1)] : 0;
        }
      }
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int j = cb + 16 * (wave * CT + c) + l16;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int e = j * rec.NG + (16 * kt) / p.group;
          const float s = bf16_to_f32(sc[c][kt]);
          int z = 1 << (rec.bits - 1);
          if (p.asym) z = is8 ? (int)zb[c][kt] : (int)((zb[c][kt] >> (4 * (e & 1))) & 15);
          const uint32_t w = is8 ? c4[c][kt] : ((c4[c][kt] >> (4 * (qd & 1))) & 0x0F0F0F0Fu);
#pragma unroll
          for (int i = 0; i < 4; ++i) S[c][kt][i] = s * ((float)((w >> (8 * i)) & 0xFFu) - (float)z);
        }
      }
    }
    __syncthreads();                   // (barrier 0) sub-block 0's inputs and gates in LDS

    for (int sb = 0; sb < nsb; ++sb) {
      const int t0 = sb * kSB;
      const int nt = min(kSB, p.T - t0);
      const int gb = sb & 1;           // gate buffer of this sub-block
      // K S and Q S of the sub-block's starting state (state as three bf16 pieces), and
      // this wave's query-key tiles Q K^T, whose operands are the same key and query tiles
      // (lane (l16, qd) holds row l16 of a tile, keys 32 kb + 4 qd + (0..3) and
      // 32 kb + 16 + 4 qd + (0..3): as the A operand a query row, as the B operand a key
      // row, in one key order)
      static_assert(CT == 1, "one column tile per consumer wave");
      v4f KS[CT][TT], QS[CT][TT], qk[3];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) KS[0][tt] = QS[0][tt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 3; ++jj) qk[jj] = v4f{0.f, 0.f, 0.f, 0.f};
      // (per wave a compile-time job list: each query-key job is issued as soon as its
      // query tile is loaded, so only the key tiles it still needs stay in registers)
      auto ks_qs = [&](auto cwc) {
        constexpr int CW = decltype(cwc)::value;
#pragma unroll
        for (int kb = 0; kb < KT / 2; ++kb) {
          const v4f s0 = S[0][2 * kb], s1 = S[0][2 * kb + 1];
          v8bf p0, p1, p2;
          split3(v8f{s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]}, p0, p1, p2);
          v8bf akt[TT];
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const int row = 16 * tt + l16;
            akt[tt] = load_2x4(&sm.K[gb][row][32 * kb + 4 * qd], &sm.K[gb][row][32 * kb + 16 + 4 * qd]);
            const v8bf aq = load_2x4(&sm.Q[row][32 * kb + 4 * qd], &sm.Q[row][32 * kb + 16 + 4 * qd]);
            KS[0][tt] = mfma_bf16(akt[tt], p0, KS[0][tt]);
            KS[0][tt] = mfma_bf16(akt[tt], p1, KS[0][tt]);
            KS[0][tt] = mfma_bf16(akt[tt], p2, KS[0][tt]);
            QS[0][tt] = mfma_bf16(aq, p0, QS[0][tt]);
            QS[0][tt] = mfma_bf16(aq, p1, QS[0][tt]);
            QS[0][tt] = mfma_bf16(aq, p2, QS[0][tt]);
#pragma unroll
            for (int jj = 0; jj < kQkCount[CW]; ++jj)
              if (kQkJobs[CW][jj][0] == tt) qk[jj] = mfma_bf16(aq, akt[kQkJobs[CW][jj][1]], qk[jj]);
          }
        }
      };
      switch (wave) {
        case 0: ks_qs(std::integral_constant<int, 0>{}); break;
        case 1: ks_qs(std::integral_constant<int, 1>{}); break;
        case 2: ks_qs(std::integral_constant<int, 2>{}); break;
        default: ks_qs(std::integral_constant<int, 3>{}); break;
      }
      // P = lower-incl [e^{g_t - g_i} q_t . k_i] of this wave's tiles
      auto qk_epi = [&](auto cwc) {
        constexpr int CW = decltype(cwc)::value;
#pragma unroll
        for (int jj = 0; jj < kQkCount[CW]; ++jj) {
          const int ti = kQkJobs[CW][jj][0], tj = kQkJobs[CW][jj][1];
          const float4 g4 = *(const float4*)&sm.g[gb][16 * ti + 4 * qd];
          const float gi = sm.g[gb][16 * tj + l16];
          const float gt[4] = {g4.x, g4.y, g4.z, g4.w};
          const int i = 16 * tj + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * ti + 4 * qd + r;
            // (the hardware exp2: decays under 2^-126 read as 0, far below any fp32 sum)
            const float dec = __builtin_amdgcn_exp2f(fminf(gt[r] - gi, 0.f));
            sm.P[t][i] = t >= i ? dec * qk[jj][r] : 0.f;
          }
        }
      };
      switch (wave) {
        case 0: qk_epi(std::integral_constant<int, 0>{}); break;
        case 1: qk_epi(std::integral_constant<int, 1>{}); break;
        case 2: qk_epi(std::integral_constant<int, 2>{}); break;
        default: qk_epi(std::integral_constant<int, 3>{}); break;
      }
      // right-hand sides R = diag(beta) V - diag(beta Gamma) K S
      v4f R[CT][TT];
      float4 gam4[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) gam4[tt] = *(const float4*)&sm.gam[gb][16 * tt + 4 * qd];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int j = cb + 16 * (wave * CT + c) + l16;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const float4 bet4 = *(const float4*)&sm.beta[gb][16 * tt + 4 * qd];
          const float bt[4] = {bet4.x, bet4.y, bet4.z, bet4.w};
          const float gt[4] = {gam4[tt].x, gam4[tt].y, gam4[tt].z, gam4[tt].w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * tt + 4 * qd + r;
            R[c][tt][r] = bt[r] * fmaf(-gt[r], KS[c][tt][r], bf16_to_f32(sm.V[t][j]));
          }
        }
      }
      __syncthreads();                 // (barrier 1) A, P and the inverses are complete;
                                       // K, Q and V are no longer read

      // blocked forward solve: U_i = Ti_i (R_i - sum_{j<i} A_ij U_j)
      v4f U[CT][TT];
#pragma unroll
      for (int ib = 0; ib < TT; ++ib) {
        v4f acc[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c] = R[c][ib];
#pragma unroll
        for (int jb = 0; jb < ib; ++jb) {
          const float4 av = *(const float4*)&sm.A[16 * ib + l16][16 * jb + 4 * qd];
          const float na[4] = {-av.x, -av.y, -av.z, -av.w};
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < CT; ++c) acc[c] = mfma4(na[r], U[c][jb][r], acc[c]);
        }
        const float4 tv = *(const float4*)&sm.Ti[ib][l16][4 * qd];
        const float ti[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          U[c][ib] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < 4; ++r) U[c][ib] = mfma4(ti[r], acc[c][r], U[c][ib]);
        }
      }

      // outputs O = diag(Gamma) Q S + P U, the four token tiles' P U chains interleaved
      {
        v4f O[TT][CT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float gr = r == 0 ? gam4[tt].x : r == 1 ? gam4[tt].y : r == 2 ? gam4[tt].z : gam4[tt].w;
              O[tt][c][r] = gr * QS[c][tt][r];
            }
#pragma unroll
        for (int ib = 0; ib < TT; ++ib) {
          float4 px[TT];
#pragma unroll
          for (int tt = ib; tt < TT; ++tt) px[tt] = *(const float4*)&sm.P[16 * tt + l16][16 * ib + 4 * qd];
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int tt = ib; tt < TT; ++tt) {
              const float pv = s == 0 ? px[tt].x : s == 1 ? px[tt].y : s == 2 ? px[tt].z : px[tt].w;
#pragma unroll
              for (int c = 0; c < CT; ++c) O[tt][c] = mfma4(pv, U[c][ib][s], O[tt][c]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int c = 0; c < CT; ++c) {
            const int j = cb + 16 * (wave * CT + c) + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 16 * tt + 4 * qd + r;
              if (t < nt) ((uint16_t*)p.o)[(((size_t)b * p.T + t0 + t) * p.Hv + h) * D + j] = f32_to_bf16_rne(O[tt][c][r]);
            }
          }
      }

      // state S' = Gamma_end S + K^T diag(e^{g_end - g}) U
      {
        const float ge = sm.gam[gb][kSB - 1];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) S[c][kt] *= ge;
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int tb = 0; tb < TT / 2; ++tb) {
            const float4 w0 = *(const float4*)&sm.wend[gb][32 * tb + 4 * qd];
            const float4 w1 = *(const float4*)&sm.wend[gb][32 * tb + 16 + 4 * qd];
            const v4f u0 = U[c][2 * tb], u1 = U[c][2 * tb + 1];
            v8bf p0, p1, p2;
            split3(v8f{u0[0] * w0.x, u0[1] * w0.y, u0[2] * w0.z, u0[3] * w0.w,
                       u1[0] * w1.x, u1[1] * w1.y, u1[2] * w1.z, u1[3] * w1.w}, p0, p1, p2);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
              // keys 16 kt + l16, tokens 32 tb + 4 qd + (0..3) and 32 tb + 16 + 4 qd + (0..3),
              // read transposed from the row-major key tile: within each 16-lane group,
              // lane i receives element i % 4 of the 8-byte pieces addressed by lanes
              // i / 4 + 4 j (j = 0..3), so lane l16 addresses token row + l16 / 4, keys
              // 16 kt + 4 (l16 % 4) .. + 3
              const uint16_t* kr = &sm.K[gb][32 * tb + 4 * qd + l16 / 4][16 * kt + 4 * (l16 % 4)];
              const v8bf ak = load_tr16_2x4(kr, kr + 16 * SmemWS<D>::LD);
              S[c][kt] = mfma_bf16(ak, p0, S[c][kt]);
              S[c][kt] = mfma_bf16(ak, p1, S[c][kt]);
              S[c][kt] = mfma_bf16(ak, p2, S[c][kt]);
            }
          }
      }
      // rounding at chunk ends and after the last token
      const int done = t0 + nt;
      if (done % p.chunk == 0 || done == p.T) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          const int j = cb + 16 * (wave * CT + c) + l16;
          if (p.group == 64) requant_tile<D, 64>(S[c], rec, j, qd);
          else requant_tile<D, 32>(S[c], rec, j, qd);
        }
      }
      __syncthreads();                 // (barrier 2) the next sub-block's inputs are in
                                       // LDS; A, P and the inverses may be replaced
    }
  } else {
    // ===================================================================== producers
    const int pw = wave - 4;
    I in;
    // this sub-block's inputs (prefetched) and gates into LDS
    auto store_inputs = [&](int gbuf) {
#pragma unroll
      for (int it = 0; it < I::NV; ++it) {
        const int i = tid + it * kThreads;
        const int t = i / I::VPR, c = (i % I::VPR) * 8;
        *(uint4*)&sm.K[gbuf][t][c] = in.k[it];
        *(uint4*)&sm.Q[t][c] = in.q[it];
        *(uint4*)&sm.V[t][c] = in.v[it];
      }
      if (pw == 0) {
        // inclusive scan of log a over the 64 tokens (a = 0 is clamped to e^-80)
        float x = fmaxf(logf(in.a), -80.f);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const float y = __shfl_up(x, o);
          if (lane >= o) x += y;
        }
        const float gend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
        sm.g[gbuf][lane] = x * 1.4426950408889634f;   // log2 units: decays are exp2 of differences
        sm.beta[gbuf][lane] = in.beta;
        sm.gam[gbuf][lane] = expf(x);
        sm.wend[gbuf][lane] = expf(gend - x);
      }
    };

    load_inputs<D, 1>(in, p, b, h, kh, 0, min(kSB, p.T), tid);
    store_inputs(0);
    __syncthreads();                   // (barrier 0)

    for (int sb = 0; sb < nsb; ++sb) {
      const int t0 = sb * kSB;
      const int gb = sb & 1;
      const bool more = sb + 1 < nsb;
      // ------------------------------------ Gram tiles of this sub-block -> A
      {
        v4f acc[3];
#pragma unroll
        for (int jj = 0; jj < 3; ++jj) acc[jj] = v4f{0.f, 0.f, 0.f, 0.f};
        // per 32-key block, the four key tiles are each read once and shared by the jobs
        // (LDS reads are what the consumers' stage contends for); the job tiles are
        // compile-time values per wave
        auto gram_mma = [&](auto pwc) {
          constexpr int PW = decltype(pwc)::value;
#pragma unroll
          for (int kb = 0; kb < D / 32; ++kb) {
            v8bf kx[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) kx[t] = load_8(&sm.K[gb][16 * t + l16][32 * kb + 8 * qd]);
#pragma unroll
            for (int jj = 0; jj < kKkCount[PW]; ++jj)
              acc[jj] = mfma_bf16(kx[kKkJobs[PW][jj][0]], kx[kKkJobs[PW][jj][1]], acc[jj]);
          }
        };
        auto gram_epi = [&](auto pwc) {
          constexpr int PW = decltype(pwc)::value;
#pragma unroll
          for (int jj = 0; jj < kKkCount[PW]; ++jj) {
            const int ti = kKkJobs[PW][jj][0], tj = kKkJobs[PW][jj][1];
            const float4 g4 = *(const float4*)&sm.g[gb][16 * ti + 4 * qd];
            const float4 b4 = *(const float4*)&sm.beta[gb][16 * ti + 4 * qd];
            const float gi = sm.g[gb][16 * tj + l16];
            const float gt[4] = {g4.x, g4.y, g4.z, g4.w};
            const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
            const int i = 16 * tj + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 16 * ti + 4 * qd + r;
              const float dec = __builtin_amdgcn_exp2f(fminf(gt[r] - gi, 0.f));
              sm.A[t][i] = t > i ? bt[r] * dec * acc[jj][r] : 0.f;
            }
          }
        };
        switch (pw) {
          case 0: gram_mma(std::integral_constant<int, 0>{}); break;
          case 1: gram_mma(std::integral_constant<int, 1>{}); break;
          case 2: gram_mma(std::integral_constant<int, 2>{}); break;
          default: gram_mma(std::integral_constant<int, 3>{}); break;
        }
        // the next sub-block's inputs, requested while these tiles are formed
        if (more) load_inputs<D, 1>(in, p, b, h, kh, t0 + kSB, min(kSB, p.T - t0 - kSB), tid);
        switch (pw) {
          case 0: gram_epi(std::integral_constant<int, 0>{}); break;
          case 1: gram_epi(std::integral_constant<int, 1>{}); break;
          case 2: gram_epi(std::integral_constant<int, 2>{}); break;
          default: gram_epi(std::integral_constant<int, 3>{}); break;
        }
      }
      // ---- inverse of diagonal block pw, written above by this wave (its job 0): a
      // wave's LDS accesses complete in order, so only the compiler must keep the reads
      // below the writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      {
        const int cc = lane & 15, base = 16 * pw;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          float acc = t == cc ? 1.f : 0.f;
#pragma unroll
          for (int i = 0; i < t; ++i) acc = fmaf(-sm.A[base + t][base + i], x[i], acc);
          x[t] = acc;
        }
        if (lane < 16) {
#pragma unroll
          for (int t = 0; t < 16; ++t) sm.Ti[pw][t][cc] = x[t];
        }
      }
      __syncthreads();                 // (barrier 1)
      if (more) store_inputs(gb ^ 1);
      __syncthreads();                 // (barrier 2)
    }
  }
}

// Compute units of the current device (one workgroup of this kernel fills a CU's LDS).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int D, int IO>
void launch_wy(const PrefillParams& p, hipStream_t stream) {
  const unsigned tiles = (unsigned)p.B * (unsigned)p.Hv;
  if constexpr (D >= 128 && IO == 1) {
    // bf16 I/O: the warp-specialised kernel, two column-block workgroups per (sequence,
    // head) whatever the number of pairs
    hipLaunchKernelGGL((prefill_ws_kernel<D>), dim3(2 * tiles), dim3(kWsThreads), 0, stream, p);
  } else {
    // fp32 I/O at d = 128: split the columns when two workgroups per pair still run in
    // one round
    if constexpr (D >= 128) {
      if (2 * tiles <= (unsigned)device_cus()) {
        hipLaunchKernelGGL((prefill_wy_kernel<D, IO, 2>), dim3(2 * tiles), dim3(kThreads), 0, stream, p);
        return;
      }
    }
    hipLaunchKernelGGL((prefill_wy_kernel<D, IO, 1>), dim3(tiles), dim3(kThreads), 0, stream, p);
  }
}

}  // namespace

size_t prefill_workspace_bytes(int B, int Hv, int dk, int dv, int T, int chunk) {
  (void)B; (void)Hv; (void)dk; (void)dv; (void)T; (void)chunk;
  return 0;
}

hipError_t launch_prefill(const PrefillParams& p, int dk, int dv, int io_bf16, hipStream_t stream) {
  (void)dv;
  if (dk == 128) {
    if (io_bf16) launch_wy<128, 1>(p, stream);
    else launch_wy<128, 0>(p, stream);
  } else {
    if (io_bf16) launch_wy<64, 1>(p, stream);
    else launch_wy<64, 0>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace pace
