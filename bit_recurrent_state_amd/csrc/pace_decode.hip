// Batched gated-delta decode step with periodic rounding and a fused flush, on a packed
// int4/int8 state with channel-aligned scale groups -- gfx950 (CDNA4, wave64).
//
// Method (PACE summary, onedev.kr "How it works" / "How it differs"; paper review
// "1. Key Terms"): each decoded token is appended to a decode buffer; the output is
// formed by replaying the buffered tokens on the last-rounded state; every dP tokens the
// buffer is folded into the state, which is rounded once.
//
// One workgroup of 2 waves owns one (sequence, value head) tile, so all B x Hv tiles of
// a layer are resident at once at B = 64 and 32 heads (eight workgroups per CU).  With S_0 the dequantised state,
// k^_i / v^_i the buffered (quantised) tokens and q the query:
//   prologue     the current token, its gates, every buffer slot of the period and the
//                tile's scales / zero points are requested at once (no address waits
//                for the count); the state codes (into registers) are requested once
//                the token phase has used them, so the whole launch's token traffic is
//                served ahead of the state stream.
//   projections  p_i = S_0^T k^_i and r = S_0^T q on the int8 matrix cores: stored codes
//                (A) times the buffer's key codes and three int8 pieces of q (B; exact
//                down to 2^-20 of max|q|),
//                one 32-key block per MFMA so every MFMA lies inside one scale group;
//                asymmetric zero points enter through a second MFMA per block (A = the
//                column's zero point in every byte), so the accumulator is the exact
//                integer sum_k (c - z) k and one scale multiply per (column, group) is
//                left.
//   replay       per value column, u_i = beta_i (v^_i - a_i y_i) with
//                y_m <- a_i y_m + (k^_i . k^_m) u_i and y_q <- a_i y_q + (k^_i . q) u_i,
//                the buffer replay written on projections; o = y_q.
//   flush        S_n = Gamma_n S_0 + K^ diag(prod_{l>i} a_l) U on the bf16 matrix cores:
//                key codes (exact in bf16) times a three-piece bf16 split of the fp32
//                weights, accumulated onto Gamma_n S_0 in fp32; every (column, g-group)
//                is then requantised in registers and written back in place.
// The state is read once per step and written only on flush.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pace_internal.h"
#include "pace_lanes.h"
#include "pace_numerics.h"

namespace pace {
namespace {

constexpr int kWaves = 2;
constexpr int kThreads = 64 * kWaves;


typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u32 __attribute__((ext_vector_type(4)));
typedef unsigned v2u32 __attribute__((ext_vector_type(2)));

// The packed state is a stream: a launch reads each tile's codes, scales and zero points
// once, writes them only on the flush, and reads nothing of them again.  When the states
// of a model's layers together exceed the last-level cache (large batches: 17.8 MB a
// layer at B = 64, 427 MB over 24 layers), its loads and stores are non-temporal (NTS), so
// that the stream does not push out of the caches the data that is reused: above all the
// decode buffer, which every step of the period reads again, and the key token and
// buffered keys that the value heads of one key head share.  Small batches keep ordinary
// accesses, so that the states stay cache-resident from one step to the next.
template <bool NT>
__device__ inline uint4 ld_state(const void* p) {
  if constexpr (NT) {
    const v4u32 v = __builtin_nontemporal_load((const v4u32*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *(const uint4*)p;
  }
}
template <bool NT>
__device__ inline uint2 ld_state2(const void* p) {
  if constexpr (NT) {
    const v2u32 v = __builtin_nontemporal_load((const v2u32*)p);
    return make_uint2(v.x, v.y);
  } else {
    return *(const uint2*)p;
  }
}
template <bool NT, class T>
__device__ inline void st_state(T* p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}
template <bool NT>
__device__ inline void st_state4(void* p, uint4 w) {
  if constexpr (NT) __builtin_nontemporal_store(v4u32{w.x, w.y, w.z, w.w}, (v4u32*)p);
  else *(uint4*)p = w;
}
template <bool NT>
__device__ inline void st_state2(void* p, uint2 w) {
  if constexpr (NT) __builtin_nontemporal_store(v2u32{w.x, w.y}, (v2u32*)p);
  else *(uint2*)p = w;
}

template <bool BF16>
__device__ inline float load_io(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  else return ((const float*)p)[i];
}
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even bf16 by the hardware conversion, packed
// (a in the low half).
__device__ inline uint32_t pk_bf16(float a, float b) {
  const v2bf h = __builtin_convertvector(v2f{a, b}, v2bf);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

template <bool BF16>
__device__ inline void store_io(void* p, size_t i, float x) {
  if constexpr (BF16) ((uint16_t*)p)[i] = (uint16_t)pk_bf16(x, 0.f);
  else ((float*)p)[i] = x;
}

// Lane permutations inside rows of 16 lanes (DPP): quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror.
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Maximum over each row of 16 lanes; every lane of the row ends with it.
__device__ inline float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}

// Sum of the 8 signed bytes of v.
__device__ inline int sum8(long v) {
  const int lo = (int)(v & 0xffffffffl), hi = (int)((unsigned long)v >> 32);
  return __builtin_amdgcn_sdot4(hi, 0x01010101, __builtin_amdgcn_sdot4(lo, 0x01010101, 0, false), false);
}

// x as three int8 pieces with power-of-two scales s1, s1/128, s1/16384, where
// s1 = 2^(e-6) for the vector's max |x| = M = m 2^e (0.5 <= m < 1), so |x / s1| < 64 and every
// piece fits in int8.  The pieces reproduce x to within s1 / 32768 = 2^(e-21), i.e. exactly
// down to 2^-20 of M (elements more than 2^12 times smaller than M lose their low bits).
// Returns the exponent of s1 in *e1 (0 for M = 0, when every piece is 0).
__device__ inline void int8_pieces(float x, float M, float& p1, float& p2, float& p3, int& e1) {
  p1 = p2 = p3 = 0.f;
  e1 = 0;
  if (M > 0.f) {
    frexpf(M, &e1);
    e1 -= 6;
    p1 = rintf(ldexpf(x, -e1));
    const float r1 = x - ldexpf(p1, e1);
    p2 = rintf(ldexpf(r1, 7 - e1));
    const float r2 = r1 - ldexpf(p2, e1 - 7);
    p3 = rintf(ldexpf(r2, 14 - e1));
  }
}

// Shared memory of one workgroup.  TOK = largest decode period this instantiation
// serves; vector slots 0..TOK-1 are buffered tokens, TOK..TOK+2 the pieces of q.
// Row strides are padded (codes: +16 bytes, projections: +4 floats) so that the 16 lanes
// of an MFMA operand or output row group hit distinct LDS banks.  The value slots, the
// scales and the zero points are sized for the instantiation's buffer kind, number of
// scale groups (NGM) and symmetry (ZP: zero points present): 16.2 KB for PACE-4.
template <int D, int TOK, int BUF, int NGM, bool ZP>
struct alignas(16) Smem {
  static constexpr int NV = 16 * ((TOK + 3 + 15) / 16);
  static constexpr int CH = TOK / 8;        // 8-token chunks of the flush
  static constexpr int KCS = D + 16;        // code row stride (bytes)
  static constexpr int PS = D + 4;          // projection row stride (floats)
  alignas(16) int8_t kc[NV][KCS];           // B-operand codes of every slot
  alignas(16) union {
    int8_t c[TOK][D];                       // int8 buffer: value codes
    uint16_t b[BUF == PACE_BUF_K4_VBF16 ? TOK : 1][D];   // mixed buffer: bf16 values
  } v;
  alignas(16) union {
    float P[NV][PS];                        // projections
    uint16_t W[CH][4][D][8];                // flush weights: 3 bf16 pieces + zeros, [col][token]
  } pw;
  alignas(16) uint16_t kT[CH][D][8];        // key codes as bf16, rows in (tile, row) order
  alignas(16) float G[NV][NV];              // Gram matrix of the slots (scaled)
  float Gq[NV];                             // k_slot . q (the q pieces combined)
  alignas(16) float scf[NGM][D];            // this tile's scales as fp32, [group][col]
  alignas(16) uint8_t zeros[ZP ? D : 1][4]; // this tile's zero points, [col][group], a byte each
  float vscale[NV];                         // key scale of each token slot / q piece scale
  float vs[TOK], ga[TOK], gb[TOK];
  float red[3][4 * kWaves];                 // row maxima of |k|, |v|, |q|
  float gamma_n;
};

// HB: 4 = every head 4-bit, 8 = every head 8-bit, 0 = per-head width from the map.
// IO: 1 = bf16 q/k/v/o, 0 = fp32.
// GT: scale-group size (32 or 64), 0 = taken from the parameters at run time.
// AS: 0 = symmetric, 1 = asymmetric, 2 = taken from the parameters at run time.
// NTS: the state's codes, scales and zero points are read and written non-temporally.
// BFS: the state is bf16 values (one dv x dk record per head, value-column-major): the
//      same buffer, replay and flush schedule, with bf16 matrix-core projections and a
//      flush that rounds each element to the nearest bf16.
// Second kernel argument: the sequence order of ordered launches, nothing otherwise (so
// that launches in plain order keep their argument block and their first addresses need
// no extra load).
template <bool ORD>
struct OrderArg : SeqOrder {};
template <>
struct OrderArg<false> {};

template <int D, int TOK, int BUF, int HB, int IO, int GT, int AS, bool NTS, bool ORD = false, bool BFS = false>
// At least eight resident workgroups per CU (four waves per SIMD) for the specialised
// dP <= 8 packed-state variants, so a 2048-tile launch runs in one round: at most 128
// VGPRs (PACE-4 needs 86 and 16.2 KB of LDS, so ten fit).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(!BFS && TOK <= 8 && GT != 0 ? 4 : 1)))
void decode_kernel(DecodeParams p, OrderArg<ORD> ord) {
  using SM = Smem<D, TOK, BUF, (GT != 0 ? D / GT : 4), AS != 0>;
  constexpr int NV = SM::NV;
  constexpr int NT = NV / 16;           // 16-vector MFMA column tiles
  constexpr int QS = TOK;               // first q-piece slot
  constexpr int CH = SM::CH;
  constexpr int KB = D / 32;            // 32-key MFMA blocks per column
  constexpr int STRIPS = D / 16;        // 16-column strips per tile
  constexpr int SPW = STRIPS / kWaves;  // strips per wave
  constexpr bool kBf16 = IO == 1;
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches and addresses
  const int l16 = lane & 15, qq = lane >> 4;
  // The value heads of one key head run on one XCD, so that the key token, the query and
  // the buffered keys they share are fetched into one L2: workgroups are dealt to the 8
  // XCDs in turn by linear id, so within each block of 8 gamma heads the heads of one key
  // head are placed 8 ids apart (power-of-two gamma, Hv a multiple of 8 gamma).
  int h = blockIdx.x;
  // the sequence of this workgroup row: the caller's order (validated as a permutation on
  // the host) in ordered launches
  int b = blockIdx.y;
  if constexpr (ORD) b = ord.seq[blockIdx.y];
  if (p.gamma > 1 && (p.gamma & (p.gamma - 1)) == 0 && p.Hv % (8 * p.gamma) == 0) {
    const int lg = __builtin_ctz(p.gamma);
    const int r = h & (8 * p.gamma - 1);
    h = ((((h >> (3 + lg)) << 3) + (r & 7)) << lg) | (r >> 3);
  }
  const int kh = h / p.gamma;

  // ---------------------------------------------------------------- prologue
  // Every global load below is unconditional with an in-bounds index, so the waves
  // issue all of them before the first wait.
  int32_t* countp = (int32_t*)p.buffer + (size_t)b * p.Hv + h;
  const int count_raw = *countp;
  __builtin_amdgcn_sched_barrier(0);          // issue the count load first

  const bool is8 = BFS ? false : (HB == 8 ? true : (HB == 4 ? false : ((p.mask8 >> h) & 1ull) != 0));
  const int bits = is8 ? 8 : 4;
  const uint64_t below = h ? (p.mask8 & ((1ull << h) - 1ull)) : 0ull;
  const uint64_t n8 = (uint64_t)__popcll(below);
  uint8_t* rec = p.state + (uint64_t)b * p.seq_stride + (uint64_t)h * p.rec4 + n8 * (p.rec8 - p.rec4);
  uint16_t* g_scales = (uint16_t*)(rec + (is8 ? p.scales_off8 : p.scales_off4));
  uint8_t* g_zeros = rec + (is8 ? p.zeros_off8 : p.zeros_off4);
  const int group = GT ? GT : p.group;
  const int NG = D / group;
  const int kpg = group / 32;           // MFMA blocks per scale group
  const int cbytes = BFS ? 2 * D : D * bits / 8;   // bytes per state column
  const bool asym = AS == 2 ? (p.asym != 0) : (AS == 1);
  const bool flush_only = p.flush_only != 0;

  // The loads are issued in the order they are consumed (the memory counters complete
  // in order): the active flag and the current token first, so that the token can be
  // quantised while the state codes and the buffered tokens are still in flight.
  // branch-free: without a mask the load reads an in-bounds stand-in and is ignored
  const uint8_t mask_v = *(p.mask ? p.mask + b : (const uint8_t*)countp);
  const bool active = !p.mask || mask_v != 0;
  // current token (a flush-only launch is given in-bounds stand-in pointers)
  const int te = tid < D ? tid : D - 1;
  const float kx = load_io<kBf16>(p.k, ((size_t)b * p.Hk + kh) * D + te);
  const float vx = load_io<kBf16>(p.v, ((size_t)b * p.Hv + h) * D + te);
  const float qx = load_io<kBf16>(p.q, ((size_t)b * p.Hk + kh) * D + te);
  // gates of the current token: lane l of each wave loads element min(l, Hv-1) of this
  // sequence's row (a vector load, issued with the others); lane h holds head h
  const float a_row = p.a[(size_t)b * p.Hv + min(lane, p.Hv - 1)];
  const float b_row = p.beta[(size_t)b * p.Hv + min(lane, p.Hv - 1)];

  // Buffered tokens.  The slots of the first half of the period are requested at once
  // (fixed-trip vector loads, indices clamped to that half), so their addresses do not
  // wait for the count; those of the second half only when the count has reached them,
  // as soon as it is known.  Slots at and past the count are loaded only in the first
  // half, and never used.
  const size_t kslot0 = ((size_t)b * p.Hk + kh) * p.dP;
  const size_t vslot0 = ((size_t)b * p.Hv + h) * p.dP;
  float* ks_buf = (float*)(p.buffer + p.off_ks);
  float* a_buf = (float*)(p.buffer + p.off_a);
  float* beta_buf = (float*)(p.buffer + p.off_beta);
  constexpr int RV = D / 16;                  // 16-byte vectors per int8 code row
  constexpr int KV4 = D / 32;                 // 16-byte vectors per 4-bit key row
  constexpr int KIT = BUF == PACE_BUF_INT8 ? (TOK * RV + kThreads - 1) / kThreads
                                           : (TOK * KV4 + kThreads - 1) / kThreads;
  constexpr int VIT = BUF == PACE_BUF_INT8 ? KIT : (TOK * (D / 8) + kThreads - 1) / kThreads;
  constexpr int VK = BUF == PACE_BUF_INT8 ? RV : KV4;        // key vectors per slot
  constexpr int VV = BUF == PACE_BUF_INT8 ? RV : D / 8;      // value vectors per slot
  const int early = min(TOK / 2, p.dP);                      // slots requested at once
  const uint4* kc_buf = (const uint4*)(p.buffer + p.off_kc + kslot0 * (BUF == PACE_BUF_INT8 ? D : D / 2));
  const uint4* v_buf = (const uint4*)(p.buffer + p.off_v + vslot0 * (BUF == PACE_BUF_INT8 ? D : 2 * D));
  uint4 kv[KIT], vv[VIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it) kv[it] = kc_buf[min(tid + it * kThreads, early * VK - 1)];
#pragma unroll
  for (int it = 0; it < VIT; ++it) vv[it] = v_buf[min(tid + it * kThreads, early * VV - 1)];
  const int si = min(tid, p.dP - 1);
  const float ks_l = ks_buf[kslot0 + si], a_l = a_buf[vslot0 + si], b_l = beta_buf[vslot0 + si];
  const float vs_l = BUF == PACE_BUF_INT8 ? ((const float*)(p.buffer + p.off_vs))[vslot0 + si] : 0.f;

  // scales and zero points of the whole tile (symmetric states read the scales twice
  // instead of a zero-point region they do not have)
  const int sc_vec = D * NG * 2 / 16;
  const int zp_vec = asym ? D * NG * bits / 8 / 16 : 1;
  uint4 sc_reg = make_uint4(0, 0, 0, 0), zp_reg = make_uint4(0, 0, 0, 0);
  if constexpr (!BFS) {
    sc_reg = ld_state<NTS>((const uint4*)g_scales + min(tid, sc_vec - 1));
    zp_reg = ld_state<NTS>((const uint4*)(asym ? (const uint8_t*)g_zeros : (const uint8_t*)g_scales) + min(tid, zp_vec - 1));
  }

  // counts outside [0, dP) cannot come from this library; clamp so that every slot
  // index stays inside the buffer whatever the buffer holds
  const int n0 = min(max(count_raw, 0), p.dP - 1);
  const int n = flush_only ? n0 : n0 + 1;
  const bool do_flush = flush_only || n >= p.dP;
  const int kvec = n0 * VK, vvec = n0 * VV;
  uint4 kvl[KIT], vvl[VIT];                   // second half of the period, slots < n0
  if (n0 > early) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int i = tid + it * kThreads;
      if (i >= early * VK && i < kvec) kvl[it] = kc_buf[i];
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int i = tid + it * kThreads;
      if (i >= early * VV && i < vvec) vvl[it] = v_buf[i];
    }
  }
  // State codes of this lane, strip by strip: strip st = wave + kWaves * s, column
  // st*16 + l16, keys of quarter qq (units qq*KB .. qq*KB + KB - 1).
  // (bf16 state: keys 32 kb + 8 qq .. + 7 of the column, 16 bytes per 32-key block)
  constexpr int AW = BFS ? 4 * KB : (HB == 4 ? KB : 2 * KB);   // state dwords per strip and lane
  uint32_t araw[SPW][AW];
  auto load_state = [&]() {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int c = (wave + kWaves * s) * 16 + l16;
      const uint8_t* colp = rec + (size_t)c * cbytes + qq * KB * bits;
      if constexpr (BFS) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const uint4 v = ld_state<NTS>(rec + (size_t)c * cbytes + (32 * kb + 8 * qq) * 2);
          araw[s][4 * kb] = v.x; araw[s][4 * kb + 1] = v.y; araw[s][4 * kb + 2] = v.z; araw[s][4 * kb + 3] = v.w;
        }
      } else if (!is8) {
        if constexpr (KB == 4) {
          const uint4 v = ld_state<NTS>(colp);
          araw[s][0] = v.x; araw[s][1] = v.y; araw[s][2] = v.z; araw[s][3] = v.w;
        } else {
          const uint2 v = ld_state2<NTS>(colp);
          araw[s][0] = v.x; araw[s][1] = v.y;
        }
      } else if constexpr (HB != 4) {
#pragma unroll
        for (int kb = 0; kb < KB; kb += 2) {
          const uint4 v = ld_state<NTS>(colp + kb * 8);
          araw[s][2 * kb] = v.x; araw[s][2 * kb + 1] = v.y; araw[s][2 * kb + 2] = v.z; araw[s][2 * kb + 3] = v.w;
        }
      }
    }
  };
  // keep the scheduler from pulling the first uses of the token (and their waits)
  // above the remaining load issues
  __builtin_amdgcn_sched_barrier(0);

  // ---------------------------------- current token -> buffer (loads still in flight)
  {
    const float m0 = row_max16(tid < D ? fabsf(kx) : 0.f);
    const float m1 = row_max16(tid < D ? fabsf(vx) : 0.f);
    const float m2 = row_max16(tid < D ? fabsf(qx) : 0.f);
    if (l16 == 0) { sm.red[0][4 * wave + qq] = m0; sm.red[1][4 * wave + qq] = m1; sm.red[2][4 * wave + qq] = m2; }
  }
  const float a_t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a_row), h));
  const float b_t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b_row), h));
  __syncthreads();
  // Inactive tiles (and flushes of an empty buffer) leave here, after the barrier: an
  // exit before it would hold every load back until the flag and the count have arrived.
  // Both are uniform over the workgroup, so the whole tile leaves together.
  if (!active || (flush_only && count_raw <= 0)) return;   // (nothing buffered: nothing to flush)
  if (!flush_only) {
    float Mk = sm.red[0][0], Mv = sm.red[1][0], Mq = sm.red[2][0];
#pragma unroll
    for (int w = 1; w < 4 * kWaves; ++w) {
      Mk = fmaxf(Mk, sm.red[0][w]); Mv = fmaxf(Mv, sm.red[1][w]); Mq = fmaxf(Mq, sm.red[2][w]);
    }
    const float kq_max = BUF == PACE_BUF_INT8 ? 127.f : 7.f;
    // the fp32 buffer scales M / 127 (M / 7), correctly rounded
    const float ks = div_rn(Mk, kq_max, BUF == PACE_BUF_INT8 ? 1.0f / 127.0f : 1.0f / 7.0f);
    if (tid < D) {
      const float kcf = ks > 0.f ? fminf(fmaxf(rintf(kx / ks), -kq_max), kq_max) : 0.f;
      sm.kc[n0][tid] = (int8_t)kcf;
      int8_t vcode = 0;
      float vs = 0.f;
      if constexpr (BUF == PACE_BUF_INT8) {
        vs = div_rn(Mv, 127.f, 1.0f / 127.0f);
        vcode = (int8_t)(vs > 0.f ? fminf(fmaxf(rintf(vx / vs), -127.f), 127.f) : 0.f);
        sm.v.c[n0][tid] = vcode;
      } else {
        sm.v.b[n0][tid] = (uint16_t)pk_bf16(vx, 0.f);
      }
      // q as three int8 pieces with power-of-two scales: a split, not a rounding to a code
      // grid; it reproduces each element exactly down to 2^-20 of max|q| (see int8_pieces)
      float q1, q2, q3;
      int e1;
      int8_pieces(qx, Mq, q1, q2, q3, e1);
      sm.kc[QS + 0][tid] = (int8_t)q1;
      sm.kc[QS + 1][tid] = (int8_t)q2;
      sm.kc[QS + 2][tid] = (int8_t)q3;
      if (tid == 0) {
        const float s1 = Mq > 0.f ? ldexpf(1.f, e1) : 0.f;
        sm.vscale[QS + 0] = s1;
        sm.vscale[QS + 1] = s1 * 0.0078125f;
        sm.vscale[QS + 2] = s1 * 0.00006103515625f;
        sm.vscale[n0] = ks;
        sm.vs[n0] = vs;
        sm.ga[n0] = a_t;
        sm.gb[n0] = b_t;
      }
      // append to the buffer unless this step empties it
      if (!do_flush) {
        const bool key_writer = (h % p.gamma) == 0;
        if (BUF == PACE_BUF_INT8) {
          if (key_writer) ((int8_t*)(p.buffer + p.off_kc))[(kslot0 + n0) * D + tid] = (int8_t)kcf;
          ((int8_t*)(p.buffer + p.off_v))[(vslot0 + n0) * D + tid] = vcode;
          if (tid == 0) ((float*)(p.buffer + p.off_vs))[vslot0 + n0] = vs;
        } else {
          ((uint16_t*)(p.buffer + p.off_v))[(vslot0 + n0) * D + tid] = (uint16_t)pk_bf16(vx, 0.f);
        }
        if (tid == 0) {
          if (key_writer) ks_buf[kslot0 + n0] = ks;
          a_buf[vslot0 + n0] = a_t;
          beta_buf[vslot0 + n0] = b_t;
        }
      }
    }
  }

  // ---------------------------------------------------------------- LDS fills
  // buffered slots [s0, s1) into LDS, from the first-half or the second-half registers
  // (chosen at compile time, so the register arrays are never addressed through memory)
  auto fill_slots = [&](int s0, int s1, auto half) {
    constexpr bool kLate = decltype(half)::value;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int i = tid + it * kThreads;
      if (i < s0 * VK || i >= s1 * VK) continue;
      if (BUF == PACE_BUF_INT8) {
        *(uint4*)&sm.kc[i / RV][16 * (i % RV)] = kLate ? kvl[it] : kv[it];
      } else {
        // 4-bit keys: 16 bytes = four 8-key units; byte w of unit m holds keys 8m+w (low
        // nibble) and 8m+4+w (high nibble), each stored as c + 8.
        const uint4 kx4 = kLate ? kvl[it] : kv[it];
        const uint32_t w4[4] = {kx4.x, kx4.y, kx4.z, kx4.w};
        uint32_t out[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // per byte, (x | 0x80) - 8 never borrows; ^ 0x80 leaves the code c = x - 8
          const uint32_t lo = w4[m] & 0x0F0F0F0Fu, hi = (w4[m] >> 4) & 0x0F0F0F0Fu;
          out[2 * m] = ((lo | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
          out[2 * m + 1] = ((hi | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
        }
        int8_t* dst = &sm.kc[i / KV4][32 * (i % KV4)];
        *(uint4*)dst = make_uint4(out[0], out[1], out[2], out[3]);
        *(uint4*)(dst + 16) = make_uint4(out[4], out[5], out[6], out[7]);
      }
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int i = tid + it * kThreads;
      if (i < s0 * VV || i >= s1 * VV) continue;
      const uint4 vx4 = kLate ? vvl[it] : vv[it];
      if constexpr (BUF == PACE_BUF_INT8) ((uint4*)&sm.v.c[0][0])[i] = vx4;
      else ((uint4*)&sm.v.b[0][0])[i] = vx4;
    }
  };
  fill_slots(0, min(n0, early), std::false_type{});
  if (BUF == PACE_BUF_INT8 && tid < n0) sm.vs[tid] = vs_l;
  if (tid < n0) {
    sm.vscale[tid] = ks_l;
    sm.ga[tid] = a_l;
    sm.gb[tid] = b_l;
  }
  // unused token slots (n .. TOK-1) and, without a query, the q slots hold zeros
#pragma unroll
  for (int it = 0; it < (NV * RV + kThreads - 1) / kThreads; ++it) {
    const int i = tid + it * kThreads;
    const int row = i / RV;
    if (i < NV * RV && row >= n && (row < QS || flush_only || row >= QS + 3))
      *(uint4*)&sm.kc[row][16 * (i % RV)] = make_uint4(0, 0, 0, 0);
  }
  if (tid >= n && tid < NV && (tid < QS || flush_only || tid >= QS + 3)) sm.vscale[tid] = 0.f;
  // scales regrouped [group][col] (a lane's four output columns of one group are one
  // vector read), zero points [col][group] (the four groups of the lane's A-operand
  // column are one read)
  const int lng = NG == 4 ? 2 : NG - 1;      // log2 NG (NG in {1, 2, 4})
  if (!BFS && tid < sc_vec) {               // 8 bf16 scales [col][group] -> fp32
    const uint32_t w[4] = {sc_reg.x, sc_reg.y, sc_reg.z, sc_reg.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int e = 8 * tid + k;
      const uint32_t u = (k & 1) ? (w[k >> 1] & 0xFFFF0000u) : (w[k >> 1] << 16);
      sm.scf[e & (NG - 1)][e >> lng] = bits_f32(u);
    }
  }
  if (!BFS && asym && tid < zp_vec) {
    const uint32_t w[4] = {zp_reg.x, zp_reg.y, zp_reg.z, zp_reg.w};
    if (is8) {                               // 16 zero points, a byte each
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int e = 16 * tid + k;
        sm.zeros[e >> lng][e & (NG - 1)] = (uint8_t)(w[k >> 2] >> (8 * (k & 3)));
      }
    } else {                                 // 32 packed 4-bit zero points (low nibble first)
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int e = 32 * tid + k;
        sm.zeros[e >> lng][e & (NG - 1)] = (uint8_t)((w[k >> 3] >> (4 * (k & 7))) & 15u);
      }
    }
  }
  // The state codes are requested only now, with the token phase done: the token-sized
  // loads of every tile (current token, buffer, scales) are then served ahead of the
  // state stream.
  load_state();
  if (n0 > early) fill_slots(early, n0, std::true_type{});   // (loads issued before the state's)

  __syncthreads();
  if (BUF == PACE_BUF_K4_VBF16 && !flush_only && !do_flush && (h % p.gamma) == 0 && tid < D / 2) {
    const int m = tid / 4, w = tid % 4;
    const int lo = sm.kc[n0][8 * m + w] + 8, hi = sm.kc[n0][8 * m + 4 + w] + 8;
    ((uint8_t*)(p.buffer + p.off_kc))[(kslot0 + n0) * (D / 2) + tid] = (uint8_t)(lo | (hi << 4));
  }

  // --------------------------------------------- B operands, group sums, Gram
  // Code-offset term of the projections, per scale group and slot vector, on MFMA with a
  // constant A operand (every output row holds the same value), used as the seed of the
  // group's accumulator.  Symmetric 4-bit states store c + 8, so each group's projection
  // carries -8 * (sum of the slot's codes over the group): an A of -8 bytes produces it.
  // Symmetric 8-bit codes and asymmetric 4-bit codes enter the MFMA as they are (no
  // term).  Asymmetric 8-bit codes enter as c - 128 and their zero-point MFMA below adds
  // (127 - z) times the sum, so the seed is the plain sum (A of ones).
  long bop[NT][KB];
  v4i zacc[NT][4];
  const long zrow = asym ? (is8 ? 0x0101010101010101l : 0l) : (is8 ? 0l : (long)0xF8F8F8F8F8F8F8F8ull);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) bop[nt][kb] = *(const long*)&sm.kc[nt * 16 + l16][32 * kb + 8 * qq];
  if (wave == kWaves - 1) {
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      if (mt * 16 >= n && mt * 16 < QS) continue;     // row tiles of empty token slots
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        v4i acc = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(bop[mt][kb], bop[nt][kb], acc, 0, 0, 0);
        const int col = nt * 16 + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mt * 16 + 4 * qq + i;
          const float gv = (float)acc[i] * sm.vscale[row] * sm.vscale[col];
          sm.G[row][col] = gv;
          // k_row . q: the three q pieces sit in columns QS..QS+2 of one 16-lane row
          if (nt == QS / 16) {
            const float gsum = gv + dpp<0x101>(gv) + dpp<0x102>(gv);
            if (col == QS) sm.Gq[row] = gsum;
          }
        }
      }
    }
  }

  // ------------------------------------------------------------ projections
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) zacc[nt][g] = v4i{0, 0, 0, 0};
    if (!BFS && zrow != 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          if (kb / kpg == g) zacc[nt][g] = __builtin_amdgcn_mfma_i32_16x16x32_i8(zrow, bop[nt][kb], zacc[nt][g], 0, 0, 0);
    }
  }
  if constexpr (BFS) {
    // bf16 state: the stored columns are the A operand as they are, the slot codes (int8,
    // exact in bf16) the B operand, fp32 accumulation; no scale groups
    v8bf bb[NT][KB];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const unsigned long x = (unsigned long)bop[nt][kb];
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w4[e] = pk_bf16((float)(int8_t)(x >> (16 * e)), (float)(int8_t)(x >> (16 * e + 8)));
        __builtin_memcpy(&bb[nt][kb], w4, 16);
      }
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int ocol = (wave + kWaves * s) * 16 + 4 * qq;
      v4f accf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) accf[nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        v8bf sa;
        __builtin_memcpy(&sa, &araw[s][4 * kb], 16);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) accf[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa, bb[nt][kb], accf[nt], 0, 0, 0);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int vi = nt * 16 + l16;
        const float vsc = sm.vscale[vi];
        *(float4*)&sm.pw.P[vi][ocol] = make_float4(accf[nt][0] * vsc, accf[nt][1] * vsc, accf[nt][2] * vsc, accf[nt][3] * vsc);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < (BFS ? 0 : SPW); ++s) {
    const int col0 = (wave + kWaves * s) * 16;
    const int ocol = col0 + 4 * qq;     // output columns ocol + i of this lane
    float proj[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) proj[nt][i] = 0.f;
    v4i acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = zacc[nt][0];
    // Asymmetric zero points: -z (4-bit) or 127 - z (8-bit, = z ^ 0x7F as a byte) of each
    // group of the lane's A-operand column, as int8 bytes; replicated over a block's eight
    // A bytes they add -z (resp. (127 - z)) times the slot's code sum to the row of that
    // column, so the accumulator ends at sum_k (c - z) k exactly.
    uint32_t zx = 0u;
    if (asym) {
      const uint32_t z4 = *(const uint32_t*)&sm.zeros[col0 + l16][0];
      // per byte, 0x80 - z never borrows (z <= 15); ^ 0x80 leaves -z
      zx = is8 ? (z4 ^ 0x7F7F7F7Fu) : ((0x80808080u - z4) ^ 0x80808080u);
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int g = kb / kpg;
      long a;
      if (!is8) {
        const uint32_t d = araw[s][kb];
        a = (long)(((unsigned long)((d >> 4) & 0x0F0F0F0Fu) << 32) | (d & 0x0F0F0F0Fu));
      } else if constexpr (HB != 4) {
        a = (long)(((unsigned long)(araw[s][2 * kb + 1] ^ 0x80808080u) << 32) | (araw[s][2 * kb] ^ 0x80808080u));
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bop[nt][kb], acc[nt], 0, 0, 0);
      if (asym) {
        const uint32_t zr = __builtin_amdgcn_perm(zx, zx, 0x01010101u * (uint32_t)g);   // byte g, four times
        const long za = (long)(((unsigned long)zr << 32) | zr);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(za, bop[nt][kb], acc[nt], 0, 0, 0);
      }
      if ((kb + 1) % kpg != 0) continue;
      // end of scale group g: one scale multiply per (column, group)
      const float4 sc4 = *(const float4*)&sm.scf[g][ocol];
      const float scv[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) proj[nt][i] += (float)acc[nt][i] * scv[i];
      if (g + 1 < NG) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          v4i nx = v4i{0, 0, 0, 0};
#pragma unroll
          for (int gg = 1; gg < 4; ++gg) nx = gg == g + 1 ? zacc[nt][gg] : nx;
          acc[nt] = nx;
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int vi = nt * 16 + l16;
      const float vsc = sm.vscale[vi];
      *(float4*)&sm.pw.P[vi][ocol] = make_float4(proj[nt][0] * vsc, proj[nt][1] * vsc, proj[nt][2] * vsc, proj[nt][3] * vsc);
    }
  }
  __syncthreads();

  // -------------------------------------------- replay, one value column / thread
  float u[TOK];
  if (tid < D) {
    const int j = tid;
    float y[TOK];
#pragma unroll
    // slots n.. hold zero codes, so their projections and Gram entries are zero and the
    // updates below may run over them unconditionally
    for (int m = 0; m < TOK; ++m) { y[m] = sm.pw.P[m][j]; u[m] = 0.f; }
    float yq = sm.pw.P[QS][j] + sm.pw.P[QS + 1][j] + sm.pw.P[QS + 2][j];
#pragma unroll
    for (int i = 0; i < TOK; ++i) {
      // (an early exit keeps the short periods cheap; the long-period instantiations keep
      // a plain guard, which the compiler still unrolls, so nothing is indexed at run time)
      if constexpr (TOK <= 8) {
        if (i >= n) break;
      } else {
        if (i >= n) continue;
      }
      const float ai = sm.ga[i];
      float vh;
      if constexpr (BUF == PACE_BUF_INT8) vh = (float)sm.v.c[i][j] * sm.vs[i];
      else vh = bf16_to_f32(sm.v.b[i][j]);
      const float ui = sm.gb[i] * (vh - ai * y[i]);
      u[i] = ui;
#pragma unroll
      for (int m = i + 1; m < TOK; ++m) y[m] = ai * y[m] + sm.G[i][m] * ui;
      yq = ai * yq + sm.Gq[i] * ui;
    }
    if (!flush_only) store_io<kBf16>(p.o, ((size_t)b * p.Hv + h) * D + j, yq);
  }
  if (!do_flush) {
    if (tid == 0) *countp = n;
    return;
  }
  __syncthreads();        // every projection is read: the weights may overwrite them

  // ------------------------------------------------------------ flush: weights
  // W_i[j] = k-scale_i * prod_{l>i} a_l * u_i[j], split into three bf16 pieces; key
  // codes transposed to [key][token] bf16 for the A operand.
  if (tid < D) {
    const int j = tid;
    float w = 1.f;
    float wv[TOK];
#pragma unroll
    for (int i = TOK - 1; i >= 0; --i) {
      wv[i] = 0.f;
      if (i < n) {
        wv[i] = w * sm.vscale[i] * u[i];
        w *= sm.ga[i];
      }
    }
    uint32_t pk[3][TOK / 2];              // pieces, two bf16 per dword, token order
#pragma unroll
    for (int e = 0; e < TOK / 2; ++e) {
      float x0 = wv[2 * e], x1 = wv[2 * e + 1];
#pragma unroll
      for (int pc = 0; pc < 3; ++pc) {
        pk[pc][e] = pk_bf16(x0, x1);
        x0 -= bits_f32(pk[pc][e] << 16);
        x1 -= bits_f32(pk[pc][e] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
#pragma unroll
      for (int pc = 0; pc < 3; ++pc)
        *(uint4*)&sm.pw.W[ch][pc][j][0] = make_uint4(pk[pc][4 * ch], pk[pc][4 * ch + 1], pk[pc][4 * ch + 2], pk[pc][4 * ch + 3]);
      *(uint4*)&sm.pw.W[ch][3][j][0] = make_uint4(0, 0, 0, 0);   // lanes of quarter 3 add nothing
    }
    if (j == 0) sm.gamma_n = w;
    // key j sits in accumulator tile t = 2 (j / 32) + (j % 8) / 4, row m = 4 ((j % 32) / 8) + j % 4
    const int t = 2 * (j / 32) + (j % 8) / 4, m = 4 * ((j % 32) / 8) + (j % 4);
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      uint32_t kw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // slots n.. hold zero codes; small integers are exact in bf16
        const int i0 = 8 * ch + 2 * e;
        kw[e] = pk_bf16((float)sm.kc[i0][j], (float)sm.kc[i0 + 1][j]);
      }
      *(uint4*)&sm.kT[ch][t * 16 + m][0] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
    }
  }
  __syncthreads();

  // ----------------------------------------- flush: fold on MFMA, requantise
  const float gn = sm.gamma_n;
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int c = (wave + kWaves * s) * 16 + l16;    // this lane's column
    // accumulator tile t = 2 kb + half holds keys 32 kb + 8 qq + 4 half + i
    v4f acc[2 * KB];
#pragma unroll
    for (int kb = 0; kb < KB && BFS; ++kb) {
      // bf16 state: dword e of block kb holds keys 8 qq + 2e, 2e + 1 of the column
      const uint32_t* w4 = &araw[s][4 * kb];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        acc[2 * kb][2 * i] = gn * bits_f32(w4[i] << 16);
        acc[2 * kb][2 * i + 1] = gn * bits_f32(w4[i] & 0xFFFF0000u);
        acc[2 * kb + 1][2 * i] = gn * bits_f32(w4[2 + i] << 16);
        acc[2 * kb + 1][2 * i + 1] = gn * bits_f32(w4[2 + i] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int kb = 0; kb < (BFS ? 0 : KB); ++kb) {
      const int g = kb / kpg;
      const float sc = sm.scf[g][c];
      const int z = asym ? (int)sm.zeros[c][g] : 1 << (bits - 1);
      const float gs = gn * sc, gz = -gs * (float)z;
      uint32_t b0, b1;            // 4 stored codes each (bytes): keys +0..3, +4..7
      if (!is8) {
        b0 = araw[s][kb] & 0x0F0F0F0Fu;
        b1 = (araw[s][kb] >> 4) & 0x0F0F0F0Fu;
        // keep the masks whole-word, so that each byte converts in one instruction
        asm("" : "+v"(b0));
        asm("" : "+v"(b1));
      } else if constexpr (HB != 4) {
        b0 = araw[s][2 * kb];
        b1 = araw[s][2 * kb + 1];
      }
      // byte i of b0 / b1 -> float via the per-byte conversions
      acc[2 * kb][0] = fmaf((float)(b0 & 255u), gs, gz);
      acc[2 * kb][1] = fmaf((float)((b0 >> 8) & 255u), gs, gz);
      acc[2 * kb][2] = fmaf((float)((b0 >> 16) & 255u), gs, gz);
      acc[2 * kb][3] = fmaf((float)(b0 >> 24), gs, gz);
      acc[2 * kb + 1][0] = fmaf((float)(b1 & 255u), gs, gz);
      acc[2 * kb + 1][1] = fmaf((float)((b1 >> 8) & 255u), gs, gz);
      acc[2 * kb + 1][2] = fmaf((float)((b1 >> 16) & 255u), gs, gz);
      acc[2 * kb + 1][3] = fmaf((float)(b1 >> 24), gs, gz);
    }
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      if (ch * 8 >= n) break;
      // K index 8 qq + token: quarters 0..2 carry the three weight pieces, quarter 3 a
      // zero piece, so the key codes can be loaded by every lane unconditionally
      const v8bf bw = *(const v8bf*)&sm.pw.W[ch][qq][c][0];
      v8bf ak[2 * KB];
#pragma unroll
      for (int t = 0; t < 2 * KB; ++t) ak[t] = *(const v8bf*)&sm.kT[ch][t * 16 + l16][0];
#pragma unroll
      for (int t = 0; t < 2 * KB; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[t], bw, acc[t], 0, 0, 0);
    }
    if constexpr (BFS) {
      // round every element to the nearest bf16 and write the column block back
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        st_state4<NTS>(rec + (size_t)c * cbytes + (32 * kb + 8 * qq) * 2,
                       make_uint4(pk_bf16(acc[2 * kb][0], acc[2 * kb][1]), pk_bf16(acc[2 * kb][2], acc[2 * kb][3]),
                                  pk_bf16(acc[2 * kb + 1][0], acc[2 * kb + 1][1]),
                                  pk_bf16(acc[2 * kb + 1][2], acc[2 * kb + 1][3])));
      continue;
    }
    // Requantise each (column, group) and write back in place.  Every group's range is
    // reduced over the four lanes (quarters) of the column; then each lane derives the
    // quantiser of one group (qq mod NG) and the others read it, rather than all four
    // lanes deriving every group.
    float lmx[4], lmn[4];                   // this lane's range of each group
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      lmx[g] = 0.f;
      lmn[g] = 0.f;
      if (g >= NG) break;
      if (asym) {
        float mx = -INFINITY, mn = INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if (kb / kpg != g) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) {       // running chains: one max3 / min3 per two values
            mx = fmaxf(fmaxf(mx, acc[2 * kb][i]), acc[2 * kb + 1][i]);
            mn = fminf(fminf(mn, acc[2 * kb][i]), acc[2 * kb + 1][i]);
          }
        }
        lmx[g] = mx;
        lmn[g] = mn;
      } else {                    // symmetric: only max |x| matters
        float mx = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if (kb / kpg != g) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(fmaxf(mx, fabsf(acc[2 * kb][i])), fabsf(acc[2 * kb + 1][i]));
        }
        lmx[g] = mx;
      }
    }
    // the range of this lane's group (row qq derives the quantiser of group qq mod NG),
    // reduced over the four rows of the column
    float mxm, mnm;
    auto reduce_own = [&](auto ng) {
      constexpr int G = decltype(ng)::value;
      mxm = rows_reduce_own<G, true>(lmx);
      mnm = asym ? rows_reduce_own<G, false>(lmn) : -mxm;
    };
    if (NG == 4) reduce_own(std::integral_constant<int, 4>{});
    else if (NG == 2) reduce_own(std::integral_constant<int, 2>{});
    else reduce_own(std::integral_constant<int, 1>{});
    const GroupQuant gq = group_quant(mnm, mxm, asym, bits);
    float rg[4];
    int zg[4];
    {                                       // the quantiser of group g from row g
      uint32_t ru[4], zu[4] = {0, 0, 0, 0};
      rows_gather(f32_bits(gq.r), NG, ru);
      if (asym) rows_gather((uint32_t)gq.z, NG, zu);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        rg[g] = bits_f32(ru[g]);
        zg[g] = (int)zu[g];
      }
    }
    if (qq < NG) {
      st_state<NTS>(&g_scales[c * NG + qq], (uint16_t)(f32_bits(gq.s) >> 16));
      if (asym) {
        const int e = c * NG + qq;
        if (is8) {
          st_state<NTS>(&g_zeros[e], (uint8_t)gq.z);
        } else if (e & 1) {                 // two 4-bit zero points a byte, low nibble first
          int zlo = zg[0];
#pragma unroll
          for (int g = 1; g < 4; ++g) zlo = g == qq - 1 ? zg[g] : zlo;
          st_state<NTS>(&g_zeros[e >> 1], (uint8_t)(zlo | (gq.z << 4)));
        }
      }
    }
    uint32_t outw[AW];
#pragma unroll
    for (int i = 0; i < AW; ++i) outw[i] = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g >= NG) break;
      const CodeRange cr = code_range(asym ? zg[g] : 1 << (bits - 1), asym, bits);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (kb / kpg != g) continue;
        // codes as the low bytes of clamped fma results; gathered four at a time
        // (symmetric: |x| r <= 2^(b-1) - 1 up to one rounding, since the scale is the
        // rounded-up max / (2^(b-1) - 1), so no clamp is needed)
        uint32_t f0[4], f1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float y0 = fmaf(acc[2 * kb][i], rg[g], cr.magic), y1 = fmaf(acc[2 * kb + 1][i], rg[g], cr.magic);
          if (asym) {                         // clamp (lo <= hi): one median-of-three each
            y0 = __builtin_amdgcn_fmed3f(y0, cr.lo, cr.hi);
            y1 = __builtin_amdgcn_fmed3f(y1, cr.lo, cr.hi);
          }
          f0[i] = f32_bits(y0);
          f1[i] = f32_bits(y1);
        }
        const uint32_t lo = __builtin_amdgcn_perm(f0[1], f0[0], 0x0c0c0400u) | __builtin_amdgcn_perm(f0[3], f0[2], 0x04000c0cu);
        const uint32_t hi = __builtin_amdgcn_perm(f1[1], f1[0], 0x0c0c0400u) | __builtin_amdgcn_perm(f1[3], f1[2], 0x04000c0cu);
        if (!is8) {
          outw[kb] = lo | (hi << 4);
        } else if constexpr (HB != 4) {
          outw[2 * kb] = lo;
          outw[2 * kb + 1] = hi;
        }
      }
    }
    uint8_t* colp = rec + (size_t)c * cbytes + qq * KB * bits;
    if (!is8) {
      if constexpr (KB == 4) st_state4<NTS>(colp, make_uint4(outw[0], outw[1], outw[2], outw[3]));
      else st_state2<NTS>(colp, make_uint2(outw[0], outw[1]));
    } else if constexpr (HB != 4) {
#pragma unroll
      for (int kb = 0; kb < KB; kb += 2)
        st_state4<NTS>(colp + kb * 8, make_uint4(outw[2 * kb], outw[2 * kb + 1], outw[2 * kb + 2], outw[2 * kb + 3]));
    }
  }
  if (tid == 0) *countp = 0;
}

template <int D, int TOK, int BUF, int HB, int IO, int GT, int AS, bool NTS = false, bool ORD = false, bool BFS = false>
hipError_t launch_t(const DecodeParams& p, const SeqOrder* order, hipStream_t stream) {
  OrderArg<ORD> ord{};
  if constexpr (ORD) static_cast<SeqOrder&>(ord) = *order;
  hipLaunchKernelGGL((decode_kernel<D, TOK, BUF, HB, IO, GT, AS, NTS, ORD, BFS>), dim3((unsigned)p.Hv, (unsigned)p.B),
                     dim3(kThreads), 0, stream, p, ord);
  return hipGetLastError();
}

// Layers whose packed states (all sequences) reach this size stream them with
// non-temporal accesses: a stack of 24-32 such layers no longer fits the 256 MB
// last-level cache of MI355X, so the states would only evict the reused data.  Measured
// on the 24-layer PACE-4 stack: B = 16 (4.4 MB a layer) is 5% faster with ordinary
// accesses, B = 32 (8.9 MB) the same either way, B = 64 (17.8 MB) 11% faster streamed.
constexpr uint64_t kStreamStateBytes = 8ull << 20;

// Specialised instantiations for the layouts the method names (d = 128, dP <= 8, bf16
// I/O; 64-key symmetric and 32-key asymmetric groups, and their mirror images), with
// group size and symmetry known at compile time; in launch order or in a given order.
template <int BUF, int HB, bool NT, bool ORD>
hipError_t launch_fast_nt(const DecodeParams& p, const SeqOrder* o, hipStream_t stream) {
  if (p.group == 64)
    return p.asym ? launch_t<128, 8, BUF, HB, 1, 64, 1, NT, ORD>(p, o, stream)
                  : launch_t<128, 8, BUF, HB, 1, 64, 0, NT, ORD>(p, o, stream);
  return p.asym ? launch_t<128, 8, BUF, HB, 1, 32, 1, NT, ORD>(p, o, stream)
                : launch_t<128, 8, BUF, HB, 1, 32, 0, NT, ORD>(p, o, stream);
}
template <int BUF, int HB, bool ORD>
hipError_t launch_fast_o(const DecodeParams& p, const SeqOrder* o, hipStream_t stream) {
  const bool stream_state = (uint64_t)p.B * p.seq_stride >= kStreamStateBytes;
  return stream_state ? launch_fast_nt<BUF, HB, true, ORD>(p, o, stream)
                      : launch_fast_nt<BUF, HB, false, ORD>(p, o, stream);
}
template <int BUF, int HB>
hipError_t launch_fast(const DecodeParams& p, const SeqOrder* o, hipStream_t stream) {
  return o ? launch_fast_o<BUF, HB, true>(p, o, stream) : launch_fast_o<BUF, HB, false>(p, nullptr, stream);
}

template <int D, int BUF, int IO>
hipError_t launch_generic(const DecodeParams& p, hipStream_t stream) {
  if (p.dP <= 8) return launch_t<D, 8, BUF, 0, IO, 0, 2>(p, nullptr, stream);
  return launch_t<D, 32, BUF, 0, IO, 0, 2>(p, nullptr, stream);
}

// bf16 states (int8 decode buffer): streamed by the same size rule as the packed states
template <int D, int IO>
hipError_t launch_bf16_state(const DecodeParams& p, hipStream_t stream) {
  constexpr int B8 = PACE_BUF_INT8;
  if (p.dP > 8) return launch_t<D, 32, B8, 4, IO, D, 0, false, false, true>(p, nullptr, stream);
  if ((uint64_t)p.B * p.seq_stride >= kStreamStateBytes)
    return launch_t<D, 8, B8, 4, IO, D, 0, true, false, true>(p, nullptr, stream);
  return launch_t<D, 8, B8, 4, IO, D, 0, false, false, true>(p, nullptr, stream);
}

template <int BUF>
hipError_t launch_buf(const DecodeParams& p, const SeqOrder* o, int dk, hipStream_t stream) {
  if (dk == 128 && p.dP <= 8 && p.io_bf16)
    return p.mask8 == 0 ? launch_fast<BUF, 4>(p, o, stream) : launch_fast<BUF, 0>(p, o, stream);
  if (dk == 128) return p.io_bf16 ? launch_generic<128, BUF, 1>(p, stream) : launch_generic<128, BUF, 0>(p, stream);
  return p.io_bf16 ? launch_generic<64, BUF, 1>(p, stream) : launch_generic<64, BUF, 0>(p, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, const SeqOrder* order, int dk, int dv, int buf_kind,
                         hipStream_t stream) {
  (void)dv;  // dk == dv is validated by the caller
  if (p.bf16_state) {   // int8 buffer only (checked by the caller); never ordered
    if (dk == 128) return p.io_bf16 ? launch_bf16_state<128, 1>(p, stream) : launch_bf16_state<128, 0>(p, stream);
    return p.io_bf16 ? launch_bf16_state<64, 1>(p, stream) : launch_bf16_state<64, 0>(p, stream);
  }
  if (buf_kind == PACE_BUF_INT8) return launch_buf<PACE_BUF_INT8>(p, order, dk, stream);
  return launch_buf<PACE_BUF_K4_VBF16>(p, order, dk, stream);
}

}  // namespace pace
