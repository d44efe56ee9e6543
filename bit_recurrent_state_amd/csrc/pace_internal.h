// Internal declarations of the PACE library: layout arithmetic shared by the host
// entry points and the launchers, and the parameter blocks the kernels take by value.
// The packed formats are specified in include/pace.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pace.h"

namespace pace {

constexpr int kMaxHeads = 64;    // head bit map is a 64-bit mask
constexpr int kMaxPeriod = 32;   // decode period dP upper bound
constexpr int kMaxOrderedBatch = 256;   // batch bound of pace_decode_step_ordered

inline size_t pad_to(size_t n, size_t a) { return (n + a - 1) / a * a; }

// Byte sizes of one (sequence, head) record of bit width `bits`.
struct RecordLayout {
  uint32_t codes, scales, zeros, total;  // part sizes after padding; total padded to 256
};

inline RecordLayout record_layout(int dk, int dv, int group, bool asym, int bits) {
  RecordLayout r;
  const size_t ng = (size_t)dk / group;
  r.codes = (uint32_t)pad_to((size_t)dv * dk * bits / 8, 16);
  r.scales = (uint32_t)pad_to((size_t)dv * ng * 2, 16);
  r.zeros = asym ? (uint32_t)pad_to((size_t)dv * ng * bits / 8, 16) : 0u;
  r.total = (uint32_t)pad_to((size_t)r.codes + r.scales + r.zeros, 256);
  return r;
}

// Offsets (bytes) of the decode-buffer regions, each padded to 256 bytes.
struct BufferLayout {
  size_t count, kc, ks, v, vs, a, beta, total;
};

inline BufferLayout buffer_layout(const pace_layer_cfg& c) {
  BufferLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += pad_to(bytes, 256); return at; };
  const size_t B = c.B, Hv = c.Hv, Hk = c.Hk, dP = c.dP, dk = c.dk, dv = c.dv;
  L.count = take(B * Hv * 4);
  if (c.buf_kind == PACE_BUF_INT8) {
    L.kc = take(B * Hk * dP * dk);
    L.ks = take(B * Hk * dP * 4);
    L.v = take(B * Hv * dP * dv);
    L.vs = take(B * Hv * dP * 4);
  } else {
    L.kc = take(B * Hk * dP * dk / 2);
    L.ks = take(B * Hk * dP * 4);
    L.v = take(B * Hv * dP * dv * 2);
    L.vs = 0;
  }
  L.a = take(B * Hv * dP * 4);
  L.beta = take(B * Hv * dP * 4);
  L.total = o;
  return L;
}

// Everything a decode / flush launch needs, passed to the kernel by value.
struct DecodeParams {
  uint8_t* state;
  uint8_t* buffer;
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* beta;
  const uint8_t* mask;  // active (decode) or seq_mask (flush); may be null
  void* o;
  uint64_t mask8;       // bit h set: head h is 8-bit
  uint32_t rec4, rec8;  // record bytes of 4-bit / 8-bit heads
  uint32_t scales_off4, zeros_off4, scales_off8, zeros_off8;  // offsets inside a record
  uint64_t seq_stride;
  uint64_t off_kc, off_ks, off_v, off_vs, off_a, off_beta;  // buffer regions
  int32_t B, Hv, Hk, gamma, dP, group, asym;
  int32_t flush_only;   // 1: pace_flush_requant (no new token)
  int32_t io_bf16;      // q, k, v, o are bf16 (else fp32)
  int32_t bf16_state;   // the state is bf16 values (one dv x dk record per head)
};

// Sequence order of an ordered decode launch, passed by value as a second kernel argument
// of its own (only the ordered instantiations take it): workgroup row y runs sequence
// seq[y], a permutation of 0..B-1 checked on the host.
struct SeqOrder {
  uint8_t seq[kMaxOrderedBatch];
};

struct PrefillParams {
  uint8_t* state;
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* beta;
  void* o;
  float* ws;            // workspace
  uint64_t mask8;
  uint32_t rec4, rec8;
  uint32_t scales_off4, zeros_off4, scales_off8, zeros_off8;
  uint64_t seq_stride;
  int32_t B, Hv, Hk, gamma, group, asym, T, chunk;
};

struct Bf16Params {
  uint16_t* state;
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* beta;
  void* o;
  int32_t B, Hv, Hk, gamma;
};

struct CalibParams {
  const void* k;
  const void* v;
  const float* a;
  const float* beta;
  double* e_h;          // [Hv] mean rounding error energy
  double* a_h;          // [Hv] mean decay
  int32_t B, Hv, Hk, gamma, T, dP, group, asym;
};

// Launchers (defined next to their kernels).  They only enqueue work.
// order: null for launch order; otherwise the specialised kernels place the sequences as
// it says (the general ones, which it cannot change the results of either, ignore it).
hipError_t launch_decode(const DecodeParams& p, const SeqOrder* order, int dk, int dv, int buf_kind,
                         hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, int dk, int dv, int io_bf16,
                          hipStream_t stream);
size_t prefill_workspace_bytes(int B, int Hv, int dk, int dv, int T, int chunk);
hipError_t launch_bf16_decode(const Bf16Params& p, int dk, int dv, int io_bf16,
                              hipStream_t stream);
hipError_t launch_calib(const CalibParams& p, int dk, int io_bf16, hipStream_t stream);

}  // namespace pace
