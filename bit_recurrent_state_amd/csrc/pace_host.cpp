// Host entry points of the PACE C ABI: argument validation, layout sizing, bit
// accounting, head allocation, and the launches of the decode / prefill / baseline
// kernels.  No call allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

#include "pace_internal.h"

using namespace pace;

namespace {

// Structural validity (PACE_EINVAL) and kernel coverage (PACE_EUNSUPPORTED).
pace_status validate(const pace_layer_cfg* c) {
  if (!c) return PACE_EINVAL;
  const bool bf16_state = c->state_kind == PACE_STATE_BF16;
  if (c->B <= 0 || c->Hv <= 0 || c->Hk <= 0 || c->dk <= 0 || c->dv <= 0 || c->dP <= 0 || c->chunk <= 0)
    return PACE_EINVAL;
  if (c->Hv % c->Hk != 0) return PACE_EINVAL;
  if (c->state_kind != PACE_STATE_SYM && c->state_kind != PACE_STATE_ASYM && !bf16_state) return PACE_EINVAL;
  // a bf16 state has no scale groups and no per-head bit widths
  if (bf16_state && c->head_bits) return PACE_EINVAL;
  if (!bf16_state && (c->group <= 0 || c->dk % c->group != 0)) return PACE_EINVAL;
  if (c->buf_kind != PACE_BUF_INT8 && c->buf_kind != PACE_BUF_K4_VBF16) return PACE_EINVAL;
  if (c->io_dtype != PACE_IO_F32 && c->io_dtype != PACE_IO_BF16) return PACE_EINVAL;
  if (c->head_bits)
    for (int h = 0; h < c->Hv; ++h)
      if (c->head_bits[h] != 4 && c->head_bits[h] != 8) return PACE_EINVAL;
  // kernel coverage
  if (!((c->dk == 64 || c->dk == 128) && c->dv == c->dk)) return PACE_EUNSUPPORTED;
  if (!bf16_state && c->group != 32 && c->group != 64) return PACE_EUNSUPPORTED;
  if (c->dP > kMaxPeriod) return PACE_EUNSUPPORTED;
  if (c->Hv > kMaxHeads || c->B > 65535) return PACE_EUNSUPPORTED;
  // the prefill kernels round where a 64-token sub-block ends on a multiple of the period
  if (c->chunk % 64 != 0) return PACE_EUNSUPPORTED;
  // 4-bit zero points pack two groups of one column per byte
  if (c->state_kind == PACE_STATE_ASYM && (c->dk / c->group) % 2 != 0) return PACE_EUNSUPPORTED;
  // a bf16 state is served with the int8 decode buffer only
  if (bf16_state && c->buf_kind != PACE_BUF_INT8) return PACE_EUNSUPPORTED;
  return PACE_OK;
}

int head_bits_of(const pace_layer_cfg* c, int h) { return c->head_bits ? c->head_bits[h] : 4; }

struct StateGeom {
  RecordLayout r4, r8;
  uint64_t mask8 = 0;
  size_t seq_stride = 0;
};

StateGeom state_geom(const pace_layer_cfg* c) {
  StateGeom g;
  if (c->state_kind == PACE_STATE_BF16) {     // one dv x dk bf16 record per head
    const uint32_t rec = (uint32_t)((size_t)c->dk * c->dv * 2);
    g.r4 = RecordLayout{rec, 0u, 0u, rec};
    g.r8 = g.r4;
    g.seq_stride = (size_t)rec * c->Hv;
    return g;
  }
  const bool asym = c->state_kind == PACE_STATE_ASYM;
  g.r4 = record_layout(c->dk, c->dv, c->group, asym, 4);
  g.r8 = record_layout(c->dk, c->dv, c->group, asym, 8);
  for (int h = 0; h < c->Hv; ++h) {
    const bool is8 = head_bits_of(c, h) == 8;
    if (is8) g.mask8 |= 1ull << h;
    g.seq_stride += is8 ? g.r8.total : g.r4.total;
  }
  return g;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

const char* pace_status_str(pace_status s) {
  switch (s) {
    case PACE_OK: return "PACE_OK";
    case PACE_EINVAL: return "PACE_EINVAL: invalid argument";
    case PACE_EUNSUPPORTED: return "PACE_EUNSUPPORTED: configuration not implemented";
    case PACE_EHIP: return "PACE_EHIP: HIP launch error";
  }
  return "unknown pace_status";
}

pace_status pace_layout(const pace_layer_cfg* cfg, pace_layout_info* out) {
  if (!out) return PACE_EINVAL;
  const pace_status st = validate(cfg);
  if (st != PACE_OK) return st;
  const StateGeom g = state_geom(cfg);
  const BufferLayout bl = buffer_layout(*cfg);
  out->seq_stride = g.seq_stride;
  out->state_bytes = g.seq_stride * (size_t)cfg->B;
  out->buffer_bytes = bl.total;
  out->workspace_bytes = 0;
  const bool asym = cfg->state_kind == PACE_STATE_ASYM;
  double payload = 0.0;
  for (int h = 0; h < cfg->Hv; ++h) {
    const double b = head_bits_of(cfg, h);
    payload += cfg->state_kind == PACE_STATE_BF16 ? 16.0 : b + (16.0 + (asym ? b : 0.0)) / cfg->group;
  }
  out->payload_bits = payload / cfg->Hv;
  const double gamma = (double)cfg->Hv / cfg->Hk;
  const double bk = cfg->buf_kind == PACE_BUF_INT8 ? 8.0 : 4.0;
  const double bv = cfg->buf_kind == PACE_BUF_INT8 ? 8.0 : 16.0;
  const double cost = (bk * cfg->dk / gamma + bv * cfg->dv + 32.0) / ((double)cfg->dk * cfg->dv);
  out->buffer_bits_model = cost * cfg->dP;
  out->buffer_bits_actual =
      (double)bl.total * 8.0 / ((double)cfg->B * cfg->Hv * cfg->dk * cfg->dv);
  return PACE_OK;
}

pace_status pace_head_alloc(int32_t Hv, int32_t dP, const double* e_h, const double* a_h,
                            int32_t n_8bit, int8_t* head_bits_out, double* E_out) {
  if (Hv <= 0 || dP <= 0 || !e_h || !a_h || !head_bits_out || n_8bit < 0 || n_8bit > Hv)
    return PACE_EINVAL;
  std::vector<double> E(Hv);
  for (int h = 0; h < Hv; ++h) {
    if (!std::isfinite(e_h[h]) || e_h[h] < 0.0 || !std::isfinite(a_h[h]) || !(a_h[h] > 0.0))
      return PACE_EINVAL;
    // retained error of one rounding: the geometric sum of its decay over the periods
    E[h] = a_h[h] >= 1.0 ? INFINITY : e_h[h] / (1.0 - std::pow(a_h[h], 2.0 * dP));
  }
  std::vector<int> order(Hv);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return E[x] > E[y]; });
  for (int h = 0; h < Hv; ++h) head_bits_out[h] = 4;
  for (int i = 0; i < n_8bit; ++i) head_bits_out[order[i]] = 8;
  if (E_out)
    for (int h = 0; h < Hv; ++h) E_out[h] = E[h];
  return PACE_OK;
}

pace_status pace_prefill_workspace_bytes(const pace_layer_cfg* cfg, int32_t T, size_t* bytes_out) {
  if (!bytes_out || T <= 0) return PACE_EINVAL;
  const pace_status st = validate(cfg);
  if (st != PACE_OK) return st;
  if (cfg->state_kind == PACE_STATE_BF16) return PACE_EUNSUPPORTED;
  *bytes_out = prefill_workspace_bytes(cfg->B, cfg->Hv, cfg->dk, cfg->dv, T, cfg->chunk);
  return PACE_OK;
}

namespace {

pace_status decode_step(const pace_layer_cfg* cfg, void* state, void* buffer, const void* q,
                        const void* k, const void* v, const float* a, const float* beta,
                        const uint8_t* active, const int32_t* seq_order, void* o, void* stream) {
  const pace_status st = validate(cfg);
  if (st != PACE_OK) return st;
  if (!state || !buffer || !q || !k || !v || !a || !beta || !o) return PACE_EINVAL;
  if (!aligned(state, 256) || !aligned(buffer, 256) || !aligned(q, 16) || !aligned(k, 16) ||
      !aligned(v, 16) || !aligned(o, 16) || !aligned(a, 4) || !aligned(beta, 4))
    return PACE_EINVAL;
  const StateGeom g = state_geom(cfg);
  const BufferLayout bl = buffer_layout(*cfg);
  DecodeParams p{};
  p.state = (uint8_t*)state;
  p.buffer = (uint8_t*)buffer;
  p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
  p.mask = active;
  p.o = o;
  p.mask8 = g.mask8;
  p.rec4 = g.r4.total; p.rec8 = g.r8.total;
  p.scales_off4 = g.r4.codes; p.zeros_off4 = g.r4.codes + g.r4.scales;
  p.scales_off8 = g.r8.codes; p.zeros_off8 = g.r8.codes + g.r8.scales;
  p.seq_stride = g.seq_stride;
  p.off_kc = bl.kc; p.off_ks = bl.ks; p.off_v = bl.v; p.off_vs = bl.vs;
  p.off_a = bl.a; p.off_beta = bl.beta;
  p.B = cfg->B; p.Hv = cfg->Hv; p.Hk = cfg->Hk; p.gamma = cfg->Hv / cfg->Hk;
  p.dP = cfg->dP; p.group = cfg->group; p.asym = cfg->state_kind == PACE_STATE_ASYM;
  p.bf16_state = cfg->state_kind == PACE_STATE_BF16;
  p.flush_only = 0;
  p.io_bf16 = cfg->io_dtype == PACE_IO_BF16;
  SeqOrder order{};
  if (seq_order) {
    // only the specialised kernels take an order (see launch_decode)
    if (!(cfg->dk == 128 && cfg->dP <= 8 && cfg->io_dtype == PACE_IO_BF16) || cfg->state_kind == PACE_STATE_BF16)
      return PACE_EUNSUPPORTED;
    // a permutation of 0..B-1, checked here so that the kernel can trust it
    if (cfg->B > kMaxOrderedBatch) return PACE_EUNSUPPORTED;
    uint8_t seen[kMaxOrderedBatch] = {};
    for (int y = 0; y < cfg->B; ++y) {
      const int32_t sb = seq_order[y];
      if (sb < 0 || sb >= cfg->B || seen[sb]) return PACE_EINVAL;
      seen[sb] = 1;
      order.seq[y] = (uint8_t)sb;
    }
  }
  const hipError_t e = launch_decode(p, seq_order ? &order : nullptr, cfg->dk, cfg->dv, cfg->buf_kind,
                                     (hipStream_t)stream);
  return e == hipSuccess ? PACE_OK : PACE_EHIP;
}

}  // namespace

pace_status pace_decode_step(const pace_layer_cfg* cfg, void* state, void* buffer,
                             const void* q, const void* k, const void* v, const float* a,
                             const float* beta, const uint8_t* active, void* o,
                             void* stream) {
  return decode_step(cfg, state, buffer, q, k, v, a, beta, active, nullptr, o, stream);
}

pace_status pace_decode_step_ordered(const pace_layer_cfg* cfg, void* state, void* buffer,
                                     const void* q, const void* k, const void* v, const float* a,
                                     const float* beta, const uint8_t* active,
                                     const int32_t* seq_order, void* o, void* stream) {
  if (!seq_order) return PACE_EINVAL;
  return decode_step(cfg, state, buffer, q, k, v, a, beta, active, seq_order, o, stream);
}

pace_status pace_flush_requant(const pace_layer_cfg* cfg, void* state, void* buffer,
                               const uint8_t* seq_mask, void* stream) {
  const pace_status st = validate(cfg);
  if (st != PACE_OK) return st;
  if (!state || !buffer) return PACE_EINVAL;
  if (!aligned(state, 256) || !aligned(buffer, 256)) return PACE_EINVAL;
  const StateGeom g = state_geom(cfg);
  const BufferLayout bl = buffer_layout(*cfg);
  DecodeParams p{};
  p.state = (uint8_t*)state;
  p.buffer = (uint8_t*)buffer;
  p.mask = seq_mask;
  p.mask8 = g.mask8;
  p.rec4 = g.r4.total; p.rec8 = g.r8.total;
  p.scales_off4 = g.r4.codes; p.zeros_off4 = g.r4.codes + g.r4.scales;
  p.scales_off8 = g.r8.codes; p.zeros_off8 = g.r8.codes + g.r8.scales;
  p.seq_stride = g.seq_stride;
  p.off_kc = bl.kc; p.off_ks = bl.ks; p.off_v = bl.v; p.off_vs = bl.vs;
  p.off_a = bl.a; p.off_beta = bl.beta;
  p.B = cfg->B; p.Hv = cfg->Hv; p.Hk = cfg->Hk; p.gamma = cfg->Hv / cfg->Hk;
  p.dP = cfg->dP; p.group = cfg->group; p.asym = cfg->state_kind == PACE_STATE_ASYM;
  p.bf16_state = cfg->state_kind == PACE_STATE_BF16;
  p.flush_only = 1;
  p.io_bf16 = cfg->io_dtype == PACE_IO_BF16;
  // no token: the kernel's unconditional token loads read the state instead (every index
  // they form is below B * Hk * dk * 4 bytes, which the state always exceeds) and never
  // use the values
  p.q = p.k = p.v = state;
  p.a = p.beta = (const float*)state;
  const hipError_t e = launch_decode(p, nullptr, cfg->dk, cfg->dv, cfg->buf_kind, (hipStream_t)stream);
  return e == hipSuccess ? PACE_OK : PACE_EHIP;
}

pace_status pace_prefill_chunk(const pace_layer_cfg* cfg, void* state, const void* q,
                               const void* k, const void* v, const float* a,
                               const float* beta, int32_t T, void* o, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const pace_status st = validate(cfg);
  if (st != PACE_OK) return st;
  if (T <= 0 || !state || !q || !k || !v || !a || !beta || !o) return PACE_EINVAL;
  if (cfg->state_kind == PACE_STATE_BF16) return PACE_EUNSUPPORTED;
  if (!aligned(state, 256) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(a, 4) || !aligned(beta, 4))
    return PACE_EINVAL;
  const size_t need = prefill_workspace_bytes(cfg->B, cfg->Hv, cfg->dk, cfg->dv, T, cfg->chunk);
  if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return PACE_EINVAL;
  const StateGeom g = state_geom(cfg);
  PrefillParams p{};
  p.state = (uint8_t*)state;
  p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta; p.o = o;
  p.ws = (float*)workspace;
  p.mask8 = g.mask8;
  p.rec4 = g.r4.total; p.rec8 = g.r8.total;
  p.scales_off4 = g.r4.codes; p.zeros_off4 = g.r4.codes + g.r4.scales;
  p.scales_off8 = g.r8.codes; p.zeros_off8 = g.r8.codes + g.r8.scales;
  p.seq_stride = g.seq_stride;
  p.B = cfg->B; p.Hv = cfg->Hv; p.Hk = cfg->Hk; p.gamma = cfg->Hv / cfg->Hk;
  p.group = cfg->group; p.asym = cfg->state_kind == PACE_STATE_ASYM;
  p.T = T; p.chunk = cfg->chunk;
  const hipError_t e = launch_prefill(p, cfg->dk, cfg->dv, cfg->io_dtype == PACE_IO_BF16,
                                      (hipStream_t)stream);
  return e == hipSuccess ? PACE_OK : PACE_EHIP;
}

pace_status pace_calibrate_heads(const pace_layer_cfg* cfg, const void* k, const void* v,
                                 const float* a, const float* beta, int32_t T,
                                 double* e_h, double* a_h, void* stream) {
  const pace_status st = validate(cfg);
  if (st != PACE_OK) return st;
  if (T <= 0 || !k || !v || !a || !beta || !e_h || !a_h) return PACE_EINVAL;
  if (cfg->state_kind == PACE_STATE_BF16) return PACE_EUNSUPPORTED;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(a, 4) || !aligned(beta, 4) ||
      !aligned(e_h, 8) || !aligned(a_h, 8))
    return PACE_EINVAL;
  CalibParams p{};
  p.k = k; p.v = v; p.a = a; p.beta = beta; p.e_h = e_h; p.a_h = a_h;
  p.B = cfg->B; p.Hv = cfg->Hv; p.Hk = cfg->Hk; p.gamma = cfg->Hv / cfg->Hk;
  p.T = T; p.dP = cfg->dP; p.group = cfg->group; p.asym = cfg->state_kind == PACE_STATE_ASYM;
  const hipError_t e = launch_calib(p, cfg->dk, cfg->io_dtype == PACE_IO_BF16, (hipStream_t)stream);
  return e == hipSuccess ? PACE_OK : PACE_EHIP;
}

pace_status pace_bf16_decode_step(const pace_layer_cfg* cfg, void* state_bf16, const void* q,
                                  const void* k, const void* v, const float* a,
                                  const float* beta, void* o, void* stream) {
  if (!cfg) return PACE_EINVAL;
  if (cfg->B <= 0 || cfg->Hv <= 0 || cfg->Hk <= 0 || cfg->Hv % cfg->Hk != 0) return PACE_EINVAL;
  if (cfg->io_dtype != PACE_IO_F32 && cfg->io_dtype != PACE_IO_BF16) return PACE_EINVAL;
  if (!((cfg->dk == 64 || cfg->dk == 128) && cfg->dv == cfg->dk)) return PACE_EUNSUPPORTED;
  if (cfg->B > 65535 || cfg->Hv > kMaxHeads) return PACE_EUNSUPPORTED;
  if (!state_bf16 || !q || !k || !v || !a || !beta || !o) return PACE_EINVAL;
  if (!aligned(state_bf16, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16))
    return PACE_EINVAL;
  Bf16Params p{};
  p.state = (uint16_t*)state_bf16;
  p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta; p.o = o;
  p.B = cfg->B; p.Hv = cfg->Hv; p.Hk = cfg->Hk; p.gamma = cfg->Hv / cfg->Hk;
  const hipError_t e = launch_bf16_decode(p, cfg->dk, cfg->dv, cfg->io_dtype == PACE_IO_BF16,
                                          (hipStream_t)stream);
  return e == hipSuccess ? PACE_OK : PACE_EHIP;
}

}  // extern "C"
