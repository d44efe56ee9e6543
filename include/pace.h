/*
 * pace.h -- C ABI of the PACE periodic / channel-aligned 4-bit recurrent-state library
 * for AMD Instinct MI355X (gfx950).
 *
 * Method source: "PACE: Periodic and Channel-Aligned Encoding of Four-Bit Recurrent
 * States" (Haller, Laitenberger, Akbik), as summarised on three web pages:
 *   [p1] onedev.kr/papers/1282 -- sections "How it works", "How it differs",
 *        "Assumptions and limits";
 *   [p2] blog.secrett2633.cloud paper review -- "1. Key Terms", "3. Method & Key Results";
 *   [p3] news.hamidun.com news item -- "Two observations".
 * Citations below name the page and the section.
 *
 * Everything here is plain C: pointers, sizes and POD structs.  No call allocates,
 * frees or synchronises device memory; all device buffers are owned by the caller.
 * Device pointers must be 16-byte aligned (state and buffer: 256-byte aligned).
 * Every call validates its arguments on the host before any launch and returns
 * PACE_EINVAL / PACE_EUNSUPPORTED without touching device memory on failure.
 * Launch failures are reported as PACE_EHIP (from hipGetLastError, no implicit sync).
 * The library keeps no global state: calls are reentrant and thread-safe, and calls
 * on different streams that touch disjoint buffers may overlap.
 *
 * ------------------------------------------------------------------------------------
 * Notation (per layer)
 *   B   sequences, Hv value heads, Hk key heads, gamma = Hv / Hk value heads per key head;
 *       value head h reads key head h / gamma (consecutive grouping).
 *   dk, dv  key / value head dimension; the state of one (sequence, value head) is
 *       S in R^{dk x dv}: rows are the key axis, columns the value channels
 *       ([p1] "What it is"; [p2] "Key Terms").
 *   Recurrence ([p2] "Key Terms", delta value):
 *       u_t = beta_t (v_t - a_t S_{t-1}^T k_t),   S_t = a_t S_{t-1} + k_t u_t^T,
 *   readout o_t = S_t^T q_t from the post-update state, before any rounding.
 *   No 1/sqrt(dk) factor is applied: callers scale q themselves.
 *
 * Quantiser ([p1] "How it differs"; [p2] "Method"): channel-aligned groups -- g
 * contiguous key-axis elements of ONE value column share one bf16 scale.
 *   symmetric, b bits:  M = max|x| over the group; s = bf16 rounded toward +inf of
 *       M / (2^(b-1) - 1); c = round-half-even(x / s), clipped to +-(2^(b-1) - 1);
 *       x^ = s c.  A group with M = 0 gets s = 0, c = 0.
 *   asymmetric, b bits: lo = min(0, min x), hi = max(0, max x);
 *       s = bf16 rounded toward +inf of (hi - lo) / (2^b - 1);
 *       z = clip(rne(-lo / s), 0, 2^b - 1); c = clip(rne(x / s) + z, 0, 2^b - 1);
 *       x^ = s (c - z).  s = 0 gives c = 0, z = 0.
 *   Scales are rounded toward +inf so that |x - x^| <= s/2 holds for every element
 *   with the stored bf16 scale.  Codes are decided on the fp32 pre-rounding state.
 *   PACE-4   = symmetric int4, g = 64, int8 decode buffer.
 *   PACE-4/8 = asymmetric, g = 32, integer zero points stored in the head's own bit
 *              width; a quarter of the heads of a layer kept at 8 bits, chosen by the
 *              retained error E_h = e_h / (1 - a_h^(2 dP)) ([p1] "How it differs").
 *
 * Rounding schedule ([p1] "How it works"; [p2] "Key Terms", periodic rounding):
 *   prefill rounds the state once per chunk of `chunk` tokens (256 in the method; any
 *   multiple of 64 is accepted, since the pages never vary it) and once at the
 *   end of the call; decode appends each token to a decode buffer and rounds the
 *   state once every dP tokens (default 8), when the buffer is folded in.
 *
 * ------------------------------------------------------------------------------------
 * PACKED STATE LAYOUT (one device allocation of pace_layout_info.state_bytes per layer)
 *
 *   Each value head h has a bit width b_h in {4, 8} (cfg.head_bits, all 4 if NULL).
 *   The record of (sequence b, head h) starts at byte
 *       b * seq_stride + head_offset(h),  head_offset(h) = sum_{h' < h} rec(b_h'),
 *       seq_stride = sum_h rec(b_h),
 *   and holds three parts, each padded to 16 bytes, the record padded to 256 bytes:
 *     codes  : dv * dk * b / 8 bytes.  Value column j (0 <= j < dv) occupies
 *              dk * b / 8 contiguous bytes starting at j * dk * b / 8.  A column is a
 *              sequence of dk/8 "units" of 8 keys; unit u (0 <= u < dk/8) sits at
 *              byte u * b within the column and holds keys base(u) .. base(u) + 7 with
 *                  base(u) = 32 * (u mod (dk/32)) + 8 * (u div (dk/32)).
 *              4-bit unit (4 bytes): byte w (0..3) holds key base+w in its low nibble
 *              and key base+4+w in its high nibble.  8-bit unit (8 bytes): byte e holds
 *              key base+e.
 *              Stored field values are unsigned, c_st in [0, 2^b - 1], and dequantise as
 *              s * (c_st - z) with z = 2^(b-1) for symmetric heads (so a symmetric code
 *              c is stored as c + 2^(b-1)) and z = the stored zero point for asymmetric
 *              heads.
 *     scales : dv * (dk/g) bf16 values; scale of (column j, key group G) at element
 *              j * (dk/g) + G.  Group G covers keys [G g, (G+1) g).
 *     zeros  : asymmetric states only; dv * (dk/g) zero points of b bits, element
 *              e = j * (dk/g) + G.  8-bit heads: byte e.  4-bit heads: byte e/2, low
 *              nibble for even e.
 *   A zero-filled state is the all-zero state S = 0 (every scale 0).
 *
 *   state_kind PACE_STATE_BF16 ([p1] "Assumptions and limits": in the pages' timing, most
 *   of the decode-time gain over per-token bf16 decode comes from the decode buffer on a
 *   bf16 state, and the 4-bit state adds the rest): the record of (b, h) is dv x dk bf16
 *   values, value-column-major -- element (key r, column j) at bf16 index j * dk + r, the
 *   layout of pace_bf16_decode_step -- at byte offset (b * Hv + h) * dk * dv * 2.  The
 *   decode buffer, the replay and the once-per-dP fold are those of the packed states; a
 *   flush rounds every element of the fp32 pre-rounding state to the nearest bf16 (ties
 *   to even).  cfg.group is ignored, cfg.head_bits must be NULL and the buffer must be
 *   PACE_BUF_INT8 (others: PACE_EUNSUPPORTED).  Only the decode
 *   calls (pace_decode_step, pace_flush_requant) take this kind; pace_prefill_chunk and
 *   pace_calibrate_heads return PACE_EUNSUPPORTED for it.  A zero-filled state is S = 0.
 *
 * DECODE BUFFER LAYOUT (pace_layout_info.buffer_bytes per layer), regions in this
 * order, each padded to 256 bytes:
 *     count : int32 [B][Hv]   tokens buffered since the last rounding (0 .. dP-1 between
 *                             calls; other values are read as clamped to that range).
 *                             All heads of one sequence advance together.
 *   buf_kind PACE_BUF_INT8 ([p1] "How it works": uniform configuration, 8-bit keys and
 *   values):
 *     kc    : int8   [B][Hk][dP][dk]  key codes, two's complement, |c| <= 127
 *     ks    : fp32   [B][Hk][dP]      key scale   (= fp32(max|k| / 127), 0 for k = 0)
 *     vc    : int8   [B][Hv][dP][dv]  value codes
 *     vs    : fp32   [B][Hv][dP]      value scale (= fp32(max|v| / 127))
 *     a     : fp32   [B][Hv][dP]      decay a_t as given
 *     beta  : fp32   [B][Hv][dP]      write strength beta_t as given
 *   buf_kind PACE_BUF_K4_VBF16 ([p1] "How it works": mixed configuration, 4-bit keys,
 *   bf16 values):
 *     kc    : uint8  [B][Hk][dP][dk/2] 4-bit symmetric key codes stored as c + 8; within
 *                                      each 8-key unit m (4 bytes), byte w holds key
 *                                      8m+w (low nibble) and 8m+4+w (high nibble)
 *     ks    : fp32   [B][Hk][dP]       key scale (= fp32(max|k| / 7))
 *     v     : bf16   [B][Hv][dP][dv]   values rounded to nearest-even bf16
 *     a     : fp32   [B][Hv][dP]
 *     beta  : fp32   [B][Hv][dP]
 *   Buffer codes: c = rne(x / scale), computed in fp32.  The token being decoded passes
 *   through the buffer quantiser before its own output is formed, so every output and
 *   every later flush see the same buffered values.  A zero-filled buffer is empty.
 *
 * I/O TENSORS (contiguous, row-major; io_dtype fp32 or bf16 for q, k, v, o):
 *   decode : q, k [B][Hk][dk];  v, o [B][Hv][dv];  a, beta fp32 [B][Hv]
 *   prefill: q, k [B][T][Hk][dk]; v, o [B][T][Hv][dv]; a, beta fp32 [B][T][Hv]
 *   Gates must satisfy 0 < a <= 1, 0 <= beta <= 1; NaN / Inf inputs are undefined.
 * ------------------------------------------------------------------------------------
 */
#ifndef PACE_H
#define PACE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PACE_OK = 0,
  PACE_EINVAL = -1,        /* malformed arguments (null pointer, bad sizes, bad enum) */
  PACE_EUNSUPPORTED = -2,  /* well-formed but outside what the kernels implement */
  PACE_EHIP = -3           /* a HIP launch reported an error */
} pace_status;

typedef enum {
  PACE_STATE_SYM = 0,   /* symmetric packed codes (PACE-4) */
  PACE_STATE_ASYM = 1,  /* asymmetric packed codes with zero points (PACE-4/8) */
  PACE_STATE_BF16 = 2   /* bf16 values: the decode buffer without the 4-bit state */
} pace_state_kind;
typedef enum { PACE_BUF_INT8 = 0, PACE_BUF_K4_VBF16 = 1 } pace_buf_kind;
typedef enum { PACE_IO_F32 = 0, PACE_IO_BF16 = 1 } pace_io_dtype;

/* One gated-delta layer.  Supported by the kernels: dk, dv in {64, 128}; g in {32, 64}
 * with g | dk (and g <= dk); 1 <= dP <= 32; chunk a multiple of 64 (256 in the method);
 * Hv % Hk == 0; Hv <= 64; 1 <= B <= 65535. */
typedef struct {
  int32_t B, Hv, Hk, dk, dv;
  int32_t group;        /* g: key-axis elements per scale group */
  int32_t state_kind;   /* pace_state_kind */
  int32_t buf_kind;     /* pace_buf_kind */
  int32_t io_dtype;     /* pace_io_dtype for q, k, v, o */
  int32_t dP;           /* decode period: tokens buffered between roundings */
  int32_t chunk;        /* prefill rounding period (tokens) */
  const int8_t* head_bits; /* host [Hv], each 4 or 8; NULL = every head 4-bit.
                              Read during the call only. */
} pace_layer_cfg;

typedef struct {
  size_t state_bytes;      /* packed state of the whole layer (all B sequences) */
  size_t buffer_bytes;     /* decode buffer of the whole layer */
  size_t workspace_bytes;  /* scratch needed by pace_prefill_chunk */
  size_t seq_stride;       /* bytes of state per sequence */
  double payload_bits;     /* mean over heads of b_h + (16 + z_h) / g, z_h = b_h if asym
                              else 0 -- bits per state value ([p1] "How it differs");
                              16 for a bf16 state */
  double buffer_bits_model;  /* c * dP, c = (b_k dk / gamma + b_v dv + 32) / (dk dv)
                                ([p1] "How it works") */
  double buffer_bits_actual; /* bytes of this buffer layout * 8 / (B Hv dk dv) */
} pace_layout_info;

/* Sizes and bit accounting of a layer configuration.  Host only.
 * Errors: PACE_EINVAL for a null pointer or malformed config, PACE_EUNSUPPORTED for a
 * configuration outside the kernels' range. */
pace_status pace_layout(const pace_layer_cfg* cfg, pace_layout_info* out);

/* Head-level precision allocation ([p1] "How it differs"; [p2] "Method", head-level
 * precision allocation).  Host only.
 *   E_h = e_h / (1 - a_h^(2 dP)), with E_h = +inf when a_h >= 1.
 *   The n_8bit heads with the largest E_h get 8 bits, the others 4 bits; ties go to the
 *   lower head index.
 * In : e_h[Hv] one-rounding error energies (>= 0), a_h[Hv] mean head decays (> 0),
 *      0 <= n_8bit <= Hv, dP >= 1.
 * Out: head_bits_out[Hv] (4 or 8); E_out[Hv] (may be NULL).
 * Errors: PACE_EINVAL on null inputs, negative or non-finite e_h, a_h <= 0, bad counts. */
pace_status pace_head_alloc(int32_t Hv, int32_t dP, const double* e_h, const double* a_h,
                            int32_t n_8bit, int8_t* head_bits_out, double* E_out);

/* Offline calibration of the head ranking inputs ([p1] "How it differs": e_h is the error
 * energy one rounding leaves, a_h the head's decay; [p2] "Method": head-level precision
 * allocation).  For each value head h, runs the exact recurrence from S = 0 over the T
 * tokens of each of the B sequences and, at every dP-th token, adds the squared Frobenius
 * error of one rounding of S by the layer's 4-bit quantiser (key groups of cfg->group,
 * bf16 scales rounded up, symmetric or asymmetric per cfg->state_kind).
 * In : k [B][T][Hk][dk], v [B][T][Hv][dv] (io_dtype), a, beta [B][T][Hv] fp32 (device).
 * Out: e_h[Hv] = mean energy over all rounding points of all sequences (0 if T < dP),
 *      a_h[Hv] = mean a_t over all tokens and sequences; fp64, device memory.
 * Feed the host copies to pace_head_alloc.  Deterministic (one workgroup per head).
 * Errors: as pace_prefill_chunk for the configuration; PACE_EINVAL for T < 1 or a null
 * pointer.  `stream` is a hipStream_t (NULL = default stream). */
pace_status pace_calibrate_heads(const pace_layer_cfg* cfg, const void* k, const void* v,
                                 const float* a, const float* beta, int32_t T,
                                 double* e_h, double* a_h, void* stream);

/* Chunked prefill ([p1] "How it works": the prefill rounding period is the chunk
 * length, 256 tokens; [p3] "Two observations": chunked kernels update the state once
 * per chunk).  Consumes T >= 1 tokens of all B sequences starting from `state`, writes
 * o for every token and leaves the state rounded: once after every `chunk` tokens of the
 * call and once after its last token.  Within a chunk the exact recurrence is applied;
 * outputs use the unrounded state.
 * Precondition: no tokens are pending in the decode buffer (count == 0); flush first.
 * `workspace` is device scratch of at least pace_layout_info.workspace_bytes for this
 * T (pass the layout of the same cfg; its size is reported per token via
 * pace_prefill_workspace_bytes).  `stream` is a hipStream_t (NULL = default stream). */
pace_status pace_prefill_chunk(const pace_layer_cfg* cfg, void* state, const void* q,
                               const void* k, const void* v, const float* a,
                               const float* beta, int32_t T, void* o, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Workspace bytes pace_prefill_chunk needs for T tokens of this configuration, written to
 * *bytes_out (0: the call needs no workspace and accepts workspace == NULL).  Host only.
 * Errors (nothing is written): PACE_EINVAL for a null pointer, T < 1 or a malformed
 * config; PACE_EUNSUPPORTED for a configuration the kernels do not implement. */
pace_status pace_prefill_workspace_bytes(const pace_layer_cfg* cfg, int32_t T, size_t* bytes_out);

/* One decode step ([p1] "How it works": decode buffer, round once per dP tokens;
 * [p2] "Key Terms": decode buffer, periodic rounding).  For every active sequence and
 * every value head: quantise (k_t, v_t) into buffer slot `count`, store (a_t, beta_t),
 * replay the buffered tokens on the dequantised state, write o_t = S_t^T q_t, and when
 * the buffer then holds dP tokens fold it into the state, requantise once and reset the
 * count -- all in one launch.  Inactive sequences (active[b] == 0) are not touched and
 * their o rows are not written.  active == NULL means all active. */
pace_status pace_decode_step(const pace_layer_cfg* cfg, void* state, void* buffer,
                             const void* q, const void* k, const void* v, const float* a,
                             const float* beta, const uint8_t* active, void* o,
                             void* stream);

/* pace_decode_step with a caller-chosen order of the sequences over the launch, for
 * continuous batching ([p1] "How it works": each serving sequence keeps its own state and
 * buffer, so sequences that joined at different times flush at different steps).  Results
 * are those of pace_decode_step, bit for bit: only the placement of the work changes.
 * seq_order: HOST array of B indices, a permutation of 0..B-1; the sequences listed first
 * are started first and spread one per compute unit (place those whose buffer holds dP-1
 * tokens, i.e. that flush at this step, first).  It is copied into the launch, so the
 * array may be reused at once (and a captured graph keeps the order it was captured with).
 * Only the kernels of the layouts the method names apply an order: dk = dv = 128, dP <= 8,
 * bf16 I/O, a packed state (either packed kind, any head map and buffer kind).  Other layouts are rejected rather
 * than run in launch order, so that a caller never believes its order took effect when it
 * did not.
 * Errors: PACE_EINVAL for a null seq_order or one that is not a permutation of 0..B-1;
 * PACE_EUNSUPPORTED for B > 256 or a layout outside the one above; otherwise as
 * pace_decode_step. */
pace_status pace_decode_step_ordered(const pace_layer_cfg* cfg, void* state, void* buffer,
                                     const void* q, const void* k, const void* v, const float* a,
                                     const float* beta, const uint8_t* active,
                                     const int32_t* seq_order, void* o, void* stream);

/* Explicit flush (sequence end, eviction, checkpoint): for every sequence with
 * seq_mask[b] != 0 (NULL = all) and 0 < count < dP, fold the buffered tokens into the
 * state, requantise once and set count = 0.  A sequence with count == 0 is untouched. */
pace_status pace_flush_requant(const pace_layer_cfg* cfg, void* state, void* buffer,
                               const uint8_t* seq_mask, void* stream);

/* Per-token bf16-state decode, the throughput comparator of [p1] "Assumptions and
 * limits" (the state is read and written every token).  state_bf16 is bf16
 * [B][Hv][dv][dk] (value-column-major like the packed codes).  Per token:
 *   u = beta (v - a S^T k);  S' = a S + k u^T;  o = S'^T q (from S' before rounding);
 *   S <- bf16_rne(S').
 * Uses cfg's B, Hv, Hk, dk, dv, io_dtype; other fields are ignored. */
pace_status pace_bf16_decode_step(const pace_layer_cfg* cfg, void* state_bf16,
                                  const void* q, const void* k, const void* v,
                                  const float* a, const float* beta, void* o, void* stream);

/* Static, human-readable name of a status code. */
const char* pace_status_str(pace_status s);

#ifdef __cplusplus
}
#endif
#endif /* PACE_H */
