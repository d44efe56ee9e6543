// Host entry points of the C ABI (bit_recurrent_state_amd/csrc/pace_host.cpp) built for
// the CPU with AddressSanitizer and UndefinedBehaviorSanitizer, linked against recording
// stand-ins of the kernel launchers (no GPU code, no device memory: the pointers passed
// are aligned stand-in addresses that nothing dereferences).  Checks that every call
// validates its arguments before any launch, fills the launch parameters from the layout
// rules of include/pace.h, and never reads or writes out of bounds while doing so.
// Built and run by tests/test_native_sanitized.py; prints "OK <checks>" on success.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../../bit_recurrent_state_amd/csrc/pace_internal.h"

using namespace pace;

static int fails = 0;
static long checks = 0;
#define EXPECT(c, ...)                                              \
  do {                                                              \
    ++checks;                                                       \
    if (!(c)) {                                                     \
      if (fails++ < 30) {                                           \
        printf("FAIL line %d: ", __LINE__);                         \
        printf(__VA_ARGS__);                                        \
        printf("\n");                                               \
      }                                                             \
    }                                                               \
  } while (0)

// ------------------------------------------------------------ recording launchers
namespace pace {
static int n_decode = 0, n_prefill = 0, n_bf16 = 0, n_calib = 0;
static DecodeParams last_decode;
static bool last_had_order = false;
static SeqOrder last_order;
static PrefillParams last_prefill;
static CalibParams last_calib;
static Bf16Params last_bf16;

hipError_t launch_decode(const DecodeParams& p, const SeqOrder* order, int, int, int, hipStream_t) {
  ++n_decode;
  last_decode = p;
  last_had_order = order != nullptr;
  if (order) last_order = *order;
  return hipSuccess;
}
hipError_t launch_prefill(const PrefillParams& p, int, int, int, hipStream_t) {
  ++n_prefill;
  last_prefill = p;
  return hipSuccess;
}
size_t prefill_workspace_bytes(int, int, int, int, int, int) { return 0; }
hipError_t launch_bf16_decode(const Bf16Params& p, int, int, int, hipStream_t) {
  ++n_bf16;
  last_bf16 = p;
  return hipSuccess;
}
hipError_t launch_calib(const CalibParams& p, int, int, hipStream_t) {
  ++n_calib;
  last_calib = p;
  return hipSuccess;
}
}  // namespace pace

static void* fake(uintptr_t a) { return (void*)a; }

static pace_layer_cfg cfg_of(int B, int Hv, int Hk, int d, int g, int kind, int buf, int io, int dP,
                             const int8_t* hb) {
  pace_layer_cfg c;
  memset(&c, 0, sizeof c);
  c.B = B; c.Hv = Hv; c.Hk = Hk; c.dk = d; c.dv = d; c.group = g;
  c.state_kind = kind; c.buf_kind = buf; c.io_dtype = io; c.dP = dP; c.chunk = 256; c.head_bits = hb;
  return c;
}

static size_t pad(size_t n, size_t a) { return (n + a - 1) / a * a; }

// record bytes by the header's rule
static size_t rec_bytes(int d, int g, bool asym, int bits) {
  const size_t codes = pad((size_t)d * d * bits / 8, 16), scales = pad((size_t)d * (d / g) * 2, 16);
  const size_t zeros = asym ? pad((size_t)d * (d / g) * bits / 8, 16) : 0;
  return pad(codes + scales + zeros, 256);
}

int main() {
  std::mt19937_64 rng(11);
  // ---------------------------------------------------------------- layout
  const int ds[] = {64, 128}, gs[] = {32, 64}, dPs[] = {1, 8, 32};
  for (int d : ds)
    for (int g : gs)
      for (int kind = 0; kind < 2; ++kind)
        for (int buf = 0; buf < 2; ++buf)
          for (int dP : dPs) {
            const int B = 1 + (int)(rng() % 9), Hk = 1 + (int)(rng() % 4), gam = 1 + (int)(rng() % 4);
            const int Hv = Hk * gam;
            if (Hv > 64) continue;
            std::vector<int8_t> hb(Hv);
            for (auto& x : hb) x = (rng() & 3) == 0 ? 8 : 4;
            pace_layer_cfg c = cfg_of(B, Hv, Hk, d, g, kind, buf, 1, dP, hb.data());
            pace_layout_info info;
            const pace_status st = pace_layout(&c, &info);
            const bool asym = kind == PACE_STATE_ASYM;
            if (asym && (d / g) % 2 != 0) {
              EXPECT(st == PACE_EUNSUPPORTED, "odd group count accepted (d=%d g=%d)", d, g);
              continue;
            }
            EXPECT(st == PACE_OK, "layout refused (d=%d g=%d kind=%d buf=%d dP=%d)", d, g, kind, buf, dP);
            size_t stride = 0;
            double payload = 0;
            for (int h = 0; h < Hv; ++h) {
              stride += rec_bytes(d, g, asym, hb[h]);
              payload += hb[h] + (16.0 + (asym ? hb[h] : 0)) / g;
            }
            EXPECT(info.seq_stride == stride && info.state_bytes == stride * B, "state bytes");
            EXPECT(std::fabs(info.payload_bits - payload / Hv) < 1e-12, "payload bits");
            EXPECT(info.workspace_bytes == 0, "workspace");
            size_t ws = 77;
            EXPECT(pace_prefill_workspace_bytes(&c, 100, &ws) == PACE_OK && ws == 0, "workspace query");
          }
  {
    pace_layout_info info;
    EXPECT(pace_layout(nullptr, &info) == PACE_EINVAL, "null cfg");
    pace_layer_cfg c = cfg_of(2, 4, 4, 64, 32, 0, 0, 1, 8, nullptr);
    EXPECT(pace_layout(&c, nullptr) == PACE_EINVAL, "null out");
    pace_layer_cfg bad = c;
    bad.Hk = 3;
    EXPECT(pace_layout(&bad, &info) == PACE_EINVAL, "Hv %% Hk");
    bad = c; bad.dk = bad.dv = 96; bad.group = 32;
    EXPECT(pace_layout(&bad, &info) == PACE_EUNSUPPORTED, "d = 96");
    bad = c; bad.state_kind = 7;
    EXPECT(pace_layout(&bad, &info) == PACE_EINVAL, "state kind");
    bad = c; bad.dP = 33;
    EXPECT(pace_layout(&bad, &info) == PACE_EUNSUPPORTED, "dP > 32");
    bad = c; bad.chunk = 100;
    EXPECT(pace_layout(&bad, &info) == PACE_EUNSUPPORTED, "chunk");
    int8_t hb[4] = {4, 8, 5, 4};
    bad = c; bad.head_bits = hb;
    EXPECT(pace_layout(&bad, &info) == PACE_EINVAL, "head bit 5");
    size_t ws = 5;
    EXPECT(pace_prefill_workspace_bytes(&c, 0, &ws) == PACE_EINVAL && ws == 5, "T = 0");
    EXPECT(pace_prefill_workspace_bytes(&c, 10, nullptr) == PACE_EINVAL, "null out");
    bad = c; bad.Hk = 3;
    EXPECT(pace_prefill_workspace_bytes(&bad, 10, &ws) == PACE_EINVAL && ws == 5, "bad cfg");
  }
  // ------------------------------------------------------------ bf16 state
  {
    pace_layer_cfg c = cfg_of(64, 32, 16, 128, 64, PACE_STATE_BF16, PACE_BUF_INT8, PACE_IO_BF16, 8, nullptr);
    pace_layout_info info;
    EXPECT(pace_layout(&c, &info) == PACE_OK, "bf16 state layout");
    EXPECT(info.seq_stride == 32u * 128 * 128 * 2 && info.state_bytes == 64u * info.seq_stride, "bf16 state bytes");
    EXPECT(info.payload_bits == 16.0, "bf16 payload");
    c.group = 0;                                   // ignored for a bf16 state
    EXPECT(pace_layout(&c, &info) == PACE_OK, "bf16 state ignores the group");
    void *st = fake(0x100000), *bu = fake(0x200000), *io = fake(0x300000);
    const float* f = (const float*)fake(0x400000);
    EXPECT(pace_decode_step(&c, st, bu, io, io, io, f, f, nullptr, io, nullptr) == PACE_OK, "bf16 state decode");
    EXPECT(last_decode.bf16_state == 1 && last_decode.rec4 == 128u * 128 * 2 && last_decode.mask8 == 0,
           "bf16 state launch parameters");
    EXPECT(pace_prefill_chunk(&c, st, io, io, io, f, f, 256, io, nullptr, 0, nullptr) == PACE_EUNSUPPORTED,
           "bf16 state prefill");
    int32_t ord[64];
    for (int i = 0; i < 64; ++i) ord[i] = i;
    EXPECT(pace_decode_step_ordered(&c, st, bu, io, io, io, f, f, nullptr, ord, io, nullptr) == PACE_EUNSUPPORTED,
           "bf16 state ordered");
    c.buf_kind = PACE_BUF_K4_VBF16;
    EXPECT(pace_layout(&c, &info) == PACE_EUNSUPPORTED, "bf16 state with the mixed buffer");
    int8_t hb[32] = {};
    for (int h = 0; h < 32; ++h) hb[h] = 4;
    c.buf_kind = PACE_BUF_INT8;
    c.head_bits = hb;
    EXPECT(pace_layout(&c, &info) == PACE_EINVAL, "bf16 state with a head map");
  }
  // ------------------------------------------------------------ head allocation
  for (int trial = 0; trial < 200; ++trial) {
    const int H = 1 + (int)(rng() % 64), n8 = (int)(rng() % (H + 1)), dP = 1 + (int)(rng() % 32);
    std::vector<double> e(H), a(H), E(H);
    std::vector<int8_t> bits(H);
    for (int h = 0; h < H; ++h) {
      e[h] = (rng() % 4) * 0.25;                 // ties on purpose
      a[h] = (rng() % 5 == 0) ? 1.0 : 0.5 + 0.1 * (double)(rng() % 5);
    }
    EXPECT(pace_head_alloc(H, dP, e.data(), a.data(), n8, bits.data(), E.data()) == PACE_OK, "head alloc");
    int got8 = 0;
    for (int h = 0; h < H; ++h) got8 += bits[h] == 8;
    EXPECT(got8 == n8, "8-bit count %d vs %d", got8, n8);
    // every 8-bit head ranks at least as high as every 4-bit head; ties go to the lower index
    for (int x = 0; x < H; ++x)
      for (int y = 0; y < H; ++y)
        if (bits[x] == 8 && bits[y] == 4)
          EXPECT(E[x] > E[y] || (E[x] == E[y] && x < y), "ranking h%d over h%d", x, y);
  }
  {
    double e[2] = {1, NAN}, a[2] = {0.9, 0.9};
    int8_t bits[2];
    EXPECT(pace_head_alloc(2, 8, e, a, 1, bits, nullptr) == PACE_EINVAL, "NaN energy");
    e[1] = 1; a[1] = 0;
    EXPECT(pace_head_alloc(2, 8, e, a, 1, bits, nullptr) == PACE_EINVAL, "zero decay");
    a[1] = 0.9;
    EXPECT(pace_head_alloc(2, 8, e, a, 3, bits, nullptr) == PACE_EINVAL, "n_8bit > H");
  }
  // ------------------------------------------------------------------ decode
  {
    int8_t hb[32];
    for (int h = 0; h < 32; ++h) hb[h] = h % 4 == 1 ? 8 : 4;
    pace_layer_cfg c = cfg_of(64, 32, 16, 128, 32, PACE_STATE_ASYM, PACE_BUF_INT8, PACE_IO_BF16, 8, hb);
    void *st = fake(0x100000), *bu = fake(0x200000), *io = fake(0x300000);
    const float* f = (const float*)fake(0x400000);
    const int before = n_decode;
    EXPECT(pace_decode_step(&c, st, bu, io, io, io, f, f, nullptr, io, nullptr) == PACE_OK, "decode");
    EXPECT(n_decode == before + 1 && !last_had_order, "one launch, plain order");
    const DecodeParams& p = last_decode;
    uint64_t mask = 0;
    for (int h = 0; h < 32; ++h) mask |= (uint64_t)(hb[h] == 8) << h;
    EXPECT(p.mask8 == mask, "head map");
    EXPECT(p.rec4 == rec_bytes(128, 32, true, 4) && p.rec8 == rec_bytes(128, 32, true, 8), "records");
    EXPECT(p.scales_off4 == 128 * 128 / 2 && p.scales_off8 == 128 * 128, "scale offsets");
    EXPECT(p.off_kc == pad(64 * 32 * 4, 256), "buffer key region after the counts");
    EXPECT(p.gamma == 2 && p.flush_only == 0 && p.io_bf16 == 1 && p.asym == 1, "fields");
    // null and misaligned pointers are refused before any launch
    EXPECT(pace_decode_step(&c, nullptr, bu, io, io, io, f, f, nullptr, io, nullptr) == PACE_EINVAL, "null");
    EXPECT(pace_decode_step(&c, fake(0x100010), bu, io, io, io, f, f, nullptr, io, nullptr) == PACE_EINVAL,
           "state alignment");
    EXPECT(pace_decode_step(&c, st, bu, fake(0x300008), io, io, f, f, nullptr, io, nullptr) == PACE_EINVAL,
           "q alignment");
    EXPECT(n_decode == before + 1, "no launch on error");
    // ordered: a permutation is copied into the launch
    std::vector<int32_t> order(64);
    for (int i = 0; i < 64; ++i) order[i] = 63 - i;
    EXPECT(pace_decode_step_ordered(&c, st, bu, io, io, io, f, f, nullptr, order.data(), io, nullptr) == PACE_OK,
           "ordered");
    EXPECT(last_had_order, "order passed");
    bool same = true;
    for (int i = 0; i < 64; ++i) same = same && last_order.seq[i] == 63 - i;
    EXPECT(same, "order copied");
    order[5] = order[6];
    EXPECT(pace_decode_step_ordered(&c, st, bu, io, io, io, f, f, nullptr, order.data(), io, nullptr) == PACE_EINVAL,
           "repeated index");
    order[5] = 64;
    EXPECT(pace_decode_step_ordered(&c, st, bu, io, io, io, f, f, nullptr, order.data(), io, nullptr) == PACE_EINVAL,
           "index past B");
    EXPECT(pace_decode_step_ordered(&c, st, bu, io, io, io, f, f, nullptr, nullptr, io, nullptr) == PACE_EINVAL,
           "null order");
    pace_layer_cfg c64 = cfg_of(4, 4, 4, 64, 32, 0, 0, PACE_IO_BF16, 8, nullptr);
    int32_t o4[4] = {3, 2, 1, 0};
    EXPECT(pace_decode_step_ordered(&c64, st, bu, io, io, io, f, f, nullptr, o4, io, nullptr) == PACE_EUNSUPPORTED,
           "ordered outside the specialised layouts");
    pace_layer_cfg big = cfg_of(300, 4, 4, 128, 64, 0, 0, PACE_IO_BF16, 8, nullptr);
    std::vector<int32_t> o300(300);
    for (int i = 0; i < 300; ++i) o300[i] = i;
    EXPECT(pace_decode_step_ordered(&big, st, bu, io, io, io, f, f, nullptr, o300.data(), io, nullptr) ==
               PACE_EUNSUPPORTED,
           "B > 256");
    // flush: no token, stand-in pointers, flush_only set
    EXPECT(pace_flush_requant(&c, st, bu, nullptr, nullptr) == PACE_OK && last_decode.flush_only == 1, "flush");
    EXPECT(pace_flush_requant(&c, st, fake(0x200010), nullptr, nullptr) == PACE_EINVAL, "buffer alignment");
  }
  // ----------------------------------------------------------------- prefill
  {
    pace_layer_cfg c = cfg_of(4, 32, 16, 128, 64, 0, 0, PACE_IO_BF16, 8, nullptr);
    void *st = fake(0x100000), *io = fake(0x300000);
    const float* f = (const float*)fake(0x400000);
    EXPECT(pace_prefill_chunk(&c, st, io, io, io, f, f, 512, io, nullptr, 0, nullptr) == PACE_OK, "prefill");
    EXPECT(last_prefill.T == 512 && last_prefill.chunk == 256 && last_prefill.gamma == 2, "prefill params");
    EXPECT(pace_prefill_chunk(&c, st, io, io, io, f, f, 0, io, nullptr, 0, nullptr) == PACE_EINVAL, "T = 0");
    EXPECT(pace_calibrate_heads(&c, io, io, f, f, 512, (double*)fake(0x500000), (double*)fake(0x500100), nullptr) ==
               PACE_OK && last_calib.T == 512,
           "calibration");
    EXPECT(pace_calibrate_heads(&c, io, io, f, f, 512, (double*)fake(0x500004), (double*)fake(0x500100), nullptr) ==
               PACE_EINVAL,
           "fp64 alignment");
    EXPECT(pace_bf16_decode_step(&c, st, io, io, io, f, f, io, nullptr) == PACE_OK && last_bf16.gamma == 2,
           "bf16 baseline");
  }
  // ----------------------------------------------------------------- strings
  const pace_status all[] = {PACE_OK, PACE_EINVAL, PACE_EUNSUPPORTED, PACE_EHIP};
  for (pace_status s : all) EXPECT(pace_status_str(s) != nullptr && strlen(pace_status_str(s)) > 0, "status string");
  if (fails) {
    printf("%d of %ld checks failed\n", fails, checks);
    return 1;
  }
  printf("OK %ld\n", checks);
  return 0;
}
