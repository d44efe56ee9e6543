// Host-side check of the quantiser's scalar numerics (bit_recurrent_state_amd/csrc/
// pace_numerics.h) against exact long-double arithmetic.  Built and run by
// tests/test_native_numerics.py; prints "OK <count>" on success.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../../bit_recurrent_state_amd/csrc/pace_numerics.h"

using namespace pace;

static int fails = 0;
#define EXPECT(c, ...) do { if (!(c)) { if (fails++ < 20) { printf("FAIL line %d: ", __LINE__); printf(__VA_ARGS__); printf("\n"); } } } while (0)

// Smallest bf16 >= d by enumeration of the 8 significant bits.
static float ref_bf16_ceil(double d) {
  if (!(d > 0)) return 0.f;
  int e;
  double m = std::frexp(d, &e);          // d = m 2^e, 0.5 <= m < 1
  double r = std::ceil(std::ldexp(m, 8));
  double v = std::ldexp(r, e - 8);
  if (d < std::ldexp(1.0, -126)) v = std::ceil(d / std::ldexp(1.0, -133)) * std::ldexp(1.0, -133);
  return (float)v;
}

// round-half-even of the exact quotient x / s.
static double ref_rne_quot(float x, float s) {
  long double q = (long double)x / (long double)s;
  long double f = std::floor(q);
  long double d = q - f;
  if (d > 0.5L) return (double)(f + 1);
  if (d < 0.5L) return (double)f;
  return std::fmod((double)f, 2.0) == 0.0 ? (double)f : (double)(f + 1);
}

int main() {
  std::mt19937_64 rng(7);
  std::uniform_real_distribution<double> U(-1.0, 1.0);
  long n = 0;
  // bf16 ceiling from double
  for (int i = 0; i < 200000; ++i) {
    double d = std::exp(U(rng) * 60.0);
    float got = bf16_ceil_from_f64(d), want = ref_bf16_ceil(d);
    EXPECT(got == want, "bf16_ceil(%.17g) = %.9g want %.9g", d, got, want);
    // values exactly on a bf16 grid point stay there
    double on = (double)want;
    EXPECT(bf16_ceil_from_f64(on) == want, "bf16_ceil on grid %.9g", want);
    n += 2;
  }
  // bf16 ceiling of m / k computed in fp32 (the kernels' scale rule)
  for (int i = 0; i < 300000; ++i) {
    const float ks[4] = {7.f, 15.f, 127.f, 255.f};
    const float k = ks[i & 3];
    float m = (float)std::exp(U(rng) * 30.0);
    if (i % 5 == 0) m = ref_bf16_ceil(std::exp(U(rng) * 20.0)) * k;   // exact multiples
    const float got = bf16_ceil_div(m, k, 1.0f / k), want = ref_bf16_ceil((double)m / (double)k);
    EXPECT(got == want, "bf16_ceil_div(%.9g, %g) = %.9g want %.9g", m, k, got, want);
    n++;
  }
  // correctly rounded quotient from a correctly rounded reciprocal, against IEEE division
  for (int i = 0; i < 400000; ++i) {
    const float ks[4] = {7.f, 15.f, 127.f, 255.f};
    const float k = ks[i & 3];
    uint32_t u = (uint32_t)(rng() % 0x7F000000u) + 1u;     // positive finite fp32 patterns
    float m;
    memcpy(&m, &u, 4);
    volatile float km = k;
    const float got = div_rn(m, k, 1.0f / km), want = m / km;
    EXPECT(got == want, "div_rn(%a, %g) = %a want %a", m, k, got, want);
    n++;
  }
  // reciprocal correction: every normal bf16 value, from each start within an ulp of the
  // correctly rounded reciprocal, lands on it (host rcp_bf16 is the IEEE division)
  for (uint32_t b = 0x0080u; b < 0x7F80u; ++b) {
    const float s = bf16_to_f32((uint16_t)b);
    volatile float vs = s;
    const float want = 1.0f / vs;
    if (!std::isfinite(want) || want < 0x1p-126f) continue;
    const float starts[3] = {std::nextafter(want, 0.f), want, std::nextafter(want, INFINITY)};
    for (float r0 : starts) {
      const float got = rcp_fix(s, r0);
      EXPECT(got == want, "rcp_fix(%a, %a) = %a want %a", s, r0, got, want);
      n++;
    }
    EXPECT(rcp_bf16(s) == want, "rcp_bf16(%a)", s);
  }
  // exact RNE quotient, including constructed exact ties and near ties
  for (int i = 0; i < 400000; ++i) {
    float s = ref_bf16_ceil(std::exp(U(rng) * 10.0));
    float x;
    const int kind = i % 4;
    if (kind == 0) {
      x = (float)(U(rng) * 8.0 * s);
    } else if (kind == 1) {                     // exact half-integer multiples
      int k = (int)std::floor(U(rng) * 128);
      x = (float)((k + 0.5) * (double)s);
    } else if (kind == 2) {                     // one fp32 ulp either side of a tie
      int k = (int)std::floor(U(rng) * 128);
      float t = (float)((k + 0.5) * (double)s);
      x = std::nextafter(t, (i & 8) ? INFINITY : -INFINITY);
    } else {
      x = (float)(U(rng) * 130.0 * s);
    }
    float r = 1.0f / s;
    double got = rne_quotient(x, s, r), want = ref_rne_quot(x, s);
    EXPECT(got == want, "rne(%.9g / %.9g) = %g want %g", x, s, got, want);
    n++;
  }
  // magic-number code decision: rne(x * r) + z clipped, equal to the exact rne(x / s) + z
  // except within a few fp32 ulps of a half-integer quotient
  for (int i = 0; i < 300000; ++i) {
    const bool asym = i & 1;
    const int bits = (i & 2) ? 8 : 4;
    float s = ref_bf16_ceil(std::exp(U(rng) * 8.0));
    const int levels = (1 << bits) - 1, zsym = 1 << (bits - 1);
    const int z = asym ? (int)(std::fabs(U(rng)) * levels) : zsym;
    float x = (float)(U(rng) * (levels + 2) * (double)s);
    CodeRange cr = code_range(z, asym, bits);
    int got = code_of(x, 1.0f / s, cr.magic, cr.lo, cr.hi);
    double q = (double)x / (double)s;
    double want = ref_rne_quot(x, s) + z;
    const double lo = asym ? 0 : 1, hi = levels;
    want = want < lo ? lo : (want > hi ? hi : want);
    const double frac = std::fabs(q - std::floor(q) - 0.5);
    EXPECT(got == (int)want || frac < 1e-5, "code_of(%.9g, s=%.9g, z=%d, bits=%d) = %d want %g", x, s, z, bits, got, want);
    n++;
  }
  // group parameters: zero group, symmetric and asymmetric ranges
  {
    GroupQuant g0 = group_quant(0.f, 0.f, false, 4);
    EXPECT(g0.s == 0.f && g0.z == 8 && g0.r == 0.f, "zero sym group");
    GroupQuant g1 = group_quant(0.f, 0.f, true, 4);
    EXPECT(g1.s == 0.f && g1.z == 0, "zero asym group");
    CodeRange cr = code_range(g0.z, false, 4);
    EXPECT(code_of(1.5f, g0.r, cr.magic, cr.lo, cr.hi) == 8, "zero scale gives stored zero");
    GroupQuant g2 = group_quant(-1.0f, 3.0f, false, 4);
    EXPECT(g2.s == ref_bf16_ceil(3.0 / 7.0) && g2.z == 8, "sym scale");
    GroupQuant g3 = group_quant(0.5f, 3.0f, true, 4);          // range forced to include 0
    EXPECT(g3.s == ref_bf16_ceil(3.0 / 15.0) && g3.z == 0, "asym scale with lo clipped to 0");
    GroupQuant g4 = group_quant(-2.0f, 1.0f, true, 4);
    EXPECT(g4.s == ref_bf16_ceil(3.0 / 15.0) && g4.z == (int)ref_rne_quot(2.0f, g4.s), "asym zero point");
    n += 6;
  }
  // asymmetric scales from random ranges, against the exact ceiling of (hi - lo) / 15
  for (int i = 0; i < 300000; ++i) {
    const float lo = -(float)std::exp(U(rng) * 12.0) * (i % 7 == 0 ? 0.f : 1.f);
    const float hi = (float)std::exp(U(rng) * 12.0) * (i % 11 == 0 ? 0.f : 1.f);
    for (int bits = 4; bits <= 8; bits += 4) {
      const GroupQuant g = group_quant(lo, hi, true, bits);
      const double levels = (double)((1 << bits) - 1);
      const float want = ref_bf16_ceil(((double)hi - (double)lo) / levels);
      EXPECT(g.s == want, "asym scale lo=%a hi=%a bits=%d: %a want %a", lo, hi, bits, g.s, want);
      if (want > 0) {
        const double zq = ref_rne_quot(-lo, want);
        const double z = zq < 0 ? 0 : (zq > levels ? levels : zq);
        EXPECT(g.z == (int)z, "asym zero point lo=%a s=%a: %d want %g", lo, want, g.z, z);
      }
      n += 2;
    }
  }
  // bf16 round-to-nearest-even of fp32
  for (int i = 0; i < 100000; ++i) {
    float x = (float)(U(rng) * std::exp(U(rng) * 20));
    uint16_t b = f32_to_bf16_rne(x);
    double v = bf16_to_f32(b);
    double lo = bf16_to_f32((uint16_t)(b - 1)), hi = bf16_to_f32((uint16_t)(b + 1));
    EXPECT(std::fabs(v - x) <= std::fabs(lo - x) && std::fabs(v - x) <= std::fabs(hi - x),
           "bf16 rne of %.9g", x);
    n++;
  }
  if (fails) {
    printf("FAILED %d\n", fails);
    return 1;
  }
  printf("OK %ld\n", n);
  return 0;
}
