// CPU checks of libflashhead's host-only code (fh_host.cpp), built with the
// address and undefined-behaviour sanitizers by tests/test_host_sanitize.py:
// the descriptor checks of flashhead_prepare, the cluster table's
// permutation check and inverse, and the INT4 centroid quantizer.  Prints
// "ok <n>" with the number of checks and exits 0, or names the first failure
// and exits 1.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <vector>

#include "../../two_stage_retrieval_amd/csrc/fh_host.h"

static int g_checks = 0;

#define CHECK(cond)                                                       \
  do {                                                                    \
    ++g_checks;                                                           \
    if (!(cond)) {                                                        \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);   \
      exit(1);                                                            \
    }                                                                     \
  } while (0)

static uint16_t to_bf16(float f) {  // truncation: any bf16 value will do here
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static double from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// code of column col in row-in-tile rin, tile t, group g, unpacked from the
// documented layout and sign-extended
static int code_at(const std::vector<uint8_t>& codes, int G, int t, int g, int rin, int col) {
  const int quarter = col / 32, j = (col % 32) / 2;
  const uint8_t byte = codes[(((size_t)t * G + g) * 64 + quarter * 16 + rin) * 16 + j];
  const int nib = (col % 2) ? (byte >> 4) : (byte & 0xF);
  return nib >= 8 ? nib - 16 : nib;
}

static void permutation_checks() {
  std::vector<int32_t> t(96);
  for (int i = 0; i < 96; ++i) t[i] = 95 - i;
  CHECK(fh::check_permutation(t.data(), 96) == FH_OK);
  std::vector<int32_t> inv(96, -1);
  fh::invert_permutation(t.data(), 96, inv.data());
  for (int i = 0; i < 96; ++i) CHECK(t[inv[i]] == i);

  std::mt19937 rng(7);
  std::vector<int32_t> p(1000);
  for (int i = 0; i < 1000; ++i) p[i] = i;
  std::shuffle(p.begin(), p.end(), rng);
  CHECK(fh::check_permutation(p.data(), 1000) == FH_OK);
  inv.assign(1000, -1);
  fh::invert_permutation(p.data(), 1000, inv.data());
  for (int i = 0; i < 1000; ++i) CHECK(inv[p[i]] == i);

  std::vector<int32_t> bad = p;
  bad[10] = bad[11];  // a repeat (and so a missing value)
  CHECK(fh::check_permutation(bad.data(), 1000) == FH_ERR_NOT_PERMUTATION);
  bad = p;
  bad[999] = 1000;  // one past the end
  CHECK(fh::check_permutation(bad.data(), 1000) == FH_ERR_NOT_PERMUTATION);
  bad = p;
  bad[0] = -1;
  CHECK(fh::check_permutation(bad.data(), 1000) == FH_ERR_NOT_PERMUTATION);
  bad = p;
  bad[500] = INT32_MAX;
  CHECK(fh::check_permutation(bad.data(), 1000) == FH_ERR_NOT_PERMUTATION);
  int32_t one = 0;
  CHECK(fh::check_permutation(&one, 1) == FH_OK);
  CHECK(fh::check_permutation(nullptr, 1) == FH_ERR_NOT_PERMUTATION);
  CHECK(fh::check_permutation(&one, 0) == FH_ERR_NOT_PERMUTATION);
}

static void desc_checks() {
  const int c = 12, b = 8, d = 256;
  const int64_t v = (int64_t)c * b;
  // the pointers are never dereferenced on the host, apart from c2t
  alignas(16) static uint8_t dummy[64];
  std::vector<int32_t> c2t(v);
  for (int64_t i = 0; i < v; ++i) c2t[i] = (int32_t)((i * 37) % v);  // gcd(37, 96) = 1
  fh_desc base;
  memset(&base, 0, sizeof base);
  base.E = dummy;
  base.v = v;
  base.d = d;
  base.lde = d;
  base.dtype = FH_DTYPE_BF16;
  base.C = nullptr;
  base.c2t = c2t.data();
  base.c = c;
  base.b = b;
  base.quant = FH_QUANT_NONE;
  base.max_batch = 16;
  base.max_p = 4;
  base.flags = 0;
  CHECK(fh::validate_desc(&base) == FH_OK);
  CHECK(fh::validate_desc(nullptr) == FH_ERR_INVALID_ARG);

  struct Case {
    const char* what;
    void (*edit)(fh_desc&);
    int want;
  };
  static const Case cases[] = {
      {"E null", [](fh_desc& x) { x.E = nullptr; }, FH_ERR_INVALID_ARG},
      {"c2t null", [](fh_desc& x) { x.c2t = nullptr; }, FH_ERR_INVALID_ARG},
      {"v != c b", [](fh_desc& x) { x.v += 1; }, FH_ERR_INVALID_ARG},
      {"c 0", [](fh_desc& x) { x.c = 0; }, FH_ERR_INVALID_ARG},
      {"b 0", [](fh_desc& x) { x.b = 0; }, FH_ERR_INVALID_ARG},
      {"d 0", [](fh_desc& x) { x.d = 0; }, FH_ERR_INVALID_ARG},
      {"max_batch 0", [](fh_desc& x) { x.max_batch = 0; }, FH_ERR_INVALID_ARG},
      {"max_batch over", [](fh_desc& x) { x.max_batch = FH_MAX_BATCH + 1; }, FH_ERR_INVALID_ARG},
      {"max_p 0", [](fh_desc& x) { x.max_p = 0; }, FH_ERR_INVALID_ARG},
      {"max_p over c", [](fh_desc& x) { x.max_p = x.c + 1; }, FH_ERR_INVALID_ARG},
      {"lde < d", [](fh_desc& x) { x.lde = x.d - 8; }, FH_ERR_INVALID_ARG},
      {"dtype", [](fh_desc& x) { x.dtype = 77; }, FH_ERR_UNSUPPORTED},
      {"row bytes % 16", [](fh_desc& x) { x.d = 4; x.lde = 4; }, FH_ERR_UNSUPPORTED},
      {"lde bytes % 16", [](fh_desc& x) { x.lde = x.d + 4; }, FH_ERR_UNSUPPORTED},
      {"row bytes over", [](fh_desc& x) { x.d = 8192; x.lde = 8192; }, FH_ERR_UNSUPPORTED},
      {"E misaligned", [](fh_desc& x) { x.E = static_cast<const uint8_t*>(x.E) + 8; },
       FH_ERR_UNSUPPORTED},
      {"C misaligned", [](fh_desc& x) { x.C = static_cast<const uint8_t*>(x.E) + 4; },
       FH_ERR_UNSUPPORTED},
      {"quant unknown", [](fh_desc& x) { x.quant = 9; }, FH_ERR_UNSUPPORTED},
      {"int4 on f32", [](fh_desc& x) { x.quant = FH_QUANT_INT4_G128; x.dtype = FH_DTYPE_F32; },
       FH_ERR_UNSUPPORTED},
      {"int4 d % 128", [](fh_desc& x) { x.quant = FH_QUANT_INT4_G128; x.d = 64; x.lde = 64; },
       FH_ERR_UNSUPPORTED},
      {"flags unknown", [](fh_desc& x) { x.flags = 16; }, FH_ERR_INVALID_ARG},
      {"both path flags", [](fh_desc& x) { x.flags = FH_FLAG_STREAM_ALL | FH_FLAG_SELECT_FIRST; },
       FH_ERR_INVALID_ARG},
      {"c over max", [](fh_desc& x) { x.c = FH_MAX_C + 1; x.b = 1; x.v = x.c; x.max_p = 1; },
       FH_ERR_UNSUPPORTED},
  };
  for (const Case& k : cases) {
    fh_desc x = base;
    k.edit(x);
    const int got = fh::validate_desc(&x);
    if (got != k.want) fprintf(stderr, "case '%s': got %d want %d\n", k.what, got, k.want);
    CHECK(got == k.want);
  }
  // accepted variants
  {
    fh_desc x = base;
    x.quant = FH_QUANT_INT4_G128_MEAN;
    CHECK(fh::validate_desc(&x) == FH_OK);
    x.flags = FH_FLAG_COOPERATIVE | FH_FLAG_BORROW_E;
    CHECK(fh::validate_desc(&x) == FH_OK);
    x.flags = FH_FLAG_STREAM_ALL;
    CHECK(fh::validate_desc(&x) == FH_OK);
    x.flags = FH_FLAG_SELECT_FIRST | FH_FLAG_BORROW_E;
    CHECK(fh::validate_desc(&x) == FH_OK);
    x = base;
    x.dtype = FH_DTYPE_F32;
    x.lde = d + 4;
    CHECK(fh::validate_desc(&x) == FH_OK);
  }
  // a table that is not a permutation, with everything else valid
  {
    std::vector<int32_t> dup = c2t;
    dup[3] = dup[4];
    fh_desc x = base;
    x.c2t = dup.data();
    CHECK(fh::validate_desc(&x) == FH_ERR_NOT_PERMUTATION);
  }
}

static void bf16_checks() {
  CHECK(fh::round_bf16(1.0) == 1.0);
  CHECK(fh::round_bf16(0.0) == 0.0);
  // 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even 1
  CHECK(fh::round_bf16(1.0 + ldexp(1.0, -8)) == 1.0);
  // 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
  CHECK(fh::round_bf16(1.0 + 3 * ldexp(1.0, -8)) == 1.0 + ldexp(1.0, -6));
  CHECK(fh::round_bf16(-3.0) == -3.0);
  CHECK(fh::round_bf16(1.0 / 3.0) == from_bf16(0x3EAB));  // 0.333984375
  for (uint32_t bits = 0; bits < 0x7F80; bits += 97) {
    const double x = from_bf16((uint16_t)bits);
    CHECK(fh::round_bf16(x) == x);
    CHECK(fh::bf16_bits(x) == bits);
    CHECK(fh::bf16_value((uint16_t)bits) == x);
  }
}

static void quantizer_checks() {
  // ragged: 37 centroid rows (3 tiles, the last with 5 rows), 3 groups
  const int c = 37, d = 384, G = d / 128;
  std::mt19937 rng(11);
  std::normal_distribution<float> nd(0.0f, 0.05f);
  std::vector<uint16_t> C((size_t)c * d);
  for (auto& x : C) x = to_bf16(nd(rng));
  // row 0, group 0: max |x| = 7 * 2^-4, so the scale is 2^-4 and x / s are integers
  for (int j = 0; j < 128; ++j) C[j] = to_bf16((float)ldexp((double)((j % 15) - 7), -4));
  // row 1, group 1: all zero -> scale 0, codes 0
  for (int j = 0; j < 128; ++j) C[(size_t)1 * d + 128 + j] = 0;
  // row 2, group 2: halfway cases at scale 1: amax 7, then 2.5 and 3.5 and -2.5
  for (int j = 0; j < 128; ++j) C[(size_t)2 * d + 256 + j] = to_bf16(0.0f);
  C[(size_t)2 * d + 256 + 0] = to_bf16(7.0f);
  C[(size_t)2 * d + 256 + 1] = to_bf16(2.5f);
  C[(size_t)2 * d + 256 + 2] = to_bf16(3.5f);
  C[(size_t)2 * d + 256 + 3] = to_bf16(-2.5f);
  C[(size_t)2 * d + 256 + 4] = to_bf16(-7.0f);

  std::vector<uint8_t> codes;
  std::vector<uint16_t> scales;
  int ntiles = 0, groups = 0;
  fh::quantize_int4(C.data(), nullptr, c, d, codes, scales, &ntiles, &groups);
  CHECK(ntiles == 3 && groups == G);
  CHECK(codes.size() == (size_t)ntiles * G * 1024 && scales.size() == (size_t)ntiles * G * 16);

  for (int k = 0; k < ntiles * 16; ++k) {
    const int t = k / 16, rin = k % 16;
    for (int g = 0; g < G; ++g) {
      const double s = from_bf16(scales[((size_t)t * G + g) * 16 + rin]);
      if (k >= c) {  // rows past c: zero scale and codes
        CHECK(s == 0.0);
        for (int col = 0; col < 128; ++col) CHECK(code_at(codes, G, t, g, rin, col) == 0);
        continue;
      }
      double amax = 0.0;
      for (int col = 0; col < 128; ++col)
        amax = fmax(amax, fabs(from_bf16(C[(size_t)k * d + g * 128 + col])));
      // the scale is a bf16 value within half a bf16 step of amax / 7
      CHECK(fabs(s - amax / 7.0) <= ldexp(amax / 7.0, -8) * 1.0000001);
      for (int col = 0; col < 128; ++col) {
        const double x = from_bf16(C[(size_t)k * d + g * 128 + col]);
        const int q = code_at(codes, G, t, g, rin, col);
        CHECK(q >= -8 && q <= 7);
        if (s == 0.0) {
          CHECK(q == 0);
        } else {
          // nearest code: the reconstruction is off by at most half a step,
          // unless the code was clipped at 7 (x / s can exceed 7 by a bf16 step)
          const double err = fabs(x - s * q);
          CHECK(err <= 0.5 * s * 1.0000001 || (q == 7 && x > 7 * s) || (q == -7 && x < -7 * s));
        }
      }
    }
  }
  // the exact rows
  for (int j = 0; j < 128; ++j) CHECK(code_at(codes, G, 0, 0, 0, j) == (j % 15) - 7);
  CHECK(from_bf16(scales[0]) == ldexp(1.0, -4));
  CHECK(from_bf16(scales[(size_t)(0 * G + 1) * 16 + 1]) == 0.0);
  CHECK(from_bf16(scales[(size_t)(0 * G + 2) * 16 + 2]) == 1.0);
  CHECK(code_at(codes, G, 0, 2, 2, 0) == 7);
  CHECK(code_at(codes, G, 0, 2, 2, 1) == 2);   // 2.5 -> 2 (ties to even)
  CHECK(code_at(codes, G, 0, 2, 2, 2) == 4);   // 3.5 -> 4
  CHECK(code_at(codes, G, 0, 2, 2, 3) == -2);  // -2.5 -> -2
  CHECK(code_at(codes, G, 0, 2, 2, 4) == -7);
  CHECK(code_at(codes, G, 0, 2, 2, 5) == 0);

  // mean shift: a matrix whose rows are one vector m plus +-u per group
  // column; the column means are m exactly, and C - shift = +-u
  {
    const int c2 = 20, d2 = 128;
    std::vector<uint16_t> M((size_t)c2 * d2);
    for (int k = 0; k < c2; ++k)
      for (int j = 0; j < d2; ++j) {
        const float m = (float)ldexp((double)(j % 9) - 4.0, -3);
        const float u = (float)ldexp(1.0 + (j % 4), -6);
        M[(size_t)k * d2 + j] = to_bf16(m + ((k % 2) ? u : -u));
      }
    std::vector<double> mu;
    fh::column_mean_shift(M.data(), c2, d2, mu);
    CHECK(mu.size() == (size_t)d2);
    for (int j = 0; j < d2; ++j) CHECK(mu[j] == ldexp((double)(j % 9) - 4.0, -3));
    std::vector<uint8_t> cs;
    std::vector<uint16_t> ss;
    int nt = 0, gg = 0;
    fh::quantize_int4(M.data(), mu.data(), c2, d2, cs, ss, &nt, &gg);
    CHECK(nt == 2 && gg == 1);
    for (int k = 0; k < c2; ++k) {
      // amax = 4 * 2^-6 -> scale bf16(2^-4 / 7); codes are round(+-u / s)
      const double s = from_bf16(ss[(size_t)(k / 16) * 16 + k % 16]);
      CHECK(s == fh::round_bf16(ldexp(4.0, -6) / 7.0));
      for (int j = 0; j < d2; ++j) {
        const double u = ldexp(1.0 + (j % 4), -6) * ((k % 2) ? 1 : -1);
        CHECK(code_at(cs, 1, k / 16, 0, k % 16, j) == (int)nearbyint(u / s));
      }
    }
  }
}

int main() {
  permutation_checks();
  desc_checks();
  bf16_checks();
  quantizer_checks();
  printf("ok %d\n", g_checks);
  return 0;
}
