// Host-only checks and the INT4 centroid quantizer (declarations and their
// contracts in fh_host.h).
#include "fh_host.h"

#include <math.h>
#include <string.h>

namespace fh {

int esize_of(int dtype) { return dtype == FH_DTYPE_F32 ? 4 : dtype == FH_DTYPE_BF16 ? 2 : 0; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_permutation(const int32_t* t, int64_t v) {
  if (!t || v < 1) return FH_ERR_NOT_PERMUTATION;
  std::vector<uint8_t> seen((size_t)v, 0);
  for (int64_t i = 0; i < v; ++i) {
    const int32_t x = t[i];
    if (x < 0 || (int64_t)x >= v || seen[(size_t)x]) return FH_ERR_NOT_PERMUTATION;
    seen[(size_t)x] = 1;
  }
  return FH_OK;
}

void invert_permutation(const int32_t* t, int64_t v, int32_t* inv) {
  for (int64_t r = 0; r < v; ++r) inv[(size_t)t[r]] = (int32_t)r;
}

int validate_desc(const fh_desc* ds) {
  if (!ds || !ds->E || !ds->c2t) return FH_ERR_INVALID_ARG;
  if (ds->c < 1 || ds->b < 1 || ds->d < 1 || ds->v != (int64_t)ds->c * ds->b)
    return FH_ERR_INVALID_ARG;
  if (ds->max_batch < 1 || ds->max_batch > FH_MAX_BATCH) return FH_ERR_INVALID_ARG;
  if (ds->max_p < 1 || ds->max_p > ds->c) return FH_ERR_INVALID_ARG;
  if (ds->lde < ds->d) return FH_ERR_INVALID_ARG;
  if (ds->v > (int64_t)INT32_MAX) return FH_ERR_UNSUPPORTED;
  const int es = esize_of(ds->dtype);
  if (!es) return FH_ERR_UNSUPPORTED;
  if (ds->c > FH_MAX_C) return FH_ERR_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)ds->d * es;
  if (row_bytes % 16 || (ds->lde * es) % 16 || row_bytes > FH_MAX_ROW_BYTES)
    return FH_ERR_UNSUPPORTED;
  if (!aligned16(ds->E) || (ds->C && !aligned16(ds->C))) return FH_ERR_UNSUPPORTED;
  if (ds->quant != FH_QUANT_NONE && ds->quant != FH_QUANT_INT4_G128 &&
      ds->quant != FH_QUANT_INT4_G128_MEAN)
    return FH_ERR_UNSUPPORTED;
  if (ds->quant != FH_QUANT_NONE && (ds->dtype != FH_DTYPE_BF16 || ds->d % 128))
    return FH_ERR_UNSUPPORTED;
  if (ds->flags & ~(FH_FLAG_COOPERATIVE | FH_FLAG_BORROW_E | FH_FLAG_STREAM_ALL |
                    FH_FLAG_SELECT_FIRST))
    return FH_ERR_INVALID_ARG;
  if ((ds->flags & FH_FLAG_STREAM_ALL) && (ds->flags & FH_FLAG_SELECT_FIRST))
    return FH_ERR_INVALID_ARG;
  return check_permutation(ds->c2t, ds->v);
}

double round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e = 0;
  (void)frexp(x, &e);
  // 8 significant bits; below the smallest normal exponent the spacing stays 2^-133
  const int se = (e - 8) > -133 ? (e - 8) : -133;
  return ldexp(nearbyint(ldexp(x, -se)), se);
}

uint16_t bf16_bits(double x) {
  const float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

void column_mean_shift(const uint16_t* C, int c, int d, std::vector<double>& mu) {
  // the sum of c bf16 values is exact in double for the c the library accepts
  mu.assign((size_t)d, 0.0);
  for (int k = 0; k < c; ++k)
    for (int j = 0; j < d; ++j) mu[(size_t)j] += bf16_value(C[(size_t)k * d + j]);
  for (int j = 0; j < d; ++j) mu[(size_t)j] = round_bf16(mu[(size_t)j] / c);
}

void quantize_int4(const uint16_t* C, const double* shift, int c, int d,
                   std::vector<uint8_t>& codes, std::vector<uint16_t>& scales, int* ntiles_out,
                   int* groups_out) {
  const int G = d / 128, ntiles = (c + 15) / 16;
  codes.assign((size_t)ntiles * G * 1024, 0);
  scales.assign((size_t)ntiles * G * 16, 0);
  int8_t q[128];
  double x[128];
  for (int k = 0; k < c; ++k) {
    const int t = k / 16, rin = k % 16;
    for (int g = 0; g < G; ++g) {
      const uint16_t* src = C + (size_t)k * d + (size_t)g * 128;
      const double* sh = shift ? shift + (size_t)g * 128 : nullptr;
      double amax = 0.0;
      for (int j = 0; j < 128; ++j) {
        // x - shift is exact in double for bf16 x and shift
        x[j] = bf16_value(src[j]) - (sh ? sh[j] : 0.0);
        amax = fmax(amax, fabs(x[j]));
      }
      const double s = round_bf16(amax / 7.0);
      for (int j = 0; j < 128; ++j) {
        double qq = s > 0.0 ? nearbyint(x[j] / s) : 0.0;
        qq = qq < -8.0 ? -8.0 : (qq > 7.0 ? 7.0 : qq);
        q[j] = (int8_t)qq;
      }
      scales[((size_t)t * G + g) * 16 + rin] = bf16_bits(s);
      for (int quarter = 0; quarter < 4; ++quarter) {
        const int lane = quarter * 16 + rin;
        uint8_t* dst = codes.data() + (((size_t)t * G + g) * 64 + lane) * 16;
        for (int j = 0; j < 16; ++j) {
          const int col = quarter * 32 + 2 * j;
          dst[j] = (uint8_t)((q[col] & 0xF) | ((q[col + 1] & 0xF) << 4));
        }
      }
    }
  }
  *ntiles_out = ntiles;
  *groups_out = G;
}

}  // namespace fh
