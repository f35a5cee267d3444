// Host-only parts of libflashhead: the checks flashhead_prepare makes of its
// descriptor (the cluster table C2T among them) and the INT4 centroid
// quantizer of the FlashHead reading notes (Module 3, selective quantization).
// Nothing here touches a device or a HIP type, so the same source also builds
// with a plain host compiler, as the sanitizer test on the CPU does.
#pragma once

#include <stdint.h>

#include <vector>

#include "../../include/flashhead.h"

namespace fh {

int esize_of(int dtype);  // bytes per element of an FH_DTYPE_*, 0 if unknown
bool aligned16(const void* p);

// FH_OK, or the status flashhead_prepare returns for this descriptor before
// it touches the device: FH_ERR_INVALID_ARG, FH_ERR_UNSUPPORTED or
// FH_ERR_NOT_PERMUTATION.  Reads ds->c2t (host memory, v entries).
int validate_desc(const fh_desc* ds);

// FH_OK when t[0..v) holds every value of [0, v) once (equal-size clusters in
// a dense c x b table: FlashHead reading notes, Module 1), else
// FH_ERR_NOT_PERMUTATION.
int check_permutation(const int32_t* t, int64_t v);

// inv[t[r]] = r for a permutation t of [0, v): the row of each token in the
// cluster-major layout.
void invert_permutation(const int32_t* t, int64_t v, int32_t* inv);

double round_bf16(double x);     // nearest bf16 value, ties to even
uint16_t bf16_bits(double x);    // bits of a value that is already a bf16 value
double bf16_value(uint16_t bits);

// bf16 of each column's mean over the c rows of C (c x d, bf16 bits): the
// shift of the mean-shifted INT4 variant.
void column_mean_shift(const uint16_t* C, int c, int d, std::vector<double>& mu);

// Symmetric INT4 codes per group of 128 columns of C - shift (shift: d values,
// or null): scale = bf16(amax / 7), code = round-half-even(x / scale) clipped
// to [-8, 7].  Codes are packed in tiles of 16 centroid rows: for tile t and
// group g, 64 lanes of 16 bytes, lane = quarter * 16 + row-in-tile, byte j of
// a lane holding columns quarter * 32 + 2j (low nibble) and + 1 (high nibble).
// Scales: [tile][group][row-in-tile] bf16 bits.  d must be a multiple of 128;
// rows past c in the last tile are left zero.
void quantize_int4(const uint16_t* C, const double* shift, int c, int d,
                   std::vector<uint8_t>& codes, std::vector<uint16_t>& scales, int* ntiles_out,
                   int* groups_out);

}  // namespace fh
