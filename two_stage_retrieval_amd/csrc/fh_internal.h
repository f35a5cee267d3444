// Host-side declarations shared by the translation units of libflashhead.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flashhead.h"

namespace fh {

// Which rows a row-dot launch visits and what it does with each dot product.
enum RowdotMode : int {
  kRowScores = 0,  // rows [0, nrows) of `base`; write key per row to `keys_out`
  kRowGather = 1,  // candidate rows C2T[sel[i / b], i % b]; decode epilogue
  kRowDense = 2,   // rows [0, nrows) of `base`; decode epilogue
};

struct RowdotArgs {
  const uint8_t* base;   // E or C
  int64_t row_bytes;     // stride between rows of `base`
  int nchunk;            // 16-byte chunks per row
  const uint8_t* H;      // B x d, row stride h_bytes
  int64_t h_bytes;
  int64_t nrows;         // logical rows per batch row
  // gather
  const int32_t* sel;    // B x sel_stride, selected clusters (ascending)
  int sel_stride;
  const int32_t* c2t;    // c x b
  int b;
  int nclusters;         // c (selected ids are clamped to [0, c))
  // scores epilogue
  float* keys_out;       // B x key_stride: selection keys (s, or s/tau + G0)
  int64_t key_stride;
  float* dbg_scores;     // optional raw scores, B x key_stride
  // decode epilogue
  uint64_t* best;        // B: running max decode key (zero between calls)
  uint32_t* counters;    // B: finished-block counters (zero between calls)
  float2* lse_part;      // B x gridDim.x partial (max, sum)
  int32_t* out_tokens;
  float* out_lse;
  int32_t* dbg_ids;      // optional, B x dbg_stride
  float* dbg_logits;
  int64_t dbg_stride;
  // sampling
  int sample;
  float inv_tau;
  const uint64_t* seeds;
};

struct SelectArgs {
  const float* keys;     // B x key_stride
  int64_t key_stride;
  int c, p;
  int32_t* sel;          // B x sel_stride, written ascending
  int sel_stride;
  uint64_t* masks;       // optional: per-cluster bitmask of selecting rows
  uint32_t* error;       // optional: set non-zero if a row selected != p
};

struct Int4Args {
  const uint8_t* codes;  // tiled, see flashhead_export_int4
  const uint16_t* scales;
  int ntiles;            // ceil(c / 16)
  int groups;            // d / 128
  int c, d;
  const uint16_t* H;     // B x d bf16
  float* keys_out;
  int64_t key_stride;
  float* dbg_scores;
  int sample;
  float inv_tau;
  const uint64_t* seeds;
};

struct FusedArgs {
  const uint8_t* C;       // c x d centroids (bf16 / fp32)
  int64_t row_bytes;      // d * element size (rows of C and of Ec)
  int nchunk;             // 16-byte chunks per row
  int c, b, p, d;
  const uint8_t* q4;      // INT4 tiles (when quantized)
  const uint16_t* q4s;
  int ntiles, groups;
  const uint8_t* H;       // one hidden vector
  const uint8_t* Ec;      // cluster-major copy of E
  const int32_t* c2t;
  float cmax;             // upper bound of the centroid norms
  int64_t rows_per_block; // stage-2 rows per workgroup (multiple of 4)
  float* keys;            // c selection keys
  uint32_t* hist;         // 2 x 4096 bins, alternating by epoch
  uint32_t* arrive;       // grid arrival counter (reset by the last block)
  uint32_t* done;         // finished-block counter (reset by the last block)
  uint32_t* epoch;        // call counter (selects the histogram buffer)
  uint32_t* error;        // bit 0: selection count, bit 1: barrier timeout
  uint64_t* best;         // running max decode key (reset by the last block)
  float2* lse_part;       // one per workgroup
  int32_t* out_tokens;
  float* out_lse;
  float* dbg_scores;
  int32_t* dbg_clusters;
  int32_t* dbg_ids;
  float* dbg_logits;
  int sample;
  float inv_tau;
  const uint64_t* seeds;
};

// Optional events recorded exactly around one kernel (hipExtLaunchKernel).
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
};

hipError_t launch_rowdot(const RowdotArgs& a, int mode, int dtype, int B, int grid_x,
                         hipStream_t s, const Timing* tm = nullptr);
int rowdot_grid(int64_t nrows, int nchunk, int mode);
hipError_t launch_select(const SelectArgs& a, int B, hipStream_t s, const Timing* tm = nullptr);
hipError_t launch_int4_gemv(const Int4Args& a, int B, hipStream_t s, const Timing* tm = nullptr);
hipError_t launch_centroid_means(const uint8_t* E, int64_t row_bytes, int dtype, int d,
                                 const int32_t* c2t, int c, int b, void* C, hipStream_t s);
int fused_grid();
int64_t fused_rows_per_block(int p, int b);
bool fused_supported(int dtype, int nchunk, int c, int quant, int p, int b);
hipError_t launch_fused(const FusedArgs& a, int dtype, int quant, hipStream_t s,
                        const Timing* tm);
hipError_t launch_cluster_major_copy(const uint8_t* E, int64_t lde_bytes, const int32_t* c2t,
                                     int64_t v, int64_t row_bytes, uint8_t* Ec, hipStream_t s);

}  // namespace fh
