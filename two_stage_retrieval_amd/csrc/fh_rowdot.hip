// Row-dot kernels: one wave computes full dot products of R rows of a
// row-major matrix with one hidden vector h (GEMV family, batch rows on
// grid.y).  Two epilogues:
//   gather  stage-2 exact logits of the candidate rows of the selected
//           clusters (notes, Overall architecture and Module 1), fused with
//           the decode (Formula 2 argmax or Formula 3 Gumbel-max sample);
//   dense   the dense head z = E h (Formula 1) with the same decode.
//
// Memory layout: lane l of a wave owns the 16-byte chunks l, l+64, ... of a
// row, so a wave reads each row as one contiguous, fully coalesced span and
// keeps its slice of h in registers for all rows it visits.  The gather
// epilogue reads the cluster-major copy of E built at prepare time: the b
// candidate rows of a cluster are one contiguous block, and C2T is read only
// for the token ids (in parallel with the row loads, not in their address
// chain).
#include "fh_rows.h"

namespace fh {

constexpr int kRowdotThreads = 256;
constexpr int kRowdotWaves = kRowdotThreads / kWave;

template <typename TE, int NCH, int R, int MODE>
__global__ __launch_bounds__(kRowdotThreads) void rowdot_kernel(RowdotArgs a) {
  __shared__ MergeSmem<kRowdotThreads> ms;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blockIdx.y;
  float hreg[NCH][Chunk<TE>::kElems];
  load_h<TE, NCH>(a.H + (int64_t)r * a.h_bytes, a.nchunk, lane, hreg);
  const uint64_t seed = a.sample ? a.seeds[r] : 0ull;
  uint64_t best = 0;
  Lse lse = lse_empty();
  // (the gather may follow an adaptive count: entries past it are skipped)
  dot_rows<TE, NCH, R, MODE, false, MODE == kRowGather>(a, r, a.sel + (int64_t)r * a.sel_stride,
                                                        hreg, seed, lane,
                                    (int64_t)blockIdx.x * kRowdotWaves + wave,
                                    (int64_t)gridDim.x * kRowdotWaves, best, lse);
  // workgroup 0 of the batch row folds every workgroup's partial
  merge_decode<kRowdotThreads>(a, r, gridDim.x, blockIdx.x, 0, best, lse, ms);
}

// Rows per wave per step: enough bytes in flight per wave without spilling.
template <int NCH> constexpr int rows_for() { return NCH <= 2 ? 8 : 4; }

template <typename TE, int MODE>
static hipError_t launch_t(const RowdotArgs& a, int B, int grid_x, hipStream_t s,
                           const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const dim3 grid(grid_x, B), block(kRowdotThreads);
  const int nch = (a.nchunk + kWave - 1) / kWave;
#define FH_ROWDOT_CASE(N)                                                              \
  case N:                                                                              \
    hipExtLaunchKernelGGL((rowdot_kernel<TE, N, rows_for<N>(), MODE>), grid, block, 0, s, e0, \
                          e1, 0, a);                                                   \
    break;
  switch (nch) {
    FH_ROWDOT_CASE(1)
    FH_ROWDOT_CASE(2)
    FH_ROWDOT_CASE(3)
    FH_ROWDOT_CASE(4)
    FH_ROWDOT_CASE(5)
    FH_ROWDOT_CASE(6)
    FH_ROWDOT_CASE(7)
    FH_ROWDOT_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef FH_ROWDOT_CASE
  return hipGetLastError();
}

int rowdot_grid(int64_t nrows, int nchunk, int mode) {
  const int nch = (nchunk + kWave - 1) / kWave;
  const int R = nch <= 2 ? 8 : 4;
  const int64_t groups = (nrows + R - 1) / R;
  int64_t blocks = (groups + kRowdotWaves - 1) / kRowdotWaves;
  // dense: cap at a few resident blocks per CU and loop (256 CUs)
  const int64_t cap = mode == kRowDense ? 2048 : 8192;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

hipError_t launch_rowdot(const RowdotArgs& a, int mode, int dtype, int B, int grid_x,
                         hipStream_t s, const Timing* tm) {
  if (dtype == FH_DTYPE_BF16) {
    if (mode == kRowGather) return launch_t<bf16_t, kRowGather>(a, B, grid_x, s, tm);
    return launch_t<bf16_t, kRowDense>(a, B, grid_x, s, tm);
  }
  if (mode == kRowGather) return launch_t<float, kRowGather>(a, B, grid_x, s, tm);
  return launch_t<float, kRowDense>(a, B, grid_x, s, tm);
}

}  // namespace fh
