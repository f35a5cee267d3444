// The single-launch batch-1 decode with the adaptive probe count compiled
// in (see fh_decode_b1.h); a translation unit of its own so that the plain
// kernels carry none of its code.
#include "fh_decode_b1.h"

namespace fh {

hipError_t decode_b1_occupancy_adaptive(int dtype, bool int4, int nchunk, int c, int* blocks) {
  return decode_b1_occupancy_impl<true>(dtype, int4, nchunk, c, blocks);
}

hipError_t launch_decode_b1_adaptive(const DecodeB1Args& a, int dtype, bool int4, int grid,
                                     bool coop, hipStream_t s, const Timing* tm) {
  return launch_decode_b1_impl<true>(a, dtype, int4, grid, coop, s, tm);
}

}  // namespace fh
