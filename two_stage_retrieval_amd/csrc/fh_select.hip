// Standalone selection kernel: one 1024-thread workgroup per batch row,
// running the block-level selection of fh_select.h on keys produced by an
// earlier kernel.
#include "fh_select.h"

namespace fh {

constexpr int kSelThreads = 1024;

template <int IPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ SelSmem sm;
  const int r = blockIdx.x;
  select_block<kSelThreads, IPT, false>(a.keys + (int64_t)r * a.key_stride, a.c,
                                        (int)a.key_stride, a.p, a.sel + (int64_t)r * a.sel_stride,
                                        a.masks, r, a.error, sm);
  if (!a.counter) return;
  // row 0's workgroup compacts the union of the selected clusters once every
  // other row has set its mask bits
  __builtin_amdgcn_s_waitcnt(0);  // this wave's mask updates have been performed
  __syncthreads();
  if (r != 0) {
    if (threadIdx.x == 0) arrive(a.counter, r);
    return;
  }
  if (threadIdx.x < kWave) {
    const bool ok = wait_arrivals(a.counter, gridDim.x - 1, threadIdx.x);
    if (!ok && threadIdx.x == 0 && a.error) atomicOr(a.error, 2u);
  }
  __syncthreads();
  compact_masks_block<kSelThreads, IPT>(a.masks, a.c, a.ulist, a.ucount, sm);
}

hipError_t launch_select(const SelectArgs& a, int B, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const int ipt = (a.c + kSelThreads - 1) / kSelThreads;
  const dim3 grid(B), block(kSelThreads);
  if (ipt <= 4) hipExtLaunchKernelGGL(select_kernel<4>, grid, block, 0, s, e0, e1, 0, a);
  else if (ipt <= 8) hipExtLaunchKernelGGL(select_kernel<8>, grid, block, 0, s, e0, e1, 0, a);
  else if (ipt <= 16) hipExtLaunchKernelGGL(select_kernel<16>, grid, block, 0, s, e0, e1, 0, a);
  else if (ipt <= 32) hipExtLaunchKernelGGL(select_kernel<32>, grid, block, 0, s, e0, e1, 0, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fh
