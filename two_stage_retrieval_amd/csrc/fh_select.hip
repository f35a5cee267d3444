// Standalone selection kernel: one 1024-thread workgroup per batch row,
// running the block-level selection of fh_select.h on keys produced by an
// earlier kernel.
#include "fh_select.h"

namespace fh {

constexpr int kSelThreads = 1024;

template <int IPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ SelSmem sm;
  __shared__ int s_last;
  const int r = blockIdx.x;
  select_block<kSelThreads, IPT, false>(a.keys + (int64_t)r * a.key_stride, a.c, a.p,
                                        a.sel + (int64_t)r * a.sel_stride, a.masks, r, a.error,
                                        sm);
  if (!a.counter) return;
  // the last row to finish compacts the union of the selected clusters
  __builtin_amdgcn_s_waitcnt(0);  // this wave's mask updates have been performed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) __hip_atomic_exchange(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  compact_masks_block<kSelThreads, IPT>(a.masks, a.c, a.ulist, a.ucount, sm);
}

hipError_t launch_select(const SelectArgs& a, int B, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const int ipt = (a.c + kSelThreads - 1) / kSelThreads;
  const dim3 grid(B), block(kSelThreads);
  if (ipt <= 1) hipExtLaunchKernelGGL(select_kernel<1>, grid, block, 0, s, e0, e1, 0, a);
  else if (ipt <= 2) hipExtLaunchKernelGGL(select_kernel<2>, grid, block, 0, s, e0, e1, 0, a);
  else if (ipt <= 4) hipExtLaunchKernelGGL(select_kernel<4>, grid, block, 0, s, e0, e1, 0, a);
  else if (ipt <= 8) hipExtLaunchKernelGGL(select_kernel<8>, grid, block, 0, s, e0, e1, 0, a);
  else if (ipt <= 16) hipExtLaunchKernelGGL(select_kernel<16>, grid, block, 0, s, e0, e1, 0, a);
  else if (ipt <= 32) hipExtLaunchKernelGGL(select_kernel<32>, grid, block, 0, s, e0, e1, 0, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fh
