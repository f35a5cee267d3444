// Standalone selection kernel: one 1024-thread workgroup per batch row,
// running the block-level selection of fh_select.h on keys produced by an
// earlier kernel.
#include <cmath>

#include "fh_select.h"

namespace fh {

constexpr int kSelThreads = 1024;

template <int IPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ SelSmem sm;
  const int r = blockIdx.x;
  uint32_t u[IPT];
  select_load_keys<IPT, false>(a.keys + (int64_t)r * a.key_stride, (int)a.key_stride, u);
  if (a.nparts > 1) {
    // the scores arrive as K-slice partials: all slices are loaded before
    // any is added, then summed in slice order; then the keys are formed
    // (sampling: score / tau + Gumbel noise of stream 0, one Philox block per
    // four consecutive ids)
    const int k0 = threadIdx.x * IPT;
    uint32_t v[kMaxKSplit - 1][IPT];
#pragma unroll
    for (int sp = 1; sp < kMaxKSplit; ++sp)
      if (sp < a.nparts)
        select_load_keys<IPT, false>(a.keys + sp * a.part_stride + (int64_t)r * a.key_stride,
                                     (int)a.key_stride, v[sp - 1]);
#pragma unroll
    for (int sp = 1; sp < kMaxKSplit; ++sp)
      if (sp < a.nparts)
#pragma unroll
        for (int j = 0; j < IPT; ++j)
          u[j] = __float_as_uint(__uint_as_float(u[j]) + __uint_as_float(v[sp - 1][j]));
    const uint64_t seed = a.sample ? a.seeds[r] : 0ull;
#pragma unroll
    for (int j4 = 0; j4 < IPT; j4 += 4) {
      float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
      if (a.sample && k0 + j4 < a.c) g = gumbel4(seed, kStreamCluster, (uint32_t)(k0 + j4) >> 2);
      const float gj[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = k0 + j4 + q;
        if (k >= a.c) continue;
        const float sc = __uint_as_float(u[j4 + q]);
        if (a.dbg_scores) a.dbg_scores[(int64_t)r * a.c + k] = sc;
        if (a.sample) u[j4 + q] = __float_as_uint(sc * a.inv_tau + gj[q]);
      }
    }
  }
  select_from_keys<kSelThreads, IPT, false>(u, a.c, a.p, a.zcut, a.sel + (int64_t)r * a.sel_stride,
                                            a.masks, r, a.error, sm);
}

// The union of the rows' selected clusters (non-zero masks), ascending, as
// the batched stage 2's work list: one workgroup, launched after the
// selection so that every row's mask bits are in (the kernel boundary
// orders them; no workgroup waits on another).
template <int IPT>
__global__ __launch_bounds__(kSelThreads) void union_kernel(SelectArgs a) {
  __shared__ SelSmem sm;
  compact_masks_block<kSelThreads, IPT>(a.masks, a.c, a.ulist, a.ucount, sm);
}

// z with upper normal tail probability q, by the rational approximation of
// Abramowitz and Stegun 26.2.23 (absolute error below 4.5e-4), for
// 0 < q <= 0.5.  Only a hint: the selection's result does not depend on it.
static double normal_upper_quantile(double q) {
  const double t = std::sqrt(-2.0 * std::log(q));
  const double num = 2.515517 + t * (0.802853 + t * 0.010328);
  const double den = 1.0 + t * (1.432788 + t * (0.189269 + t * 0.001308));
  return t - num / den;
}

float select_zcut(int c, int p) {
  if (c < 2048 || p < 1) return 0.0f;
  const double q = 4.0 * (double)p / (double)c;
  if (q >= 0.5) return 0.0f;
  return (float)normal_upper_quantile(q);
}

hipError_t launch_select(const SelectArgs& a, int B, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const int ipt = (a.c + kSelThreads - 1) / kSelThreads;
  const dim3 grid(B), block(kSelThreads);
  // with a union list, the events bracket both launches
  hipEvent_t es = a.ulist ? nullptr : e1;
#define FH_SEL_IPT(N)                                                                         \
  if (ipt <= N) {                                                                             \
    hipExtLaunchKernelGGL(select_kernel<N>, grid, block, 0, s, e0, es, 0, a);                 \
    if (a.ulist)                                                                              \
      hipExtLaunchKernelGGL(union_kernel<N>, dim3(1), block, 0, s, nullptr, e1, 0, a);        \
    return hipGetLastError();                                                                 \
  }
  FH_SEL_IPT(4)
  FH_SEL_IPT(8)
  FH_SEL_IPT(16)
  FH_SEL_IPT(32)
#undef FH_SEL_IPT
  return hipErrorInvalidValue;
}

}  // namespace fh
