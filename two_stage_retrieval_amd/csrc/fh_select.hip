// Standalone selection kernel: one 1024-thread workgroup per batch row,
// running the block-level selection of fh_select.h on keys produced by an
// earlier kernel.
#include <cmath>

#include "fh_select.h"

namespace fh {

constexpr int kSelThreads = 1024;

// The values the first loads need (the keys or K-slice partials of the
// row) arrive as leading scalar kernel arguments, which the dispatcher
// preloads into scalar registers, so the loads need not wait for the
// argument struct; the rest comes in SelectArgs.
struct SelectFirst {
  const float* keys;
  int key_stride, nparts, part_stride;
};

// The selection of batch row r (the whole workgroup).
template <int IPT>
__device__ __forceinline__ void select_row(const SelectFirst& f, const SelectArgs& a, int r,
                                           SelSmem& sm) {
  uint32_t u[IPT];
  // every slice of the row is requested before anything else is read
  uint32_t v[kMaxKSplit - 1][IPT];
  select_load_keys<IPT, false>(f.keys + (int64_t)r * f.key_stride, f.key_stride, u);
#pragma unroll
  for (int sp = 1; sp < kMaxKSplit; ++sp)
    if (sp < f.nparts)
      select_load_keys<IPT, false>(f.keys + (int64_t)sp * f.part_stride + (int64_t)r * f.key_stride,
                                   f.key_stride, v[sp - 1]);
  int p = a.p;  // the row's probe count
  if (f.nparts > 1 || a.form_keys) {
    // the scores arrive as K-slice partials (or, with form_keys, as plain
    // scores): all slices were loaded before any is added, then summed in
    // slice order; then the keys are formed
    // (sampling: score / tau + Gumbel noise of stream 0, one Philox block per
    // four consecutive ids)
    const int k0 = threadIdx.x * IPT;
#pragma unroll
    for (int sp = 1; sp < kMaxKSplit; ++sp)
      if (sp < f.nparts)
#pragma unroll
        for (int j = 0; j < IPT; ++j)
          u[j] = __float_as_uint(__uint_as_float(u[j]) + __uint_as_float(v[sp - 1][j]));
    // the adaptive count reads the plain scores, before any noise
    if (a.ad.on) p = adaptive_count<kSelThreads, IPT>(u, a.c, a.ad, a.p, sm);
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
  } else if (a.ad.on) {
    if (a.raw) {  // the keys carry noise: count on the plain scores beside them
      uint32_t us[IPT];
      select_load_keys<IPT, false>(a.raw + (int64_t)r * a.key_stride, (int)a.key_stride, us);
      p = adaptive_count<kSelThreads, IPT>(us, a.c, a.ad, a.p, sm);
    } else {
      p = adaptive_count<kSelThreads, IPT>(u, a.c, a.ad, a.p, sm);  // greedy: keys are scores
    }
  }
  if (a.ad.on && a.ad.out_p && threadIdx.x == 0) a.ad.out_p[r] = p;
  select_from_keys<kSelThreads, IPT, false>(u, a.c, p, a.zcut, a.sel + (int64_t)r * a.sel_stride,
                                            a.masks, r, a.error, sm, nullptr,
                                            a.ad.on ? a.p : 0);
}

template <int IPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* keys, int key_stride,
                                                             int nparts, int part_stride,
                                                             SelectArgs a) {
  __shared__ SelSmem sm;
  const SelectFirst f{keys, key_stride, nparts, part_stride};
  select_row<IPT>(f, a, blockIdx.x, sm);
}

// Selection of batch row r, then the fold of the records the all-cluster
// stream left for its selected clusters: the best decode key (the token) and
// the log-sum-exp over exactly the candidates of those clusters.
template <int IPT>
__global__ __launch_bounds__(kSelThreads) void select_fold_kernel(const float* keys,
                                                                  int key_stride, int nparts,
                                                                  int part_stride, SelectArgs a) {
  const SelectFirst f{keys, key_stride, nparts, part_stride};
  __shared__ SelSmem sm;
  __shared__ uint64_t s_b[kSelThreads / kWave];
  __shared__ float2 s_l[kSelThreads / kWave];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  select_row<IPT>(f, a, r, sm);
  __threadfence_block();  // this workgroup's writes of the row's selection
  __syncthreads();
  const int32_t* sr = a.sel + (int64_t)r * a.sel_stride;
  uint64_t bb = 0ull;
  Lse ll = lse_empty();
  for (int j = t; j < a.p; j += kSelThreads) {
    const int32_t k = sr[j];
    if (k == kUnusedEntry) continue;  // past an adaptive count
    for (int m = 0; m < a.fold_sub; ++m) {
      const int64_t rec = ((int64_t)k * a.fold_sub + m) * a.fold_pitch + r;
      const uint64_t x = a.fold_best[rec];
      bb = x > bb ? x : bb;
      if (a.fold_lse) {
        const float2 l = a.fold_lse[rec];
        ll = lse_merge(ll, Lse{l.x, l.y});
      }
    }
  }
  bb = wave_max_u64(bb);
  if (a.fold_lse) ll = wave_lse(ll);
  if ((t & (kWave - 1)) == 0) {
    s_b[t / kWave] = bb;
    s_l[t / kWave] = make_float2(ll.m, ll.s);
  }
  __syncthreads();
  if (t == 0) {
    uint64_t b0 = s_b[0];
    Lse l0{s_l[0].x, s_l[0].y};
#pragma unroll
    for (int w = 1; w < kSelThreads / kWave; ++w) {
      b0 = s_b[w] > b0 ? s_b[w] : b0;
      l0 = lse_merge(l0, Lse{s_l[w].x, s_l[w].y});
    }
    a.out_tokens[r] = (int32_t)key_id(b0);
    if (a.out_lse) a.out_lse[r] = l0.m + logf(l0.s);
  }
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

hipError_t launch_select_fold(const SelectArgs& a, int B, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const int ipt = (a.c + kSelThreads - 1) / kSelThreads;
  const dim3 grid(B), block(kSelThreads);
#define FH_SEL_IPT(N)                                                                \
  if (ipt <= N) {                                                                    \
    hipExtLaunchKernelGGL(select_fold_kernel<N>, grid, block, 0, s, e0, e1, 0, a.keys,  \
                          (int)a.key_stride, a.nparts, (int)a.part_stride, a);      \
    return hipGetLastError();                                                        \
  }
  FH_SEL_IPT(4)
  FH_SEL_IPT(8)
  FH_SEL_IPT(16)
  FH_SEL_IPT(32)
#undef FH_SEL_IPT
  return hipErrorInvalidValue;
}

hipError_t launch_select(const SelectArgs& a, int B, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const int ipt = (a.c + kSelThreads - 1) / kSelThreads;
  const dim3 grid(B), block(kSelThreads);
  // with a union list, the events bracket both launches
  hipEvent_t es = a.ulist ? nullptr : e1;
#define FH_SEL_IPT(N)                                                                         \
  if (ipt <= N) {                                                                             \
    hipExtLaunchKernelGGL(select_kernel<N>, grid, block, 0, s, e0, es, 0, a.keys,             \
                          (int)a.key_stride, a.nparts, (int)a.part_stride, a);                \
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
