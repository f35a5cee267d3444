// Monte Carlo marginal of the two-stage head (notes, Module 4 and Formula 7):
// N independent draws S_1..S_N of the probed clusters share one stage-1
// scoring of h; draw i contributes p(v | h, S_i), the softmax of z / tau
// over the candidates of S_i (zero for a token outside them), and the
// estimate of p(v | h) is the mean over the draws.
//
// The draws share more than stage 1: a cluster's candidate logits do not
// depend on the draw, so each cluster that some draw selects is read once.
//  1. mc_select_kernel   one workgroup per draw: keys s / tau + Gumbel noise
//                        of stream 0 under the draw's seed (Gumbel-top-p, as
//                        in sampling mode), the block-level selection, and
//                        the draw's clusters flagged in the union;
//  2. mc_cluster_kernel  one wave per flagged cluster: its b candidate
//                        logits, folded into (max, sum of exp) of z / tau;
//                        clears the flag for the next call;
//  3. mc_query_kernel    one wave per query token: its exact logit and its
//                        cluster;
//  4. mc_draw_kernel     one workgroup per draw: the lse of the draw's
//                        candidates from the per-cluster pairs, then each
//                        query token's conditional probability (a binary
//                        search of its cluster in the ascending selection);
//  5. mc_reduce_kernel   one workgroup per query token: the mean over the
//                        draws, summed in a fixed order.
#include "fh_rows.h"
#include "fh_select.h"

namespace fh {

constexpr int kMcSelThreads = 1024;
constexpr int kMcThreads = 256;
constexpr int kMcWaves = kMcThreads / kWave;

// Each draw's selection is a chain of short dependent steps, so draws on one
// compute unit overlap: up to 16 keys per thread the registers are held to
// 80, six waves per SIMD (three 512-thread draws per compute unit instead
// of two; 10 000 draws at the Llama-3.2-1B head shape: 350 -> 323 us per
// estimate), without spilling.
template <int NT, int IPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(IPT <= 16 ? 6 : 1)))
void mc_select_kernel(McArgs a) {
  __shared__ SelSmem sm;
  const int i = blockIdx.x;
  const int k0 = threadIdx.x * IPT;
  uint32_t u[IPT];
  select_load_keys<IPT, false>(a.scores, (int)a.score_stride, u);
  const uint64_t seed = a.seeds[i];
#pragma unroll
  for (int j4 = 0; j4 < IPT; j4 += 4) {
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k0 + j4 < a.c) g = gumbel4(seed, kStreamCluster, (uint32_t)(k0 + j4) >> 2);
    const float gj[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (k0 + j4 + q < a.c)
        u[j4 + q] = __float_as_uint(__uint_as_float(u[j4 + q]) * a.inv_tau + gj[q]);
  }
  int32_t* out = a.sel + (int64_t)i * a.p;
  select_from_keys<NT, IPT, false>(u, a.c, a.p, a.zcut, out, nullptr, 0, a.error, sm);
  __syncthreads();  // the draw's ids are visible to the whole workgroup
  // flag the draw's clusters (plain stores of one: every writer stores the
  // same value, so no atomics)
  for (int j = threadIdx.x; j < a.p; j += NT) {
    const int32_t k = out[j];
    if (k >= 0 && k < a.c) a.flags[k] = 1u;
  }
}

// one wave per cluster: the (max, sum) pair of z / tau over its b rows
template <typename TE, int NCH, int R>
__global__ __launch_bounds__(kMcThreads) void mc_cluster_kernel(McArgs a, RowdotArgs ra) {
  __shared__ int32_t s_k[kMcWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int k = blockIdx.x * kMcWaves + wave;
  if (k >= a.c || a.flags[k] == 0u) return;  // wave-uniform
  float hreg[NCH][Chunk<TE>::kElems];
  load_h<TE, NCH>(a.H, ra.nchunk, lane, hreg);
  if (lane == 0) s_k[wave] = k;
  uint64_t best = 0;
  Lse lse = lse_empty();
  dot_rows<TE, NCH, R, kRowGather, false>(ra, 0, &s_k[wave], hreg, 0ull, lane, 0, 1, best, lse,
                                          a.error);
  lse = wave_lse(lse);
  if (lane == 0) {
    a.cl[k] = make_float2(lse.m, lse.s);
    a.flags[k] = 0u;
  }
}

// one wave per query token: its exact logit and its cluster
template <typename TE, int NCH>
__global__ __launch_bounds__(kMcThreads) void mc_query_kernel(McArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int q = blockIdx.x * kMcWaves + (threadIdx.x >> 6);
  if (q >= a.q) return;  // wave-uniform
  int32_t tok = a.tokens[q];
  if (tok < 0 || (int64_t)tok >= a.v) {
    if (lane == 0 && a.error) atomicOr(a.error, 16u);
    tok = 0;
  }
  const int32_t row = a.t2row[tok];  // its row in the cluster-major order
  float hreg[NCH][Chunk<TE>::kElems];
  load_h<TE, NCH>(a.H, a.nchunk, lane, hreg);
  const uint8_t* rowp = a.Ec + (int64_t)(a.borrowed ? tok : row) * a.row_bytes;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = lane + kWave * i;
    const uint4 w = ch < a.nchunk ? *reinterpret_cast<const uint4*>(rowp + (int64_t)ch * 16)
                                  : make_uint4(0u, 0u, 0u, 0u);
    acc = Chunk<TE>::dot(w, hreg[i], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    a.zq[q] = acc;
    a.qcl[q] = row / a.b;
  }
}

// one workgroup per draw: the draw's lse, then each query token's term
__global__ __launch_bounds__(kMcThreads) void mc_draw_kernel(McArgs a) {
  __shared__ int32_t s_sel[kMcMaxP];
  __shared__ float2 s_lse[kMcWaves];
  const int i = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  const int32_t* sel = a.sel + (int64_t)i * a.p;
  Lse l = lse_empty();
  for (int j = t; j < a.p; j += kMcThreads) {
    int32_t k = sel[j];
    k = k < 0 ? 0 : (k >= a.c ? a.c - 1 : k);
    s_sel[j] = k;
    const float2 cl = a.cl[k];
    l = lse_merge(l, Lse{cl.x, cl.y});
  }
  l = wave_lse(l);
  if (lane == 0) s_lse[wave] = make_float2(l.m, l.s);
  __syncthreads();
  Lse tot{s_lse[0].x, s_lse[0].y};
#pragma unroll
  for (int w = 1; w < kMcWaves; ++w) tot = lse_merge(tot, Lse{s_lse[w].x, s_lse[w].y});
  const float lse_i = tot.m + logf(tot.s);
  if (t == 0 && a.out_lse) a.out_lse[i] = lse_i;
  for (int q = t; q < a.q; q += kMcThreads) {
    const int32_t kq = a.qcl[q];
    int lo = 0, hi = a.p;  // the selection is ascending
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_sel[mid] < kq) lo = mid + 1;
      else hi = mid;
    }
    const bool member = lo < a.p && s_sel[lo] == kq;
    a.contrib[(int64_t)q * a.n + i] = member ? expf(a.zq[q] * a.inv_tau - lse_i) : 0.0f;
  }
}

// one workgroup per query token: the mean of its terms over the draws, in a
// fixed order (thread t sums draws t, t + 256, ... of the token's contiguous
// row; then a fixed-order DPP reduction per wave and the waves in order)
__global__ __launch_bounds__(kMcThreads) void mc_reduce_kernel(McArgs a) {
  __shared__ float s_part[kMcWaves];
  const int t = threadIdx.x;
  const int q = blockIdx.x;
  const float* row = a.contrib + (int64_t)q * a.n;
  float s = 0.0f;
  for (int i = t; i < a.n; i += kMcThreads) s += row[i];
  s = wave_sum(s);
  if ((t & (kWave - 1)) == 0) s_part[t >> 6] = s;
  __syncthreads();
  if (t == 0) {
    float tot = s_part[0];
#pragma unroll
    for (int w = 1; w < kMcWaves; ++w) tot += s_part[w];
    a.out_prob[q] = tot / (float)a.n;
  }
}

template <typename TE, int NCH>
static hipError_t launch_mc_t(const McArgs& a, const RowdotArgs& ra, hipStream_t s) {
  constexpr int R = NCH <= 2 ? 8 : 4;
  // 512-thread workgroups (16 keys per thread, up to 8192 clusters) measured
  // faster for the many independent draws than 1024-thread ones
  const int ipt512 = (a.c + 511) / 512;
  const int ipt1k = (a.c + kMcSelThreads - 1) / kMcSelThreads;
  const dim3 gsel(a.n);
  if (ipt512 <= 4) hipLaunchKernelGGL((mc_select_kernel<512, 4>), gsel, dim3(512), 0, s, a);
  else if (ipt512 <= 8) hipLaunchKernelGGL((mc_select_kernel<512, 8>), gsel, dim3(512), 0, s, a);
  else if (ipt512 <= 16) hipLaunchKernelGGL((mc_select_kernel<512, 16>), gsel, dim3(512), 0, s, a);
  else if (ipt1k <= 16) hipLaunchKernelGGL((mc_select_kernel<1024, 16>), gsel, dim3(1024), 0, s, a);
  else if (ipt1k <= 32) hipLaunchKernelGGL((mc_select_kernel<1024, 32>), gsel, dim3(1024), 0, s, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mc_cluster_kernel<TE, NCH, R>), dim3((a.c + kMcWaves - 1) / kMcWaves),
                     dim3(kMcThreads), 0, s, a, ra);
  hipLaunchKernelGGL((mc_query_kernel<TE, NCH>), dim3((a.q + kMcWaves - 1) / kMcWaves),
                     dim3(kMcThreads), 0, s, a);
  hipLaunchKernelGGL(mc_draw_kernel, dim3(a.n), dim3(kMcThreads), 0, s, a);
  hipLaunchKernelGGL(mc_reduce_kernel, dim3(a.q), dim3(kMcThreads), 0, s, a);
  return hipGetLastError();
}

template <typename TE>
static hipError_t launch_mc_nch(const McArgs& a, const RowdotArgs& ra, hipStream_t s) {
  switch ((a.nchunk + kWave - 1) / kWave) {
    case 1: return launch_mc_t<TE, 1>(a, ra, s);
    case 2: return launch_mc_t<TE, 2>(a, ra, s);
    case 3: return launch_mc_t<TE, 3>(a, ra, s);
    case 4: return launch_mc_t<TE, 4>(a, ra, s);
    case 5: return launch_mc_t<TE, 5>(a, ra, s);
    case 6: return launch_mc_t<TE, 6>(a, ra, s);
    case 7: return launch_mc_t<TE, 7>(a, ra, s);
    case 8: return launch_mc_t<TE, 8>(a, ra, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mc(const McArgs& a, const RowdotArgs& ra, int dtype, hipStream_t s) {
  if (dtype == FH_DTYPE_BF16) return launch_mc_nch<bf16_t>(a, ra, s);
  return launch_mc_nch<float>(a, ra, s);
}

}  // namespace fh
