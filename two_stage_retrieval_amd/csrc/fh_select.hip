// Cluster selection (notes, Module 2): the p clusters with the largest keys,
// ties to the lower cluster id.  Keys are the stage-1 scores (greedy mode)
// or scores / tau + Gumbel noise (sampling mode: Gumbel-top-p draws p
// clusters without replacement from softmax(scores / tau)); the noise is
// added by the stage-1 kernel, so this kernel only selects.
//
// One 1024-thread workgroup per batch row; thread t owns the keys
// [t*IPT, t*IPT + IPT) in registers as order-preserving uint32 values.
//  1. block min / max of the keys;
//  2. histogram of 2048 equal-width value buckets over [min, max] in LDS
//     (the bucket index is a monotone function of the key, so bucket order
//     is key order); a block scan from the top finds the boundary bucket
//     holding the p-th largest key;
//  3. the boundary bucket is resolved exactly: by all-pairs rank when it
//     holds at most 1024 keys, else (degenerate, heavily tied inputs) by an
//     8-bit radix select on the ordered keys plus a scan for the lowest ids
//     among exact ties;
//  4. a block scan in cluster-id order writes the p ids ascending, and in
//     batched mode marks the row in each selected cluster's bitmask.
#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBuckets = 2048;
constexpr int kCandMax = 1024;

__device__ __forceinline__ float from_ordered(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// inclusive scan over the workgroup in thread order
__device__ __forceinline__ int block_incl_scan(int x, int* s_wsum, int lane, int wave) {
  const int incl = wave_incl_scan(x, lane);
  __syncthreads();
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) off += (w < wave) ? s_wsum[w] : 0;
  return incl + off;
}

template <int IPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ int s_hist[kBuckets];
  __shared__ uint32_t s_cu[kCandMax];
  __shared__ int s_ck[kCandMax];
  __shared__ uint32_t s_bits[FH_MAX_C / 32];
  __shared__ float s_fmin[kSelWaves], s_fmax[kSelWaves];
  __shared__ int s_wsum[kSelWaves];
  __shared__ int s_misc[8];

  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  const int c = a.c, p = a.p;
  const int k0 = t * IPT;
  const float* keys = a.keys + (int64_t)r * a.key_stride;

  uint32_t u[IPT];
  float lmax = -INFINITY, lmin = INFINITY;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int k = k0 + j;
    const float f = (k < c) ? keys[k] : -INFINITY;
    u[j] = ordered_u32(f);
    if (k < c) { lmax = fmaxf(lmax, f); lmin = fminf(lmin, f); }
  }
  lmax = wave_max(lmax);
  lmin = wave_min(lmin);
  if (lane == 0) { s_fmax[wave] = lmax; s_fmin[wave] = lmin; }
  for (int i = t; i < kBuckets; i += kSelThreads) s_hist[i] = 0;
  for (int i = t; i < FH_MAX_C / 32; i += kSelThreads) s_bits[i] = 0u;
  if (t < 8) s_misc[t] = 0;
  __syncthreads();
  float fmax = s_fmax[0], fmin = s_fmin[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) { fmax = fmaxf(fmax, s_fmax[w]); fmin = fminf(fmin, s_fmin[w]); }
  const float range = fmax - fmin;
  const float scale = (float)kBuckets / range;
  const bool degen = !(range > 0.0f) || !(scale < INFINITY);

  // bucket of a key: monotone non-decreasing in the key
  auto bucket_of = [&](uint32_t uu) -> int {
    const int bb = (int)((from_ordered(uu) - fmin) * scale);
    return bb < 0 ? 0 : (bb < kBuckets - 1 ? bb : kBuckets - 1);
  };

  int beta = -1, ngt = 0;
  if (!degen) {
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      if (k0 + j < c) atomicAdd(&s_hist[bucket_of(u[j])], 1);
    __syncthreads();
    // thread t owns buckets kBuckets-1-2t and kBuckets-2-2t (descending)
    const int b1 = kBuckets - 1 - 2 * t, b2 = kBuckets - 2 - 2 * t;
    const int h1 = s_hist[b1], h2 = s_hist[b2];
    const int incl = block_incl_scan(h1 + h2, s_wsum, lane, wave);
    const int excl = incl - h1 - h2;
    if (excl < p && p <= incl) {
      if (excl + h1 >= p) { s_misc[0] = b1; s_misc[1] = excl; }
      else { s_misc[0] = b2; s_misc[1] = excl + h1; }
    }
    __syncthreads();
    beta = s_misc[0];
    ngt = s_misc[1];
  }
  const int need = p - ngt;
  const int m = degen ? c : s_hist[beta];

  uint32_t candmask = 0u, chosenmask = 0u, abovemask = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    if (k0 + j >= c) continue;
    if (degen) { candmask |= 1u << j; continue; }
    const int bb = bucket_of(u[j]);
    if (bb > beta) abovemask |= 1u << j;
    else if (bb == beta) candmask |= 1u << j;
  }

  if (need == m) {
    chosenmask = candmask;
  } else if (m <= kCandMax) {
    // all-pairs rank inside the boundary bucket
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      if (candmask & (1u << j)) {
        const int pos = atomicAdd(&s_misc[2], 1);
        s_cu[pos] = u[j];
        s_ck[pos] = k0 + j;
      }
    }
    __syncthreads();
    if (t < m) {
      const uint32_t uu = s_cu[t];
      const int kk = s_ck[t];
      int rank = 0;
      for (int q = 0; q < m; ++q) {
        const uint32_t uq = s_cu[q];
        rank += (uq > uu) || (uq == uu && s_ck[q] < kk);
      }
      if (rank < need) atomicOr(&s_bits[kk >> 5], 1u << (kk & 31));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int k = k0 + j;
      if ((candmask & (1u << j)) && ((s_bits[k >> 5] >> (k & 31)) & 1u)) chosenmask |= 1u << j;
    }
  } else {
    // radix select on the ordered keys of the boundary bucket
    uint32_t prefix = 0u, pmask = 0u;
    int rem = need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      if (t < 256) s_hist[t] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < IPT; ++j)
        if ((candmask & (1u << j)) && (u[j] & pmask) == prefix)
          atomicAdd(&s_hist[(u[j] >> shift) & 255u], 1);
      __syncthreads();
      if (wave == 0) {
        int dq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) dq[q] = s_hist[255 - 4 * lane - q];
        const int cnt = dq[0] + dq[1] + dq[2] + dq[3];
        const int incl = wave_incl_scan(cnt, lane);
        int acc = incl - cnt;
        if (acc < rem && rem <= incl) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (acc + dq[q] >= rem) { s_misc[3] = 255 - 4 * lane - q; s_misc[4] = acc; break; }
            acc += dq[q];
          }
        }
      }
      __syncthreads();
      rem -= s_misc[4];
      prefix |= (uint32_t)s_misc[3] << shift;
      pmask |= 0xFFu << shift;
    }
    int ties = 0;
#pragma unroll
    for (int j = 0; j < IPT; ++j) ties += ((candmask >> j) & 1u) && u[j] == prefix;
    int run = block_incl_scan(ties, s_wsum, lane, wave) - ties;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      if (!(candmask & (1u << j))) continue;
      if (u[j] > prefix) chosenmask |= 1u << j;
      else if (u[j] == prefix) { if (run < rem) chosenmask |= 1u << j; ++run; }
    }
  }

  const uint32_t selmask = abovemask | chosenmask;
  const int cnt = __popc(selmask);
  const int incl = block_incl_scan(cnt, s_wsum, lane, wave);
  int pos = incl - cnt;
  int32_t* out = a.sel + (int64_t)r * a.sel_stride;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    if ((selmask & (1u << j)) && pos < p) {
      out[pos++] = k0 + j;
      if (a.masks) atomicOr(reinterpret_cast<unsigned long long*>(a.masks + k0 + j),
                            1ull << r);
    }
  }
  if (t == kSelThreads - 1 && incl != p && a.error) atomicOr(a.error, 1u);
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
