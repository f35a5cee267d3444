// Block-level cluster selection (notes, Module 2): the p clusters with the
// largest keys, ties to the lower cluster id.  Keys are the stage-1 scores
// (greedy mode) or scores / tau + Gumbel noise (sampling mode, Gumbel-top-p:
// p draws without replacement from softmax(scores / tau)); the noise is added
// where the scores are produced, so this code only selects.
//
// Item j of thread t is cluster t + j*NT (coalesced loads).
//  1. block min / max of the keys (DPP wave reductions, one barrier);
//  2. LDS histogram of 2048 equal-width value bins over [min, max] (a
//     monotone function of the key, so bin order is key order); a block scan
//     from the top finds the boundary bin holding the p-th largest key;
//  3. the boundary bin is resolved exactly: all-pairs rank when it holds at
//     most 1024 keys, else (heavily tied keys) an 8-bit radix select on the
//     order-preserving key bits plus the lowest ids among exact ties;
//  4. the selection becomes a bitmap in cluster-id order (one ballot per 64
//     consecutive ids); a block scan of per-word popcounts gives every
//     selected cluster its rank, and the ids are written ascending.
// Block scans use DPP inside the wave and one barrier each.
#pragma once
#include "fh_device.h"
#include "fh_internal.h"

// Optional phase hook for measurement builds (empty in the library).
#ifndef FH_SEL_TRACE
#define FH_SEL_TRACE(i)
#endif

namespace fh {

constexpr int kSelBins = 2048;
constexpr int kSelCandMax = 1024;

struct SelSmem {
  int hist[kSelBins];
  uint32_t cu[kSelCandMax];
  int ck[kSelCandMax];
  uint32_t bits[FH_MAX_C / 32];  // chosen keys of the boundary bin / exact ties
  uint32_t sel[FH_MAX_C / 32];   // selection bitmap, cluster-id order
  float fmin[16], fmax[16];
  int w[2][16];                   // block-scan wave totals, alternating buffers
  int misc[8];
};

__device__ __forceinline__ float sel_from_ordered(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Inclusive scan over the workgroup in thread order with one barrier: DPP
// scan inside the wave, wave totals through one of two alternating LDS
// buffers (a buffer is rewritten only after a later barrier, so no reader
// of its previous contents remains).
template <int NT>
__device__ __forceinline__ int sel_scan(int x, SelSmem& sm, int& parity, int lane, int wave) {
  const int incl = wave_incl_scan_dpp(x);
  int* buf = sm.w[parity];
  parity ^= 1;
  if (lane == kWave - 1) buf[wave] = incl;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) off += (w < wave) ? buf[w] : 0;
  return incl + off;
}

template <bool COHERENT>
__device__ __forceinline__ float sel_load(const float* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// Selects p of the c keys; writes the ids ascending to out[0..p).  With
// `masks`, also sets bit `row` of masks[k] for every selected k.  Sets bit 0
// of *error if the selection did not produce exactly p ids.  COHERENT reads
// keys written by other workgroups of the running kernel.
template <int NT, int IPT, bool COHERENT>
__device__ void select_block(const float* keys, int c, int p, int32_t* out, uint64_t* masks,
                             int row, uint32_t* error, SelSmem& sm) {
  constexpr int NW = NT / kWave;
  constexpr int BPT = kSelBins / NT;                  // bins per thread
  constexpr int WPT = (FH_MAX_C / 32 + NT - 1) / NT;  // bitmap words per thread
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  int parity = 0;

  // ---- keys, block min / max --------------------------------------------------
  FH_SEL_TRACE(0);
  uint32_t u[IPT];
  float lmax = -INFINITY, lmin = INFINITY;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int k = t + j * NT;
    const float f = k < c ? sel_load<COHERENT>(keys + k) : -INFINITY;
    u[j] = ordered_u32(f);
    if (k < c) { lmax = fmaxf(lmax, f); lmin = fminf(lmin, f); }
  }
  for (int i = t; i < kSelBins; i += NT) sm.hist[i] = 0;
  for (int i = t; i < FH_MAX_C / 32; i += NT) { sm.bits[i] = 0u; sm.sel[i] = 0u; }
  if (t < 8) sm.misc[t] = 0;
  FH_SEL_TRACE(1);
  lmax = wave_max_dpp(lmax);
  lmin = wave_min_dpp(lmin);
  if (lane == 0) { sm.fmax[wave] = lmax; sm.fmin[wave] = lmin; }
  __syncthreads();
  FH_SEL_TRACE(2);
  float fmax = sm.fmax[0], fmin = sm.fmin[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { fmax = fmaxf(fmax, sm.fmax[w]); fmin = fminf(fmin, sm.fmin[w]); }
  const float range = fmax - fmin;
  const float scale = (float)kSelBins / range;
  const bool flat = !(range > 0.0f) || !(scale < INFINITY);
  auto bin_of = [&](uint32_t uu) -> int {
    const int b = (int)((sel_from_ordered(uu) - fmin) * scale);
    return b < 0 ? 0 : (b < kSelBins - 1 ? b : kSelBins - 1);
  };

  // ---- histogram and the boundary bin -----------------------------------------
  int beta = 0, ngt = 0;
  if (!flat) {
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      if (t + j * NT < c) atomicAdd(&sm.hist[bin_of(u[j])], 1);
    __syncthreads();
    FH_SEL_TRACE(3);
    int hb[BPT];
    int hs = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      hb[q] = sm.hist[kSelBins - 1 - t * BPT - q];  // descending bins
      hs += hb[q];
    }
    const int incl = sel_scan<NT>(hs, sm, parity, lane, wave);
    int acc = incl - hs;
    if (acc < p && p <= incl) {
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (acc + hb[q] >= p) { sm.misc[0] = kSelBins - 1 - t * BPT - q; sm.misc[1] = acc; break; }
        acc += hb[q];
      }
    }
    __syncthreads();
    beta = sm.misc[0];
    ngt = sm.misc[1];
  }
  FH_SEL_TRACE(4);
  const int need = p - ngt;
  const int m = flat ? c : sm.hist[beta];

  uint32_t candmask = 0u, abovemask = 0u, chosenmask = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    if (t + j * NT >= c) continue;
    if (flat) { candmask |= 1u << j; continue; }
    const int b = bin_of(u[j]);
    if (b > beta) abovemask |= 1u << j;
    else if (b == beta) candmask |= 1u << j;
  }

  // ---- exact resolution of the boundary bin -----------------------------------
  if (need == m) {
    chosenmask = candmask;
  } else if (m <= kSelCandMax) {
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      if (candmask & (1u << j)) {
        const int pos = atomicAdd(&sm.misc[2], 1);
        sm.cu[pos] = u[j];
        sm.ck[pos] = t + j * NT;
      }
    }
    __syncthreads();
    for (int i = t; i < m; i += NT) {
      const uint32_t uu = sm.cu[i];
      const int kk = sm.ck[i];
      int rank = 0;
      for (int q = 0; q < m; ++q) {
        const uint32_t uq = sm.cu[q];
        rank += (uq > uu) || (uq == uu && sm.ck[q] < kk);
      }
      if (rank < need) atomicOr(&sm.bits[kk >> 5], 1u << (kk & 31));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int k = t + j * NT;
      if ((candmask & (1u << j)) && ((sm.bits[k >> 5] >> (k & 31)) & 1u)) chosenmask |= 1u << j;
    }
  } else {
    // heavily tied keys: 8-bit radix select on the order-preserving bits
    uint32_t prefix = 0u, pmask = 0u;
    int rem = need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      if (t < 256) sm.hist[t] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < IPT; ++j)
        if ((candmask & (1u << j)) && (u[j] & pmask) == prefix)
          atomicAdd(&sm.hist[(u[j] >> shift) & 255u], 1);
      __syncthreads();
      if (wave == 0) {
        int dq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) dq[q] = sm.hist[255 - 4 * lane - q];
        const int cnt = dq[0] + dq[1] + dq[2] + dq[3];
        const int incl = wave_incl_scan_dpp(cnt);
        int acc = incl - cnt;
        if (acc < rem && rem <= incl) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (acc + dq[q] >= rem) { sm.misc[3] = 255 - 4 * lane - q; sm.misc[4] = acc; break; }
            acc += dq[q];
          }
        }
      }
      __syncthreads();
      rem -= sm.misc[4];
      prefix |= (uint32_t)sm.misc[3] << shift;
      pmask |= 0xFFu << shift;
    }
    // exact ties at the threshold as a bitmap in id order
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const bool tie = ((candmask >> j) & 1u) && u[j] == prefix;
      const uint64_t bal = __ballot(tie);
      const int k = j * NT + wave * kWave;  // first id of this wave's 64
      if (lane == 0 && k < c) {
        sm.bits[k >> 5] = (uint32_t)bal;
        if ((k >> 5) + 1 < FH_MAX_C / 32) sm.bits[(k >> 5) + 1] = (uint32_t)(bal >> 32);
      }
      if ((candmask & (1u << j)) && u[j] > prefix) chosenmask |= 1u << j;
    }
    __syncthreads();
    // keep the `rem` lowest tie ids
    const int words = (c + 31) >> 5;
    int wc = 0;
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int w = t * WPT + q;
      if (w < words) wc += __popc(sm.bits[w]);
    }
    int below = sel_scan<NT>(wc, sm, parity, lane, wave) - wc;
    uint32_t keep[WPT];
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int w = t * WPT + q;
      keep[q] = 0u;
      if (w >= words) continue;
      uint32_t bw = sm.bits[w];
      while (bw) {
        const int bit = __ffs(bw) - 1;
        if (below < rem) keep[q] |= 1u << bit;
        ++below;
        bw &= bw - 1u;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int w = t * WPT + q;
      if (w < words) sm.bits[w] = keep[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int k = t + j * NT;
      if ((candmask & (1u << j)) && u[j] == prefix && ((sm.bits[k >> 5] >> (k & 31)) & 1u))
        chosenmask |= 1u << j;
    }
  }
  FH_SEL_TRACE(5);

  // ---- selection bitmap in id order, ranks, ascending ids -----------------------
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const bool sj = ((abovemask | chosenmask) >> j) & 1u;
    const uint64_t bal = __ballot(sj);
    const int k = j * NT + wave * kWave;
    if (lane == 0 && k < c) {
      sm.sel[k >> 5] = (uint32_t)bal;
      if ((k >> 5) + 1 < FH_MAX_C / 32) sm.sel[(k >> 5) + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();
  FH_SEL_TRACE(6);
  const int words = (c + 31) >> 5;
  uint32_t mw[WPT];
  int wc = 0;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    const int w = t * WPT + q;
    mw[q] = w < words ? sm.sel[w] : 0u;
    wc += __popc(mw[q]);
  }
  const int incl = sel_scan<NT>(wc, sm, parity, lane, wave);
  FH_SEL_TRACE(7);
  int rank = incl - wc;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    uint32_t bw = mw[q];
    while (bw) {
      const int k = ((t * WPT + q) << 5) + __ffs(bw) - 1;
      if (rank < p) {
        out[rank] = k;
        if (masks) atomicOr(reinterpret_cast<unsigned long long*>(masks + k), 1ull << row);
      }
      ++rank;
      bw &= bw - 1u;
    }
  }
  FH_SEL_TRACE(8);
  if (t == NT - 1 && incl != p && error) atomicOr(error, 1u);
}

// The clusters whose row mask is non-zero, ascending, into ulist / ucount.
// Masks are read coherently (they were set by atomics of other workgroups).
template <int NT, int IPT>
__device__ void compact_masks_block(const uint64_t* masks, int c, int32_t* ulist, int32_t* ucount,
                                    SelSmem& sm) {
  constexpr int WPT = (FH_MAX_C / 32 + NT - 1) / NT;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  int parity = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int k = t + j * NT;
    const bool nz = k < c && __hip_atomic_load(masks + k, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) != 0ull;
    const uint64_t bal = __ballot(nz);
    const int k0 = j * NT + wave * kWave;
    if (lane == 0 && k0 < c) {
      sm.sel[k0 >> 5] = (uint32_t)bal;
      if ((k0 >> 5) + 1 < FH_MAX_C / 32) sm.sel[(k0 >> 5) + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();
  const int words = (c + 31) >> 5;
  uint32_t mw[WPT];
  int wc = 0;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    const int w = t * WPT + q;
    mw[q] = w < words ? sm.sel[w] : 0u;
    wc += __popc(mw[q]);
  }
  const int incl = sel_scan<NT>(wc, sm, parity, lane, wave);
  int pos = incl - wc;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    uint32_t bw = mw[q];
    while (bw) {
      ulist[pos++] = ((t * WPT + q) << 5) + __ffs(bw) - 1;
      bw &= bw - 1u;
    }
  }
  if (t == NT - 1) *ucount = incl;
}

}  // namespace fh
