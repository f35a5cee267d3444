// Block-level cluster selection (notes, Module 2): the p clusters with the
// largest keys, ties to the lower cluster id.  Keys are the stage-1 scores
// (greedy mode) or scores / tau + Gumbel noise (sampling mode, Gumbel-top-p:
// p draws without replacement from softmax(scores / tau)); the noise is added
// where the scores are produced, so this code only selects.
//
// Thread t owns the IPT consecutive ids [t*IPT, t*IPT + IPT), read with
// 16-byte loads, so that a scan of per-thread counts is already in id order.
//  1. block min / max (and sum / sum of squares) of the keys (DPP wave
//     reductions, one barrier);
//  2. LDS histogram of 2048 equal-width value bins over [lo, max] (a
//     monotone function of the key, so bin order is key order), lo = min,
//     or a point the moments place below the p-th largest key (then the
//     keys under it skip the histogram; if it turns out to leave fewer than
//     p keys, the pass is redone with lo = min); each item's bin is
//     computed once and kept; a block scan from the top finds the boundary
//     bin holding the p-th largest key;
//  3. the boundary bin is resolved exactly.  Up to 64 keys (the usual case:
//     a handful) are gathered and wave 0 ranks each against the others in
//     (key descending, id ascending) order, taking the ones needed.  Larger
//     bins (heavily tied or skewed keys) first go through 8-bit radix passes
//     on the order-preserving key bits; keys that stay exactly equal are
//     taken lowest id first through a block scan;
//  4. each thread counts its selected ids; one block scan gives every thread
//     its output offset and the ids are written ascending.
// Block scans use DPP inside the wave and one barrier each.
#pragma once
#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

constexpr int kSelBins = 2048;
constexpr int kSelWaveMax = 64;           // boundary bins up to this size go to one wave
constexpr int32_t kCachePolicySc1 = 16;   // buffer-load cache policy: device-coherent read

struct SelSmem {
  int hist[kSelBins];
  uint32_t cu[kSelWaveMax];        // gathered boundary keys (order-preserving bits)
  int ck[kSelWaveMax];             // and their ids
  uint32_t chosen[FH_MAX_C / 32];  // ids picked inside the boundary bin (id bitmap)
  float fmin[16], fmax[16], fsum[16], fsq[16];
  int w[2][16];                    // block-scan wave totals, alternating buffers
  int misc[8];
  float amax[16];                  // adaptive count: wave maxima and counts
  int acnt[16];
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

// Buffer resource over `bytes` bytes at `base`: loads past the end read as
// zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sel_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// One 16-byte load.  COHERENT reads data that other workgroups of the
// running kernel wrote with device-scope stores.  The compiler treats these
// loads as plain reads: a loop that polls with them needs poll_barrier()
// in every round, or the reloads are merged with the first load.
template <bool COHERENT>
__device__ __forceinline__ uint4 sel_load4(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  const auto v =
      __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, COHERENT ? kCachePolicySc1 : 0);
  return __builtin_bit_cast(uint4, v);
}

// Compiler-only memory barrier (no instruction): memory may have changed,
// so loads after it are not merged with loads before it.
__device__ __forceinline__ void poll_barrier() { asm volatile("" ::: "memory"); }

// Loads this thread's IPT keys (thread t owns [t*IPT, t*IPT + IPT)) as raw
// fp32 bits.  `keys` is 16-byte aligned with room for `stride` floats
// (stride >= c, a multiple of 4); words past `stride` read as zero.
// COHERENT: the keys were written by other workgroups of the running kernel.
template <int IPT, bool COHERENT>
__device__ __forceinline__ void select_load_keys(const float* keys, int stride,
                                                 uint32_t (&u)[IPT]) {
  const int k0 = threadIdx.x * IPT;
  const __amdgpu_buffer_rsrc_t rs = sel_rsrc(keys, (uint32_t)stride * 4u);
#pragma unroll
  for (int q = 0; q < IPT / 4; ++q) {
    const uint4 v = sel_load4<COHERENT>(rs, (uint32_t)(k0 + 4 * q) * 4u);
    u[4 * q] = v.x;
    u[4 * q + 1] = v.y;
    u[4 * q + 2] = v.z;
    u[4 * q + 3] = v.w;
  }
}

// Clears what the selection accumulates into (histogram, boundary id bitmap
// words of [0, c), counters).  Needs no key, so a caller that waits for the
// keys can do it beforehand.
template <int NT>
__device__ __forceinline__ void select_clear(int c, SelSmem& sm) {
  const int t = threadIdx.x;
  for (int i = t; i < kSelBins; i += NT) sm.hist[i] = 0;
  for (int i = t; i < (c + 31) / 32; i += NT) sm.chosen[i] = 0u;
  if (t < 8) sm.misc[t] = 0;
}

// The wave's min, max, sum and sum of squares of the keys its threads own
// (raw fp32 bits; items past c are skipped) into sm.fmin / fmax / fsum /
// fsq[wave].  The sums only steer the histogram range (see below).
template <int IPT>
__device__ __forceinline__ void select_wave_range(const uint32_t (&u)[IPT], int c, SelSmem& sm) {
  const int t = threadIdx.x;
  const int k0 = t * IPT;
  const int nvalid = c - k0 < 0 ? 0 : (c - k0 < IPT ? c - k0 : IPT);
  float lmax = -INFINITY, lmin = INFINITY, lsum = 0.0f, lsq = 0.0f;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const float f = __uint_as_float(u[j]);
    if (j < nvalid) {
      lmax = fmaxf(lmax, f);
      lmin = fminf(lmin, f);
      lsum += f;
      lsq = fmaf(f, f, lsq);
    }
  }
  lmax = wave_max(lmax);
  lmin = wave_min(lmin);
  lsum = wave_sum(lsum);
  lsq = wave_sum(lsq);
  if ((t & (kWave - 1)) == 0) {
    sm.fmax[t >> 6] = lmax;
    sm.fmin[t >> 6] = lmin;
    sm.fsum[t >> 6] = lsum;
    sm.fsq[t >> 6] = lsq;
  }
}

// Selects p of the c keys held by the workgroup (raw fp32 bits in u, from
// select_load_keys); writes the ids ascending to out[0..p) (global or LDS
// memory).  COHERENT_OUT stores the ids device-coherently for readers in
// the running kernel.  With `masks`, also sets bit `row` of masks[k] for
// every selected k.  Sets bit 0 of *error (if given) when the selection did
// not produce exactly p ids.  Needs NT * IPT >= c.  PREPARED: the caller has
// run select_clear and select_wave_range on these keys, followed by a
// barrier.
//
// zcut > 0 narrows the histogram to [mean + zcut * sd, max] of the keys
// (keys below are not counted): with zcut chosen so that a normal sample
// would leave a few times p keys in that range, most keys skip the
// histogram and the bins are finer.  If fewer than p keys fall in the
// range, the histogram is redone over [min, max]; the result never depends
// on zcut.
//
// `early` (device memory, written device-coherently; out is then the LDS
// copy): the selection is published in two parts.  As soon as the boundary
// bin is known, the keys in the bins above it, all selected, are written
// ascending to out[0 .. ngt) and stored to early[0 .. ngt); the ids taken
// from the boundary bin follow, ascending, at [ngt, p).  Readers that wait
// for the entries they need start on most of them before the boundary bin
// is resolved.  Without it the p ids are ascending.
//
// p_fill > p (an adaptive count p below the call's p_fill): out[p .. p_fill)
// (and early[p .. p_fill)) are set to kUnusedEntry.
template <int NT, int IPT, bool COHERENT_OUT, bool PREPARED = false>
__device__ __forceinline__ void select_from_keys(uint32_t (&u)[IPT], int c, int p, float zcut,
                                                 int32_t* out, uint64_t* masks, int row,
                                                 uint32_t* error, SelSmem& sm,
                                                 int32_t* early = nullptr, int p_fill = 0) {
  static_assert(IPT % 4 == 0 && IPT <= 32 && (IPT & (IPT - 1)) == 0, "items per thread");
  constexpr int NW = NT / kWave;
  constexpr int BPT = kSelBins / NT;  // histogram bins per thread in the scan
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  const int k0 = t * IPT;
  const int nvalid = c - k0 < 0 ? 0 : (c - k0 < IPT ? c - k0 : IPT);
  int parity = 0;

  // ---- block min / max / moments --------------------------------------------------
  // u keeps the raw fp32 bits; the order-preserving form is made where the
  // bits themselves are compared (boundary candidates, radix passes)
  FH_TRACE_SEL(0);
  if constexpr (!PREPARED) {
    select_clear<NT>(c, sm);
    select_wave_range<IPT>(u, c, sm);
    __syncthreads();
  }
  FH_TRACE_SEL(2);
  float fmax = sm.fmax[0], fmin = sm.fmin[0], fsum = sm.fsum[0], fsq = sm.fsq[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    fmax = fmaxf(fmax, sm.fmax[w]);
    fmin = fminf(fmin, sm.fmin[w]);
    fsum += sm.fsum[w];
    fsq += sm.fsq[w];
  }
  float lo = fmin;
  if (zcut > 0.0f) {
    const float mean = fsum / (float)c;
    const float sd = sqrtf(fmaxf(fsq / (float)c - mean * mean, 0.0f));
    const float t0 = fmaf(zcut, sd, mean);
    if (t0 > fmin && t0 < fmax) lo = t0;  // false for NaN or infinite moments
  }

  // ---- histogram and the boundary bin -----------------------------------------
  // bins[j / 2] holds this thread's item bins + 1 in 16 bits each (0: below
  // the histogram's range)
  uint32_t bins[IPT / 2];
  int beta = 0, ngt = 0, nb = 0;
  for (;;) {  // at most two passes (block-uniform)
    const float range = fmax - lo;
    const float scale = (float)kSelBins / range;
    const float offset = -lo * scale;
    const bool flat =
        !(range > 0.0f) || !(scale < INFINITY) || !(offset > -INFINITY && offset < INFINITY);
    if (flat) {  // all keys equal (lo == fmin here): one bin holds all
#pragma unroll
      for (int j = 0; j < IPT / 2; ++j)
        bins[j] = (2 * j < nvalid ? 1u : 0u) | (2 * j + 1 < nvalid ? 0x10000u : 0u);
      beta = 0;
      ngt = 0;
      nb = c;
      break;
    }
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      // (f - lo) * scale as one fma: a monotone map of f, clamped to the bins
      const float f = __uint_as_float(u[j]);
      const int b = min(max((int)fmaf(f, scale, offset), 0), kSelBins - 1);
      const bool in = j < nvalid && f >= lo;
      const uint32_t bp = in ? (uint32_t)b + 1u : 0u;
      bins[j / 2] = (j & 1) ? (bins[j / 2] | (bp << 16)) : bp;
      if (in) atomicAdd(&sm.hist[b], 1);
    }
    __syncthreads();
    FH_TRACE_SEL(3);
    int hb[BPT];
    int hs = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      hb[q] = sm.hist[kSelBins - 1 - t * BPT - q];  // descending bins
      hs += hb[q];
    }
    const int incl = sel_scan<NT>(hs, sm, parity, lane, wave);
    int acc = incl - hs;
    if (t == NT - 1) sm.misc[7] = incl;  // keys in the histogram
    if (acc < p && p <= incl) {
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (acc + hb[q] >= p) {
          sm.misc[0] = kSelBins - 1 - t * BPT - q;
          sm.misc[1] = acc;
          sm.misc[2] = hb[q];
          break;
        }
        acc += hb[q];
      }
    }
    __syncthreads();
    beta = sm.misc[0];
    ngt = sm.misc[1];
    nb = sm.misc[2];
    if (sm.misc[7] >= p || lo == fmin) break;
    // fewer than p keys in the narrowed range: again over [min, max]
    lo = fmin;
    for (int i = t; i < kSelBins; i += NT) sm.hist[i] = 0;
    __syncthreads();
  }
  FH_TRACE_COUNT(2, nb);  // keys in the boundary bin
  FH_TRACE_SEL(4);
  int need = p - ngt;  // ids still to take from the boundary bin

  // (branch-free: items past c carry bin 0, below every key's)
  uint32_t above = 0u, cand = 0u;
  const uint32_t bb = (uint32_t)beta + 1u;  // the boundary bin in the stored form
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const uint32_t b = (bins[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
    above |= (uint32_t)(b > bb) << j;
    cand |= (uint32_t)(b == bb) << j;
  }
  const uint32_t first = early ? above : 0u;  // published before the boundary bin
  if (early) {  // (block-uniform)
    // each thread publishes its own ids at their ranks: consecutive threads
    // hold consecutive ranks, so a wave's stores stay mostly contiguous
    const int ca = __popc(above);
    int r = sel_scan<NT>(ca, sm, parity, lane, wave) - ca;
    for (uint32_t mm = above; mm != 0u; mm &= mm - 1u, ++r) {
      const int id = k0 + __ffs(mm) - 1;
      out[r] = id;
      __hip_atomic_store(early + r, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    FH_TRACE_SEL(12);
  }

  // ---- large boundary bin: 8-bit radix passes on the key bits -----------------
  // (block-uniform control flow: need and nb are the same in every thread)
  for (int shift = 24; need < nb && nb > kSelWaveMax && shift >= 0; shift -= 8) {
    __syncthreads();
    if (t < 256) sm.hist[t] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      if ((cand >> j) & 1u)
        atomicAdd(&sm.hist[(ordered_u32(__uint_as_float(u[j])) >> shift) & 255u], 1);
    __syncthreads();
    if (wave == 0) {
      int dq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) dq[q] = sm.hist[255 - 4 * lane - q];
      const int cnt = dq[0] + dq[1] + dq[2] + dq[3];
      const int incl = wave_incl_scan_dpp(cnt);
      int acc = incl - cnt;
      if (acc < need && need <= incl) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (acc + dq[q] >= need) {
            sm.misc[3] = 255 - 4 * lane - q;
            sm.misc[4] = acc;
            sm.misc[5] = dq[q];
            break;
          }
          acc += dq[q];
        }
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)sm.misc[3];
    need -= sm.misc[4];
    nb = sm.misc[5];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      if (!((cand >> j) & 1u)) continue;
      const uint32_t dj = (ordered_u32(__uint_as_float(u[j])) >> shift) & 255u;
      if (dj > digit) {
        above |= 1u << j;
        cand &= ~(1u << j);
      } else if (dj < digit) {
        cand &= ~(1u << j);
      }
    }
  }

  if (need >= nb) {
    above |= cand;  // the whole boundary set is taken
  } else if (nb <= kSelWaveMax) {
    // ---- gather the boundary keys; wave 0 picks `need` of them ---------------
    // (few threads hold a candidate: the others skip the per-item loop)
    const int cc = __popc(cand);
    const int wincl = wave_incl_scan_dpp(cc);
    int base = 0;
    if (lane == kWave - 1 && wincl > 0) base = atomicAdd(&sm.misc[6], wincl);
    base = __shfl(base, kWave - 1, kWave) + wincl - cc;
    FH_TRACE_SEL(8);
    if (cand) {
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        if ((cand >> j) & 1u) {
          sm.cu[base] = ordered_u32(__uint_as_float(u[j]));
          sm.ck[base] = k0 + j;
          ++base;
        }
      }
    }
    __syncthreads();
    FH_TRACE_SEL(9);
    if (wave == 0) {
      // each candidate's rank in (key descending, id ascending); the `need`
      // first are taken (candidate j is read from lane j's registers)
      const bool live = lane < nb;
      const uint32_t uu = live ? sm.cu[lane] : 0u;
      const uint32_t kk = live ? (uint32_t)sm.ck[lane] : 0u;
      int rank = 0;
      for (int j = 0; j < nb; ++j) {
        const uint32_t uj = (uint32_t)__builtin_amdgcn_readlane((int)uu, j);
        const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)kk, j);
        rank += (uj > uu || (uj == uu && kj < kk)) ? 1 : 0;
      }
      if (live && rank < need) atomicOr(&sm.chosen[kk >> 5], 1u << (kk & 31));
    }
    __syncthreads();
    FH_TRACE_SEL(10);
    // the thread's ids [k0, k0 + IPT) lie in one word of the bitmap (IPT is
    // a power of two up to 32 and k0 a multiple of it)
    if (cand) above |= cand & (sm.chosen[k0 >> 5] >> (k0 & 31));
  } else {
    // ---- more than kSelWaveMax exactly equal keys: lowest ids first ----------
    const int cc = __popc(cand);
    int r = sel_scan<NT>(cc, sm, parity, lane, wave) - cc;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      if ((cand >> j) & 1u) {
        if (r < need) above |= 1u << j;
        ++r;
      }
    }
  }
  FH_TRACE_SEL(5);

  // ---- ascending ids -------------------------------------------------------------
  // (with `early`: the boundary bin's ids, after the ngt already published)
  const uint32_t rest = above & ~first;
  const int cnt = __popc(rest);
  const int incl = sel_scan<NT>(cnt, sm, parity, lane, wave) + (early ? ngt : 0);
  FH_TRACE_SEL(6);
  // one step per selected id of the thread, lowest first
  int rank = incl - cnt;
  for (uint32_t m = rest; m != 0u && rank < p; m &= m - 1u, ++rank) {
    const int k = k0 + __ffs(m) - 1;
    if constexpr (COHERENT_OUT) {
      __hip_atomic_store(out + rank, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      out[rank] = k;
    }
    if (masks) atomicOr(reinterpret_cast<unsigned long long*>(masks + k), 1ull << row);
  }
  for (int i = p + t; i < p_fill; i += NT) {  // entries past an adaptive count
    if constexpr (COHERENT_OUT) {
      __hip_atomic_store(out + i, kUnusedEntry, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      out[i] = kUnusedEntry;
    }
  }
  if (early) {
    __syncthreads();
    for (int i = ngt + t; i < p; i += NT)
      __hip_atomic_store(early + i, out[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = p + t; i < p_fill; i += NT)
      __hip_atomic_store(early + i, kUnusedEntry, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  FH_TRACE_SEL(7);
  if (t == NT - 1 && incl != p && error) atomicOr(error, 1u);
}

// ---------------------------------------------------------------------------
// The adaptive probe count of one row (reading of the notes' "Potential
// improvements": fewer probes for easy tokens, more for hard ones; the rule
// is the design's): every cluster whose score s satisfies
//   s * rt >= max_k (s_k * rt) - L,   rt = 1 / tau, L = ln(1 / eps),
// that is every cluster whose softmax weight at temperature tau is at least
// eps times the largest, counts; the count is clamped to [p_min, p_max].
// `us` holds the row's plain scores as thread t owns them (raw fp32 bits,
// ids [t * IPT, t * IPT + IPT)).  Two barriers; the result is the same in
// every thread.
// ---------------------------------------------------------------------------
template <int NT, int IPT>
__device__ __forceinline__ int adaptive_count(const uint32_t (&us)[IPT], int c, const Adaptive& ad,
                                              int p_max, SelSmem& sm) {
  constexpr int NW = NT / kWave;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  const int k0 = t * IPT;
  const int nvalid = c - k0 < 0 ? 0 : (c - k0 < IPT ? c - k0 : IPT);
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < IPT; ++j)
    if (j < nvalid) mx = fmaxf(mx, __uint_as_float(us[j]) * ad.rt);
  mx = wave_max(mx);
  if (lane == 0) sm.amax[wave] = mx;
  __syncthreads();
  float m = sm.amax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, sm.amax[w]);
  const float thr = m - ad.L;
  uint32_t n = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j)
    n += (j < nvalid && __uint_as_float(us[j]) * ad.rt >= thr) ? 1u : 0u;
  n = wave_sum_u32(n);
  if (lane == 0) sm.acnt[wave] = (int)n;
  __syncthreads();
  int tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) tot += sm.acnt[w];
  return tot < ad.p_min ? ad.p_min : (tot > p_max ? p_max : tot);
}

// Loads the keys and selects (see select_load_keys / select_from_keys).
template <int NT, int IPT, bool COHERENT>
__device__ __forceinline__ void select_block(const float* keys, int c, int stride, int p,
                                             float zcut, int32_t* out, uint64_t* masks, int row,
                                             uint32_t* error, SelSmem& sm) {
  uint32_t u[IPT];
  select_load_keys<IPT, COHERENT>(keys, stride, u);
  select_from_keys<NT, IPT, COHERENT>(u, c, p, zcut, out, masks, row, error, sm);
}

// The clusters whose row mask is non-zero, ascending, into ulist / ucount.
// Masks are read coherently (they were set by atomics of other workgroups);
// thread t owns the IPT consecutive clusters [t*IPT, t*IPT + IPT).  `masks`
// is 16-byte aligned with room for c rounded up to even entries.
template <int NT, int IPT>
__device__ void compact_masks_block(const uint64_t* masks, int c, int32_t* ulist, int32_t* ucount,
                                    SelSmem& sm) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  const int k0 = t * IPT;
  int parity = 0;
  const __amdgpu_buffer_rsrc_t rs = sel_rsrc(masks, (uint32_t)((c + 1) & ~1) * 8u);
  uint32_t nz = 0u;
#pragma unroll
  for (int q = 0; q < IPT / 2; ++q) {
    const uint4 v = sel_load4<true>(rs, (uint32_t)(k0 + 2 * q) * 8u);
    if ((v.x | v.y) && k0 + 2 * q < c) nz |= 1u << (2 * q);
    if ((v.z | v.w) && k0 + 2 * q + 1 < c) nz |= 1u << (2 * q + 1);
  }
  const int cnt = __popc(nz);
  const int incl = sel_scan<NT>(cnt, sm, parity, lane, wave);
  int pos = incl - cnt;
#pragma unroll
  for (int j = 0; j < IPT; ++j)
    if ((nz >> j) & 1u) ulist[pos++] = k0 + j;
  if (t == NT - 1) *ucount = incl;
}

}  // namespace fh
