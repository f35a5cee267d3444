// Fused single-launch decode step for one hidden vector (batch 1): stage-1
// centroid scores, cluster selection and stage-2 candidate logits with the
// decode, in one persistent grid of one workgroup per CU.
//
// What it computes is the same as the three-kernel path (notes, Overall
// architecture and Figure 1; Module 2 for the selection; Formulas 2-3 for
// the decode).  How:
//   phase 1  every wave scores R centroid rows (bf16/fp32 rows, or 16-row
//            INT4 tiles) and publishes each selection key with a coherent
//            store; each key also increments one of 4096 global histogram
//            bins.  The bins split [-bound, bound] evenly, where bound
//            bounds every key: |C_k h| <= max_k |C_k| |h|, plus the range of
//            the Gumbel noise in sampling mode.  Every block computes the
//            same bound from h, so the binning is one monotone function.
//   barrier  each block counts itself in once its stores have completed and
//            waits (bounded) for all blocks.
//   phase 2  every block selects redundantly (no second barrier): the
//            histogram gives the boundary bin; the keys in it are ranked
//            exactly (ties to the lower cluster id); a block scan over the
//            selection flags in cluster-id order gives each selected
//            cluster its rank, and the block keeps the clusters whose
//            candidate rows fall in its own rank window.
//   phase 3  each wave computes the exact logits of R candidate rows of the
//            cluster-major copy of E and keeps the best 64-bit decode key;
//            blocks merge through device atomics and the last block writes
//            the token (and the log-sum-exp in sampling mode) and resets the
//            shared state.  Two histogram buffers alternate by a device
//            epoch so the next call finds a zeroed one.
// All cross-block data move through device-scope atomics or coherent loads
// and stores; no cache write-back or invalidate is issued.
#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

constexpr int kFThreads = 512;
constexpr int kFWaves = kFThreads / kWave;
constexpr int kFBins = 4096;
constexpr int kFCandMax = 1024;
constexpr int kFR = 4;  // rows per wave step
constexpr uint64_t kSpinLimit = 1ull << 22;
constexpr int kFWin = 64;  // clusters of one block's stage-2 row window

__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Binning {
  float lo, scale;
  bool flat;
  __device__ __forceinline__ int operator()(float key) const {
    if (flat) return 0;
    const int b = (int)((key - lo) * scale);
    return b < 0 ? 0 : (b < kFBins - 1 ? b : kFBins - 1);
  }
};

// inclusive scan over the block in thread order
__device__ __forceinline__ int fblock_scan(int x, int* s_w, int lane, int wave) {
  const int incl = wave_incl_scan(x, lane);
  __syncthreads();
  if (lane == kWave - 1) s_w[wave] = incl;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) off += (w < wave) ? s_w[w] : 0;
  return incl + off;
}

template <typename TE, int NCH, int IPT, bool INT4>
__global__ __launch_bounds__(kFThreads) void fused_step_kernel(FusedArgs a) {
  using CK = Chunk<TE>;
  constexpr int EPC = CK::kElems;
  __shared__ int s_hist[kFBins];
  __shared__ uint32_t s_cu[kFCandMax];
  __shared__ int s_ck[kFCandMax];
  __shared__ uint32_t s_bits[FH_MAX_C / 32];
  __shared__ uint32_t s_sel[FH_MAX_C / 32];
  __shared__ int s_win[kFWin];
  __shared__ int s_w[kFWaves];
  __shared__ int s_misc[8];
  __shared__ uint64_t s_best[kFWaves];
  __shared__ float2 s_lse[kFThreads];
  __shared__ float s_h[INT4 ? FH_MAX_ROW_BYTES / 2 : 1];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = threadIdx.x;
  const int G = gridDim.x;
  const int gw = blockIdx.x * kFWaves + wave;  // global wave id
  const int nwaves = G * kFWaves;
  const uint64_t seed = a.sample ? a.seeds[0] : 0ull;

  // ---- h slice in registers, |h|, and the key binning -----------------------
  float hreg[NCH][EPC];
  float hss = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = lane + kWave * i;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (ch < a.nchunk) w = *reinterpret_cast<const uint4*>(a.H + (int64_t)ch * 16);
    CK::unpack(w, hreg[i]);
#pragma unroll
    for (int e = 0; e < EPC; ++e) hss = fmaf(hreg[i][e], hreg[i][e], hss);
  }
  if constexpr (INT4) {
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(a.H);
    for (int i = t; i < a.d; i += kFThreads) s_h[i] = __uint_as_float((uint32_t)hb[i] << 16);
  }
  hss = wave_sum(hss);  // identical in every wave of every block
  Binning bin;
  {
    const float bound = sqrtf(hss) * a.cmax * 1.001f * a.inv_tau + (a.sample ? 17.0f : 0.0f);
    bin.flat = !(bound > 0.0f) || !(bound < 3.0e38f);
    bin.lo = -bound;
    bin.scale = bin.flat ? 0.0f : (float)kFBins / (2.0f * bound);
  }
  const uint32_t epoch = ld_coherent(a.epoch);
  uint32_t* hist = a.hist + (epoch & 1u) * kFBins;
  uint32_t* hist_next = a.hist + ((epoch + 1u) & 1u) * kFBins;
  if constexpr (INT4) __syncthreads();

  // ---- phase 1: stage-1 keys ----------------------------------------------
  if constexpr (!INT4) {
    const int ngroups = (a.c + kFR - 1) / kFR;
    for (int g = gw; g < ngroups; g += nwaves) {
      const int row0 = g * kFR;
      uint4 data[kFR][NCH];
#pragma unroll
      for (int rr = 0; rr < kFR; ++rr) {
        const int row = row0 + rr < a.c ? row0 + rr : a.c - 1;
        const uint8_t* rowp = a.C + (int64_t)row * a.row_bytes;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int ch = lane + kWave * i;
          data[rr][i] = ch < a.nchunk ? *reinterpret_cast<const uint4*>(rowp + (int64_t)ch * 16)
                                      : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      float acc[kFR];
#pragma unroll
      for (int rr = 0; rr < kFR; ++rr) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) s = CK::dot(data[rr][i], hreg[i], s);
        acc[rr] = wave_sum(s);
      }
      float mine = acc[0];
#pragma unroll
      for (int rr = 1; rr < kFR; ++rr)
        if (lane == rr) mine = acc[rr];
      const int row = row0 + lane;
      if (lane < kFR && row < a.c) {
        const float key =
            a.sample ? mine * a.inv_tau + gumbel(seed, kStreamCluster, (uint32_t)row) : mine;
        st_coherent(a.keys + row, key);
        __hip_atomic_fetch_add(hist + bin(key), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (a.dbg_scores) a.dbg_scores[row] = mine;
      }
    }
  } else {
    const int q = lane >> 4, rin = lane & 15;
    const int Gq = a.groups;
    for (int tile = gw; tile < a.ntiles; tile += nwaves) {
      const uint4* codes = reinterpret_cast<const uint4*>(a.q4) + (int64_t)tile * Gq * kWave + lane;
      const uint16_t* sc = a.q4s + (int64_t)tile * Gq * 16 + rin;
      float acc = 0.0f;
#pragma unroll 4
      for (int g = 0; g < Gq; ++g) {
        const uint4 w = codes[(int64_t)g * kWave];
        const float s = __uint_as_float((uint32_t)sc[g * 16] << 16);
        acc = fmaf(s, int4_dot_chunk(w, s_h + g * 128 + q * 32), acc);
      }
      acc += __shfl_xor(acc, 16, kWave);
      acc += __shfl_xor(acc, 32, kWave);
      const int row = tile * 16 + rin;
      if (q == 0 && row < a.c) {
        const float key =
            a.sample ? acc * a.inv_tau + gumbel(seed, kStreamCluster, (uint32_t)row) : acc;
        st_coherent(a.keys + row, key);
        __hip_atomic_fetch_add(hist + bin(key), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (a.dbg_scores) a.dbg_scores[row] = acc;
      }
    }
  }

  // ---- grid arrival barrier -------------------------------------------------
  __builtin_amdgcn_s_waitcnt(0);  // this wave's key stores and bin increments are done
  __syncthreads();
  if (t == 0) {
    __hip_atomic_fetch_add(a.arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t spins = 0;
    while (ld_coherent(a.arrive) < (uint32_t)G) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        __hip_atomic_fetch_or(a.error, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // ---- phase 2: selection, redundantly in every block -------------------------
  for (int i = t; i < kFBins; i += kFThreads) s_hist[i] = (int)ld_coherent(hist + i);
  for (int i = t; i < FH_MAX_C / 32; i += kFThreads) { s_bits[i] = 0u; s_sel[i] = 0u; }
  if (t < 8) s_misc[t] = 0;
  // keys, coalesced: item j of thread t is cluster t + j * kFThreads
  uint32_t u[IPT];
  float fk[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int k = t + j * kFThreads;
    fk[j] = k < a.c ? ld_coherent(a.keys + k) : -INFINITY;
    u[j] = ordered_u32(fk[j]);
  }
  __syncthreads();
  constexpr int BPT = kFBins / kFThreads;  // bins per thread, descending order
  int hb[BPT];
  int hsum = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    hb[q] = s_hist[kFBins - 1 - t * BPT - q];
    hsum += hb[q];
  }
  {
    const int incl = fblock_scan(hsum, s_w, lane, wave);
    int acc = incl - hsum;
    if (acc < a.p && a.p <= incl) {
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (acc + hb[q] >= a.p) { s_misc[0] = kFBins - 1 - t * BPT - q; s_misc[1] = acc; break; }
        acc += hb[q];
      }
    }
  }
  __syncthreads();
  const int beta = s_misc[0];
  const int need = a.p - s_misc[1];
  const int m = s_hist[beta];
  uint32_t candmask = 0u, abovemask = 0u, chosenmask = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    if (t + j * kFThreads >= a.c) continue;
    const int bb = bin(fk[j]);
    if (bb > beta) abovemask |= 1u << j;
    else if (bb == beta) candmask |= 1u << j;
  }
  if (need == m) {
    chosenmask = candmask;
  } else if (m <= kFCandMax) {
    // exact rank among the keys of the boundary bin (ties: lower cluster id)
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      if (candmask & (1u << j)) {
        const int pos = atomicAdd(&s_misc[2], 1);
        s_cu[pos] = u[j];
        s_ck[pos] = t + j * kFThreads;
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
      const int k = t + j * kFThreads;
      if ((candmask & (1u << j)) && ((s_bits[k >> 5] >> (k & 31)) & 1u)) chosenmask |= 1u << j;
    }
  } else {
    // heavily tied keys: radix select on the ordered keys of the boundary bin,
    // then the lowest cluster ids among exact ties (bitmap in id order)
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
    // ties at the threshold key, as a bitmap in cluster-id order
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const bool tie = ((candmask >> j) & 1u) && u[j] == prefix;
      const uint64_t bal = __ballot(tie);
      const int k = t + j * kFThreads;
      if (lane == 0 && (k >> 5) < FH_MAX_C / 32) {
        s_bits[k >> 5] = (uint32_t)bal;
        if ((k >> 5) + 1 < FH_MAX_C / 32) s_bits[(k >> 5) + 1] = (uint32_t)(bal >> 32);
      }
      if ((candmask & (1u << j)) && u[j] > prefix) chosenmask |= 1u << j;
    }
    __syncthreads();
    // the lowest `rem` tie ids: rank each tie by the ties below it
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int k = t + j * kFThreads;
      if (!((candmask >> j) & 1u) || u[j] != prefix) continue;
      int below = 0;
      for (int w = 0; w < (k >> 5); ++w) below += __popc(s_bits[w]);
      below += __popc(s_bits[k >> 5] & ((1u << (k & 31)) - 1u));
      if (below < rem) chosenmask |= 1u << j;
    }
  }
  // selection bitmap in cluster-id order (one ballot per 64 consecutive ids)
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const bool selj = ((abovemask | chosenmask) >> j) & 1u;
    const uint64_t bal = __ballot(selj);
    const int k = j * kFThreads + wave * kWave;  // first id of this wave's 64
    if (lane == 0 && k < a.c) {
      s_sel[k >> 5] = (uint32_t)bal;
      s_sel[(k >> 5) + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();
  // ranks: thread t scans ids [t * IPT, t * IPT + IPT)
  const int id0 = t * IPT;
  uint32_t mybits = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int k = id0 + j;
    if (k < a.c && ((s_sel[k >> 5] >> (k & 31)) & 1u)) mybits |= 1u << j;
  }
  const int cnt = __popc(mybits);
  const int incl = fblock_scan(cnt, s_w, lane, wave);
  if (t == kFThreads - 1) s_misc[5] = incl;
  const int64_t nrows2 = (int64_t)a.p * a.b;
  const int64_t rows_per_block = a.rows_per_block;  // multiple of kFR
  const int64_t wrow0 = (int64_t)blockIdx.x * rows_per_block;
  const int rank_lo = (int)(wrow0 / a.b);
  {
    int rank = incl - cnt;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      if (mybits & (1u << j)) {
        const int slot = rank - rank_lo;
        if (slot >= 0 && slot < kFWin) s_win[slot] = id0 + j;
        if (blockIdx.x == 0 && a.dbg_clusters && rank < a.p) a.dbg_clusters[rank] = id0 + j;
        ++rank;
      }
    }
  }
  __syncthreads();
  if (t == 0 && blockIdx.x == 0 && s_misc[5] != a.p)
    __hip_atomic_fetch_or(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- phase 3: candidate logits and decode ----------------------------------
  // zero this block's slice of the other histogram buffer for the next call
  for (int i = blockIdx.x * kFThreads + t; i < kFBins; i += G * kFThreads) st_coherent(hist_next + i, 0u);
  uint64_t best = 0;
  Lse lse = lse_empty();
  {
    const int64_t wend = wrow0 + rows_per_block < nrows2 ? wrow0 + rows_per_block : nrows2;
    using CE = Chunk<TE>;
    for (int64_t row0 = wrow0 + (int64_t)wave * kFR; row0 < wend; row0 += (int64_t)kFWaves * kFR) {
      int64_t phys[kFR];
#pragma unroll
      for (int rr = 0; rr < kFR; ++rr) {
        int64_t i = row0 + rr < wend ? row0 + rr : wend - 1;
        const int64_t rank = i / a.b;
        int64_t k = s_win[rank - rank_lo];
        k = k < 0 ? 0 : (k >= a.c ? a.c - 1 : k);
        phys[rr] = k * a.b + (i - rank * a.b);
      }
      uint4 data[kFR][NCH];
#pragma unroll
      for (int rr = 0; rr < kFR; ++rr) {
        const uint8_t* rowp = a.Ec + phys[rr] * a.row_bytes;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int ch = lane + kWave * i;
          data[rr][i] = ch < a.nchunk ? *reinterpret_cast<const uint4*>(rowp + (int64_t)ch * 16)
                                      : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      int64_t myphys = phys[0];
#pragma unroll
      for (int rr = 1; rr < kFR; ++rr)
        if (lane == rr) myphys = phys[rr];
      const uint32_t mytok = lane < kFR ? (uint32_t)a.c2t[myphys] : 0u;
      float acc[kFR];
#pragma unroll
      for (int rr = 0; rr < kFR; ++rr) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) s = CE::dot(data[rr][i], hreg[i], s);
        acc[rr] = wave_sum(s);
      }
      float mine = acc[0];
#pragma unroll
      for (int rr = 1; rr < kFR; ++rr)
        if (lane == rr) mine = acc[rr];
      const int64_t myrow = row0 + lane;
      if (lane < kFR && myrow < wend) {
        const float x = mine * a.inv_tau;
        const float kx = a.sample ? x + gumbel(seed, kStreamToken, mytok) : mine;
        const uint64_t key = decode_key(kx, mytok);
        best = key > best ? key : best;
        if (a.out_lse) lse = lse_add(lse, x);
        if (a.dbg_logits) {
          a.dbg_ids[myrow] = (int32_t)mytok;
          a.dbg_logits[myrow] = mine;
        }
      }
    }
  }

  // ---- merge across blocks; the last block finalizes and resets -------------
  best = wave_max_u64(best);
  if (a.out_lse) lse = wave_lse(lse);
  if (lane == 0) {
    s_best[wave] = best;
    s_lse[wave] = make_float2(lse.m, lse.s);
  }
  __syncthreads();
  __shared__ int s_last;
  if (t == 0) {
    uint64_t bb = s_best[0];
    Lse ll{s_lse[0].x, s_lse[0].y};
    for (int w = 1; w < kFWaves; ++w) {
      bb = s_best[w] > bb ? s_best[w] : bb;
      ll = lse_merge(ll, Lse{s_lse[w].x, s_lse[w].y});
    }
    if (bb) __hip_atomic_fetch_max(reinterpret_cast<unsigned long long*>(a.best),
                                   (unsigned long long)bb, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    if (a.out_lse) {
      const unsigned long long packed =
          ((unsigned long long)__float_as_uint(ll.s) << 32) | __float_as_uint(ll.m);
      __hip_atomic_exchange(reinterpret_cast<unsigned long long*>(a.lse_part) + blockIdx.x,
                            packed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    const uint32_t prev =
        __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)G - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (a.out_lse) {
    Lse ll = lse_empty();
    for (int j = t; j < G; j += kFThreads) {
      const unsigned long long pr = __hip_atomic_fetch_add(
          reinterpret_cast<unsigned long long*>(a.lse_part) + j, 0ull, __ATOMIC_RELAXED,
          __HIP_MEMORY_SCOPE_AGENT);
      ll = lse_merge(ll, Lse{__uint_as_float((uint32_t)pr), __uint_as_float((uint32_t)(pr >> 32))});
    }
    s_lse[t] = make_float2(ll.m, ll.s);
    __syncthreads();
    for (int w = kFThreads / 2; w >= 1; w >>= 1) {
      if (t < w) {
        const Lse x = lse_merge(Lse{s_lse[t].x, s_lse[t].y}, Lse{s_lse[t + w].x, s_lse[t + w].y});
        s_lse[t] = make_float2(x.m, x.s);
      }
      __syncthreads();
    }
    if (t == 0) a.out_lse[0] = s_lse[0].x + logf(s_lse[0].y);
  }
  if (t == 0) {
    unsigned long long* gb = reinterpret_cast<unsigned long long*>(a.best);
    const uint64_t k = __hip_atomic_fetch_add(gb, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.out_tokens[0] = (int32_t)key_id(k);
    __hip_atomic_exchange(gb, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_exchange(a.arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_exchange(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(a.epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename TE, int NCH, bool INT4>
static hipError_t launch_ipt(const FusedArgs& a, int grid, hipStream_t s, const Timing* tm) {
  const int ipt = (a.c + kFThreads - 1) / kFThreads;
  void* args[] = {const_cast<FusedArgs*>(&a)};
  const void* fn = nullptr;
  if (ipt <= 8) fn = reinterpret_cast<const void*>(&fused_step_kernel<TE, NCH, 8, INT4>);
  else if (ipt <= 16) fn = reinterpret_cast<const void*>(&fused_step_kernel<TE, NCH, 16, INT4>);
  else if (ipt <= 32) fn = reinterpret_cast<const void*>(&fused_step_kernel<TE, NCH, 32, INT4>);
  else return hipErrorInvalidValue;
  if (tm && tm->start) {
    const hipError_t e = hipEventRecord(tm->start, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kFThreads), args, 0, s);
  if (e != hipSuccess) return e;
  if (tm && tm->stop) e = hipEventRecord(tm->stop, s);
  return e;
}

int fused_grid() {
  static int grid = 0;
  if (!grid) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    grid = cus;
  }
  return grid;
}

int64_t fused_rows_per_block(int p, int b) {
  const int grid = fused_grid();
  if (grid <= 0) return -1;
  const int64_t rows = (int64_t)p * b;
  return ((rows + grid - 1) / grid + kFR - 1) / kFR * kFR;
}

bool fused_supported(int dtype, int nchunk, int c, int quant, int p, int b) {
  const int nch = (nchunk + kWave - 1) / kWave;
  if (c > kFThreads * 32) return false;
  const int64_t rpb = fused_rows_per_block(p, b);
  if (rpb <= 0 || rpb / b + 2 > kFWin) return false;
  if (quant == FH_QUANT_INT4_G128) return dtype == FH_DTYPE_BF16 && nch <= 4;
  return nch >= 1 && nch <= 4;
}

hipError_t launch_fused(const FusedArgs& a, int dtype, int quant, hipStream_t s,
                        const Timing* tm) {
  const int grid = fused_grid();
  if (grid <= 0) return hipErrorInvalidDevice;
  const int nch = (a.nchunk + kWave - 1) / kWave;
  if (quant == FH_QUANT_INT4_G128) {
    switch (nch) {
      case 1: return launch_ipt<bf16_t, 1, true>(a, grid, s, tm);
      case 2: return launch_ipt<bf16_t, 2, true>(a, grid, s, tm);
      case 3: return launch_ipt<bf16_t, 3, true>(a, grid, s, tm);
      case 4: return launch_ipt<bf16_t, 4, true>(a, grid, s, tm);
      default: return hipErrorInvalidValue;
    }
  }
  if (dtype == FH_DTYPE_BF16) {
    switch (nch) {
      case 1: return launch_ipt<bf16_t, 1, false>(a, grid, s, tm);
      case 2: return launch_ipt<bf16_t, 2, false>(a, grid, s, tm);
      case 3: return launch_ipt<bf16_t, 3, false>(a, grid, s, tm);
      case 4: return launch_ipt<bf16_t, 4, false>(a, grid, s, tm);
      default: return hipErrorInvalidValue;
    }
  }
  switch (nch) {
    case 1: return launch_ipt<float, 1, false>(a, grid, s, tm);
    case 2: return launch_ipt<float, 2, false>(a, grid, s, tm);
    case 3: return launch_ipt<float, 3, false>(a, grid, s, tm);
    case 4: return launch_ipt<float, 4, false>(a, grid, s, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fh
