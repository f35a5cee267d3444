// Row-dot building blocks shared by the GEMV kernels (stage 1 at small
// batch, stage 2 gather, the dense head, and the single-launch batch-1
// decode).  A wave computes full dot products of whole rows with one hidden
// vector: lane l owns the 16-byte chunks l, l+64, ... of a row, so a wave
// reads each row as one contiguous, fully coalesced span, and keeps its
// slice of h in registers for every row it visits.
#pragma once
#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

// h (one row of H): chunk lane + 64 i of the row, raw, then unpacked.
template <int NCH>
__device__ __forceinline__ void load_h_raw(const uint8_t* hrow, int nchunk, int lane,
                                           uint4 (&hraw)[NCH]) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = lane + kWave * i;
    hraw[i] = ch < nchunk ? *reinterpret_cast<const uint4*>(hrow + (int64_t)ch * 16)
                          : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <typename TE, int NCH>
__device__ __forceinline__ void unpack_h(const uint4 (&hraw)[NCH],
                                         float (&hreg)[NCH][Chunk<TE>::kElems]) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) Chunk<TE>::unpack(hraw[i], hreg[i]);
}

template <typename TE, int NCH>
__device__ __forceinline__ void load_h(const uint8_t* hrow, int nchunk, int lane,
                                       float (&hreg)[NCH][Chunk<TE>::kElems]) {
  uint4 hraw[NCH];
  load_h_raw<NCH>(hrow, nchunk, lane, hraw);
  unpack_h<TE, NCH>(hraw, hreg);
}

// ---------------------------------------------------------------------------
// Stage 1 (notes, Overall architecture and Figure 1: inner products of h with
// the c centroids).  Key = score, or score / tau + Gumbel noise of stream 0
// keyed by the cluster id in sampling mode (Gumbel-top-p).  COHERENT stores
// the keys device-coherently for a reader in the same launch.
// ---------------------------------------------------------------------------
// The raw bits of an unwritten key for readers that poll (a NaN that no
// finite score produces).
constexpr uint32_t kKeyPending = 0xFFFFFFFFu;

// With `keys_next`, also marks the row pending in the key buffer of the next
// launch (single-launch batch-1 decode).
// With `raw`, also stores the plain score there (adaptive sampling: the
// probe count is taken on scores, the selection on keys).
template <bool COHERENT>
__device__ __forceinline__ float publish_key(const Stage1Args& a, float* keys, float* keys_next,
                                             float* dbg, uint64_t seed, int row, float score,
                                             float* raw = nullptr) {
  const float key =
      a.sample ? score * a.inv_tau + gumbel(seed, kStreamCluster, (uint32_t)row) : score;
  if constexpr (COHERENT) {
    __hip_atomic_store(keys + row, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (raw) __hip_atomic_store(raw + row, score, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    keys[row] = key;
    if (raw) raw[row] = score;
  }
  if (keys_next) keys_next[row] = __uint_as_float(kKeyPending);
  if (dbg) dbg[row] = score;
  return key;
}

// A lane's running best (key, row) as one orderable word: larger key, then
// lower row; 0 means none.
__device__ __forceinline__ void track_best_key(uint64_t* best, float key, int row) {
  if (!best) return;
  const uint64_t w = ((uint64_t)ordered_u32(key) << 32) | (0xFFFFFFFFu - (uint32_t)row);
  *best = w > *best ? w : *best;
}


constexpr int kS1Rows = 4;  // centroid rows per wave step (bf16 / fp32)

// bf16 / fp32 centroid rows: wave w0, w0 + wstride, ... take groups of 4 rows.
// h arrives raw (its loads issued by the caller) and is unpacked into hreg
// only after the first group's rows have been requested, so that neither
// waits for the other.
template <typename TE, int NCH>
__device__ __forceinline__ void load_centroid_group(const Stage1Args& a, int g, int lane,
                                                    uint4 (&data)[kS1Rows][NCH]) {
  const int row0 = g * kS1Rows;
#pragma unroll
  for (int rr = 0; rr < kS1Rows; ++rr) {
    const int row = row0 + rr < a.c ? row0 + rr : a.c - 1;
    const uint8_t* rowp = a.C + (int64_t)row * a.row_bytes;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = lane + kWave * i;
      data[rr][i] = ch < a.nchunk ? *reinterpret_cast<const uint4*>(rowp + (int64_t)ch * 16)
                                  : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// Groups g, g + wstride, ...; the rows of group g are already in `data` (if
// g < number of groups).
template <typename TE, int NCH, bool COHERENT>
__device__ __forceinline__ void score_rows_from(const Stage1Args& a, float* keys,
                                                float* keys_next, float* dbg, uint64_t seed,
                                                const uint4 (&hraw)[NCH],
                                                float (&hreg)[NCH][Chunk<TE>::kElems], int lane,
                                                int g, int wstride,
                                                uint4 (&data)[kS1Rows][NCH],
                                                uint64_t* best_key = nullptr,
                                                float* raw = nullptr) {
  using CK = Chunk<TE>;
  const int ngroups = (a.c + kS1Rows - 1) / kS1Rows;
  unpack_h<TE, NCH>(hraw, hreg);
  while (g < ngroups) {
    const int row0 = g * kS1Rows;
    float acc[kS1Rows];
#pragma unroll
    for (int rr = 0; rr < kS1Rows; ++rr) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) s = CK::dot(data[rr][i], hreg[i], s);
      acc[rr] = wave_sum(s);
    }
    float mine = acc[0];
#pragma unroll
    for (int rr = 1; rr < kS1Rows; ++rr)
      if (lane == rr) mine = acc[rr];
    if (lane < kS1Rows && row0 + lane < a.c)
      track_best_key(best_key,
                     publish_key<COHERENT>(a, keys, keys_next, dbg, seed, row0 + lane, mine, raw),
                     row0 + lane);
    g += wstride;
    if (g < ngroups) load_centroid_group<TE, NCH>(a, g, lane, data);
  }
}

template <typename TE, int NCH, bool COHERENT>
__device__ __forceinline__ void score_rows(const Stage1Args& a, float* keys, float* keys_next,
                                           float* dbg, uint64_t seed, const uint4 (&hraw)[NCH],
                                           float (&hreg)[NCH][Chunk<TE>::kElems], int lane,
                                           int w0, int wstride, float* raw = nullptr) {
  uint4 data[kS1Rows][NCH];
  if (w0 < (a.c + kS1Rows - 1) / kS1Rows) load_centroid_group<TE, NCH>(a, w0, lane, data);
  score_rows_from<TE, NCH, COHERENT>(a, keys, keys_next, dbg, seed, hraw, hreg, lane, w0,
                                     wstride, data, nullptr, raw);
}

// INT4 centroids (notes, Module 3): one 16-row group tile per wave step,
// one coalesced 1 KB load per 128-column group; lane l owns row l mod 16 and
// 32 of the group's columns; h comes from LDS (s_h, d floats).
template <bool COHERENT>
__device__ __forceinline__ void score_int4_tiles(const Stage1Args& a, float* keys,
                                                 float* keys_next, float* dbg, uint64_t seed,
                                                 const float* s_h, int lane, int w0,
                                                 int wstride, uint64_t* best_key = nullptr,
                                                 float* raw = nullptr) {
  const int q = lane >> 4, rin = lane & 15;
  const int G = a.groups;
  for (int tile = w0; tile < a.ntiles; tile += wstride) {
    const uint4* codes = reinterpret_cast<const uint4*>(a.q4) + (int64_t)tile * G * kWave + lane;
    const uint16_t* sc = a.q4s + (int64_t)tile * G * 16 + rin;
    float acc = 0.0f;
#pragma unroll 4
    for (int g = 0; g < G; ++g) {
      const uint4 w = codes[(int64_t)g * kWave];
      const float s = __uint_as_float((uint32_t)sc[g * 16] << 16);
      acc = fmaf(s, int4_dot_chunk(w, s_h + g * 128 + q * 32), acc);
    }
    acc += __shfl_xor(acc, 16, kWave);
    acc += __shfl_xor(acc, 32, kWave);
    const int row = tile * 16 + rin;
    if (q == 0 && row < a.c)
      track_best_key(best_key,
                     publish_key<COHERENT>(a, keys, keys_next, dbg, seed, row, acc, raw), row);
  }
}

// ---------------------------------------------------------------------------
// Row dots with the decode epilogue (notes, Formulas 2 and 3): stage 2 over
// the candidate rows of the selected clusters, or the dense head over all
// rows.  Each candidate's decode key is (ordered z or z / tau + G1(t)) << 32
// | ~t; the running maximum and the online log-sum-exp of z / tau stay in
// the lane that owns the row.
// ---------------------------------------------------------------------------
// `sel_row`: the batch row's selected clusters.  POLL: they are being
// published by another workgroup of the running kernel; an entry reads -1
// until it is written (bounded wait; on timeout bit 2 of *error is set).
template <bool POLL>
__device__ __forceinline__ int64_t selected_cluster(const int32_t* sel_row, int64_t j,
                                                    uint32_t* error) {
  if constexpr (!POLL) {
    return sel_row[j];
  } else {
    int32_t k = -1;
    for (int it = 0; it < kArriveSpinLimit; ++it) {
      k = __hip_atomic_load(sel_row + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (k >= 0) return k;
      __builtin_amdgcn_s_sleep(1);
    }
    if (error) atomicOr(error, 4u);
    return 0;
  }
}

// `win` (optional): entries [wlo, wlo + wn) of the selection already in
// LDS; other entries are read from sel_row.  SKIP: entries may be
// kUnusedEntry (past an adaptive probe count); their rows are skipped.
template <typename TE, int NCH, int R, int MODE, bool POLL = false, bool SKIP = false>
__device__ __forceinline__ void dot_rows(const RowdotArgs& a, int r, const int32_t* sel_row,
                                         const float (&hreg)[NCH][Chunk<TE>::kElems],
                                         uint64_t seed, int lane, int64_t w0, int64_t wstride,
                                         uint64_t& best, Lse& lse, uint32_t* error = nullptr,
                                         const int32_t* win = nullptr, int64_t wlo = 0,
                                         int64_t wn = 0) {
  using CK = Chunk<TE>;
  const int64_t ngroups = (a.nrows + R - 1) / R;
  auto entry = [&](int64_t j) -> int64_t {
    const int64_t q = j - wlo;
    if (win && q >= 0 && q < wn) return win[q];
    return selected_cluster<POLL>(sel_row, j, error);
  };
  for (int64_t g = w0; g < ngroups; g += wstride) {
    const int64_t row0 = g * R;
    int64_t phys[R];
    bool live[R];  // gather: rows of an entry past the row's probe count are not
#pragma unroll   // read or folded (their entry is kUnusedEntry)
    for (int rr = 0; rr < R; ++rr) live[rr] = true;
    if constexpr (MODE == kRowGather) {
      // candidate i is slot i mod b of selection entry i / b (candidate
      // indices fit 32 bits: there are at most v of them); one division per
      // group, and one selection entry per cluster the group touches
      const uint32_t b = (uint32_t)a.b;
      uint32_t j = (uint32_t)row0 / b;
      uint32_t slot = (uint32_t)row0 - j * b;
      int64_t k = entry(j);
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        if (rr > 0 && row0 + rr >= a.nrows) {
          phys[rr] = phys[rr - 1];  // tail: reread a row, result dropped
          live[rr] = false;
          continue;
        }
        if (rr > 0 && ++slot == b) {
          slot = 0;
          k = entry(++j);
        }
        if constexpr (SKIP) live[rr] = k >= 0 && k < a.nclusters;
        const int64_t kc = k < 0 ? 0 : (k >= a.nclusters ? a.nclusters - 1 : k);  // stay in the table
        phys[rr] = kc * (int64_t)b + slot;  // row of the cluster-major copy
      }
      if constexpr (SKIP) {
        bool any = false;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) any = any || live[rr];
        if (!any) continue;  // a group wholly past the row's probe count
      }
      if (a.borrowed) {
        // the caller's E: candidate row = token C2T[k, slot], looked up
        // before the row can be requested (lane rr fetches entry rr)
        int64_t mine = phys[0];
#pragma unroll
        for (int rr = 1; rr < R; ++rr)
          if (lane == rr) mine = phys[rr];
        const int32_t tk = lane < R ? a.c2t[mine] : 0;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) phys[rr] = (uint32_t)__builtin_amdgcn_readlane(tk, rr);
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const int64_t i = row0 + rr;
        phys[rr] = i < a.nrows ? i : a.nrows - 1;  // tail: reread the last row, result dropped
      }
    }
    uint4 data[R][NCH];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const uint8_t* rowp = a.base + phys[rr] * a.row_bytes;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ch = lane + kWave * i;
        data[rr][i] = (ch < a.nchunk) ? *reinterpret_cast<const uint4*>(rowp + (int64_t)ch * 16)
                                      : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // token ids of the rows (lane rr fetches row rr's id)
    int64_t myphys = phys[0];
#pragma unroll
    for (int rr = 1; rr < R; ++rr)
      if (lane == rr) myphys = phys[rr];
    uint32_t mytok = (uint32_t)myphys;
    if constexpr (MODE == kRowGather) {
      if (lane < R && !a.borrowed) mytok = (uint32_t)a.c2t[myphys];
    }
    float acc[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) s = CK::dot(data[rr][i], hreg[i], s);
      acc[rr] = wave_sum(s);
    }
    float mine = acc[0];
    bool mylive = live[0];
#pragma unroll
    for (int rr = 1; rr < R; ++rr)
      if (lane == rr) {
        mine = acc[rr];
        mylive = live[rr];
      }
    const int64_t myrow = row0 + lane;
    if (lane < R && myrow < a.nrows && mylive) {
      const float x = mine * a.inv_tau;
      const float kx = a.sample ? x + gumbel(seed, kStreamToken, mytok) : mine;
      const uint64_t key = decode_key(kx, mytok);
      best = key > best ? key : best;
      if (a.out_lse) lse = lse_add(lse, x);
      if (a.dbg_logits) {
        a.dbg_ids[(int64_t)r * a.dbg_stride + myrow] = (int32_t)mytok;
        a.dbg_logits[(int64_t)r * a.dbg_stride + myrow] = mine;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-workgroup decode merge.  Every workgroup folds its waves' (best, lse)
// in LDS; workgroups other than `finisher` store theirs into their own slot
// with device-scope stores, wait for them to complete and count themselves
// arrived (spread counters); the finisher, after its own share, waits for
// every arrival and folds all partials in a fixed order (deterministic),
// then writes the token and the lse.  No same-address atomics, no L2
// write-back or invalidate.  Returns true in the finisher.
// ---------------------------------------------------------------------------
template <int NT>
struct MergeSmem {
  uint64_t best[NT / kWave];
  float2 lse[NT / kWave];
};

template <int NT>
__device__ __forceinline__ bool merge_decode(const RowdotArgs& a, int r, int nblocks, int block,
                                             int finisher, uint64_t best, Lse lse,
                                             MergeSmem<NT>& ms) {
  constexpr int NW = NT / kWave;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  best = wave_max_u64(best);
  if (a.out_lse) lse = wave_lse(lse);
  if (lane == 0) {
    ms.best[wave] = best;
    ms.lse[wave] = make_float2(lse.m, lse.s);
  }
  __syncthreads();
  uint64_t* pbest = a.part_best + (int64_t)r * nblocks;
  unsigned long long* plse = reinterpret_cast<unsigned long long*>(a.lse_part + (int64_t)r * nblocks);
  uint32_t* ctr = a.counters + (int64_t)r * kArriveWords;
  uint64_t bb = ms.best[0];
  Lse ll{ms.lse[0].x, ms.lse[0].y};
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    bb = ms.best[w] > bb ? ms.best[w] : bb;
    ll = lse_merge(ll, Lse{ms.lse[w].x, ms.lse[w].y});
  }
  if (block != finisher) {
    if (t == 0) {
      __hip_atomic_store(pbest + block, bb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.out_lse) {
        const unsigned long long packed =
            ((unsigned long long)__float_as_uint(ll.s) << 32) | __float_as_uint(ll.m);
        __hip_atomic_store(plse + block, packed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0);  // the partial is visible device-wide
      arrive(ctr, block);
    }
    return false;
  }
  // finisher: wave 0 waits for the others, then folds every partial
  if (wave != 0) return true;
  wait_arrivals(ctr, nblocks - 1, lane);
  if (lane != 0) {
    bb = 0ull;
    ll = lse_empty();
  }
  for (int j = lane; j < nblocks; j += kWave) {
    if (j == finisher) continue;
    const uint64_t x = __hip_atomic_load(pbest + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bb = x > bb ? x : bb;
    if (a.out_lse) {
      const unsigned long long pr =
          __hip_atomic_load(plse + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ll = lse_merge(ll, Lse{__uint_as_float((uint32_t)pr), __uint_as_float((uint32_t)(pr >> 32))});
    }
  }
  bb = wave_max_u64(bb);
  if (a.out_lse) ll = wave_lse(ll);
  if (lane == 0) {
    a.out_tokens[r] = (int32_t)key_id(bb);
    if (a.out_lse) a.out_lse[r] = ll.m + logf(ll.s);
  }
  return true;
}

// ---------------------------------------------------------------------------
// The same merge with the data as its own flag (single-launch batch-1
// decode): workgroups other than 0 store their partial key into their slot
// of `slot` (zero = not yet written; a published key is never zero) after
// their lse partial, if any, has been performed; workgroup 0's wave 0 polls
// the slots until every one is written and folds them.  Workgroup 0 also
// clears all of `slot_next`, the set the next launch uses.  Slot j is word
// j * kSlotWords: one 128-byte line per writer.  Returns true in workgroup 0.
// ---------------------------------------------------------------------------
constexpr int kSlotWords = 16;  // u64 words per slot
template <int NT>
__device__ __forceinline__ bool merge_decode_slots(const RowdotArgs& a, int nblocks,
                                                   uint64_t* slot, uint64_t* slot_next,
                                                   unsigned long long* lse_slot, uint64_t best,
                                                   Lse lse, uint32_t* error, MergeSmem<NT>& ms) {
  constexpr int NW = NT / kWave;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  const int block = blockIdx.x;
  best = wave_max_u64(best);
  if (a.out_lse) lse = wave_lse(lse);
  if (lane == 0) {
    ms.best[wave] = best;
    ms.lse[wave] = make_float2(lse.m, lse.s);
  }
  __syncthreads();
  uint64_t bb = ms.best[0];
  Lse ll{ms.lse[0].x, ms.lse[0].y};
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    bb = ms.best[w] > bb ? ms.best[w] : bb;
    ll = lse_merge(ll, Lse{ms.lse[w].x, ms.lse[w].y});
  }
  // Workgroup 0 clears every slot of the set the next launch uses, not only
  // the slots of this launch's grid: the grid depends on p, so a slot beyond
  // it may still hold a key from two launches back.  Nothing in this launch
  // reads or writes that set.
  if (block == 0)
    for (int j = t; j < kDecodeB1MaxGrid; j += NT) slot_next[j * kSlotWords] = 0ull;
  if (block != 0) {
    if (t == 0) {
      if (a.out_lse) {
        const unsigned long long packed =
            ((unsigned long long)__float_as_uint(ll.s) << 32) | __float_as_uint(ll.m);
        __hip_atomic_store(lse_slot + block * kSlotWords, packed, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);  // the lse partial is performed before the key
      }
      __hip_atomic_store(slot + block * kSlotWords, bb ? bb : 1ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      FH_TRACE_BLOCK(4);  // partial published
    }
    return false;
  }
  if (wave != 0) return true;
  // workgroup 0, wave 0: poll every other slot until all are written
  if (lane != 0) {
    bb = 0ull;
    ll = lse_empty();
  }
  // a round issues all of a lane's pending loads before looking at any (one
  // memory round trip per round); a lane rereads only slots not yet written
  constexpr int kQ = kDecodeB1MaxGrid / kWave;
  uint64_t got = bb;
  uint32_t todo = 0u;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int j = lane + kWave * q;
    if (j != 0 && j < nblocks) todo |= 1u << q;
  }
  for (int it = 0;; ++it) {
    FH_TRACE_COUNT(1, it + 1);  // merge poll rounds
    uint64_t xs[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      xs[q] = ((todo >> q) & 1u) ? __hip_atomic_load(slot + (lane + kWave * q) * kSlotWords,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : 0ull;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (((todo >> q) & 1u) && xs[q] != 0ull) {
        todo &= ~(1u << q);
        got = xs[q] > got ? xs[q] : got;
      }
    }
    if (!__any(todo != 0u)) break;
    if (it == kArriveSpinLimit) {
      if (lane == 0 && error) atomicOr(error, 8u);
      break;
    }
  }
  bb = wave_max_u64(got);
  if (a.out_lse) {
    for (int j = lane; j < nblocks; j += kWave) {
      if (j == 0) continue;
      const unsigned long long pr = __hip_atomic_load(lse_slot + j * kSlotWords, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
      ll = lse_merge(ll, Lse{__uint_as_float((uint32_t)pr), __uint_as_float((uint32_t)(pr >> 32))});
    }
    ll = wave_lse(ll);
  }
  if (lane == 0) {
    a.out_tokens[0] = (int32_t)key_id(bb);
    if (a.out_lse) a.out_lse[0] = ll.m + logf(ll.s);
  }
  return true;
}

}  // namespace fh
