// The single-launch batch-1 decode (its kernel template and launchers).
// fh_stage1.hip instantiates the plain kernels, fh_decode_b1_adapt.hip the
// ones with the adaptive probe count compiled in (ADAPT), so that the plain
// step carries none of its code and the two compile in parallel.
#pragma once
#include "fh_rows.h"
#include "fh_select.h"

namespace fh {

constexpr int kS1Threads = 512;
constexpr int kS1Waves = kS1Threads / kWave;
// selection entries the rows of one workgroup's first groups can touch
// (kS1Waves groups of at most 8 rows, at least one row per entry)
constexpr int kB1Window = 2 * kWave;
static_assert(kS1Waves * 8 + 1 <= kB1Window, "stage-2 entry window");

// ---------------------------------------------------------------------------
// Stage-1 shares of the single-launch decode.  In pass k workgroup b scores
// one contiguous run of rows (32 bf16 / fp32 rows, or 64 rows of INT4
// tiles); the scores meet in LDS (double-buffered, one barrier per pass)
// and wave 0 forms the keys and stores them as whole 128-byte lines with one
// device-coherent store, marks the same rows pending in the next launch's
// key buffer and writes the debug scores.  A line stored whole by one wave
// reaches the polling workgroup sooner than partial lines stored by several.
// ---------------------------------------------------------------------------
// One key of the pass: lane `i` of wave 0 owns row `row` (score in LDS).
// `raw` (this launch's plain-score buffer, adaptive sampling only) gets the
// score too; workgroup 0 marks it pending again once it has read it.
__device__ __forceinline__ void b1_publish_key(const Stage1Args& a, float* keys, float* keys_next,
                                               float* raw, uint64_t seed, int row, float score,
                                               uint64_t* best_key) {
  const float key =
      a.sample ? score * a.inv_tau + gumbel(seed, kStreamCluster, (uint32_t)row) : score;
  if (raw) __hip_atomic_store(raw + row, score, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(keys + row, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  keys_next[row] = __uint_as_float(kKeyPending);
  if (a.dbg_scores) a.dbg_scores[row] = score;
  track_best_key(best_key, key, row);
}

// bf16 / fp32 centroid rows: wave w scores the 4 rows of group
// (k * grid + b) * 8 + w; its first group's rows are already in `data`.
template <typename TE, int NCH>
__device__ __forceinline__ void b1_score_rows(const Stage1Args& a, float* keys, float* keys_next,
                                              float* raw, uint64_t seed,
                                              const uint4 (&hraw)[NCH],
                                              float (&hreg)[NCH][Chunk<TE>::kElems], int lane,
                                              int wave, uint4 (&data)[kS1Rows][NCH],
                                              float (*s_stage)[kS1Waves * kS1Rows],
                                              uint64_t* best_key) {
  using CK = Chunk<TE>;
  constexpr int kRun = kS1Waves * kS1Rows;  // rows per workgroup and pass
  const int ngroups = (a.c + kS1Rows - 1) / kS1Rows;
  const int wstride = gridDim.x * kS1Waves;
  unpack_h<TE, NCH>(hraw, hreg);
  for (int k = 0;; ++k) {
    const int gbase = (k * (int)gridDim.x + (int)blockIdx.x) * kS1Waves;
    if (gbase >= ngroups) break;  // the same in every wave of the workgroup
    float* st = s_stage[k & 1];
    const int g = gbase + wave;
    if (g < ngroups) {
      float acc[kS1Rows];
#pragma unroll
      for (int rr = 0; rr < kS1Rows; ++rr) {
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) sum = CK::dot(data[rr][i], hreg[i], sum);
        acc[rr] = wave_sum(sum);
      }
      float mine = acc[0];
#pragma unroll
      for (int rr = 1; rr < kS1Rows; ++rr)
        if (lane == rr) mine = acc[rr];
      if (lane < kS1Rows) st[wave * kS1Rows + lane] = mine;
      if (g + wstride < ngroups) load_centroid_group<TE, NCH>(a, g + wstride, lane, data);
    }
    __syncthreads();
    if (wave == 0 && lane < kRun) {
      const int row = gbase * kS1Rows + lane;
      if (row < a.c)
        b1_publish_key(a, keys, keys_next, raw, seed, row, st[lane], best_key);
    }
  }
}

// INT4 tiles (notes, Module 3): the two waves 2i and 2i + 1 of a workgroup
// share tile (k * grid + b) * 4 + i, each taking half of its 128-column
// groups (one coalesced 1 KB load per group, all issued before any is
// used); lane l owns row l mod 16 and 32 of a group's columns, h comes from
// LDS.  The halves' partial scores are added in LDS.
__device__ __forceinline__ void b1_score_int4(const Stage1Args& a, float* keys, float* keys_next,
                                              float* raw, uint64_t seed, const float* s_h,
                                              int lane, int wave,
                                              float (*s_part)[kS1Waves][16],
                                              uint64_t* best_key) {
  constexpr int kTilesPerPass = kS1Waves / 2;
  constexpr int kBatch = 8;  // group loads in flight per wave
  const int q = lane >> 4, rin = lane & 15;
  const int G = a.groups, Gh = (G + 1) / 2;
  const int g_lo = (wave & 1) * Gh;
  const int g_hi = g_lo + Gh < G ? g_lo + Gh : G;
  for (int k = 0;; ++k) {
    const int tbase = (k * (int)gridDim.x + (int)blockIdx.x) * kTilesPerPass;
    if (tbase >= a.ntiles) break;  // the same in every wave of the workgroup
    const int tile = tbase + (wave >> 1);
    if (tile < a.ntiles) {
      const uint4* codes =
          reinterpret_cast<const uint4*>(a.q4) + (int64_t)tile * G * kWave + lane;
      const uint16_t* sc = a.q4s + (int64_t)tile * G * 16 + rin;
      float acc = 0.0f;
      for (int g0 = g_lo; g0 < g_hi; g0 += kBatch) {
        uint4 w[kBatch];
        uint32_t sb[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          if (g0 + i < g_hi) {
            w[i] = codes[(int64_t)(g0 + i) * kWave];
            sb[i] = sc[(g0 + i) * 16];
          }
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (g0 + i < g_hi)
            acc = fmaf(__uint_as_float(sb[i] << 16),
                       int4_dot_chunk(w[i], s_h + (g0 + i) * 128 + q * 32), acc);
      }
      acc += __shfl_xor(acc, 16, kWave);
      acc += __shfl_xor(acc, 32, kWave);
      if (q == 0) s_part[k & 1][wave][rin] = acc;
    }
    __syncthreads();
    if (wave == 0) {  // lane = 16 * (tile of the pass) + row in the tile
      const int tl = tbase + (lane >> 4);
      const int row = tl * 16 + (lane & 15);
      if (tl < a.ntiles && row < a.c) {
        const int pr = lane >> 4;
        const float score = s_part[k & 1][2 * pr][lane & 15] + s_part[k & 1][2 * pr + 1][lane & 15];
        b1_publish_key(a, keys, keys_next, raw, seed, row, score, best_key);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The whole batch-1 decode step in one launch (notes, Overall architecture
// and Figure 1): one workgroup per compute unit, all resident at once.  No
// counters and no flags: the data are their own flags.
//  A  every workgroup scores its share of the centroids and stores the keys
//     device-coherently into this launch's key buffer (and marks the same
//     rows pending in the other buffer, which the next launch uses);
//  B  workgroup 0 polls the key buffer until no key is pending, runs the
//     block-level selection and publishes the p cluster ids, device-
//     coherently, into this launch's selection buffer, whose entries read -1
//     until written (it also clears the other buffer for the next launch);
//  C  every workgroup computes the exact logits of its share of the p*b
//     candidate rows, with the hidden vector still in registers, waiting
//     only for the selection entries its rows need;
//  D  partials meet in zero-initialised slots polled by workgroup 0
//     (merge_decode_slots), which finally advances the launch epoch that
//     picks the buffer sets.
// Every wait is bounded; running out of patience sets a bit of the error
// word instead of hanging.
// ---------------------------------------------------------------------------
// The values the prologue's first requests need (h, the centroid rows and
// their sizes) come as leading scalar arguments, which the dispatcher can
// preload into scalar registers before the waves start; everything else is
// read from `args`, behind those requests.
template <typename TE, int NCH, int R, int IPT, bool INT4, bool ADAPT>
__global__ __launch_bounds__(kS1Threads) void decode_b1_kernel(const uint8_t* pre_H,
                                                               const uint8_t* pre_C, int pre_c,
                                                               int pre_row_bytes, int pre_nchunk,
                                                               DecodeB1Args args) {
  __shared__ SelSmem sm;
  __shared__ float s_h[INT4 ? FH_MAX_ROW_BYTES / 2 : 1];
  __shared__ MergeSmem<kS1Threads> ms;
  __shared__ int32_t s_sel[kDecodeB1MaxP];
  __shared__ float s_stage[2][kS1Waves * kS1Rows];
  __shared__ float s_part[INT4 ? 2 : 1][kS1Waves][16];
  const Stage1Args& a = args.s1;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int w0 = blockIdx.x * kS1Waves + wave, wstride = gridDim.x * kS1Waves;

  // ---- A: stage-1 share ----------------------------------------------------------
  // h and the wave's first centroid rows are requested before anything else
  // is waited for (the buffer set and the seed are needed only when keys
  // are stored)
  FH_TRACE_BLOCK(0);  // start
  // Straight-line prologue: bounds-checked buffer loads (a chunk past the
  // row, or a group past the last, reads as zero without a memory access),
  // so that the requests go out after one wait for the few arguments they
  // need, ahead of everything the rest of the kernel loads.
  float hreg[NCH][Chunk<TE>::kElems];
  uint4 hraw[NCH];
  uint4 data[kS1Rows][NCH];
  {
    const __amdgpu_buffer_rsrc_t hrs = sel_rsrc(pre_H, (uint32_t)pre_nchunk * 16u);
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      hraw[i] = sel_load4<false>(hrs, (uint32_t)(lane + kWave * i) * 16u);
    if constexpr (!INT4) {
      const __amdgpu_buffer_rsrc_t crs = sel_rsrc(pre_C, (uint32_t)(pre_c * pre_row_bytes));
      const bool have = w0 < (pre_c + kS1Rows - 1) / kS1Rows;
#pragma unroll
      for (int rr = 0; rr < kS1Rows; ++rr) {
        const int row = w0 * kS1Rows + rr < pre_c ? w0 * kS1Rows + rr : pre_c - 1;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int ch = lane + kWave * i;
          const uint32_t off = (have && ch < pre_nchunk)
                                   ? (uint32_t)(row * pre_row_bytes) + (uint32_t)ch * 16u
                                   : 0xFFFFFFF0u;
          data[rr][i] = sel_load4<false>(crs, off);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    FH_TRACE_WAVE(0);  // stage-1 requests issued
  }
  const uint32_t epoch = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(args.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const int cur = (int)(epoch & 1u);
  float* keys = a.keys + (int64_t)cur * a.key_stride;
  float* keys_next = a.keys + (int64_t)(1 - cur) * a.key_stride;
  float* raw = (ADAPT && a.raw) ? args.raw + (int64_t)cur * a.key_stride : nullptr;
  int32_t* sel = args.sel + (int64_t)cur * kDecodeB1MaxP;
  int32_t* sel_next = args.sel + (int64_t)(1 - cur) * kDecodeB1MaxP;
  const uint64_t seed = a.sample ? a.seeds[0] : 0ull;
  uint64_t best_key = 0;  // this lane's best (key, row), for the prefetch below
  if constexpr (!INT4) {
    b1_score_rows<TE, NCH>(a, keys, keys_next, raw, seed, hraw, hreg, lane, wave, data, s_stage,
                           &best_key);
  } else {
    // h in LDS as floats for the INT4 tiles, written by wave 0 from its
    // registers (lane l holds bf16 elements 8 (l + 64 i) .. 8 (l + 64 i) + 7)
    unpack_h<TE, NCH>(hraw, hreg);
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ch = lane + kWave * i;
        if (ch < args.s2.nchunk) {
          const uint32_t wv[4] = {hraw[i].x, hraw[i].y, hraw[i].z, hraw[i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s_h[ch * 8 + 2 * e] = bf16_lo(wv[e]);
            s_h[ch * 8 + 2 * e + 1] = bf16_hi(wv[e]);
          }
        }
      }
    }
    __syncthreads();
    b1_score_int4(a, keys, keys_next, raw, seed, s_h, lane, wave, s_part, &best_key);
  }
  FH_TRACE_WAVE(1);  // stage-1 share done


  // ---- B: workgroup 0 waits for all keys, selects and publishes ------------------
  if (blockIdx.x == 0) {
    for (int i = t; i < kDecodeB1MaxP; i += kS1Threads) sel_next[i] = -1;
    select_clear<kS1Threads>(a.c, sm);  // ordered before the selection by the polls' barriers
    uint32_t u[IPT];
    const int k0 = t * IPT;
    const int nvalid = a.c - k0 < 0 ? 0 : (a.c - k0 < IPT ? a.c - k0 : IPT);
    // each wave polls its own keys (no block barrier per round); a thread
    // rereads only the 16-byte chunks that still hold a pending key
    // With 32 keys per thread, plain loads after an acquire fence (which
    // drops this compute unit's stale cache lines) bring the keys in about
    // 0.9 us sooner than device-coherent loads, which go out one 16-byte
    // request per lane; with fewer keys per thread the fence costs more than
    // it saves (measured at 8016 and 16384 clusters).
    constexpr bool kFenced = IPT >= 32;
    const __amdgpu_buffer_rsrc_t krs = sel_rsrc(keys, (uint32_t)a.key_stride * 4u);
    if (kFenced) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    select_load_keys<IPT, !kFenced>(keys, (int)a.key_stride, u);
    // adaptive sampling: the plain scores are polled beside the keys
    uint32_t us[IPT];
    const __amdgpu_buffer_rsrc_t rrs = sel_rsrc(raw ? raw : keys, (uint32_t)a.key_stride * 4u);
    if (raw) select_load_keys<IPT, !kFenced>(raw, (int)a.key_stride, us);
    for (int it = 0;; ++it) {
      uint32_t pend = 0u;  // chunks with a pending key
#pragma unroll
      for (int j = 0; j < IPT; ++j)
        if (j < nvalid && (u[j] == kKeyPending || (raw && us[j] == kKeyPending)))
          pend |= 1u << (j / 4);
      FH_TRACE_COUNT(0, it + 1);  // key poll rounds
      if (!__any(pend != 0u)) break;
      if (it == kArriveSpinLimit) {
        if (lane == 0 && a.error) atomicOr(a.error, 2u);
        break;
      }
      poll_barrier();
      if (kFenced) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      FH_TRACE_SEL(11);  // a reload round issued (the last one counts)
#pragma unroll
      for (int q = 0; q < IPT / 4; ++q) {
        if ((pend >> q) & 1u) {
          const uint4 v = sel_load4<!kFenced>(krs, (uint32_t)(k0 + 4 * q) * 4u);
          u[4 * q] = v.x;
          u[4 * q + 1] = v.y;
          u[4 * q + 2] = v.z;
          u[4 * q + 3] = v.w;
          if (raw) {
            const uint4 w = sel_load4<!kFenced>(rrs, (uint32_t)(k0 + 4 * q) * 4u);
            us[4 * q] = w.x;
            us[4 * q + 1] = w.y;
            us[4 * q + 2] = w.z;
            us[4 * q + 3] = w.w;
          }
        }
      }
    }
    FH_TRACE_BLOCK(7);  // every key in this thread's registers
    select_wave_range<IPT>(u, a.c, sm);
    __syncthreads();
    if (t == 0) {  // every key is in: the other workgroups may prefetch
      __hip_atomic_store(args.go + cur, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      args.go[1 - cur] = 0u;
    }
    FH_TRACE_BLOCK(1);  // every key seen
    int p = a.p;
    if (ADAPT && a.ad.on) {  // the adaptive count, on the plain scores
      p = raw ? adaptive_count<kS1Threads, IPT>(us, a.c, a.ad, a.p, sm)
              : adaptive_count<kS1Threads, IPT>(u, a.c, a.ad, a.p, sm);
      if (a.ad.out_p && t == 0) a.ad.out_p[0] = p;
      if (raw)  // read: pending again for the next launch that uses this set
        for (int j = 0; j < IPT; ++j)
          if (j < nvalid) raw[k0 + j] = __uint_as_float(kKeyPending);
    }
    // the selection goes to LDS and out in two coalesced device-coherent
    // passes: the clusters above the boundary bin first, then the ones taken
    // from it (stage 2 starts on the first before the second are known);
    // entries past an adaptive count read kUnusedEntry
    select_from_keys<kS1Threads, IPT, false, true>(u, a.c, p, a.zcut, s_sel, nullptr, 0, a.error,
                                                   sm, sel, (ADAPT && a.ad.on) ? a.p : 0);
    __syncthreads();  // s_sel complete for this workgroup's own stage-2 share
    FH_TRACE_BLOCK(2);  // selection published
  }

  // ---- C: stage-2 share ---------------------------------------------------------
  // While workgroup 0 selects, memory is idle.  Once it holds every key (the
  // go word), each other workgroup requests the rows of the cluster with its
  // own best key, which is very likely selected, so that stage 2 finds them
  // in the memory-side cache.  The requests are direct-to-LDS loads into a
  // scratch area nobody reads: no register waits on them.  Requesting them
  // right after stage 1 instead slows workgroup 0's key polls more than it
  // gains; two clusters per workgroup outlast the selection.
  //
  // The entries of the workgroup's first groups (one group per wave when the
  // grid covers the rows) are then fetched once, by wave 0, into LDS: one
  // coherent round trip per workgroup instead of one per wave.  Workgroup 0
  // has the whole selection in LDS already.
  __shared__ int32_t s_win[kB1Window];
  __shared__ uint64_t s_best[kS1Waves];
  __shared__ uint4 s_prefetch[kS1Waves][kWave];
  int64_t wlo = 0, wn = 0;
  if (blockIdx.x != 0) {
    const uint64_t wbest = wave_max_u64(best_key);
    if (lane == 0) s_best[wave] = wbest;
    if (wave == 0) {
      for (int it = 0;; ++it) {
        if (__hip_atomic_load(args.go + cur, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
          break;
        if (it == kArriveSpinLimit) {
          if (lane == 0 && a.error) atomicOr(a.error, 4u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    if (wave >= 1) {
      uint64_t m = 0;
#pragma unroll
      for (int w = 0; w < kS1Waves; ++w) m = s_best[w] > m ? s_best[w] : m;
      if (m != 0 && !args.s2.borrowed) {
        // waves 1 .. kS1Waves - 1 split the cluster's rows in 1 KB requests
        const int64_t k = (int64_t)(0xFFFFFFFFu - (uint32_t)m);  // < c
        const int64_t bytes = (int64_t)args.s2.b * args.s2.row_bytes;
        const uint8_t* src = args.s2.base + k * bytes;
        constexpr int kParts = kS1Waves - 1;
        const int64_t per = ((bytes + kParts - 1) / kParts + 1023) & ~(int64_t)1023;
        const int64_t lo = (int64_t)(wave - 1) * per;
        const int64_t hi = lo + per < bytes ? lo + per : bytes;
        for (int64_t off = lo; off + 1024 <= hi; off += 1024)
          __builtin_amdgcn_global_load_lds(
              (const void*)(src + off + lane * 16),
              (void __attribute__((address_space(3)))*)&s_prefetch[wave][0], 16, 0, 0);
      }
    }
    const int64_t ngroups = (args.s2.nrows + R - 1) / R;
    const int64_t g0 = (int64_t)(gridDim.x - 1 - blockIdx.x) * kS1Waves;
    if (g0 < ngroups) {
      const int64_t g1 = g0 + kS1Waves < ngroups ? g0 + kS1Waves : ngroups;
      const int64_t rend = g1 * R < args.s2.nrows ? g1 * R : args.s2.nrows;
      wlo = g0 * R / args.s2.b;
      wn = (rend - 1) / args.s2.b - wlo + 1;
    }
    if (wave == 0 && wn > 0) {
      const bool n0 = lane < wn, n1 = lane + kWave < wn;
      int32_t e0 = -1, e1 = -1;
      for (int it = 0;; ++it) {
        if (n0 && e0 < 0)
          e0 = __hip_atomic_load(sel + wlo + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n1 && e1 < 0)
          e1 = __hip_atomic_load(sel + wlo + lane + kWave, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        if (!__any((n0 && e0 < 0) || (n1 && e1 < 0))) break;
        if (it == kArriveSpinLimit) {
          if (lane == 0 && a.error) atomicOr(a.error, 4u);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (n0) s_win[lane] = e0;
      if (n1) s_win[lane + kWave] = e1;
    }
    __syncthreads();
    FH_TRACE_BLOCK(3);  // stage-2 entries in LDS
  }
  // stage-2 groups in reverse workgroup order: workgroup 0, which holds the
  // whole selection in LDS, takes the last entries of the list (the boundary
  // bin's, known last), and the last workgroups the first entries
  uint64_t best = 0;
  Lse lse = lse_empty();
  const int w2 = (int)(gridDim.x - 1 - blockIdx.x) * kS1Waves + wave;
  if (blockIdx.x == 0) {
    dot_rows<TE, NCH, R, kRowGather, true, ADAPT>(args.s2, 0, sel, hreg, seed, lane, w2, wstride,
                                                  best, lse, a.error, s_sel, 0, a.p);
  } else {
    dot_rows<TE, NCH, R, kRowGather, true, ADAPT>(args.s2, 0, sel, hreg, seed, lane, w2, wstride,
                                                  best, lse, a.error, s_win, wlo, wn);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no direct-to-LDS load outlives the workgroup
  FH_TRACE_WAVE(2);  // stage-2 share done

  // ---- D: the decode merge; workgroup 0 then advances the epoch --------------------
  uint64_t* slots = args.s2.part_best + (int64_t)cur * args.slot_stride;
  uint64_t* slots_next = args.s2.part_best + (int64_t)(1 - cur) * args.slot_stride;
  if (merge_decode_slots<kS1Threads>(args.s2, gridDim.x, slots, slots_next,
                                     reinterpret_cast<unsigned long long*>(args.s2.lse_part),
                                     best, lse, a.error, ms) &&
      t == 0) {
    __hip_atomic_store(args.epoch, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    FH_TRACE_BLOCK(5);  // token written
  }
  FH_TRACE_BLOCK(6);  // end
}

// One launch of the decode kernel.  COOPERATIVE: through the cooperative
// launch API, whose runtime guarantees that all workgroups are resident
// together (the kernel uses no grid barrier of that API; the events are then
// recorded around the launch instead of exactly at the kernel).
template <typename K>
hipError_t launch_one(K kernel, const DecodeB1Args& a, int grid, bool coop, hipStream_t s,
                             hipEvent_t e0, hipEvent_t e1) {
  const dim3 g(grid), block(kS1Threads);
  const uint8_t* H = a.s1.H;
  const uint8_t* C = a.s1.C;
  int c = a.s1.c, row_bytes = (int)a.s1.row_bytes, nchunk = a.s1.nchunk;
  if (!coop) {
    hipExtLaunchKernelGGL(kernel, g, block, 0, s, e0, e1, 0, H, C, c, row_bytes, nchunk, a);
    return hipGetLastError();
  }
  if (e0) (void)hipEventRecord(e0, s);
  DecodeB1Args copy = a;
  void* params[] = {&H, &C, &c, &row_bytes, &nchunk, &copy};
  const hipError_t e =
      hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel), g, block, params, 0, s);
  if (e != hipSuccess) return e;
  if (e1) (void)hipEventRecord(e1, s);
  return hipSuccess;
}

template <typename TE, int NCH, bool INT4, bool ADAPT>
hipError_t launch_b1_nch(const DecodeB1Args& a, int grid, bool coop, hipStream_t s,
                         hipEvent_t e0, hipEvent_t e1) {
  constexpr int R = NCH <= 2 ? 8 : 4;
  const int c = a.s1.c;
  if (c <= kS1Threads * 4)
    return launch_one(decode_b1_kernel<TE, NCH, R, 4, INT4, ADAPT>, a, grid, coop, s, e0, e1);
  if (c <= kS1Threads * 16)
    return launch_one(decode_b1_kernel<TE, NCH, R, 16, INT4, ADAPT>, a, grid, coop, s, e0, e1);
  if (c <= kS1Threads * 32)
    return launch_one(decode_b1_kernel<TE, NCH, R, 32, INT4, ADAPT>, a, grid, coop, s, e0, e1);
  return hipErrorInvalidValue;
}

template <typename TE, bool INT4, bool ADAPT>
hipError_t launch_b1_t(const DecodeB1Args& a, int grid, bool coop, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1) {
  switch ((a.s2.nchunk + kWave - 1) / kWave) {
    case 1: return launch_b1_nch<TE, 1, INT4, ADAPT>(a, grid, coop, s, e0, e1);
    case 2: return launch_b1_nch<TE, 2, INT4, ADAPT>(a, grid, coop, s, e0, e1);
    case 3: return launch_b1_nch<TE, 3, INT4, ADAPT>(a, grid, coop, s, e0, e1);
    case 4: return launch_b1_nch<TE, 4, INT4, ADAPT>(a, grid, coop, s, e0, e1);
    case 5: return launch_b1_nch<TE, 5, INT4, ADAPT>(a, grid, coop, s, e0, e1);
    case 6: return launch_b1_nch<TE, 6, INT4, ADAPT>(a, grid, coop, s, e0, e1);
    case 7: return launch_b1_nch<TE, 7, INT4, ADAPT>(a, grid, coop, s, e0, e1);
    case 8: return launch_b1_nch<TE, 8, INT4, ADAPT>(a, grid, coop, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

template <typename TE, int NCH, bool INT4, bool ADAPT>
hipError_t occ_nch(int c, int* blocks) {
  constexpr int R = NCH <= 2 ? 8 : 4;
  if (c <= kS1Threads * 4)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks, decode_b1_kernel<TE, NCH, R, 4, INT4, ADAPT>, kS1Threads, 0);
  if (c <= kS1Threads * 16)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks, decode_b1_kernel<TE, NCH, R, 16, INT4, ADAPT>, kS1Threads, 0);
  if (c <= kS1Threads * 32)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks, decode_b1_kernel<TE, NCH, R, 32, INT4, ADAPT>, kS1Threads, 0);
  return hipSuccess;  // more clusters than the single launch selects: none
}

template <typename TE, bool INT4, bool ADAPT>
hipError_t occ_t(int nchunk, int c, int* blocks) {
  switch ((nchunk + kWave - 1) / kWave) {
    case 1: return occ_nch<TE, 1, INT4, ADAPT>(c, blocks);
    case 2: return occ_nch<TE, 2, INT4, ADAPT>(c, blocks);
    case 3: return occ_nch<TE, 3, INT4, ADAPT>(c, blocks);
    case 4: return occ_nch<TE, 4, INT4, ADAPT>(c, blocks);
    case 5: return occ_nch<TE, 5, INT4, ADAPT>(c, blocks);
    case 6: return occ_nch<TE, 6, INT4, ADAPT>(c, blocks);
    case 7: return occ_nch<TE, 7, INT4, ADAPT>(c, blocks);
    case 8: return occ_nch<TE, 8, INT4, ADAPT>(c, blocks);
    default: return hipSuccess;  // rows wider than any instantiation: none
  }
}

// The kernels of one variant (ADAPT: the adaptive probe count compiled in).
template <bool ADAPT>
hipError_t decode_b1_occupancy_impl(int dtype, bool int4, int nchunk, int c, int* blocks) {
  *blocks = 0;
  if (int4) return occ_t<bf16_t, true, ADAPT>(nchunk, c, blocks);
  if (dtype == FH_DTYPE_BF16) return occ_t<bf16_t, false, ADAPT>(nchunk, c, blocks);
  return occ_t<float, false, ADAPT>(nchunk, c, blocks);
}

template <bool ADAPT>
hipError_t launch_decode_b1_impl(const DecodeB1Args& a, int dtype, bool int4, int grid, bool coop,
                                 hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  if (int4) return launch_b1_t<bf16_t, true, ADAPT>(a, grid, coop, s, e0, e1);
  if (dtype == FH_DTYPE_BF16) return launch_b1_t<bf16_t, false, ADAPT>(a, grid, coop, s, e0, e1);
  return launch_b1_t<float, false, ADAPT>(a, grid, coop, s, e0, e1);
}


}  // namespace fh
