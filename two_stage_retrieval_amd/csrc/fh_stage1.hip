// Stage 1 (notes, Overall architecture and Figure 1: inner products of h
// with the c centroids; Module 3 for INT4 centroids) fused with the cluster
// selection (Module 2).
//
// grid = (blocks, B): the blocks of batch row r score all c centroids
// against h_r.  bf16 / fp32 centroid rows: a wave reads R = 4 whole rows
// (lane l owns the 16-byte chunks l, l+64, ... of a row and keeps the
// matching slice of h in registers).  INT4 centroids: a wave reads one
// 16-row group tile per 128-column group (one coalesced 1 KB load each; lane
// l owns row l mod 16 and 32 of the group's columns), scales each group's
// integer dot product by the group's bf16 scale, and the four lanes of a row
// combine their sums.  Each key (the score, or score / tau + Gumbel noise in
// sampling mode) is stored with a coherent store.
//
// Workgroup 0 of a batch row waits, after its own share, until every other
// workgroup of the row has stored its keys (arrival counters spread over
// separate lines, see fh_device.h), then reads the row's c keys and runs the
// block-level selection, writing the p selected cluster ids in ascending
// order for stage 2.
#include "fh_rows.h"
#include "fh_select.h"

// Optional timeline hook for measurement builds (empty in the library).
#ifndef FH_S1_TRACE
#define FH_S1_TRACE(slot)
#endif
#ifndef FH_S1_WAVE_TRACE
#define FH_S1_WAVE_TRACE(wave)
#endif
#ifndef FH_S1_ISSUE_TRACE
#define FH_S1_ISSUE_TRACE(wave)
#endif
#ifndef FH_S2_WAVE_TRACE
#define FH_S2_WAVE_TRACE(wave)
#endif
#ifndef FH_S1_TRACE_END
#define FH_S1_TRACE_END()
#endif
#ifndef FH_S1_POLL_TRACE
#define FH_S1_POLL_TRACE(round)
#endif

namespace fh {

constexpr int kS1Threads = 512;
constexpr int kS1Waves = kS1Threads / kWave;
// selection entries the rows of one workgroup's first groups can touch
// (kS1Waves groups of at most 8 rows, at least one row per entry)
constexpr int kB1Window = 2 * kWave;
static_assert(kS1Waves * 8 + 1 <= kB1Window, "stage-2 entry window");

template <typename TE, int NCH, int IPT, bool INT4, bool SELECT>
__global__ __launch_bounds__(kS1Threads) void stage1_kernel(Stage1Args a) {
  __shared__ SelSmem sm;
  __shared__ float s_h[INT4 ? FH_MAX_ROW_BYTES / 2 : 1];
  const int r = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint8_t* hrow = a.H + (int64_t)r * a.h_bytes;
  FH_S1_TRACE(0);
  const uint64_t seed = a.sample ? a.seeds[r] : 0ull;
  float* keys = a.keys + (int64_t)r * a.key_stride;
  float* dbg = a.dbg_scores ? a.dbg_scores + (int64_t)r * a.c : nullptr;
  const int w0 = blockIdx.x * kS1Waves + wave, wstride = gridDim.x * kS1Waves;

  if constexpr (!INT4) {
    uint4 hraw[NCH];
    float hreg[NCH][Chunk<TE>::kElems];
    load_h_raw<NCH>(hrow, a.nchunk, lane, hraw);
    score_rows<TE, NCH, SELECT>(a, keys, nullptr, dbg, seed, hraw, hreg, lane, w0, wstride);
  } else {
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(hrow);
    for (int i = t; i < a.d; i += kS1Threads) s_h[i] = __uint_as_float((uint32_t)hb[i] << 16);
    __syncthreads();
    score_int4_tiles<SELECT>(a, keys, nullptr, dbg, seed, s_h, lane, w0, wstride);
  }
  FH_S1_TRACE(1);
  if constexpr (!SELECT) return;

  // ---- workgroup 0 of this batch row selects, once every other workgroup
  // of the row has stored its keys -----------------------------------------
  uint32_t* ctr = a.counters + (int64_t)r * kArriveWords;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's key stores have been performed
  __syncthreads();
  if (blockIdx.x != 0) {
    if (t == 0) arrive(ctr, blockIdx.x);
    return;
  }
  if (wave == 0) {
    const bool ok = wait_arrivals(ctr, gridDim.x - 1, lane);
    if (!ok && lane == 0 && a.error) atomicOr(a.error, 2u);
  }
  __syncthreads();
  FH_S1_TRACE(2);
  select_block<kS1Threads, IPT, true>(keys, a.c, (int)a.key_stride, a.p, a.zcut,
                                      a.sel + (int64_t)r * a.sel_stride, a.masks, r, a.error, sm);
  FH_S1_TRACE(3);
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
template <typename TE, int NCH, int R, int IPT, bool INT4>
__global__ __launch_bounds__(kS1Threads) void decode_b1_kernel(DecodeB1Args args) {
  __shared__ SelSmem sm;
  __shared__ float s_h[INT4 ? FH_MAX_ROW_BYTES / 2 : 1];
  __shared__ MergeSmem<kS1Threads> ms;
  __shared__ int32_t s_sel[kDecodeB1MaxP];
  const Stage1Args& a = args.s1;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int w0 = blockIdx.x * kS1Waves + wave, wstride = gridDim.x * kS1Waves;

  // ---- A: stage-1 share ----------------------------------------------------------
  // h and the wave's first centroid rows are requested before anything else
  // is waited for (the buffer set and the seed are needed only when keys
  // are stored)
  FH_S1_TRACE(0);
  // Straight-line prologue: bounds-checked buffer loads (a chunk past the
  // row, or a group past the last, reads as zero without a memory access),
  // so that the requests go out after one wait for the few arguments they
  // need, ahead of everything the rest of the kernel loads.
  float hreg[NCH][Chunk<TE>::kElems];
  uint4 hraw[NCH];
  uint4 data[kS1Rows][NCH];
  {
    const int nch2 = args.s2.nchunk;
    const __amdgpu_buffer_rsrc_t hrs = sel_rsrc(a.H, (uint32_t)nch2 * 16u);
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      hraw[i] = sel_load4<false>(hrs, (uint32_t)(lane + kWave * i) * 16u);
    if constexpr (!INT4) {
      const __amdgpu_buffer_rsrc_t crs = sel_rsrc(a.C, (uint32_t)(a.c * a.row_bytes));
      const bool have = w0 < (a.c + kS1Rows - 1) / kS1Rows;
#pragma unroll
      for (int rr = 0; rr < kS1Rows; ++rr) {
        const int row = w0 * kS1Rows + rr < a.c ? w0 * kS1Rows + rr : a.c - 1;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int ch = lane + kWave * i;
          const uint32_t off = (have && ch < a.nchunk)
                                   ? (uint32_t)(row * a.row_bytes) + (uint32_t)ch * 16u
                                   : 0xFFFFFFF0u;
          data[rr][i] = sel_load4<false>(crs, off);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    FH_S1_ISSUE_TRACE(wave);
  }
  const uint32_t epoch = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(args.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const int cur = (int)(epoch & 1u);
  float* keys = a.keys + (int64_t)cur * a.key_stride;
  float* keys_next = a.keys + (int64_t)(1 - cur) * a.key_stride;
  int32_t* sel = args.sel + (int64_t)cur * kDecodeB1MaxP;
  int32_t* sel_next = args.sel + (int64_t)(1 - cur) * kDecodeB1MaxP;
  const uint64_t seed = a.sample ? a.seeds[0] : 0ull;
  uint64_t best_key = 0;  // this lane's best (key, row), for the prefetch below
  if constexpr (!INT4) {
    score_rows_from<TE, NCH, true>(a, keys, keys_next, a.dbg_scores, seed, hraw, hreg, lane, w0,
                                   wstride, data, &best_key);
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
    score_int4_tiles<true>(a, keys, keys_next, a.dbg_scores, seed, s_h, lane, w0, wstride,
                           &best_key);
  }
  FH_S1_TRACE(1);
  FH_S1_WAVE_TRACE(wave);


  // ---- B: workgroup 0 waits for all keys, selects and publishes ------------------
  if (blockIdx.x == 0) {
    for (int i = t; i < kDecodeB1MaxP; i += kS1Threads) sel_next[i] = -1;
    select_clear<kS1Threads>(a.c, sm);  // ordered before the selection by the polls' barriers
    uint32_t u[IPT];
    const int k0 = t * IPT;
    const int nvalid = a.c - k0 < 0 ? 0 : (a.c - k0 < IPT ? a.c - k0 : IPT);
    // each wave polls its own keys (no block barrier per round); a thread
    // rereads only the 16-byte chunks that still hold a pending key
    const __amdgpu_buffer_rsrc_t krs = sel_rsrc(keys, (uint32_t)a.key_stride * 4u);
    select_load_keys<IPT, true>(keys, (int)a.key_stride, u);
    for (int it = 0;; ++it) {
      uint32_t pend = 0u;  // chunks with a pending key
#pragma unroll
      for (int j = 0; j < IPT; ++j)
        if (j < nvalid && u[j] == kKeyPending) pend |= 1u << (j / 4);
      FH_S1_POLL_TRACE(it);
      if (!__any(pend != 0u)) break;
      if (it == kArriveSpinLimit) {
        if (lane == 0 && a.error) atomicOr(a.error, 2u);
        break;
      }
      poll_barrier();
#pragma unroll
      for (int q = 0; q < IPT / 4; ++q) {
        if ((pend >> q) & 1u) {
          const uint4 v = sel_load4<true>(krs, (uint32_t)(k0 + 4 * q) * 4u);
          u[4 * q] = v.x;
          u[4 * q + 1] = v.y;
          u[4 * q + 2] = v.z;
          u[4 * q + 3] = v.w;
        }
      }
    }
    select_wave_range<IPT>(u, a.c, sm);
    __syncthreads();
    if (t == 0) {  // every key is in: the other workgroups may prefetch
      __hip_atomic_store(args.go + cur, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      args.go[1 - cur] = 0u;
    }
    FH_S1_TRACE(2);
    // the selection goes to LDS, then out in one coalesced device-coherent pass
    select_from_keys<kS1Threads, IPT, false, true>(u, a.c, a.p, a.zcut, s_sel, nullptr, 0, a.error,
                                                   sm);
    __syncthreads();
    for (int i = t; i < a.p; i += kS1Threads)
      __hip_atomic_store(sel + i, s_sel[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    FH_S1_TRACE(3);
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
      if (m != 0) {
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
    const int64_t g0 = (int64_t)blockIdx.x * kS1Waves;
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
    FH_S1_TRACE(7);
  }
  uint64_t best = 0;
  Lse lse = lse_empty();
  if (blockIdx.x == 0) {
    dot_rows<TE, NCH, R, kRowGather, true>(args.s2, 0, sel, hreg, seed, lane, w0, wstride, best,
                                           lse, a.error, s_sel, 0, a.p);
  } else {
    dot_rows<TE, NCH, R, kRowGather, true>(args.s2, 0, sel, hreg, seed, lane, w0, wstride, best,
                                           lse, a.error, s_win, wlo, wn);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no direct-to-LDS load outlives the workgroup
  FH_S2_WAVE_TRACE(wave);
  FH_S1_TRACE(5);

  // ---- D: the decode merge; workgroup 0 then advances the epoch --------------------
  uint64_t* slots = args.s2.part_best + (int64_t)cur * args.slot_stride;
  uint64_t* slots_next = args.s2.part_best + (int64_t)(1 - cur) * args.slot_stride;
  if (merge_decode_slots<kS1Threads>(args.s2, gridDim.x, slots, slots_next,
                                     reinterpret_cast<unsigned long long*>(args.s2.lse_part),
                                     best, lse, a.error, ms) &&
      t == 0) {
    __hip_atomic_store(args.epoch, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    FH_S1_TRACE(6);
  }
  FH_S1_TRACE_END();
}

int stage1_blocks(const Stage1Args& a, bool int4) {
  const int64_t units = int4 ? a.ntiles : (a.c + kS1Rows - 1) / kS1Rows;
  int64_t blocks = (units + kS1Waves - 1) / kS1Waves;
  return (int)(blocks < 1 ? 1 : blocks);
}

bool stage1_selects(int c) { return c <= kS1Threads * 32; }

template <typename TE, int NCH, bool INT4>
static hipError_t launch_nch(const Stage1Args& a, int B, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const dim3 grid(stage1_blocks(a, INT4), B), block(kS1Threads);
  if (!a.select) {
    hipExtLaunchKernelGGL((stage1_kernel<TE, NCH, 4, INT4, false>), grid, block, 0, s, e0, e1, 0,
                          a);
    return hipGetLastError();
  }
  const int ipt = (a.c + kS1Threads - 1) / kS1Threads;
#define FH_S1_IPT(N)                                                                          \
  if (ipt <= N) {                                                                             \
    hipExtLaunchKernelGGL((stage1_kernel<TE, NCH, N, INT4, true>), grid, block, 0, s, e0, e1, \
                          0, a);                                                              \
    return hipGetLastError();                                                                 \
  }
  FH_S1_IPT(4)
  FH_S1_IPT(8)
  FH_S1_IPT(16)
  FH_S1_IPT(32)
#undef FH_S1_IPT
  return hipErrorInvalidValue;
}

hipError_t launch_stage1(const Stage1Args& a, int dtype, bool int4, int B, hipStream_t s,
                         const Timing* tm) {
  if (int4) return launch_nch<bf16_t, 1, true>(a, B, s, tm);
  const int nch = (a.nchunk + kWave - 1) / kWave;
  if (dtype == FH_DTYPE_BF16) {
    switch (nch) {
      case 1: return launch_nch<bf16_t, 1, false>(a, B, s, tm);
      case 2: return launch_nch<bf16_t, 2, false>(a, B, s, tm);
      case 3: return launch_nch<bf16_t, 3, false>(a, B, s, tm);
      case 4: return launch_nch<bf16_t, 4, false>(a, B, s, tm);
      case 5: return launch_nch<bf16_t, 5, false>(a, B, s, tm);
      case 6: return launch_nch<bf16_t, 6, false>(a, B, s, tm);
      case 7: return launch_nch<bf16_t, 7, false>(a, B, s, tm);
      case 8: return launch_nch<bf16_t, 8, false>(a, B, s, tm);
      default: return hipErrorInvalidValue;
    }
  }
  switch (nch) {
    case 1: return launch_nch<float, 1, false>(a, B, s, tm);
    case 2: return launch_nch<float, 2, false>(a, B, s, tm);
    case 3: return launch_nch<float, 3, false>(a, B, s, tm);
    case 4: return launch_nch<float, 4, false>(a, B, s, tm);
    case 5: return launch_nch<float, 5, false>(a, B, s, tm);
    case 6: return launch_nch<float, 6, false>(a, B, s, tm);
    case 7: return launch_nch<float, 7, false>(a, B, s, tm);
    case 8: return launch_nch<float, 8, false>(a, B, s, tm);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// single-launch batch-1 decode
// ---------------------------------------------------------------------------
int decode_b1_grid(const DecodeB1Args& a, bool int4, int num_cu) {
  if (!stage1_selects(a.s1.c) || num_cu < 1 || a.s1.p > kDecodeB1MaxP) return 0;
  const int nch = (a.s2.nchunk + kWave - 1) / kWave;
  if (nch < 1 || nch > 8) return 0;
  const int R = nch <= 2 ? 8 : 4;
  const int64_t units1 = int4 ? a.s1.ntiles : (a.s1.c + kS1Rows - 1) / kS1Rows;
  const int64_t units2 = (a.s2.nrows + R - 1) / R;
  const int64_t units = units1 > units2 ? units1 : units2;
  int64_t g = (units + kS1Waves - 1) / kS1Waves;
  if (g > num_cu) g = num_cu;  // one resident workgroup per compute unit
  if (g > kDecodeB1MaxGrid) g = kDecodeB1MaxGrid;  // slots the merge's polling wave tracks
  return (int)(g < 1 ? 1 : g);
}

template <typename TE, int NCH, bool INT4>
static hipError_t launch_b1_nch(const DecodeB1Args& a, int grid, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1) {
  constexpr int R = NCH <= 2 ? 8 : 4;
  const int c = a.s1.c;
  const dim3 g(grid), block(kS1Threads);
  if (c <= kS1Threads * 4) {
    hipExtLaunchKernelGGL((decode_b1_kernel<TE, NCH, R, 4, INT4>), g, block, 0, s, e0, e1, 0, a);
  } else if (c <= kS1Threads * 16) {
    hipExtLaunchKernelGGL((decode_b1_kernel<TE, NCH, R, 16, INT4>), g, block, 0, s, e0, e1, 0, a);
  } else if (c <= kS1Threads * 32) {
    hipExtLaunchKernelGGL((decode_b1_kernel<TE, NCH, R, 32, INT4>), g, block, 0, s, e0, e1, 0, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TE, bool INT4>
static hipError_t launch_b1_t(const DecodeB1Args& a, int grid, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1) {
  switch ((a.s2.nchunk + kWave - 1) / kWave) {
    case 1: return launch_b1_nch<TE, 1, INT4>(a, grid, s, e0, e1);
    case 2: return launch_b1_nch<TE, 2, INT4>(a, grid, s, e0, e1);
    case 3: return launch_b1_nch<TE, 3, INT4>(a, grid, s, e0, e1);
    case 4: return launch_b1_nch<TE, 4, INT4>(a, grid, s, e0, e1);
    case 5: return launch_b1_nch<TE, 5, INT4>(a, grid, s, e0, e1);
    case 6: return launch_b1_nch<TE, 6, INT4>(a, grid, s, e0, e1);
    case 7: return launch_b1_nch<TE, 7, INT4>(a, grid, s, e0, e1);
    case 8: return launch_b1_nch<TE, 8, INT4>(a, grid, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_b1(const DecodeB1Args& a, int dtype, bool int4, int grid,
                            hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  if (int4) return launch_b1_t<bf16_t, true>(a, grid, s, e0, e1);
  if (dtype == FH_DTYPE_BF16) return launch_b1_t<bf16_t, false>(a, grid, s, e0, e1);
  return launch_b1_t<float, false>(a, grid, s, e0, e1);
}

}  // namespace fh
