// Batched decode steps (B rows per call) on the matrix cores.
//
// Stage 1 at batch is the product S = C H^T (notes, Figure 1: inner products
// of every hidden vector with the c centroids), a GEMM with M = c, N = B,
// K = d that reads C once; stage 2 (notes, Overall architecture) computes
// exact logits of the candidate rows.  With the configs' independent hidden
// vectors the union of the rows' selected clusters covers most of the
// vocabulary, so stage 2 reads each selected cluster once (deduplicated
// across the batch) and computes its logits for all B rows, keeping those
// of the rows that selected it (a per-cluster bitmask of rows).
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l feeds row l mod 16 of A and
// column l mod 16 of B with the 8 values of k-slice l div 16, and receives
// D[4 (l div 16) + q][l mod 16], q = 0..3.  Any fixed assignment of actual
// k indices to (slice, element) works as long as A and B use the same one;
// here lane l's 16-byte load from a row covers k = 32 s + 8 (l div 16) +
// [0, 8) at step s, so every load is a contiguous 16-byte piece of a row.
#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// stage 1, INT4 centroids (notes, Module 3).  One 16-row group tile per wave;
// per 128-column group the wave runs 4 MFMA steps on the codes (small
// integers are exact in bf16) into a fresh accumulator, then adds
// scale[row, g] times it to the row's total.
// ---------------------------------------------------------------------------
constexpr int kS1qThreads = 256;

__device__ __forceinline__ uint32_t int4_pair_bf16(uint32_t w, int i) {
  // codes i and i+1 of the word as two bf16 (exact), low half first
  const uint32_t lo = __float_as_uint(int4_at(w, i)) >> 16;
  const uint32_t hi = __float_as_uint(int4_at(w, i + 1)) & 0xFFFF0000u;
  return lo | hi;
}

template <int NT>
__global__ __launch_bounds__(kS1qThreads) void stage1_int4_mfma_kernel(Stage1Args a, int B) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = lane >> 4, lr = lane & 15;
  const uint8_t* hp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int j = nt * 16 + lr;
    j = j < B ? j : B - 1;
    hp[nt] = a.H + (int64_t)j * a.h_bytes + (int64_t)(32 * slice) * 2;
  }
  const int tile = blockIdx.x * (kS1qThreads / kWave) + wave;
  if (tile >= a.ntiles) return;
  const int G = a.groups;
  const uint4* codes = reinterpret_cast<const uint4*>(a.q4) + (int64_t)tile * G * kWave + lane;
  f32x4_t tot[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) tot[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < G; ++g) {
    const uint4 w = codes[(int64_t)g * kWave];
    // scales of the 4 output rows of this lane: 4 (l div 16) + q
    const uint2 sc2 = *reinterpret_cast<const uint2*>(a.q4s + ((int64_t)tile * G + g) * 16 + 4 * slice);
    const float sc[4] = {__uint_as_float(sc2.x << 16), __uint_as_float(sc2.x & 0xFFFF0000u),
                         __uint_as_float(sc2.y << 16), __uint_as_float(sc2.y & 0xFFFF0000u)};
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    f32x4_t part[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) part[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // lane's codes for this step: columns 128 g + 32 slice + 8 s + [0, 8)
      const uint4 av = make_uint4(int4_pair_bf16(ws[s], 0), int4_pair_bf16(ws[s], 2),
                                  int4_pair_bf16(ws[s], 4), int4_pair_bf16(ws[s], 6));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint4 bv = *reinterpret_cast<const uint4*>(hp[nt] + (int64_t)(128 * g + 8 * s) * 2);
        part[nt] = mfma_bf16(av, bv, part[nt]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[nt][q] = fmaf(sc[q], part[nt][q], tot[nt][q]);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + lr;
    if (r >= B) continue;
    // the lane's 4 consecutive clusters share one Philox block
    const int kq0 = tile * 16 + 4 * slice;
    const float4 g4 = a.sample ? gumbel4(a.seeds[r], kStreamCluster, (uint32_t)kq0 >> 2)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
    const float gq[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = kq0 + q;
      if (k >= a.c) continue;
      const float s = tot[nt][q];
      const float key = a.sample ? s * a.inv_tau + gq[q] : s;
      a.keys[(int64_t)r * a.key_stride + k] = key;
      if (a.dbg_scores) a.dbg_scores[(int64_t)r * a.c + k] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny GEMM engine: rows of a bf16 matrix (16-row items) times H^T (B
// columns), K = d in chunks of 128.  A workgroup of 4 waves owns 4 * IT
// consecutive items (each wave IT of them) and walks K chunk by chunk: the
// chunk of H (B x 128) is staged once in LDS for all four waves (padded rows
// against bank conflicts, double-buffered), while each wave streams its
// items' rows with the next chunk's loads issued before the current chunk's
// matrix products.  Epilogues:
//   SCORES  stage-1 keys: item rows are centroids; key = score (or score /
//           tau + Gumbel noise) for every (batch row, centroid);
//   FLASH   stage 2: item rows are the candidate rows of a selected cluster
//           (cluster ulist[i / (b/16)] of the cluster-major copy of E, or
//           cluster i / (b/16) when there is no list, unselected ones
//           skipped); per
//           batch row, candidates of clusters the row selected (its bit in
//           the cluster's mask) are folded into a running best decode key
//           and log-sum-exp;
//   DENSE   the batched dense head: item rows are rows of E, every token a
//           candidate for every batch row.
// FLASH and DENSE write one partial per (workgroup, batch row).
// ---------------------------------------------------------------------------
constexpr int kGmThreads = 256;
constexpr int kGmWaves = kGmThreads / kWave;
enum GmMode : int { kGmScores = 0, kGmFlash = 1, kGmDense = 2 };

// KC: K per chunk (KC / 32 MFMA steps); a wave requests KC * 2 contiguous
// bytes of each of its rows per chunk
template <int NT, int IT, int MODE, int KC>
__global__ __launch_bounds__(kGmThreads) __attribute__((amdgpu_waves_per_eu(2))) void gemm_engine_kernel(Stage2mArgs a) {
  constexpr int kSteps = KC / 32;
  constexpr int kHRow = KC + 8;  // LDS row pitch in bf16 (16-byte pad)
  constexpr int kHP = NT * 16 * (KC / 8) / kGmThreads;  // H pieces per thread per chunk
  static_assert(kHP * kGmThreads == NT * 16 * (KC / 8), "H staging");
  __shared__ uint4 s_h[2][NT * 16 * kHRow / 8];
  __shared__ uint64_t s_best[kGmWaves][NT * 16];
  __shared__ float2 s_lse[kGmWaves][NT * 16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = lane >> 4, lr = lane & 15;
  const int B = a.B;
  const int sub = a.b / 16;
  const int64_t nrows_total = MODE == kGmScores ? (int64_t)a.c : a.v;
  // FLASH walks the union list when there is one, else every cluster
  // (skipping the ones no row selected)
  const int64_t nitems = MODE == kGmFlash
                             ? (a.ulist ? (int64_t)(*a.ucount) : (int64_t)a.c) * sub
                             : (nrows_total + 15) / 16;
  const int nchunks = a.d / KC;
  uint64_t best[NT];
  Lse lse[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) { best[nt] = 0ull; lse[nt] = lse_empty(); }

  // work units: groups of kGmWaves * IT items times ksplit slices of K (the
  // waves of a workgroup share the slice, so the staged H chunk is shared),
  // grid-stride (uniform per workgroup)
  const int S = MODE == kGmScores ? a.ksplit : 1;
  const int64_t nunits = ((nitems + kGmWaves * IT - 1) / (kGmWaves * IT)) * S;
  for (int64_t unit = blockIdx.x; unit < nunits; unit += gridDim.x) {
  __syncthreads();  // the previous group's readers of both LDS buffers are done
  const int64_t item0 = (unit / S) * kGmWaves * IT;
  const int sp = (int)(unit % S);
  if constexpr (MODE == kGmFlash) {
    if (!a.ulist) {
      // a group whose clusters no row selected is skipped by the whole
      // workgroup (every thread reads the same masks)
      bool any = false;
      for (int w = 0; w < kGmWaves * IT; ++w) {
        const int64_t it = item0 + w;
        any = any || (it < nitems && a.masks[it / sub] != 0ull);
      }
      if (!any) continue;
    }
  }
  const int cbeg = sp * nchunks / S, cend = (sp + 1) * nchunks / S;

  // this wave's items
  int64_t row0[IT], kc[IT];
  uint64_t mask[IT];
  const uint8_t* ap[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    int64_t it = item0 + wave * IT + i;
    const bool live = it < nitems;
    it = live ? it : nitems - 1;
    if constexpr (MODE == kGmFlash) {
      kc[i] = a.ulist ? a.ulist[it / sub] : it / sub;
      row0[i] = kc[i] * a.b + (it % sub) * 16;
      mask[i] = live ? a.masks[kc[i]] : 0ull;
    } else {
      kc[i] = 0;
      row0[i] = it * 16;
      mask[i] = live ? ~0ull : 0ull;
    }
    int64_t arow = row0[i] + lr;
    if constexpr (MODE != kGmFlash) arow = arow < nrows_total ? arow : nrows_total - 1;
    ap[i] = a.base + arow * a.row_bytes + (int64_t)(8 * slice) * 2;
  }
  // H chunk staging: thread t moves kHP 16-byte pieces per chunk
  const uint8_t* hsrc[kHP];
  int hdst[kHP];
#pragma unroll
  for (int n = 0; n < kHP; ++n) {
    const int piece = threadIdx.x + n * kGmThreads;  // KC / 8 pieces per H row
    int j = piece / (KC / 8);
    const int kp = piece % (KC / 8);
    hdst[n] = j * (kHRow / 8) + kp;
    j = j < B ? j : B - 1;
    hsrc[n] = a.H + (int64_t)j * a.h_bytes + (int64_t)kp * 16;
  }
  f32x4_t acc[IT][NT];
#pragma unroll
  for (int i = 0; i < IT; ++i)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the H staging registers are a native vector type: as an array of uint4
  // they were kept in scratch memory, which made every prefetch wait
  uint4 a0[IT][kSteps], a1[IT][kSteps];
  u32x4_t hreg[kHP];
  // a wave whose items no row needs (a cluster no row selected, the tail)
  // reads no rows and runs no MFMA; it still stages H for the others
  bool wlive = false;
#pragma unroll
  for (int i = 0; i < IT; ++i) wlive = wlive || mask[i] != 0ull;
  auto load_a = [&](uint4 (&dst)[IT][kSteps], int c) {
    if (!wlive) return;
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int u = 0; u < kSteps; ++u)
        dst[i][u] = *reinterpret_cast<const uint4*>(ap[i] + (int64_t)c * KC * 2 + u * 64);
  };
  auto load_h = [&](int c) {
#pragma unroll
    for (int n = 0; n < kHP; ++n)
      hreg[n] = *reinterpret_cast<const u32x4_t*>(hsrc[n] + (int64_t)c * KC * 2);
  };
  auto store_h = [&](int buf) {
#pragma unroll
    for (int n = 0; n < kHP; ++n) reinterpret_cast<u32x4_t*>(s_h[buf])[hdst[n]] = hreg[n];
  };
  auto compute = [&](const uint4 (&av)[IT][kSteps], int buf) {
    if (!wlive) return;
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      uint4 bv[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bv[nt] = s_h[buf][(nt * 16 + lr) * (kHRow / 8) + u * 4 + slice];
#pragma unroll
      for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[i][nt] = mfma_bf16(av[i][u], bv[nt], acc[i][nt]);
    }
  };

  load_h(cbeg);
  load_a(a0, cbeg);
  store_h(0);
  for (int c = cbeg; c < cend; c += 2) {
    // chunk c from buffer 0 / registers a0; prefetch chunk c + 1
    __syncthreads();
    if (c + 1 < cend) { load_h(c + 1); load_a(a1, c + 1); }
    compute(a0, 0);
    if (c + 1 >= cend) break;
    store_h(1);
    // chunk c + 1 from buffer 1 / registers a1; prefetch chunk c + 2
    __syncthreads();
    if (c + 2 < cend) { load_h(c + 2); load_a(a0, c + 2); }
    compute(a1, 1);
    if (c + 2 < cend) store_h(0);
  }

  if constexpr (MODE == kGmScores) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      if (!mask[i]) continue;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + lr;
        if (r >= B) continue;
        // the lane's 4 consecutive clusters share one Philox block
        const int64_t kq0 = row0[i] + 4 * slice;
        const float4 g4 = (a.sample && S == 1)
                              ? gumbel4(a.seeds[r], kStreamCluster, (uint32_t)kq0 >> 2)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        const float gq[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t k = kq0 + q;
          if (k >= a.c) continue;
          const float sc = acc[i][nt][q];
          if (S > 1) {  // partial score over this K slice; the select sums the slices
            a.keys[sp * a.part_stride + (int64_t)r * a.key_stride + k] = sc;
            continue;
          }
          const float key = a.sample ? sc * a.inv_tau + gq[q] : sc;
          a.keys[(int64_t)r * a.key_stride + k] = key;
          if (a.dbg_scores) a.dbg_scores[(int64_t)r * a.c + k] = sc;
        }
      }
    }
    continue;
  }

#pragma unroll
  for (int i = 0; i < IT; ++i) {
    if (!mask[i]) continue;
    uint32_t tok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = row0[i] + 4 * slice + q;
      if constexpr (MODE == kGmDense) tok[q] = (uint32_t)row;
      else tok[q] = (uint32_t)a.c2t[row];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = nt * 16 + lr;
      const bool rowsel = r < B && ((mask[i] >> r) & 1ull);
      if (!rowsel) continue;
      const uint64_t seed = a.sample ? a.seeds[r] : 0ull;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = row0[i] + 4 * slice + q;
        if (MODE == kGmDense && row >= a.v) continue;
        const float x = acc[i][nt][q];
        const float xs = x * a.inv_tau;
        const float kx = a.sample ? xs + gumbel(seed, kStreamToken, tok[q]) : x;
        const uint64_t key = decode_key(kx, tok[q]);
        best[nt] = key > best[nt] ? key : best[nt];
        if (a.with_lse) lse[nt] = lse_add(lse[nt], xs);
        if (MODE == kGmFlash && a.dbg_logits) {
          // position of cluster k in row r's ascending selection
          const int64_t k = kc[i];
          const int32_t* sr = a.sel + (int64_t)r * a.sel_stride;
          int lo = 0, hi = a.p - 1;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sr[mid] < k) lo = mid + 1; else hi = mid;
          }
          const int64_t pos = (int64_t)lo * a.b + (row - k * a.b);
          a.dbg_ids[(int64_t)r * a.dbg_stride + pos] = (int32_t)tok[q];
          a.dbg_logits[(int64_t)r * a.dbg_stride + pos] = x;
        }
      }
    }
  }
  }  // groups
  if constexpr (MODE == kGmScores) return;
  // combine the 4 lanes that share a batch column, then the waves
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const uint64_t y = __shfl_xor(best[nt], o, kWave);
      best[nt] = y > best[nt] ? y : best[nt];
      if (a.with_lse) lse[nt] = lse_merge(lse[nt], Lse{__shfl_xor(lse[nt].m, o, kWave),
                                                       __shfl_xor(lse[nt].s, o, kWave)});
    }
    if (slice == 0) {
      s_best[wave][nt * 16 + lr] = best[nt];
      s_lse[wave][nt * 16 + lr] = make_float2(lse[nt].m, lse[nt].s);
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < B; r += kGmThreads) {
    uint64_t bb = s_best[0][r];
    Lse ll{s_lse[0][r].x, s_lse[0][r].y};
    for (int w = 1; w < kGmWaves; ++w) {
      bb = s_best[w][r] > bb ? s_best[w][r] : bb;
      ll = lse_merge(ll, Lse{s_lse[w][r].x, s_lse[w][r].y});
    }
    // row-major partials ([row][workgroup]): the fold of a row reads them
    // contiguously
    a.part_best[(int64_t)r * gridDim.x + blockIdx.x] = bb;
    if (a.with_lse) a.part_lse[(int64_t)r * gridDim.x + blockIdx.x] = make_float2(ll.m, ll.s);
  }
}

// per batch row: fold the per-block partials (a contiguous run per row) into
// the token (and lse), wave by wave and then the waves in order; the rows'
// workgroups together clear the cluster masks of this call's union
__global__ __launch_bounds__(256) void finalize_kernel(Stage2mArgs a, int nblocks) {
  __shared__ uint64_t s_b[256 / kWave];
  __shared__ float2 s_l[256 / kWave];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const uint64_t* pb = a.part_best + (int64_t)r * nblocks;
  const float2* pl = a.part_lse + (int64_t)r * nblocks;
  uint64_t bb = 0ull;
  Lse ll = lse_empty();
  for (int j = t; j < nblocks; j += 256) {
    const uint64_t x = pb[j];
    bb = x > bb ? x : bb;
    if (a.with_lse) ll = lse_merge(ll, Lse{pl[j].x, pl[j].y});
  }
  bb = wave_max_u64(bb);
  if (a.with_lse) ll = wave_lse(ll);
  if ((t & (kWave - 1)) == 0) {
    s_b[t / kWave] = bb;
    s_l[t / kWave] = make_float2(ll.m, ll.s);
  }
  __syncthreads();
  if (t == 0) {
    uint64_t b0 = s_b[0];
    Lse l0{s_l[0].x, s_l[0].y};
#pragma unroll
    for (int w = 1; w < 256 / kWave; ++w) {
      b0 = s_b[w] > b0 ? s_b[w] : b0;
      l0 = lse_merge(l0, Lse{s_l[w].x, s_l[w].y});
    }
    a.out_tokens[r] = (int32_t)key_id(b0);
    if (a.out_lse) a.out_lse[r] = l0.m + logf(l0.s);
  }
  if (a.masks) {
    if (a.ulist) {
      const int u = *a.ucount;
      for (int i = r * 256 + t; i < u; i += (int)gridDim.x * 256) a.masks[a.ulist[i]] = 0ull;
    } else {
      for (int i = r * 256 + t; i < a.c; i += (int)gridDim.x * 256) a.masks[i] = 0ull;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
bool batched_supported(int dtype, int d, int B, bool int4) {
  if (dtype != FH_DTYPE_BF16 || B < 2 || B > FH_MAX_BATCH) return false;
  return d % 128 == 0;
}

// Tiling (measured on the 2048-wide heads at B = 16, 32, 64): one 16-row
// item per wave, and as long a K chunk as d allows (256, 8 MFMA steps, when
// d % 256 == 0; else 128) for the streaming modes, where it gives each row
// 512-byte contiguous requests.  Stage-1 scores keep 128: their K slices
// are short.  The kernel is capped at 256 registers (two waves per SIMD):
// with one wave per SIMD the wider tiles stalled on HBM latency.
constexpr int kGmItems = 1;

template <int NT, int MODE, int KC>
static void launch_engine_kc(const Stage2mArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                             hipEvent_t e1) {
  hipExtLaunchKernelGGL((gemm_engine_kernel<NT, kGmItems, MODE, KC>), dim3(grid),
                        dim3(kGmThreads), 0, s, e0, e1, 0, a);
}

template <int MODE, int KC>
static hipError_t launch_engine_nt(const Stage2mArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                                   hipEvent_t e1) {
  switch ((a.B + 15) / 16) {
    case 1: launch_engine_kc<1, MODE, KC>(a, grid, s, e0, e1); break;
    case 2: launch_engine_kc<2, MODE, KC>(a, grid, s, e0, e1); break;
    case 3: launch_engine_kc<3, MODE, KC>(a, grid, s, e0, e1); break;
    case 4: launch_engine_kc<4, MODE, KC>(a, grid, s, e0, e1); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_engine(const Stage2mArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1) {
  if (a.d % 256 == 0) return launch_engine_nt<MODE, 256>(a, grid, s, e0, e1);
  return launch_engine_nt<MODE, 128>(a, grid, s, e0, e1);
}

static int engine_grid(int64_t nrows16) {
  const int64_t per = (int64_t)kGmWaves * kGmItems;
  const int64_t g = (nrows16 + per - 1) / per;
  return g < 1 ? 1 : (int)g;
}

hipError_t launch_stage1_mfma(const Stage1Args& a, bool int4, int B, hipStream_t s,
                              const Timing* tm, int* ksplit) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const int NT = (B + 15) / 16;
  *ksplit = 1;
  if (int4) {
    const dim3 grid((a.ntiles + kS1qThreads / kWave - 1) / (kS1qThreads / kWave));
    switch (NT) {
      case 1: hipExtLaunchKernelGGL(stage1_int4_mfma_kernel<1>, grid, dim3(kS1qThreads), 0, s, e0, e1, 0, a, B); break;
      case 2: hipExtLaunchKernelGGL(stage1_int4_mfma_kernel<2>, grid, dim3(kS1qThreads), 0, s, e0, e1, 0, a, B); break;
      case 3: hipExtLaunchKernelGGL(stage1_int4_mfma_kernel<3>, grid, dim3(kS1qThreads), 0, s, e0, e1, 0, a, B); break;
      case 4: hipExtLaunchKernelGGL(stage1_int4_mfma_kernel<4>, grid, dim3(kS1qThreads), 0, s, e0, e1, 0, a, B); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  Stage2mArgs m{};
  m.base = a.C;
  m.row_bytes = a.row_bytes;
  m.c = a.c;
  m.b = 16;
  m.d = a.d;
  m.B = B;
  m.H = a.H;
  m.h_bytes = a.h_bytes;
  m.sample = a.sample;
  m.inv_tau = a.inv_tau;
  m.seeds = a.seeds;
  m.keys = a.keys;
  m.key_stride = a.key_stride;
  m.dbg_scores = a.dbg_scores;
  // one 16-row item per wave and enough K slices to give the chip ~2 x 256
  // workgroups (slices are whole K chunks)
  constexpr int kKC = 128;
  const int nchunks = a.d / kKC;
  const int64_t groups = ((int64_t)(a.c + 15) / 16 + kGmWaves - 1) / kGmWaves;
  int S = (int)((512 + groups - 1) / groups);
  S = S < 1 ? 1 : (S > kMaxKSplit ? kMaxKSplit : S);
  S = S > nchunks ? nchunks : S;
  m.ksplit = S;
  m.part_stride = a.part_stride;
  *ksplit = S;
  const int64_t units = groups * S;
  const int grid = (int)(units < 4096 ? units : 4096);
  return launch_engine_nt<kGmScores, kKC>(m, grid, s, e0, e1);
}

int stage2_mfma_grid() { return 4096; }

hipError_t launch_stage2_mfma(const Stage2mArgs& a, bool dense, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  // flash: the union is known on the device only; launch for every cluster
  const int64_t items = dense ? (a.v + 15) / 16 : (int64_t)a.c * (a.b / 16);
  int grid = engine_grid(items);
  grid = grid < stage2_mfma_grid() ? grid : stage2_mfma_grid();
  hipError_t e = dense ? launch_engine<kGmDense>(a, grid, s, e0, e1)
                       : launch_engine<kGmFlash>(a, grid, s, e0, e1);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(finalize_kernel, dim3(a.B), dim3(256), 0, s, a, grid);
  return hipGetLastError();
}

}  // namespace fh
