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
#include <type_traits>

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

// Scores of one INT4 tile (16 centroid rows) against the B hidden rows: lane
// l ends with centroid rows 4 (l div 16) + q of the tile for batch rows
// nt * 16 + (l mod 16) in tot[nt][q].
template <int NT>
__device__ __forceinline__ void int4_tile_scores(const uint8_t* q4, const uint16_t* q4s, int G,
                                                 const uint8_t* H, int64_t h_bytes, int B,
                                                 int tile, int lane, f32x4_t (&tot)[NT]) {
  const int slice = lane >> 4, lr = lane & 15;
  const uint8_t* hp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int j = nt * 16 + lr;
    j = j < B ? j : B - 1;
    hp[nt] = H + (int64_t)j * h_bytes + (int64_t)(32 * slice) * 2;
  }
  const uint4* codes = reinterpret_cast<const uint4*>(q4) + (int64_t)tile * G * kWave + lane;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) tot[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < G; ++g) {
    const uint4 w = codes[(int64_t)g * kWave];
    // scales of the 4 output rows of this lane: 4 (l div 16) + q
    const uint2 sc2 = *reinterpret_cast<const uint2*>(q4s + ((int64_t)tile * G + g) * 16 + 4 * slice);
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
}

// The batched INT4 stage 1 as its own kernel.  A workgroup owns TPW
// consecutive tiles and its 4 waves split the 128-column groups (wave w
// takes groups [w G / 4, (w + 1) G / 4)): each H fragment a wave loads feeds
// the products of all TPW tiles, so a workgroup reads H once, and the codes
// and scales of a batch of kS1qGB groups of every tile are requested before
// the first product (one round trip per batch, not one per group).  The
// waves' partial scores meet in LDS; wave i adds them in wave order for
// tile i and stores its keys.
constexpr int kS1qWaves = kS1qThreads / kWave;
constexpr int kS1qGB = 4;  // groups per batch of loads

template <int NT, int TPW>
__global__ __launch_bounds__(kS1qThreads) void stage1_int4_mfma_kernel(
    const uint8_t* pq4, const uint16_t* pq4s, const uint8_t* pH, int ph_bytes, int pgroups,
    int pntiles, int B, Stage1Args a) {
  static_assert(TPW <= kS1qWaves, "one finishing wave per tile");
  __shared__ f32x4_t s_red[kS1qWaves][TPW][NT][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = lane >> 4, lr = lane & 15;
  const int G = pgroups;
  const int tile0 = blockIdx.x * TPW;
  const int g_lo = wave * G / kS1qWaves, g_hi = (wave + 1) * G / kS1qWaves;
  // lane (slice, lr) feeds H row nt * 16 + lr, columns 128 g + 32 slice +
  // 8 s + [0, 8) at step s (rows past the batch repeat the last one; their
  // results are dropped); tiles past the last repeat the last one too
  const uint8_t* hp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int j = nt * 16 + lr < B ? nt * 16 + lr : B - 1;
    hp[nt] = pH + (int64_t)j * ph_bytes + (int64_t)(32 * slice) * 2;
  }
  const uint4* codes[TPW];
  const uint16_t* scl[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tl = tile0 + i < pntiles ? tile0 + i : pntiles - 1;
    codes[i] = reinterpret_cast<const uint4*>(pq4) + (int64_t)tl * G * kWave + lane;
    scl[i] = pq4s + (int64_t)tl * G * 16 + 4 * slice;
  }
  f32x4_t tot[TPW][NT];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) tot[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the H fragments of one group (4 MFMA steps): with one or two column
  // tiles the next group's are requested before the current group's
  // products (two buffers), else each group's just before its own
  constexpr int kHB = NT <= 2 ? 2 : 1;
  uint4 hb[kHB][4][NT];
  auto load_hg = [&](uint4 (&dst)[4][NT], int g) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        dst[s][nt] = *reinterpret_cast<const uint4*>(hp[nt] + (int64_t)(128 * g + 8 * s) * 2);
  };
  for (int g0 = g_lo; g0 < g_hi; g0 += kS1qGB) {
    uint4 w[TPW][kS1qGB];
    uint2 sc[TPW][kS1qGB];
#pragma unroll
    for (int gi = 0; gi < kS1qGB; ++gi) {
      if (g0 + gi < g_hi) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          w[i][gi] = codes[i][(int64_t)(g0 + gi) * kWave];
          // scales of the lane's 4 output rows of the tile: 4 slice + q
          sc[i][gi] = *reinterpret_cast<const uint2*>(scl[i] + (g0 + gi) * 16);
        }
      }
    }
    if constexpr (kHB == 2) load_hg(hb[0], g0);
#pragma unroll
    for (int gi = 0; gi < kS1qGB; ++gi) {
      if (g0 + gi >= g_hi) break;  // uniform over the wave
      if constexpr (kHB == 2) {
        if (gi + 1 < kS1qGB && g0 + gi + 1 < g_hi) load_hg(hb[(gi + 1) & 1], g0 + gi + 1);
      } else {
        load_hg(hb[0], g0 + gi);
      }
      __builtin_amdgcn_sched_barrier(0);  // the loads go out before the products
      const uint4 (&bv)[4][NT] = hb[kHB == 2 ? (gi & 1) : 0];
      f32x4_t part[TPW][NT];
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) part[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          const uint32_t ws = s == 0 ? w[i][gi].x : s == 1 ? w[i][gi].y : s == 2 ? w[i][gi].z
                                                                                 : w[i][gi].w;
          // the lane's codes for this step as bf16 (exact for -8..7)
          const uint4 av = make_uint4(int4_pair_bf16(ws, 0), int4_pair_bf16(ws, 2),
                                      int4_pair_bf16(ws, 4), int4_pair_bf16(ws, 6));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) part[i][nt] = mfma_bf16(av, bv[s][nt], part[i][nt]);
        }
      }
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const float scq[4] = {__uint_as_float(sc[i][gi].x << 16),
                              __uint_as_float(sc[i][gi].x & 0xFFFF0000u),
                              __uint_as_float(sc[i][gi].y << 16),
                              __uint_as_float(sc[i][gi].y & 0xFFFF0000u)};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int q = 0; q < 4; ++q) tot[i][nt][q] = fmaf(scq[q], part[i][nt][q], tot[i][nt][q]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) s_red[wave][i][nt][lane] = tot[i][nt];
  __syncthreads();
  if (wave >= TPW) return;
  const int tile = tile0 + wave;
  if (tile >= pntiles) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + lr;
    if (r >= B) continue;
    f32x4_t sum = s_red[0][wave][nt][lane];
#pragma unroll
    for (int w = 1; w < kS1qWaves; ++w) sum += s_red[w][wave][nt][lane];
    // the lane's 4 consecutive clusters share one Philox block
    const int kq0 = tile * 16 + 4 * slice;
    const float4 g4 = a.sample ? gumbel4(a.seeds[r], kStreamCluster, (uint32_t)kq0 >> 2)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
    const float gq[4] = {g4.x, g4.y, g4.z, g4.w};
    float kv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // raw_keys: the plain score (the select forms the key after counting)
      kv[q] = (a.sample && !a.raw_keys) ? sum[q] * a.inv_tau + gq[q] : sum[q];
      if (a.dbg_scores && kq0 + q < a.c) a.dbg_scores[(int64_t)r * a.c + kq0 + q] = sum[q];
    }
    float* kr = a.keys + (int64_t)r * a.key_stride + kq0;
    if (kq0 + 3 < a.c) {
      *reinterpret_cast<float4*>(kr) = make_float4(kv[0], kv[1], kv[2], kv[3]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (kq0 + q < a.c) kr[q] = kv[q];
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
//   ALL     stage 1 and stage 2 in one pass, before any selection: items
//           [0, n1) are stage-1 items (16 centroid rows, or one INT4 tile
//           scored by int4_tile_scores) with the SCORES epilogue; every
//           later item is 16 candidate rows of a cluster, and each batch row
//           gets one record per item (best decode key, and log-sum-exp), for
//           every cluster whether or not the row will select it.  The
//           select-and-fold kernel then keeps the records of the row's
//           selected clusters only.
// FLASH and DENSE write one partial per (workgroup, batch row).
// ---------------------------------------------------------------------------
constexpr int kGmThreads = 256;
// buffer resource word 3 for untyped 32-bit-element reads on gfx950
constexpr int kBufferFlags = 0x00020000;
constexpr int kGmWaves = kGmThreads / kWave;
enum GmMode : int { kGmScores = 0, kGmFlash = 1, kGmDense = 2, kGmAll = 3, kGmAllQ4 = 4 };
// ALL with INT4 stage-1 tiles (kGmAllQ4) or 16-row bf16 centroid items (kGmAll)

// KC: K per chunk (KC / 32 MFMA steps); a wave requests KC * 2 contiguous
// bytes of each of its rows per chunk
// NCH > 0: d = NCH * KC and one K slice; the K walk is unrolled, so the
// buffers of every chunk are fixed at compile time and each chunk's loads
// are issued ahead of the previous chunk's products.
template <int NT, int IT, int MODE, int KC, int NCH = 0>
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
  // the unrolled walk serves greedy calls only (its launcher checks)
  const bool sample = NCH > 0 ? false : a.sample;
  constexpr bool ALL = MODE == kGmAll || MODE == kGmAllQ4;
  constexpr bool Q4 = MODE == kGmAllQ4;
  const int64_t nrows_total = MODE == kGmScores ? (int64_t)a.c : a.v;
  // FLASH walks the union list when there is one, else every cluster
  // (skipping the ones no row selected); ALL walks the stage-1 items, then
  // every cluster
  const int64_t nitems = MODE == kGmFlash
                             ? (a.ulist ? (int64_t)(*a.ucount) : (int64_t)a.c) * sub
                         : ALL ? a.n1 + (int64_t)a.c * sub
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

  // this wave's items: item i streams rows of abase[i] at the lane's byte
  // offset aoff[i] (32 bits in the unrolled walk, whose launcher checks the
  // matrix sizes; the base is uniform over the wave)
  int64_t row0[IT], kc[IT];
  uint64_t mask[IT];
  const uint8_t* abase[IT];
  uint32_t ftok[IT][4];  // FLASH: the token ids of the item's rows for this lane
  using AOff = std::conditional_t<(NCH > 0), uint32_t, int64_t>;
  AOff aoff[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    int64_t it = item0 + wave * IT + i;
    const bool live = it < nitems;
    it = live ? it : nitems - 1;
    if constexpr (ALL) {
      if (it < a.n1) {
        // stage-1 item: 16 centroid rows (none to stream for an INT4 tile)
        kc[i] = -1;
        row0[i] = it * 16;
        mask[i] = (live && !Q4) ? ~0ull : 0ull;
        int64_t crow = row0[i] + lr;
        crow = crow < a.c ? crow : a.c - 1;
        abase[i] = a.cbase;
        aoff[i] = (AOff)(crow * a.c_row_bytes + (int64_t)(8 * slice) * 2);
      } else {
        // item ie is rows [16 ie, 16 ie + 16) of the cluster-major order
        // (cluster ie / (b/16), its 16-row part ie % (b/16))
        const int64_t ie = it - a.n1;
        kc[i] = -1;
        row0[i] = ie * 16;
        mask[i] = live ? ~0ull : 0ull;
        int64_t arow = row0[i] + lr;
        if (a.borrowed) arow = a.c2t[arow];
        abase[i] = a.base;
        aoff[i] = (AOff)(arow * a.row_bytes + (int64_t)(8 * slice) * 2);
      }
      continue;
    }
    if constexpr (MODE == kGmFlash) {
      kc[i] = a.ulist ? a.ulist[it / sub] : it / sub;
      row0[i] = kc[i] * a.b + (it % sub) * 16;
      mask[i] = live ? a.masks[kc[i]] : 0ull;
      // the candidates' token ids, loaded now so that the epilogue does not
      // wait for them after the K walk
#pragma unroll
      for (int q = 0; q < 4; ++q) ftok[i][q] = (uint32_t)a.c2t[row0[i] + 4 * slice + q];
    } else {
      kc[i] = 0;
      row0[i] = it * 16;
      mask[i] = live ? ~0ull : 0ull;
    }
    int64_t arow = row0[i] + lr;
    if constexpr (MODE != kGmFlash) arow = arow < nrows_total ? arow : nrows_total - 1;
    if constexpr (MODE == kGmFlash) {
      if (a.borrowed) arow = a.c2t[arow];  // the caller's E: the candidate's token row
    }
    abase[i] = a.base;
    aoff[i] = (AOff)(arow * a.row_bytes + (int64_t)(8 * slice) * 2);
  }
  // H chunk staging: thread t moves kHP 16-byte pieces per chunk; piece
  // t + n * kGmThreads is H row j0 + n * kHStep, 16-byte column kp.  H is
  // read through a buffer resource that ends with row B - 1: a piece is the
  // lane's row-j0 offset plus a uniform row offset (one register for all
  // pieces; 64 rows of at most FH_MAX_ROW_BYTES fit 31 bits), and the
  // pieces of rows past the batch read as zeros (their columns are dropped)
  constexpr int kHStep = kGmThreads / (KC / 8);
  static_assert(kHStep * (KC / 8) == kGmThreads, "H staging rows");
  static_assert((int64_t)64 * FH_MAX_ROW_BYTES < ((int64_t)1 << 31), "H offsets");
  const int j0 = threadIdx.x / (KC / 8), kp = threadIdx.x % (KC / 8);
  const int hdst0 = j0 * (kHRow / 8) + kp;
  const __amdgpu_buffer_rsrc_t hrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.H), (short)0, (int)((B - 1) * a.h_bytes + (int64_t)a.d * 2),
      kBufferFlags);
  const uint32_t hoff0 = (uint32_t)(j0 * a.h_bytes) + (uint32_t)kp * 16;
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
  // (the unrolled walk serves the modes where every wave streams: its tail
  // rows are clamped to valid ones and their results dropped)
  bool wlive = NCH > 0;
#pragma unroll
  for (int i = 0; i < IT; ++i) wlive = wlive || mask[i] != 0ull;
  auto load_a = [&](uint4 (&dst)[IT][kSteps], int c) {
    if (!wlive) return;
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int u = 0; u < kSteps; ++u)
        dst[i][u] = *reinterpret_cast<const uint4*>(abase[i] + aoff[i] + (int64_t)c * KC * 2 +
                                                    u * 64);
  };
  auto load_h = [&](int c) {
#pragma unroll
    for (int n = 0; n < kHP; ++n)
      hreg[n] = __builtin_amdgcn_raw_buffer_load_b128(
          hrsrc, hoff0 + (uint32_t)(c * KC * 2), (int)(n * kHStep * a.h_bytes), 0);
  };
  auto store_h = [&](int buf) {
#pragma unroll
    for (int n = 0; n < kHP; ++n)
      reinterpret_cast<u32x4_t*>(s_h[buf])[hdst0 + n * kHStep * (kHRow / 8)] = hreg[n];
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

  // a unit of INT4 stage-1 tiles only streams no rows: it skips the K walk
  const bool unit_rows = !Q4 || item0 + kGmWaves * IT > a.n1;
  // ALL: the candidates' token ids of the records, loaded with the last
  // chunk (whose next-chunk registers are free) so that the records do not
  // wait for them
  uint32_t tokp[IT][4];
  if constexpr (NCH > 0) {
    if (unit_rows) {
      load_h(0);
      load_a(a0, 0);
      store_h(0);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        __syncthreads();
        if (c + 1 < NCH) {
          load_h(c + 1);
          if ((c & 1) == 0) load_a(a1, c + 1); else load_a(a0, c + 1);
        } else if constexpr (ALL) {
#pragma unroll
          for (int i = 0; i < IT; ++i) {
            const int64_t t0 = row0[i] + 4 * slice;  // clamped to a cluster row
            const int64_t tr = item0 + wave * IT + i < a.n1 ? 0 : t0;
#pragma unroll
            for (int q = 0; q < 4; ++q) tokp[i][q] = (uint32_t)a.c2t[tr + q];
          }
        }
        // keep the next chunk's loads ahead of this chunk's products
        __builtin_amdgcn_sched_barrier(0);
        if ((c & 1) == 0) compute(a0, 0); else compute(a1, 1);
        if (c + 1 < NCH) store_h((c + 1) & 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  } else {
  if (unit_rows) {
  load_h(cbeg);
  load_a(a0, cbeg);
  store_h(0);
  }
  for (int c = cbeg; unit_rows && c < cend; c += 2) {
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
  }

  if constexpr (ALL) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int64_t it = item0 + wave * IT + i;  // uniform over the wave
      if (it >= nitems) continue;
      if (it < a.n1) {
        // stage-1 keys of 16 centroids for every batch row
        f32x4_t sc[NT];
        if constexpr (Q4) {
          int4_tile_scores<NT>(a.q4, a.q4s, a.groups, a.H, a.h_bytes, B, (int)it, lane, sc);
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) sc[nt] = acc[i][nt];
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int r = nt * 16 + lr;
          if (r >= B) continue;
          const int64_t kq0 = it * 16 + 4 * slice;
          // raw_scores: the plain score (the select counts on it, then forms
          // the key)
          const bool keyed = sample && !a.raw_scores;
          const float4 g4 = keyed ? gumbel4(a.seeds[r], kStreamCluster, (uint32_t)kq0 >> 2)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
          const float gq[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t k = kq0 + q;
            if (k >= a.c) continue;
            const float x = sc[nt][q];
            a.keys[(int64_t)r * a.key_stride + k] = keyed ? x * a.inv_tau + gq[q] : x;
            if (a.dbg_scores && !a.raw_scores) a.dbg_scores[(int64_t)r * a.c + k] = x;
          }
        }
        continue;
      }
      // one record per batch row for these 16 candidates: the lane's 4
      // tokens, then the 4 lanes that share a batch row
      uint32_t tok[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        tok[q] = NCH > 0 ? tokp[i][q] : (uint32_t)a.c2t[row0[i] + 4 * slice + q];
      const int64_t rec = (it - a.n1) * a.B;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + lr;
        const uint64_t seed = (sample && r < B) ? a.seeds[r] : 0ull;
        uint64_t bk = 0ull;
        Lse ll = lse_empty();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x = acc[i][nt][q];
          const float xs = x * a.inv_tau;
          const float kx = sample ? xs + gumbel(seed, kStreamToken, tok[q]) : x;
          const uint64_t key = decode_key(kx, tok[q]);
          bk = key > bk ? key : bk;
          if (a.with_lse) ll = lse_add(ll, xs);
        }
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
          const uint64_t y = __shfl_xor(bk, o, kWave);
          bk = y > bk ? y : bk;
          if (a.with_lse) ll = lse_merge(ll, Lse{__shfl_xor(ll.m, o, kWave),
                                                 __shfl_xor(ll.s, o, kWave)});
        }
        if (slice == 0 && r < B) {
          a.part_best[rec + r] = bk;
          if (a.with_lse) a.part_lse[rec + r] = make_float2(ll.m, ll.s);
        }
      }
    }
    continue;
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
        const float4 g4 = (sample && S == 1)
                              ? gumbel4(a.seeds[r], kStreamCluster, (uint32_t)kq0 >> 2)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        const float gq[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t k = kq0 + q;
          if (k >= a.c) continue;
          const float sc = acc[i][nt][q];
          if (S > 1 || a.raw_scores) {  // partial or plain score; the select forms the key
            a.keys[sp * a.part_stride + (int64_t)r * a.key_stride + k] = sc;
            continue;
          }
          const float key = sample ? sc * a.inv_tau + gq[q] : sc;
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
      else tok[q] = ftok[i][q];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = nt * 16 + lr;
      const bool rowsel = r < B && ((mask[i] >> r) & 1ull);
      if (!rowsel) continue;
      const uint64_t seed = sample ? a.seeds[r] : 0ull;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = row0[i] + 4 * slice + q;
        if (MODE == kGmDense && row >= a.v) continue;
        const float x = acc[i][nt][q];
        const float xs = x * a.inv_tau;
        const float kx = sample ? xs + gumbel(seed, kStreamToken, tok[q]) : x;
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
  if constexpr (MODE == kGmScores || ALL) return;
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
// (the partials' addresses, count and the lse switch come as leading scalar
// arguments, preloaded into scalar registers, so the partials' loads need
// not wait for the argument struct)
__global__ __launch_bounds__(256) void finalize_kernel(const uint64_t* part_best,
                                                       const float2* part_lse, int nblocks,
                                                       int with_lse, Stage2mArgs a) {
  __shared__ uint64_t s_b[256 / kWave];
  __shared__ float2 s_l[256 / kWave];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const uint64_t* pb = part_best + (int64_t)r * nblocks;
  const float2* pl = part_lse + (int64_t)r * nblocks;
  uint64_t bb = 0ull;
  Lse ll = lse_empty();
  // every partial of the thread is requested before the first is folded
  // (one round trip instead of one per partial), then folded in j order
  constexpr int kPer = 16;  // the engine's grid is at most 16 * 256 workgroups
  uint64_t xb[kPer];
  float2 xl[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = t + 256 * i;
    if (j < nblocks) {
      xb[i] = pb[j];
      if (with_lse) xl[i] = pl[j];
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = t + 256 * i;
    if (j < nblocks) {
      bb = xb[i] > bb ? xb[i] : bb;
      if (with_lse) ll = lse_merge(ll, Lse{xl[i].x, xl[i].y});
    }
  }
  for (int j = t + 256 * kPer; j < nblocks; j += 256) {
    const uint64_t x = pb[j];
    bb = x > bb ? x : bb;
    if (with_lse) ll = lse_merge(ll, Lse{pl[j].x, pl[j].y});
  }
  bb = wave_max_u64(bb);
  if (with_lse) ll = wave_lse(ll);
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
// Batched bf16 stage 1 in one round of loads.  A workgroup's unit is 4
// consecutive 16-row items (one per wave) times one K slice of at most
// kScChunks chunks of 128 columns.  Every thread requests all of its A rows'
// pieces and its share of the slice's H before anything is waited for; H
// goes to LDS (padded rows, one buffer per chunk), then the waves run the
// products chunk by chunk, in the order the engine's SCORES walk uses, and
// store the slice's partial scores (or, with one slice, the keys).
// ---------------------------------------------------------------------------
constexpr int kScChunks = 4;
constexpr int kScKC = 128;

template <int NT>
__global__ __launch_bounds__(kGmThreads) void scores_mfma_kernel(
    const uint8_t* pbase, const uint8_t* pH, int prow_bytes, int ph_bytes, int pc, int pd, int pB,
    int pS, Stage2mArgs a) {
  constexpr int kSteps = kScKC / 32;
  constexpr int kHRow = kScKC + 8;                       // LDS row pitch in bf16
  constexpr int kHP = NT * 16 * (kScKC / 8) / kGmThreads;  // H pieces per thread per chunk
  static_assert(kHP * kGmThreads == NT * 16 * (kScKC / 8), "H staging");
  __shared__ uint4 s_h[kScChunks][NT * 16 * kHRow / 8];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = lane >> 4, lr = lane & 15;
  const int B = pB;
  const int S = pS;
  const int unit = blockIdx.x;
  const int sp = unit % S;
  const int64_t item = (int64_t)(unit / S) * kGmWaves + wave;
  const int64_t nitems = ((int64_t)pc + 15) / 16;
  const bool live = item < nitems;  // uniform over the wave
  const int nchunks = pd / kScKC;
  const int cbeg = sp * nchunks / S, nc = (sp + 1) * nchunks / S - cbeg;  // nc <= kScChunks
  const int64_t row0 = (live ? item : nitems - 1) * 16;
  int64_t arow = row0 + lr;
  arow = arow < pc ? arow : pc - 1;
  const uint8_t* ap = pbase + arow * prow_bytes + (int64_t)(8 * slice) * 2 +
                      (int64_t)cbeg * kScKC * 2;
  // H through a buffer resource that ends with row B - 1: pieces of rows past
  // the batch read as zeros (their columns are dropped)
  constexpr int kHStep = kGmThreads / (kScKC / 8);
  const int j0 = threadIdx.x / (kScKC / 8), kp = threadIdx.x % (kScKC / 8);
  const __amdgpu_buffer_rsrc_t hrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(pH), (short)0, (int)((B - 1) * ph_bytes + (int64_t)pd * 2),
      kBufferFlags);
  const uint32_t hoff0 = (uint32_t)(j0 * ph_bytes) + (uint32_t)kp * 16 + (uint32_t)cbeg * kScKC * 2;
  uint4 av[kScChunks][kSteps];
  u32x4_t hreg[kScChunks][kHP];
#pragma unroll
  for (int c = 0; c < kScChunks; ++c) {
    if (c < nc) {
#pragma unroll
      for (int n = 0; n < kHP; ++n)
        hreg[c][n] = __builtin_amdgcn_raw_buffer_load_b128(
            hrsrc, hoff0 + (uint32_t)(c * kScKC * 2), (int)(n * kHStep * ph_bytes), 0);
      if (live) {
#pragma unroll
        for (int u = 0; u < kSteps; ++u)
          av[c][u] = *reinterpret_cast<const uint4*>(ap + (int64_t)c * kScKC * 2 + u * 64);
      }
    }
  }
  const int hdst0 = j0 * (kHRow / 8) + kp;
#pragma unroll
  for (int c = 0; c < kScChunks; ++c)
    if (c < nc)
#pragma unroll
      for (int n = 0; n < kHP; ++n)
        reinterpret_cast<u32x4_t*>(s_h[c])[hdst0 + n * kHStep * (kHRow / 8)] = hreg[c][n];
  __syncthreads();
  if (!live) return;
  f32x4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kScChunks; ++c) {
    if (c >= nc) break;
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      uint4 bv[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bv[nt] = s_h[c][(nt * 16 + lr) * (kHRow / 8) + u * 4 + slice];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_bf16(av[c][u], bv[nt], acc[nt]);
    }
  }
  // lane: centroid rows row0 + 4 slice + q for batch row nt * 16 + lr
  const bool keyed = S == 1 && !a.raw_scores;  // else partial or plain scores (the select keys them)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + lr;
    if (r >= B) continue;
    const int64_t kq0 = row0 + 4 * slice;
    // the lane's 4 consecutive clusters share one Philox block
    const float4 g4 = (keyed && a.sample) ? gumbel4(a.seeds[r], kStreamCluster, (uint32_t)kq0 >> 2)
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
    const float gq[4] = {g4.x, g4.y, g4.z, g4.w};
    float kv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sc = acc[nt][q];
      kv[q] = (keyed && a.sample) ? sc * a.inv_tau + gq[q] : sc;
      if (keyed && a.dbg_scores && kq0 + q < pc) a.dbg_scores[(int64_t)r * pc + kq0 + q] = sc;
    }
    float* kr = a.keys + (keyed ? 0 : (int64_t)sp * a.part_stride) + (int64_t)r * a.key_stride + kq0;
    if (kq0 + 3 < pc) {
      *reinterpret_cast<float4*>(kr) = make_float4(kv[0], kv[1], kv[2], kv[3]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (kq0 + q < pc) kr[q] = kv[q];
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

// Four column tiles (B = 49-64) at d = 2048 in the streaming modes: two
// items per wave with the unrolled K walk (measured on the 2048-wide head at
// B = 64: 107 us against 118 us for one item per wave).
constexpr int kWideItems = 2;
static bool engine_wide(const Stage2mArgs& a, int mode) {
  const int64_t lim = (int64_t)1 << 31;
  return (mode == kGmDense || mode == kGmAll) && !a.sample && (a.B + 15) / 16 == 4 &&
         a.d == 8 * 256 && a.v * a.row_bytes < lim && (int64_t)a.c * a.c_row_bytes < lim;
}
static int engine_items(const Stage2mArgs& a, int mode) {
  return engine_wide(a, mode) ? kWideItems : kGmItems;
}

template <int MODE, int KC>
static hipError_t launch_engine_nt(const Stage2mArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                                   hipEvent_t e1) {
  if constexpr ((MODE == kGmDense || MODE == kGmAll) && KC == 256) {
    if (engine_wide(a, MODE)) {
      hipExtLaunchKernelGGL((gemm_engine_kernel<4, kWideItems, MODE, 256, 8>), dim3(grid),
                            dim3(kGmThreads), 0, s, e0, e1, 0, a);
      return hipGetLastError();
    }
  }
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

static int engine_grid(int64_t nrows16, int items_per_wave) {
  const int64_t per = (int64_t)kGmWaves * items_per_wave;
  const int64_t g = (nrows16 + per - 1) / per;
  return g < 1 ? 1 : (int)g;
}

hipError_t launch_stage1_mfma(const Stage1Args& a, bool int4, int B, hipStream_t s,
                              const Timing* tm, int* ksplit) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const int NT = (B + 15) / 16;
  *ksplit = 1;
  if (int4) {
    // tiles per workgroup: as many as keep at least 256 workgroups (one per
    // compute unit), at most 4 (2 from three column tiles on, for registers)
    int tpw = NT <= 2 ? 4 : 2;
    while (tpw > 1 && (a.ntiles + tpw - 1) / tpw < 256) tpw /= 2;
    const dim3 grid((a.ntiles + tpw - 1) / tpw), block(kS1qThreads);
#define FH_S1Q(N, T)                                                                         \
  if (NT == N && tpw == T) {                                                                 \
    hipExtLaunchKernelGGL(stage1_int4_mfma_kernel<N, T>, grid, block, 0, s, e0, e1, 0, a.q4,   \
                          a.q4s, a.H, (int)a.h_bytes, a.groups, a.ntiles, B, a);              \
    return hipGetLastError();                                                                \
  }
    FH_S1Q(1, 4) FH_S1Q(1, 2) FH_S1Q(1, 1)
    FH_S1Q(2, 4) FH_S1Q(2, 2) FH_S1Q(2, 1)
    FH_S1Q(3, 2) FH_S1Q(3, 1)
    FH_S1Q(4, 2) FH_S1Q(4, 1)
#undef FH_S1Q
    return hipErrorInvalidValue;
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
  m.raw_scores = a.raw_keys;
  *ksplit = S;
  if (nchunks <= kMaxKSplit * kScChunks) {
    // one round of loads per unit: at most kScChunks chunks per K slice
    const int smin = (nchunks + kScChunks - 1) / kScChunks;
    S = S < smin ? smin : S;
    m.ksplit = S;
    *ksplit = S;
    const dim3 grid((unsigned)(groups * S)), block(kGmThreads);
    // the values the first loads need, as leading scalar arguments
#define SC_ARGS m.base, m.H, (int)m.row_bytes, (int)m.h_bytes, m.c, m.d, m.B, m.ksplit, m
    switch ((B + 15) / 16) {
      case 1: hipExtLaunchKernelGGL(scores_mfma_kernel<1>, grid, block, 0, s, e0, e1, 0, SC_ARGS); break;
      case 2: hipExtLaunchKernelGGL(scores_mfma_kernel<2>, grid, block, 0, s, e0, e1, 0, SC_ARGS); break;
      case 3: hipExtLaunchKernelGGL(scores_mfma_kernel<3>, grid, block, 0, s, e0, e1, 0, SC_ARGS); break;
      case 4: hipExtLaunchKernelGGL(scores_mfma_kernel<4>, grid, block, 0, s, e0, e1, 0, SC_ARGS); break;
      default: return hipErrorInvalidValue;
    }
#undef SC_ARGS
    return hipGetLastError();
  }
  const int64_t units = groups * S;
  const int grid = (int)(units < 4096 ? units : 4096);
  return launch_engine_nt<kGmScores, kKC>(m, grid, s, e0, e1);
}

int stage2_mfma_grid() { return 4096; }

hipError_t launch_stream_all(const Stage2mArgs& a, const SelectArgs& sa, hipStream_t s,
                             const Timing* t1, const Timing* t2) {
  hipEvent_t e0 = t1 ? t1->start : nullptr, e1 = t1 ? t1->stop : nullptr;
  // one unit of kGmWaves items per workgroup, stage-1 units first in the
  // grid (the dispatcher starts them first)
  const int64_t items = a.n1 + (int64_t)a.c * (a.b / 16);
  const int per = kGmWaves * engine_items(a, a.q4 ? kGmAllQ4 : kGmAll);
  int64_t grid = (items + per - 1) / per;
  grid = grid < (1 << 20) ? grid : (1 << 20);
  const hipError_t e = a.q4 ? launch_engine<kGmAllQ4>(a, (int)grid, s, e0, e1)
                            : launch_engine<kGmAll>(a, (int)grid, s, e0, e1);
  if (e != hipSuccess) return e;
  return launch_select_fold(sa, a.B, s, t2);
}

hipError_t launch_stage2_mfma(const Stage2mArgs& a, bool dense, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  // flash: the union is known on the device only; launch for every cluster
  const int64_t items = dense ? (a.v + 15) / 16 : (int64_t)a.c * (a.b / 16);
  int grid = engine_grid(items, engine_items(a, dense ? kGmDense : kGmFlash));
  grid = grid < stage2_mfma_grid() ? grid : stage2_mfma_grid();
  hipError_t e = dense ? launch_engine<kGmDense>(a, grid, s, e0, e1)
                       : launch_engine<kGmFlash>(a, grid, s, e0, e1);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(finalize_kernel, dim3(a.B), dim3(256), 0, s,
                     static_cast<const uint64_t*>(a.part_best),
                     static_cast<const float2*>(a.part_lse), grid, a.with_lse, a);
  return hipGetLastError();
}

}  // namespace fh
