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

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// stage 1, bf16 centroids.  Block: 32 centroid rows x all batch columns.
// 8 waves = 2 row tiles x 4 quarters of K; each wave issues all its A loads
// first (16 rows x d/4 columns), then walks K with B fragments from H.  The
// four K-partials are summed through LDS in fixed order.
// ---------------------------------------------------------------------------
constexpr int kS1mThreads = 512;
constexpr int kS1mRows = 32;
constexpr int kS1mSteps = 16;  // k-steps of 32 per load round

template <int NT>
__global__ __launch_bounds__(kS1mThreads) void stage1_mfma_kernel(Stage1Args a, int B) {
  __shared__ float red[4][NT * 16][kS1mRows + 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mt = wave >> 2, kq = wave & 3;
  const int qd = a.d / 4;            // columns per K-quarter (multiple of 32)
  const int ksteps = qd / 32;
  const int slice = lane >> 4, lr = lane & 15;
  int arow = blockIdx.x * kS1mRows + mt * 16 + lr;
  arow = arow < a.c ? arow : a.c - 1;
  const uint8_t* ap = a.C + (int64_t)arow * a.row_bytes + (int64_t)(kq * qd + 8 * slice) * 2;
  const uint8_t* hp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int j = nt * 16 + lr;
    j = j < B ? j : B - 1;
    hp[nt] = a.H + (int64_t)j * a.h_bytes + (int64_t)(kq * qd + 8 * slice) * 2;
  }
  f32x4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ksteps; s0 += kS1mSteps) {
    uint4 av[kS1mSteps];
#pragma unroll
    for (int u = 0; u < kS1mSteps; ++u)
      av[u] = s0 + u < ksteps ? *reinterpret_cast<const uint4*>(ap + (int64_t)(s0 + u) * 64)
                              : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < kS1mSteps; ++u) {
      if (s0 + u >= ksteps) break;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint4 bv = *reinterpret_cast<const uint4*>(hp[nt] + (int64_t)(s0 + u) * 64);
        acc[nt] = mfma_bf16(av[u], bv, acc[nt]);
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[kq][nt * 16 + lr][mt * 16 + 4 * slice + q] = acc[nt][q];
  __syncthreads();
  // outputs (batch row r, centroid k): consecutive threads take consecutive k
  for (int o = threadIdx.x; o < NT * 16 * kS1mRows; o += kS1mThreads) {
    const int r = o / kS1mRows, kk = o % kS1mRows;
    const int k = blockIdx.x * kS1mRows + kk;
    if (r >= B || k >= a.c) continue;
    const float s = ((red[0][r][kk] + red[1][r][kk]) + red[2][r][kk]) + red[3][r][kk];
    const float key = a.sample ? s * a.inv_tau + gumbel(a.seeds[r], kStreamCluster, (uint32_t)k) : s;
    a.keys[(int64_t)r * a.key_stride + k] = key;
    if (a.dbg_scores) a.dbg_scores[(int64_t)r * a.key_stride + k] = s;
  }
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
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = tile * 16 + 4 * slice + q;
      if (k >= a.c) continue;
      const float s = tot[nt][q];
      const float key =
          a.sample ? s * a.inv_tau + gumbel(a.seeds[r], kStreamCluster, (uint32_t)k) : s;
      a.keys[(int64_t)r * a.key_stride + k] = key;
      if (a.dbg_scores) a.dbg_scores[(int64_t)r * a.key_stride + k] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// stage 2 (and the batched dense head).  Work item = 16 consecutive rows:
// FLASH mode, 16 rows of a selected cluster in the cluster-major copy of E
// (cluster ulist[i / (b/16)]); DENSE mode, rows 16 i .. 16 i + 15 of E.  A
// wave computes the 16 x B logits of an item and folds, per batch row, the
// candidates the row selected (its bit in the cluster's mask) into a running
// best decode key and log-sum-exp; the block writes one partial per row.
// ---------------------------------------------------------------------------
constexpr int kS2mThreads = 256;
constexpr int kS2mWaves = kS2mThreads / kWave;
constexpr int kS2mSteps = 16;

template <int NT, bool DENSE>
__global__ __launch_bounds__(kS2mThreads) void stage2_mfma_kernel(Stage2mArgs a) {
  __shared__ uint64_t s_best[kS2mWaves][NT * 16];
  __shared__ float2 s_lse[kS2mWaves][NT * 16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = lane >> 4, lr = lane & 15;
  const int B = a.B;
  const int sub = a.b / 16;  // items per cluster (FLASH)
  const int64_t nitems = DENSE ? (a.v + 15) / 16 : (int64_t)(*a.ucount) * sub;
  const int ksteps = a.d / 32;
  const uint8_t* hp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int j = nt * 16 + lr;
    j = j < B ? j : B - 1;
    hp[nt] = a.H + (int64_t)j * a.h_bytes + (int64_t)(8 * slice) * 2;
  }
  uint64_t best[NT];
  Lse lse[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) { best[nt] = 0ull; lse[nt] = lse_empty(); }

  for (int64_t it = (int64_t)blockIdx.x * kS2mWaves + wave; it < nitems;
       it += (int64_t)gridDim.x * kS2mWaves) {
    int64_t row0, k = 0;
    uint64_t mask;
    if constexpr (DENSE) {
      row0 = it * 16;
      mask = ~0ull;
    } else {
      k = a.ulist[it / sub];
      row0 = k * a.b + (it % sub) * 16;
      mask = a.masks[k];
    }
    int64_t arow = row0 + lr;
    if constexpr (DENSE) arow = arow < a.v ? arow : a.v - 1;
    const uint8_t* ap = a.base + arow * a.row_bytes + (int64_t)(8 * slice) * 2;
    f32x4_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ksteps; s0 += kS2mSteps) {
      uint4 av[kS2mSteps];
#pragma unroll
      for (int u = 0; u < kS2mSteps; ++u)
        av[u] = s0 + u < ksteps ? *reinterpret_cast<const uint4*>(ap + (int64_t)(s0 + u) * 64)
                                : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < kS2mSteps; ++u) {
        if (s0 + u >= ksteps) break;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint4 bv = *reinterpret_cast<const uint4*>(hp[nt] + (int64_t)(s0 + u) * 64);
          acc[nt] = mfma_bf16(av[u], bv, acc[nt]);
        }
      }
    }
    // epilogue: rows 4 slice + q of the item, batch column nt*16 + lr
    uint32_t tok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = row0 + 4 * slice + q;
      if constexpr (DENSE) tok[q] = (uint32_t)row;
      else tok[q] = (uint32_t)a.c2t[row];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = nt * 16 + lr;
      const bool rowsel = r < B && ((mask >> r) & 1ull);
      const uint64_t seed = (a.sample && r < B) ? a.seeds[r] : 0ull;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = row0 + 4 * slice + q;
        const bool ok = rowsel && (!DENSE || row < a.v);
        if (!ok) continue;
        const float x = acc[nt][q];
        const float xs = x * a.inv_tau;
        const float kx = a.sample ? xs + gumbel(seed, kStreamToken, tok[q]) : x;
        const uint64_t key = decode_key(kx, tok[q]);
        best[nt] = key > best[nt] ? key : best[nt];
        if (a.with_lse) lse[nt] = lse_add(lse[nt], xs);
        if (!DENSE && a.dbg_logits) {
          // position of cluster k in row r's ascending selection
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
  for (int r = threadIdx.x; r < B; r += kS2mThreads) {
    uint64_t bb = s_best[0][r];
    Lse ll{s_lse[0][r].x, s_lse[0][r].y};
    for (int w = 1; w < kS2mWaves; ++w) {
      bb = s_best[w][r] > bb ? s_best[w][r] : bb;
      ll = lse_merge(ll, Lse{s_lse[w][r].x, s_lse[w][r].y});
    }
    a.part_best[(int64_t)blockIdx.x * B + r] = bb;
    if (a.with_lse) a.part_lse[(int64_t)blockIdx.x * B + r] = make_float2(ll.m, ll.s);
  }
}

// per batch row: fold the per-block partials into the token (and lse);
// block 0 also clears the cluster masks of this call's union
__global__ __launch_bounds__(256) void finalize_kernel(Stage2mArgs a, int nblocks) {
  __shared__ uint64_t s_b[256];
  __shared__ float2 s_l[256];
  const int r = blockIdx.x;
  uint64_t bb = 0ull;
  Lse ll = lse_empty();
  for (int j = threadIdx.x; j < nblocks; j += 256) {
    const uint64_t x = a.part_best[(int64_t)j * a.B + r];
    bb = x > bb ? x : bb;
    if (a.with_lse) {
      const float2 pl = a.part_lse[(int64_t)j * a.B + r];
      ll = lse_merge(ll, Lse{pl.x, pl.y});
    }
  }
  s_b[threadIdx.x] = bb;
  s_l[threadIdx.x] = make_float2(ll.m, ll.s);
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) {
      if (s_b[threadIdx.x + w] > s_b[threadIdx.x]) s_b[threadIdx.x] = s_b[threadIdx.x + w];
      const Lse x = lse_merge(Lse{s_l[threadIdx.x].x, s_l[threadIdx.x].y},
                              Lse{s_l[threadIdx.x + w].x, s_l[threadIdx.x + w].y});
      s_l[threadIdx.x] = make_float2(x.m, x.s);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.out_tokens[r] = (int32_t)key_id(s_b[0]);
    if (a.out_lse) a.out_lse[r] = s_l[0].x + logf(s_l[0].y);
  }
  if (r == 0 && a.masks) {
    const int u = *a.ucount;
    for (int i = threadIdx.x; i < u; i += 256) a.masks[a.ulist[i]] = 0ull;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
bool batched_supported(int dtype, int d, int B, bool int4) {
  if (dtype != FH_DTYPE_BF16 || B < 2 || B > FH_MAX_BATCH) return false;
  return d % 128 == 0;
}

hipError_t launch_stage1_mfma(const Stage1Args& a, bool int4, int B, hipStream_t s,
                              const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const int NT = (B + 15) / 16;
  if (int4) {
    const dim3 grid((a.ntiles + kS1qThreads / kWave - 1) / (kS1qThreads / kWave));
    const uint32_t shm = 0;
    switch (NT) {
      case 1: hipExtLaunchKernelGGL(stage1_int4_mfma_kernel<1>, grid, dim3(kS1qThreads), shm, s, e0, e1, 0, a, B); break;
      case 2: hipExtLaunchKernelGGL(stage1_int4_mfma_kernel<2>, grid, dim3(kS1qThreads), shm, s, e0, e1, 0, a, B); break;
      case 3: hipExtLaunchKernelGGL(stage1_int4_mfma_kernel<3>, grid, dim3(kS1qThreads), shm, s, e0, e1, 0, a, B); break;
      case 4: hipExtLaunchKernelGGL(stage1_int4_mfma_kernel<4>, grid, dim3(kS1qThreads), shm, s, e0, e1, 0, a, B); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 grid((a.c + kS1mRows - 1) / kS1mRows);
  switch (NT) {
    case 1: hipExtLaunchKernelGGL(stage1_mfma_kernel<1>, grid, dim3(kS1mThreads), 0, s, e0, e1, 0, a, B); break;
    case 2: hipExtLaunchKernelGGL(stage1_mfma_kernel<2>, grid, dim3(kS1mThreads), 0, s, e0, e1, 0, a, B); break;
    case 3: hipExtLaunchKernelGGL(stage1_mfma_kernel<3>, grid, dim3(kS1mThreads), 0, s, e0, e1, 0, a, B); break;
    case 4: hipExtLaunchKernelGGL(stage1_mfma_kernel<4>, grid, dim3(kS1mThreads), 0, s, e0, e1, 0, a, B); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int stage2_mfma_grid() { return 1024; }

hipError_t launch_stage2_mfma(const Stage2mArgs& a, bool dense, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const int NT = (a.B + 15) / 16;
  const dim3 grid(stage2_mfma_grid()), block(kS2mThreads);
#define FH_S2M(N)                                                                             \
  case N:                                                                                     \
    if (dense) hipExtLaunchKernelGGL((stage2_mfma_kernel<N, true>), grid, block, 0, s, e0, e1, 0, a); \
    else hipExtLaunchKernelGGL((stage2_mfma_kernel<N, false>), grid, block, 0, s, e0, e1, 0, a); \
    break;
  switch (NT) {
    FH_S2M(1)
    FH_S2M(2)
    FH_S2M(3)
    FH_S2M(4)
    default: return hipErrorInvalidValue;
  }
#undef FH_S2M
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(finalize_kernel, dim3(a.B), dim3(256), 0, s, a, stage2_mfma_grid());
  return hipGetLastError();
}

}  // namespace fh
