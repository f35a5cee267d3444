// Row-dot kernels: one wave computes full dot products of R rows of a
// row-major matrix with one hidden vector h (GEMV family, batch rows on
// grid.y).  Two epilogues:
//   gather  stage-2 exact logits of the candidate rows of the selected
//           clusters (notes, Overall architecture and Module 1), fused with
//           the decode (Formula 2 argmax or Formula 3 Gumbel-max sample);
//   dense   the dense head z = E h (Formula 1) with the same decode.
//
// Memory layout: lane l of a wave owns the 16-byte chunks l, l+64, ... of a
// row, so a wave reads each row as one contiguous, fully coalesced span and
// keeps its slice of h in registers for all rows it visits.  The gather
// epilogue reads the cluster-major copy of E built at prepare time: the b
// candidate rows of a cluster are one contiguous block, and C2T is read only
// for the token ids (in parallel with the row loads, not in their address
// chain).
#include "fh_device.h"
#include "fh_internal.h"

// Optional timeline hook for measurement builds (empty in the library).
#ifndef FH_S2_TRACE
#define FH_S2_TRACE(slot)
#endif

namespace fh {

constexpr int kRowdotThreads = 256;
constexpr int kRowdotWaves = kRowdotThreads / kWave;

template <typename TE, int NCH, int R, int MODE>
__global__ __launch_bounds__(kRowdotThreads) void rowdot_kernel(RowdotArgs a) {
  using CK = Chunk<TE>;
  constexpr int EPC = CK::kElems;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blockIdx.y;
  FH_S2_TRACE(0);

  float hreg[NCH][EPC];
  {
    const uint8_t* hrow = a.H + (int64_t)r * a.h_bytes;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = lane + kWave * i;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (ch < a.nchunk) w = *reinterpret_cast<const uint4*>(hrow + (int64_t)ch * 16);
      CK::unpack(w, hreg[i]);
    }
  }
  const uint64_t seed = a.sample ? a.seeds[r] : 0ull;
  const int64_t ngroups = (a.nrows + R - 1) / R;
  const int64_t wstride = (int64_t)gridDim.x * kRowdotWaves;
  uint64_t best = 0;
  Lse lse = lse_empty();

  for (int64_t g = (int64_t)blockIdx.x * kRowdotWaves + wave; g < ngroups; g += wstride) {
    const int64_t row0 = g * R;
    int64_t phys[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      int64_t i = row0 + rr;
      if (i >= a.nrows) i = a.nrows - 1;  // tail: reread the last row, result dropped
      if constexpr (MODE == kRowGather) {
        const int64_t j = i / a.b;
        int64_t k = a.sel[(int64_t)r * a.sel_stride + j];
        k = k < 0 ? 0 : (k >= a.nclusters ? a.nclusters - 1 : k);  // never leave the table
        phys[rr] = k * a.b + (i - j * a.b);  // row of the cluster-major copy
      } else {
        phys[rr] = i;
      }
    }
    uint4 data[R][NCH];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const uint8_t* rowp = a.base + phys[rr] * a.row_bytes;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ch = lane + kWave * i;
        data[rr][i] = (ch < a.nchunk)
                          ? *reinterpret_cast<const uint4*>(rowp + (int64_t)ch * 16)
                          : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // token ids of the gathered rows (lane rr fetches row rr's id)
    int64_t myphys = phys[0];
#pragma unroll
    for (int rr = 1; rr < R; ++rr)
      if (lane == rr) myphys = phys[rr];
    uint32_t mytok = (uint32_t)myphys;
    if constexpr (MODE == kRowGather) {
      if (lane < R) mytok = (uint32_t)a.c2t[myphys];
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
#pragma unroll
    for (int rr = 1; rr < R; ++rr)
      if (lane == rr) mine = acc[rr];
    const int64_t myrow = row0 + lane;
    const bool valid = lane < R && myrow < a.nrows;
    {
      if (valid) {
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
  // ---- block reduction; workgroup 0 of this batch row finishes -----------
  // Every workgroup stores its partial (best key, lse pair) into its own slot
  // with device-scope stores, waits for them to complete and counts itself
  // arrived (spread counters, fh_device.h); workgroup 0, after its own share,
  // waits for all arrivals and folds the partials in a fixed order.  No
  // same-address atomics, no L2 write-back or invalidate on this path.
  __shared__ uint64_t s_best[kRowdotThreads];
  __shared__ float2 s_lse[kRowdotThreads];
  FH_S2_TRACE(1);
  best = wave_max_u64(best);
  if (a.out_lse) lse = wave_lse(lse);
  if (lane == 0) {
    s_best[wave] = best;
    s_lse[wave] = make_float2(lse.m, lse.s);
  }
  __syncthreads();
  uint64_t* pbest = a.part_best + (int64_t)r * gridDim.x;
  unsigned long long* plse =
      reinterpret_cast<unsigned long long*>(a.lse_part + (int64_t)r * gridDim.x);
  uint32_t* ctr = a.counters + (int64_t)r * kArriveWords;
  if (threadIdx.x == 0) {
    uint64_t bb = s_best[0];
    Lse ll{s_lse[0].x, s_lse[0].y};
    for (int w = 1; w < kRowdotWaves; ++w) {
      bb = s_best[w] > bb ? s_best[w] : bb;
      ll = lse_merge(ll, Lse{s_lse[w].x, s_lse[w].y});
    }
    if (blockIdx.x != 0) {
      __hip_atomic_store(pbest + blockIdx.x, bb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.out_lse) {
        const unsigned long long packed =
            ((unsigned long long)__float_as_uint(ll.s) << 32) | __float_as_uint(ll.m);
        __hip_atomic_store(plse + blockIdx.x, packed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0);  // the partial is visible device-wide
      arrive(ctr, blockIdx.x);
    } else {
      s_best[kRowdotThreads - 1] = bb;  // workgroup 0's own partial
      s_lse[kRowdotThreads - 1] = make_float2(ll.m, ll.s);
    }
  }
  if (blockIdx.x != 0) return;
  __syncthreads();
  const uint64_t own_best = s_best[kRowdotThreads - 1];
  const float2 own_lse = s_lse[kRowdotThreads - 1];
  if (wave == 0) wait_arrivals(ctr, gridDim.x - 1, lane);
  __syncthreads();
  FH_S2_TRACE(2);
  // deterministic fold: fixed strided order, fixed tree
  uint64_t bb = threadIdx.x == 0 ? own_best : 0ull;
  Lse ll = threadIdx.x == 0 ? Lse{own_lse.x, own_lse.y} : lse_empty();
  for (int j = 1 + threadIdx.x; j < (int)gridDim.x; j += kRowdotThreads) {
    const uint64_t x = __hip_atomic_load(pbest + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bb = x > bb ? x : bb;
    if (a.out_lse) {
      const unsigned long long pr =
          __hip_atomic_load(plse + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ll = lse_merge(ll, Lse{__uint_as_float((uint32_t)pr), __uint_as_float((uint32_t)(pr >> 32))});
    }
  }
  __syncthreads();
  s_best[threadIdx.x] = bb;
  s_lse[threadIdx.x] = make_float2(ll.m, ll.s);
  __syncthreads();
  for (int w = kRowdotThreads / 2; w >= 1; w >>= 1) {
    if (threadIdx.x < w) {
      if (s_best[threadIdx.x + w] > s_best[threadIdx.x]) s_best[threadIdx.x] = s_best[threadIdx.x + w];
      if (a.out_lse) {
        const Lse x = lse_merge(Lse{s_lse[threadIdx.x].x, s_lse[threadIdx.x].y},
                                Lse{s_lse[threadIdx.x + w].x, s_lse[threadIdx.x + w].y});
        s_lse[threadIdx.x] = make_float2(x.m, x.s);
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.out_tokens[r] = (int32_t)key_id(s_best[0]);
    if (a.out_lse) a.out_lse[r] = s_lse[0].x + logf(s_lse[0].y);
  }
  FH_S2_TRACE(3);
}

// Rows per wave per step: enough bytes in flight per wave without spilling.
template <int NCH> constexpr int rows_for() { return NCH <= 2 ? 8 : 4; }

template <typename TE, int MODE>
static hipError_t launch_t(const RowdotArgs& a, int B, int grid_x, hipStream_t s,
                           const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  const dim3 grid(grid_x, B), block(kRowdotThreads);
  const int nch = (a.nchunk + kWave - 1) / kWave;
#define FH_ROWDOT_CASE(N)                                                              \
  case N:                                                                              \
    hipExtLaunchKernelGGL((rowdot_kernel<TE, N, rows_for<N>(), MODE>), grid, block, 0, s, e0, \
                          e1, 0, a);                                                   \
    break;
  switch (nch) {
    FH_ROWDOT_CASE(1)
    FH_ROWDOT_CASE(2)
    FH_ROWDOT_CASE(3)
    FH_ROWDOT_CASE(4)
    FH_ROWDOT_CASE(5)
    FH_ROWDOT_CASE(6)
    FH_ROWDOT_CASE(7)
    FH_ROWDOT_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef FH_ROWDOT_CASE
  return hipGetLastError();
}

int rowdot_grid(int64_t nrows, int nchunk, int mode) {
  const int nch = (nchunk + kWave - 1) / kWave;
  const int R = nch <= 2 ? 8 : 4;
  const int64_t groups = (nrows + R - 1) / R;
  int64_t blocks = (groups + kRowdotWaves - 1) / kRowdotWaves;
  // dense: cap at a few resident blocks per CU and loop (256 CUs)
  const int64_t cap = mode == kRowDense ? 2048 : 8192;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

hipError_t launch_rowdot(const RowdotArgs& a, int mode, int dtype, int B, int grid_x,
                         hipStream_t s, const Timing* tm) {
  if (dtype == FH_DTYPE_BF16) {
    if (mode == kRowGather) return launch_t<bf16_t, kRowGather>(a, B, grid_x, s, tm);
    return launch_t<bf16_t, kRowDense>(a, B, grid_x, s, tm);
  }
  if (mode == kRowGather) return launch_t<float, kRowGather>(a, B, grid_x, s, tm);
  return launch_t<float, kRowDense>(a, B, grid_x, s, tm);
}

}  // namespace fh
