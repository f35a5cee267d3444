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
#include "fh_select.h"

// Optional timeline hook for measurement builds (empty in the library).
#ifndef FH_S1_TRACE
#define FH_S1_TRACE(slot)
#endif

namespace fh {

constexpr int kS1Threads = 512;
constexpr int kS1Waves = kS1Threads / kWave;
constexpr int kS1R = 4;

template <typename TE, int NCH, int IPT, bool INT4, bool SELECT>
__global__ __launch_bounds__(kS1Threads) void stage1_kernel(Stage1Args a) {
  using CK = Chunk<TE>;
  constexpr int EPC = CK::kElems;
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

  auto publish = [&](int row, float score) {
    const float key =
        a.sample ? score * a.inv_tau + gumbel(seed, kStreamCluster, (uint32_t)row) : score;
    if constexpr (SELECT) {
      __hip_atomic_store(keys + row, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      keys[row] = key;
    }
    if (dbg) dbg[row] = score;
  };

  if constexpr (!INT4) {
    float hreg[NCH][EPC];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = lane + kWave * i;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (ch < a.nchunk) w = *reinterpret_cast<const uint4*>(hrow + (int64_t)ch * 16);
      CK::unpack(w, hreg[i]);
    }
    const int ngroups = (a.c + kS1R - 1) / kS1R;
    for (int g = blockIdx.x * kS1Waves + wave; g < ngroups; g += gridDim.x * kS1Waves) {
      const int row0 = g * kS1R;
      uint4 data[kS1R][NCH];
#pragma unroll
      for (int rr = 0; rr < kS1R; ++rr) {
        const int row = row0 + rr < a.c ? row0 + rr : a.c - 1;
        const uint8_t* rowp = a.C + (int64_t)row * a.row_bytes;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int ch = lane + kWave * i;
          data[rr][i] = ch < a.nchunk ? *reinterpret_cast<const uint4*>(rowp + (int64_t)ch * 16)
                                      : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      float acc[kS1R];
#pragma unroll
      for (int rr = 0; rr < kS1R; ++rr) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) s = CK::dot(data[rr][i], hreg[i], s);
        acc[rr] = wave_sum(s);
      }
      float mine = acc[0];
#pragma unroll
      for (int rr = 1; rr < kS1R; ++rr)
        if (lane == rr) mine = acc[rr];
      if (lane < kS1R && row0 + lane < a.c) publish(row0 + lane, mine);
    }
  } else {
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(hrow);
    for (int i = t; i < a.d; i += kS1Threads) s_h[i] = __uint_as_float((uint32_t)hb[i] << 16);
    __syncthreads();
    const int q = lane >> 4, rin = lane & 15;
    const int G = a.groups;
    for (int tile = blockIdx.x * kS1Waves + wave; tile < a.ntiles;
         tile += gridDim.x * kS1Waves) {
      const uint4* codes =
          reinterpret_cast<const uint4*>(a.q4) + (int64_t)tile * G * kWave + lane;
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
      if (q == 0 && row < a.c) publish(row, acc);
    }
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
  select_block<kS1Threads, IPT, true>(keys, a.c, (int)a.key_stride, a.p,
                                      a.sel + (int64_t)r * a.sel_stride, a.masks, r, a.error, sm);
  FH_S1_TRACE(3);
}

int stage1_blocks(const Stage1Args& a, bool int4) {
  const int64_t units = int4 ? a.ntiles : (a.c + kS1R - 1) / kS1R;
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

}  // namespace fh
