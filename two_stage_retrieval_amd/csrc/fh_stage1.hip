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
#include "fh_decode_b1.h"

namespace fh {


template <typename TE, int NCH, int IPT, bool INT4, bool SELECT>
__global__ __launch_bounds__(kS1Threads) void stage1_kernel(Stage1Args a) {
  __shared__ SelSmem sm;
  __shared__ float s_h[INT4 ? FH_MAX_ROW_BYTES / 2 : 1];
  const int r = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint8_t* hrow = a.H + (int64_t)r * a.h_bytes;
  const uint64_t seed = a.sample ? a.seeds[r] : 0ull;
  float* keys = a.keys + (int64_t)r * a.key_stride;
  float* dbg = a.dbg_scores ? a.dbg_scores + (int64_t)r * a.c : nullptr;
  float* raw = a.raw ? a.raw + (int64_t)r * a.key_stride : nullptr;
  const int w0 = blockIdx.x * kS1Waves + wave, wstride = gridDim.x * kS1Waves;

  if constexpr (!INT4) {
    uint4 hraw[NCH];
    float hreg[NCH][Chunk<TE>::kElems];
    load_h_raw<NCH>(hrow, a.nchunk, lane, hraw);
    score_rows<TE, NCH, SELECT>(a, keys, nullptr, dbg, seed, hraw, hreg, lane, w0, wstride, raw);
  } else {
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(hrow);
    for (int i = t; i < a.d; i += kS1Threads) s_h[i] = __uint_as_float((uint32_t)hb[i] << 16);
    __syncthreads();
    score_int4_tiles<SELECT>(a, keys, nullptr, dbg, seed, s_h, lane, w0, wstride, nullptr, raw);
  }
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
  uint32_t u[IPT];
  select_load_keys<IPT, true>(keys, (int)a.key_stride, u);
  int p = a.p;
  if (a.ad.on) {  // the adaptive count, on the plain scores
    if (raw) {
      uint32_t us[IPT];
      select_load_keys<IPT, true>(raw, (int)a.key_stride, us);
      p = adaptive_count<kS1Threads, IPT>(us, a.c, a.ad, a.p, sm);
    } else {
      p = adaptive_count<kS1Threads, IPT>(u, a.c, a.ad, a.p, sm);
    }
    if (a.ad.out_p && t == 0) a.ad.out_p[r] = p;
  }
  select_from_keys<kS1Threads, IPT, true>(u, a.c, p, a.zcut, a.sel + (int64_t)r * a.sel_stride,
                                          a.masks, r, a.error, sm, nullptr,
                                          a.ad.on ? a.p : 0);
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
int decode_b1_grid(int c, int p, int nchunk, int ntiles, int64_t nrows, bool int4,
                   int num_cu) {
  if (!stage1_selects(c) || num_cu < 1 || p < 1 || p > kDecodeB1MaxP) return 0;
  const int nch = (nchunk + kWave - 1) / kWave;
  if (nch < 1 || nch > 8) return 0;
  const int R = nch <= 2 ? 8 : 4;
  const int64_t units1 = int4 ? 2 * (int64_t)ntiles : (c + kS1Rows - 1) / kS1Rows;
  const int64_t units2 = (nrows + R - 1) / R;
  const int64_t units = units1 > units2 ? units1 : units2;
  int64_t g = (units + kS1Waves - 1) / kS1Waves;
  if (g > num_cu) g = num_cu;  // one resident workgroup per compute unit
  if (g > kDecodeB1MaxGrid) g = kDecodeB1MaxGrid;  // slots the merge's polling wave tracks
  return (int)(g < 1 ? 1 : g);
}


hipError_t decode_b1_occupancy(int dtype, bool int4, int nchunk, int c, int* blocks) {
  // the fewer of the two variants' resident workgroups
  int plain = 0, adapt = 0;
  hipError_t e = decode_b1_occupancy_impl<false>(dtype, int4, nchunk, c, &plain);
  if (e == hipSuccess) e = decode_b1_occupancy_adaptive(dtype, int4, nchunk, c, &adapt);
  *blocks = plain < adapt ? plain : adapt;
  return e;
}

hipError_t launch_decode_b1(const DecodeB1Args& a, int dtype, bool int4, int grid, bool coop,
                            hipStream_t s, const Timing* tm) {
  if (a.s1.ad.on) return launch_decode_b1_adaptive(a, dtype, int4, grid, coop, s, tm);
  return launch_decode_b1_impl<false>(a, dtype, int4, grid, coop, s, tm);
}

}  // namespace fh

// The decode kernel's timeline (the measurement build's hooks, see
// fh_trace.h): copied to the host and cleared.
extern "C" int flashhead_trace_read(uint64_t* host, int64_t max_words, int64_t* words,
                                    int64_t* clock_khz) {
  if (!words || !clock_khz) return FH_ERR_INVALID_ARG;
  *words = 0;
  *clock_khz = 0;
#ifdef FH_TRACE
  if (!host || max_words < fh::kTraceWords) return FH_ERR_INVALID_ARG;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return FH_ERR_HIP;
  const size_t bytes = (size_t)fh::kTraceWords * 8;
  if (hipMemcpyFromSymbol(host, HIP_SYMBOL(fh::fh_trace_buf), bytes, 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return FH_ERR_HIP;
  void* dptr = nullptr;
  if (hipGetSymbolAddress(&dptr, HIP_SYMBOL(fh::fh_trace_buf)) != hipSuccess ||
      hipMemset(dptr, 0, bytes) != hipSuccess)
    return FH_ERR_HIP;
  *words = fh::kTraceWords;
  *clock_khz = khz;
  return FH_OK;
#else
  (void)host;
  (void)max_words;
  return FH_ERR_UNSUPPORTED;
#endif
}
