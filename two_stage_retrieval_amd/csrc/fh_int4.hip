// Stage-1 scores on INT4 centroids (notes, Module 3: stage 1 may run on
// 4-bit centroids because it only shortlists; stage 2 stays bf16).
//
// s_k = sum_g scale[k, g] * sum_{j in group g} q[k, j] * h[j]
//
// Codes are stored in 16-row group tiles: tile (t, g) is 1024 bytes, one
// 16-byte word per lane; lane l owns row 16t + (l mod 16) and the 32 columns
// 128g + 32(l div 16) + [0, 32), two codes per byte (low nibble first).  A
// wave streams tile row t group by group with one coalesced 1 KB load per
// group; products of 4-bit integers with bf16 h are exact in fp32.  The four
// lanes that share a row combine their partial sums at the end.
#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

constexpr int kI4Threads = 256;
constexpr int kI4Waves = kI4Threads / kWave;

__global__ __launch_bounds__(kI4Threads) void int4_gemv_kernel(Int4Args a) {
  extern __shared__ float s_h[];
  const int r = blockIdx.y;
  const uint16_t* hrow = a.H + (int64_t)r * a.d;
  for (int i = threadIdx.x; i < a.d; i += kI4Threads) s_h[i] = __uint_as_float((uint32_t)hrow[i] << 16);
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, rin = lane & 15;
  const uint64_t seed = a.sample ? a.seeds[r] : 0ull;
  const int G = a.groups;
  for (int tile = blockIdx.x * kI4Waves + wave; tile < a.ntiles; tile += gridDim.x * kI4Waves) {
    const uint4* codes = reinterpret_cast<const uint4*>(a.codes) + (int64_t)tile * G * kWave + lane;
    const uint16_t* sc = a.scales + (int64_t)tile * G * 16 + rin;
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
    if (q == 0 && row < a.c) {
      float key = acc;
      if (a.sample) key = acc * a.inv_tau + gumbel(seed, kStreamCluster, (uint32_t)row);
      a.keys_out[(int64_t)r * a.key_stride + row] = key;
      if (a.dbg_scores) a.dbg_scores[(int64_t)r * a.key_stride + row] = acc;
    }
  }
}

hipError_t launch_int4_gemv(const Int4Args& a, int B, hipStream_t s, const Timing* tm) {
  hipEvent_t e0 = tm ? tm->start : nullptr, e1 = tm ? tm->stop : nullptr;
  int blocks = (a.ntiles + kI4Waves - 1) / kI4Waves;
  if (blocks > 2048) blocks = 2048;
  hipExtLaunchKernelGGL(int4_gemv_kernel, dim3(blocks, B), dim3(kI4Threads),
                        (uint32_t)(a.d * sizeof(float)), s, e0, e1, 0, a);
  return hipGetLastError();
}

}  // namespace fh
