// Prepare-time device work (not on the decode path).
//  * centroid means (notes, Module 1 / Formula 5): c_k = unit(sum of the
//    cluster's rows), bf16 by round-to-nearest-even for bf16 heads;
//  * the cluster-major copy of E: row k*b + j holds E[C2T[k, j]], so that the
//    candidate rows of one cluster form one contiguous block.
#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

constexpr int kPrepThreads = 256;

template <typename TE>
__device__ __forceinline__ float load_elem(const uint8_t* row, int col);
template <>
__device__ __forceinline__ float load_elem<float>(const uint8_t* row, int col) {
  return reinterpret_cast<const float*>(row)[col];
}
template <>
__device__ __forceinline__ float load_elem<bf16_t>(const uint8_t* row, int col) {
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[col] << 16);
}

template <typename TE>
__global__ __launch_bounds__(kPrepThreads) void centroid_means_kernel(
    const uint8_t* E, int64_t row_bytes, int d, const int32_t* c2t, int b, void* C) {
  extern __shared__ float s_sum[];
  __shared__ float s_red[kPrepThreads / kWave];
  const int k = blockIdx.x;
  float ss = 0.0f;
  for (int col = threadIdx.x; col < d; col += kPrepThreads) {
    float acc = 0.0f;
    for (int j = 0; j < b; ++j)
      acc += load_elem<TE>(E + (int64_t)c2t[(int64_t)k * b + j] * row_bytes, col);
    s_sum[col] = acc;
    ss = fmaf(acc, acc, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & (kWave - 1)) == 0) s_red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
  for (int w = 0; w < kPrepThreads / kWave; ++w) tot += s_red[w];
  const float inv = tot > 0.0f ? 1.0f / sqrtf(tot) : 0.0f;
  for (int col = threadIdx.x; col < d; col += kPrepThreads) {
    const float x = s_sum[col] * inv;
    if constexpr (sizeof(TE) == sizeof(float))
      reinterpret_cast<float*>(C)[(int64_t)k * d + col] = x;
    else
      reinterpret_cast<uint16_t*>(C)[(int64_t)k * d + col] = f32_to_bf16_rne(x);
  }
}

hipError_t launch_centroid_means(const uint8_t* E, int64_t row_bytes, int dtype, int d,
                                 const int32_t* c2t, int c, int b, void* C, hipStream_t s) {
  const size_t shm = (size_t)d * sizeof(float);
  if (dtype == FH_DTYPE_BF16)
    hipLaunchKernelGGL(centroid_means_kernel<bf16_t>, dim3(c), dim3(kPrepThreads), shm, s, E,
                       row_bytes, d, c2t, b, C);
  else
    hipLaunchKernelGGL(centroid_means_kernel<float>, dim3(c), dim3(kPrepThreads), shm, s, E,
                       row_bytes, d, c2t, b, C);
  return hipGetLastError();
}

// one wave per destination row, 16-byte chunks
__global__ __launch_bounds__(kPrepThreads) void cluster_major_copy_kernel(
    const uint8_t* E, int64_t lde_bytes, const int32_t* c2t, int64_t v, int nchunk,
    uint8_t* Ec, int64_t row_bytes) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (kPrepThreads / kWave);
  for (int64_t dst = (int64_t)blockIdx.x * (kPrepThreads / kWave) + (threadIdx.x >> 6); dst < v;
       dst += waves) {
    const uint8_t* src = E + (int64_t)c2t[dst] * lde_bytes;
    uint8_t* out = Ec + dst * row_bytes;
    for (int ch = lane; ch < nchunk; ch += kWave)
      reinterpret_cast<uint4*>(out)[ch] = reinterpret_cast<const uint4*>(src)[ch];
  }
}

hipError_t launch_cluster_major_copy(const uint8_t* E, int64_t lde_bytes, const int32_t* c2t,
                                     int64_t v, int64_t row_bytes, uint8_t* Ec, hipStream_t s) {
  hipLaunchKernelGGL(cluster_major_copy_kernel, dim3(4096), dim3(kPrepThreads), 0, s, E,
                     lde_bytes, c2t, v, (int)(row_bytes / 16), Ec, row_bytes);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plain streaming read (measurement reference and cache flush): every
// 16-byte word of the buffer is read once, grid-stride, eight words in
// flight per thread (non-temporal: streamed, not kept); one word that depends on all of them is written so that the
// reads cannot be dropped.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* p, int64_t n,
                                                          uint32_t* sink) {
  uint32_t acc = 0u;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(q + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].w;
  }
  for (; i < n; i += stride) acc ^= p[i].x;
  if (acc == 0x9E3779B9u) sink[0] = acc;  // data dependent, practically never
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int num_cu,
                              hipStream_t s) {
  const int64_t n = bytes / 16;
  int64_t grid = (int64_t)num_cu * 8;
  const int64_t need = (n + 255) / 256;
  if (grid > need) grid = need < 1 ? 1 : need;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const uint4*>(buf), n, sink);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fill of n 32-bit words (for memory a caller may capture into a graph,
// where a memset node is avoided).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, uint32_t value, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t grid = (n + 255) / 256;
  if (grid > 1024) grid = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)grid), dim3(256), 0, s, p, value, n);
  return hipGetLastError();
}

// The single launch's selection, for the debug output: the launch used the
// buffer set its epoch picked, one below the epoch it left behind.  Read on
// the device, so that it holds for launches replayed from a captured graph.
__global__ __launch_bounds__(256) void b1_copy_sel_kernel(const uint32_t* epoch,
                                                          const int32_t* sets, int64_t set_stride,
                                                          int32_t* dst, int p) {
  const uint32_t used = (*epoch - 1u) & 1u;
  const int32_t* src = sets + (int64_t)used * set_stride;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < p; i += gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_b1_copy_sel(const uint32_t* epoch, const int32_t* sets, int64_t set_stride,
                              int32_t* dst, int p, hipStream_t s) {
  hipLaunchKernelGGL(b1_copy_sel_kernel, dim3((unsigned)((p + 255) / 256)), dim3(256), 0, s, epoch,
                     sets, set_stride, dst, p);
  return hipGetLastError();
}

}  // namespace fh
