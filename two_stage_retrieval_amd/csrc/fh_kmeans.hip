// Equal-size spherical k-means (notes, Module 1; Formula 4: the summed
// cosine of every token to its cluster's unit centroid; Formula 5: the
// centroid is the unit-normalised mean of its cluster's rows), the offline
// step that turns an embedding matrix E into the c x b table C2T.
//
// Every cluster holds exactly b = v / c tokens.  The pages do not say how
// the size constraint is enforced; here a token goes to its most similar
// cluster that still has room, pairs taken in descending cosine (ties: the
// lower token id, then the lower cluster id).  With tokens and clusters
// ranking each other by the same cosine that is the unique stable
// assignment, which deferred acceptance reaches in parallel rounds:
//   propose  every unplaced token proposes to its best cluster below the
//            last one it proposed to (one wave scans the token's row of
//            cosines);
//   bucket   proposals are counted per cluster, offsets scanned, and the
//            token ids scattered into per-cluster runs;
//   accept   one workgroup per cluster ranks what it holds together with
//            its new proposals by (cosine desc, token id asc), keeps the
//            first b and sends the rest back to the unplaced list.
// The rounds end when every token is placed (a token can always place:
// total room equals v).  Cosines, centroids and their sums are float64, so
// the integer decisions rest on float64 comparisons, as in a plain CPU
// implementation of the same definition.
//
// Iteration: cosines S = X C^T of the unit rows X against the centroids,
// the assignment, then (unless it repeats the previous assignment) the
// Formula 5 update.  The initial centroids are the unit rows of c distinct
// caller-chosen token ids.
#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

namespace {

constexpr int kKmThreads = 256;
constexpr int kKmWaves = kKmThreads / kWave;

template <typename TE> __device__ __forceinline__ double elem(const uint8_t* row, int j);
template <> __device__ __forceinline__ double elem<float>(const uint8_t* row, int j) {
  return (double)reinterpret_cast<const float*>(row)[j];
}
template <> __device__ __forceinline__ double elem<bf16_t>(const uint8_t* row, int j) {
  const uint32_t w = reinterpret_cast<const uint16_t*>(row)[j];
  return (double)__uint_as_float(w << 16);
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// block sum of a double (all threads get it); sm holds kKmWaves doubles
__device__ __forceinline__ double block_sum_f64(double x, double* sm) {
  x = wave_sum_f64(x);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sm[wave] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kKmWaves; ++w) t += sm[w];
  return t;
}

// X[i] = E[i] / ||E[i]|| in float64 (a zero row stays zero); one wave per row
template <typename TE>
__global__ __launch_bounds__(kKmThreads) void unit_rows_kernel(const uint8_t* E, int64_t lde_bytes,
                                                               int64_t v, int d, double* X) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t i = (int64_t)blockIdx.x * kKmWaves + (threadIdx.x >> 6);
  if (i >= v) return;  // wave-uniform
  const uint8_t* row = E + i * lde_bytes;
  double ss = 0.0;
  for (int j = lane; j < d; j += kWave) {
    const double x = elem<TE>(row, j);
    ss += x * x;
  }
  const double n = sqrt(wave_sum_f64(ss));
  double* xr = X + i * d;
  for (int j = lane; j < d; j += kWave) xr[j] = n > 0.0 ? elem<TE>(row, j) / n : 0.0;
}

// C[k] = X[init[k]]
__global__ __launch_bounds__(kKmThreads) void gather_rows_kernel(const double* X, const int32_t* idx,
                                                                 int d, double* C) {
  const int k = blockIdx.x;
  const double* src = X + (int64_t)idx[k] * d;
  for (int j = threadIdx.x; j < d; j += kKmThreads) C[(int64_t)k * d + j] = src[j];
}

// S (v x c) = X (v x d) C^T (C c x d), float64.  64 x 64 output tile per
// workgroup, 4 x 4 per thread, K staged through LDS 16 at a time; each
// output is a sum over j ascending.
constexpr int kSimTile = 64, kSimK = 16;
__global__ __launch_bounds__(kKmThreads) void cosine_kernel(const double* X, const double* C,
                                                            int64_t v, int c, int d, double* S) {
  __shared__ double sa[kSimK][kSimTile + 1];
  __shared__ double sb[kSimK][kSimTile + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t i0 = (int64_t)blockIdx.y * kSimTile;
  const int k0 = blockIdx.x * kSimTile;
  double acc[4][4] = {};
  for (int j0 = 0; j0 < d; j0 += kSimK) {
    // 64 rows x 16 columns of each operand: 4 elements per thread
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = threadIdx.x + q * kKmThreads;  // [0, 1024)
      const int r = e >> 4, jj = e & 15;
      const int64_t gi = i0 + r;
      const int gk = k0 + r;
      const int gj = j0 + jj;
      sa[jj][r] = (gi < v && gj < d) ? X[gi * d + gj] : 0.0;
      sb[jj][r] = (gk < c && gj < d) ? C[(int64_t)gk * d + gj] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < kSimK; ++jj) {
      double a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = sa[jj][ty * 4 + q];
        b[q] = sb[jj][tx * 4 + q];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = fma(a[p], b[q], acc[p][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t gi = i0 + ty * 4 + p;
    if (gi >= v) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int gk = k0 + tx * 4 + q;
      if (gk < c) S[gi * c + gk] = acc[p][q];
    }
  }
}

struct Round {
  const double* S;
  int64_t v;
  int c, b;
  const int32_t* freel;   // unplaced tokens of this round
  int32_t nfree;
  int32_t* last;          // per token: the cluster of its last proposal (-1: none)
  int32_t* cnt;           // per cluster: proposals this round
  int32_t* off;           // per cluster: start of its run in bucket (c + 1)
  int32_t* fill;          // per cluster: scatter cursor
  int32_t* bucket;        // proposals grouped by cluster
  double* bucket_s;       // and their cosines
  int32_t* holds;         // c x b: the tokens a cluster holds
  double* holds_s;        // and their cosines
  int32_t* hn;            // per cluster: how many it holds
  int32_t* freel_next;    // tokens sent back this round
  int32_t* counters;      // [0] unplaced after this round, [1] no-candidate flag
};

// does (s1, id1) rank before (s2, id2): larger cosine, then lower id
__device__ __forceinline__ bool before(double s1, int id1, double s2, int id2) {
  return s1 > s2 || (s1 == s2 && id1 < id2);
}

// one wave per unplaced token: the best cluster after its last proposal in
// its own order (cosine desc, cluster id asc)
__global__ __launch_bounds__(kKmThreads) void propose_kernel(Round r) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kKmWaves + (threadIdx.x >> 6);
  if (t >= r.nfree) return;  // wave-uniform
  const int32_t i = r.freel[t];
  const double* row = r.S + (int64_t)i * r.c;
  const int lk = r.last[i];
  const double ls = lk >= 0 ? row[lk] : 0.0;
  double bs = 0.0;
  int bk = -1;
  for (int k = lane; k < r.c; k += kWave) {
    const double s = row[k];
    const bool after = lk < 0 || s < ls || (s == ls && k > lk);
    if (after && (bk < 0 || before(s, k, bs, bk))) { bs = s; bk = k; }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const double os = __shfl_xor(bs, o, kWave);
    const int ok = __shfl_xor(bk, o, kWave);
    if (ok >= 0 && (bk < 0 || before(os, ok, bs, bk))) { bs = os; bk = ok; }
  }
  if (lane == 0) {
    if (bk < 0) {
      r.counters[1] = 1;  // only with non-finite cosines
      r.last[i] = -2;
      return;
    }
    r.last[i] = bk;
    atomicAdd(&r.cnt[bk], 1);
  }
}

// exclusive scan of the per-cluster counts (one 1024-thread workgroup);
// clears the scatter cursors
__global__ __launch_bounds__(1024) void offsets_kernel(Round r) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (r.c + 1023) / 1024;
  const int b0 = t * per;
  int s = 0;
  for (int k = b0; k < b0 + per && k < r.c; ++k) s += r.cnt[k];
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    const int x = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  int run = part[t] - s;
  for (int k = b0; k < b0 + per && k < r.c; ++k) {
    r.off[k] = run;
    run += r.cnt[k];
    r.fill[k] = 0;
  }
  if (t == 1023) r.off[r.c] = part[1023];
}

__global__ __launch_bounds__(kKmThreads) void scatter_kernel(Round r) {
  const int t = blockIdx.x * kKmThreads + threadIdx.x;
  if (t >= r.nfree) return;
  const int32_t i = r.freel[t];
  const int k = r.last[i];
  if (k < 0) return;
  const int pos = r.off[k] + atomicAdd(&r.fill[k], 1);
  r.bucket[pos] = i;
  r.bucket_s[pos] = r.S[(int64_t)i * r.c + k];
}

// one workgroup per cluster with proposals: rank held + proposed tokens,
// keep the first b (written in rank order), send back the rest
__global__ __launch_bounds__(kKmThreads) void accept_kernel(Round r) {
  __shared__ int32_t sh_id[kMaxKmB];
  __shared__ double sh_s[kMaxKmB];
  const int k = blockIdx.x;
  const int np = r.cnt[k];
  if (np == 0) return;
  const int h = r.hn[k];
  const int m = h + np;
  const int b = r.b;
  __syncthreads();  // every wave has read hn[k] before thread 0 rewrites it
  int32_t* hold = r.holds + (int64_t)k * b;
  double* hold_s = r.holds_s + (int64_t)k * b;
  const int32_t* pid = r.bucket + r.off[k];
  const double* ps = r.bucket_s + r.off[k];
  if (m <= b) {
    for (int j = threadIdx.x; j < np; j += kKmThreads) {
      hold[h + j] = pid[j];
      hold_s[h + j] = ps[j];
    }
    if (threadIdx.x == 0) r.hn[k] = m;
    return;
  }
  for (int j = threadIdx.x; j < h; j += kKmThreads) {
    sh_id[j] = hold[j];
    sh_s[j] = hold_s[j];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < m; j += kKmThreads) {
    const int32_t id = j < h ? sh_id[j] : pid[j - h];
    const double s = j < h ? sh_s[j] : ps[j - h];
    int rank = 0;
    for (int l = 0; l < h; ++l) rank += before(sh_s[l], sh_id[l], s, id);
    for (int l = 0; l < np; ++l) rank += before(ps[l], pid[l], s, id);
    if (rank < b) {
      hold[rank] = id;
      hold_s[rank] = s;
    } else {
      r.freel_next[atomicAdd(&r.counters[0], 1)] = id;
    }
  }
  if (threadIdx.x == 0) r.hn[k] = b;
}

// each cluster's tokens ascending into c2t; flags a change from prev
__global__ __launch_bounds__(kKmThreads) void table_kernel(const int32_t* holds, int b,
                                                           int32_t* c2t, const int32_t* prev,
                                                           int32_t* changed) {
  const int k = blockIdx.x;
  const int32_t* hk = holds + (int64_t)k * b;
  for (int j = threadIdx.x; j < b; j += kKmThreads) {
    const int32_t id = hk[j];
    int rank = 0;
    for (int l = 0; l < b; ++l) rank += hk[l] < id;
    const int64_t o = (int64_t)k * b + rank;
    c2t[o] = id;
    if (prev && prev[o] != id) *changed = 1;
  }
}

// Formula 5 in float64: C[k] = mean of the cluster's raw rows (in c2t
// order), scaled to unit norm (a zero mean stays zero)
template <typename TE>
__global__ __launch_bounds__(kKmThreads) void centroid_kernel(const uint8_t* E, int64_t lde_bytes,
                                                              const int32_t* c2t, int b, int d,
                                                              double* C) {
  __shared__ double red[kKmWaves];
  const int k = blockIdx.x;
  const int32_t* members = c2t + (int64_t)k * b;
  double* ck = C + (int64_t)k * d;
  double ss = 0.0;
  for (int j = threadIdx.x; j < d; j += kKmThreads) {
    double sum = 0.0;
    for (int l = 0; l < b; ++l) sum += elem<TE>(E + (int64_t)members[l] * lde_bytes, j);
    const double mean = sum / b;
    ck[j] = mean;
    ss += mean * mean;
  }
  const double n = sqrt(block_sum_f64(ss, red));
  for (int j = threadIdx.x; j < d; j += kKmThreads) ck[j] = n > 0.0 ? ck[j] / n : 0.0;
}

__global__ void iota_kernel(int32_t* x, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) x[t] = (int32_t)t;
}

struct Buffers {
  std::vector<void*> ptrs;
  ~Buffers() {
    for (void* p : ptrs) (void)hipFree(p);
  }
  template <typename T> hipError_t get(T** p, size_t n) {
    void* q = nullptr;
    const hipError_t e = hipMalloc(&q, n * sizeof(T) > 0 ? n * sizeof(T) : 16);
    if (e != hipSuccess) return e;
    ptrs.push_back(q);
    *p = static_cast<T*>(q);
    return hipSuccess;
  }
};

#define KM_TRY(expr)                            \
  do {                                          \
    const hipError_t e_ = (expr);               \
    if (e_ != hipSuccess) return e_;            \
  } while (0)

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t run_kmeans(const KMeansArgs& a, hipStream_t s, int* iters, int* status) {
  *iters = 0;
  *status = 0;
  const int64_t v = a.v;
  const int c = a.c, d = a.d, b = (int)(v / c);
  Buffers buf;
  double *X, *C, *S, *bucket_s, *holds_s;
  int32_t *init, *fa, *fb, *last, *cnt, *off, *fill, *bucket, *holds, *hn, *prev, *ctr;
  KM_TRY(buf.get(&X, (size_t)v * d));
  KM_TRY(buf.get(&C, (size_t)c * d));
  KM_TRY(buf.get(&S, (size_t)v * c));
  KM_TRY(buf.get(&bucket_s, (size_t)v));
  KM_TRY(buf.get(&holds_s, (size_t)v));
  KM_TRY(buf.get(&init, (size_t)c));
  KM_TRY(buf.get(&fa, (size_t)v));
  KM_TRY(buf.get(&fb, (size_t)v));
  KM_TRY(buf.get(&last, (size_t)v));
  KM_TRY(buf.get(&cnt, (size_t)c));
  KM_TRY(buf.get(&off, (size_t)c + 1));
  KM_TRY(buf.get(&fill, (size_t)c));
  KM_TRY(buf.get(&bucket, (size_t)v));
  KM_TRY(buf.get(&holds, (size_t)v));
  KM_TRY(buf.get(&hn, (size_t)c));
  KM_TRY(buf.get(&prev, (size_t)v));
  KM_TRY(buf.get(&ctr, 4));
  int32_t* host_ctr = nullptr;
  KM_TRY(hipHostMalloc((void**)&host_ctr, 4 * sizeof(int32_t), 0));
  struct HostFree {
    int32_t* p;
    ~HostFree() { (void)hipHostFree(p); }
  } host_free{host_ctr};

  KM_TRY(hipMemcpyAsync(init, a.init_host, (size_t)c * 4, hipMemcpyHostToDevice, s));
  const unsigned gv = blocks_for(v, kKmWaves);
  if (a.dtype == FH_DTYPE_BF16)
    hipLaunchKernelGGL(unit_rows_kernel<bf16_t>, dim3(gv), dim3(kKmThreads), 0, s, a.E, a.lde_bytes,
                       v, d, X);
  else
    hipLaunchKernelGGL(unit_rows_kernel<float>, dim3(gv), dim3(kKmThreads), 0, s, a.E, a.lde_bytes,
                       v, d, X);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(c), dim3(kKmThreads), 0, s, X, init, d, C);
  KM_TRY(hipGetLastError());

  const dim3 gsim(blocks_for(c, kSimTile), blocks_for(v, kSimTile));
  for (int it = 0; it < a.max_iter; ++it) {
    hipLaunchKernelGGL(cosine_kernel, gsim, dim3(kKmThreads), 0, s, X, C, v, c, d, S);
    KM_TRY(hipMemsetAsync(hn, 0, (size_t)c * 4, s));
    KM_TRY(hipMemsetAsync(last, 0xFF, (size_t)v * 4, s));  // -1: no proposal yet
    KM_TRY(hipMemsetAsync(ctr, 0, 4 * 4, s));
    hipLaunchKernelGGL(iota_kernel, dim3(blocks_for(v, 256)), dim3(256), 0, s, fa, v);
    KM_TRY(hipGetLastError());
    int32_t nfree = (int32_t)v;
    int64_t rounds = 0;
    while (nfree > 0) {
      Round r{};
      r.S = S;
      r.v = v;
      r.c = c;
      r.b = b;
      r.freel = fa;
      r.nfree = nfree;
      r.last = last;
      r.cnt = cnt;
      r.off = off;
      r.fill = fill;
      r.bucket = bucket;
      r.bucket_s = bucket_s;
      r.holds = holds;
      r.holds_s = holds_s;
      r.hn = hn;
      r.freel_next = fb;
      r.counters = ctr;
      KM_TRY(hipMemsetAsync(cnt, 0, (size_t)c * 4, s));
      KM_TRY(hipMemsetAsync(ctr, 0, 4, s));  // unplaced count of this round
      hipLaunchKernelGGL(propose_kernel, dim3(blocks_for(nfree, kKmWaves)), dim3(kKmThreads), 0, s, r);
      hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(1024), 0, s, r);
      hipLaunchKernelGGL(scatter_kernel, dim3(blocks_for(nfree, kKmThreads)), dim3(kKmThreads), 0, s, r);
      hipLaunchKernelGGL(accept_kernel, dim3(c), dim3(kKmThreads), 0, s, r);
      KM_TRY(hipGetLastError());
      KM_TRY(hipMemcpyAsync(host_ctr, ctr, 2 * 4, hipMemcpyDeviceToHost, s));
      KM_TRY(hipStreamSynchronize(s));
      if (host_ctr[1]) {
        *status = 1;  // a token found no cluster: non-finite cosines
        return hipSuccess;
      }
      nfree = host_ctr[0];
      int32_t* t = fa;
      fa = fb;
      fb = t;
      // every round places or re-places at least one proposal; a token
      // proposes to each cluster at most once
      if (++rounds > v * (int64_t)c) {
        *status = 1;
        return hipSuccess;
      }
    }
    KM_TRY(hipMemsetAsync(ctr + 2, 0, 4, s));
    hipLaunchKernelGGL(table_kernel, dim3(c), dim3(kKmThreads), 0, s, holds, b, a.c2t,
                       it > 0 ? prev : nullptr, ctr + 2);
    KM_TRY(hipGetLastError());
    KM_TRY(hipMemcpyAsync(host_ctr + 2, ctr + 2, 4, hipMemcpyDeviceToHost, s));
    KM_TRY(hipStreamSynchronize(s));
    *iters = it + 1;
    if (it > 0 && host_ctr[2] == 0) break;  // the centroids are already its means
    if (a.dtype == FH_DTYPE_BF16)
      hipLaunchKernelGGL(centroid_kernel<bf16_t>, dim3(c), dim3(kKmThreads), 0, s, a.E,
                         a.lde_bytes, a.c2t, b, d, C);
    else
      hipLaunchKernelGGL(centroid_kernel<float>, dim3(c), dim3(kKmThreads), 0, s, a.E,
                         a.lde_bytes, a.c2t, b, d, C);
    KM_TRY(hipGetLastError());
    KM_TRY(hipMemcpyAsync(prev, a.c2t, (size_t)v * 4, hipMemcpyDeviceToDevice, s));
  }
  if (a.centroids)
    KM_TRY(hipMemcpyAsync(a.centroids, C, (size_t)c * d * 8, hipMemcpyDeviceToDevice, s));
  KM_TRY(hipStreamSynchronize(s));
  return hipSuccess;
}

}  // namespace fh
