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
//            last one it proposed to (one workgroup scans the token's row of
//            cosines) and takes a slot of that cluster's proposal block; a
//            token that finds the block full proposes again next round
//            (deferred acceptance ends in the same assignment whatever the
//            order of the proposals);
//   accept   one workgroup per cluster with proposals ranks what it holds
//            together with them by (cosine desc, token id asc), keeps the
//            first b and sends the rest back to the unplaced list.
// When 8 or fewer tokens are left unplaced, one workgroup finishes the
// assignment one proposal at a time (a round would cost about as much as
// 6 proposals).  It ends when every token is placed (a token can always
// place: total room equals v).  Cosines, centroids and their sums are
// float64, so the integer decisions rest on float64 comparisons, as in a
// plain CPU implementation of the same definition.
//
// Iteration: cosines S = X C^T of the unit rows X against the centroids,
// the assignment, then (unless it repeats the previous assignment) the
// Formula 5 update.  The initial centroids are the unit rows of c distinct
// caller-chosen token ids.
#include <hip/hip_runtime.h>

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

// S (v x c) = X (v x d) C^T (C c x d), float64 on the matrix cores
// (v_mfma_f64_16x16x4f64: lane l feeds A[l mod 16][l div 16] and
// B[l div 16][l mod 16] and holds D[l div 16 + 4 r][l mod 16], r = 0..3).
// A 128 x 128 output tile per workgroup, a 64 x 64 quarter (4 x 4 blocks of
// 16 x 16) per wave, K staged through LDS 16 at a time.
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kSimTile = 128, kSimK = 16;
__global__ __launch_bounds__(kKmThreads) void cosine_kernel(const double* X, const double* C,
                                                            int64_t v, int c, int d, double* S) {
  __shared__ double sa[kSimK][kSimTile + 1];  // [k][row]
  __shared__ double sb[kSimK][kSimTile + 1];  // [k][column]
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;  // the wave's quarter
  const int li = lane & 15, lk = lane >> 4;
  const int64_t i0 = (int64_t)blockIdx.y * kSimTile;
  const int k0 = blockIdx.x * kSimTile;
  f64x4_t acc[4][4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[p][q] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  // 128 rows x 16 columns of each operand per K step: 8 elements per
  // thread, the next step's loaded into registers while this one computes
  double na[8], nb[8];
  auto fetch = [&](int j0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = threadIdx.x + q * kKmThreads;  // [0, 2048)
      const int r = e >> 4, jj = e & 15;
      const int64_t gi = i0 + r;
      const int gk = k0 + r;
      const int gj = j0 + jj;
      na[q] = (gi < v && gj < d) ? X[gi * d + gj] : 0.0;
      nb[q] = (gk < c && gj < d) ? C[(int64_t)gk * d + gj] : 0.0;
    }
  };
  fetch(0);
  for (int j0 = 0; j0 < d; j0 += kSimK) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = threadIdx.x + q * kKmThreads;
      sa[e & 15][e >> 4] = na[q];
      sb[e & 15][e >> 4] = nb[q];
    }
    __syncthreads();
    if (j0 + kSimK < d) fetch(j0 + kSimK);
#pragma unroll
    for (int k4 = 0; k4 < kSimK; k4 += 4) {
      double a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = sa[k4 + lk][wr + 16 * q + li];
        b[q] = sb[k4 + lk][wc + 16 * q + li];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[p][q] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[p], b[q], acc[p][q], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t gi = i0 + wr + 16 * p + lk + 4 * r;
      if (gi >= v) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gk = k0 + wc + 16 * q + li;
        if (gk < c) S[gi * c + gk] = acc[p][q][r];
      }
    }
}

constexpr int kKmQ = 256;  // proposal slots per cluster and round
// counters (int32): unplaced after the round and clusters with proposals,
// each by round parity; the no-candidate and table-changed flags
constexpr int kCtrFree = 0, kCtrAct = 2, kCtrBad = 4, kCtrChanged = 5, kCtrWords = 8;

struct Round {
  const double* S;
  int64_t v;
  int c, b;
  int par;                // round parity: which counter pair this round uses
  const int32_t* freel;   // unplaced tokens of this round
  int32_t nfree;
  int32_t* last;          // per token: the cluster of its last proposal (-1: none)
  int32_t* pcnt;          // per cluster: proposals this round (may exceed kKmQ)
  int32_t* prop;          // c x kKmQ proposal slots
  double* prop_s;         // and their cosines
  int32_t* act;           // clusters with proposals this round
  int32_t* holds;         // c x b: the tokens a cluster holds
  double* holds_s;        // and their cosines
  int32_t* hn;            // per cluster: how many it holds
  int32_t* freel_next;    // unplaced tokens for the next round
  int32_t* counters;
};

// does (s1, id1) rank before (s2, id2): larger cosine, then lower id
__device__ __forceinline__ bool before(double s1, int id1, double s2, int id2) {
  return s1 > s2 || (s1 == s2 && id1 < id2);
}

// keep (os, ok) in (bs, bk) if it ranks before it (bk < 0: nothing kept yet)
__device__ __forceinline__ void better_pair(double& bs, int& bk, double os, int ok) {
  if (ok >= 0 && (bk < 0 || before(os, ok, bs, bk))) { bs = os; bk = ok; }
}

// The best cluster of token i after its last proposal lk (cosine desc,
// cluster id asc), by the whole workgroup; the result is valid in thread 0
// (bk < 0: no cluster left, only with non-finite cosines).  Ends with the
// workgroup's LDS scratch free again.
template <int NT>
__device__ __forceinline__ void best_after(const Round& r, int32_t i, int lk, double* w_s, int* w_k,
                                           double& bs, int& bk) {
  constexpr int kLoads = 8192 / NT;  // loads in flight per thread (c <= 8192: one batch)
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const double* row = r.S + (int64_t)i * r.c;
  const double ls = lk >= 0 ? row[lk] : 0.0;
  bs = 0.0;
  bk = -1;
  // kLoads loads in flight per thread, then their comparisons
  for (int k0 = threadIdx.x; k0 < r.c; k0 += kLoads * NT) {
    double vals[kLoads];
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int k = k0 + q * NT;
      vals[q] = k < r.c ? row[k] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int k = k0 + q * NT;
      const double sv = vals[q];
      const bool after = lk < 0 || sv < ls || (sv == ls && k > lk);
      if (k < r.c && after) better_pair(bs, bk, sv, k);
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1)
    better_pair(bs, bk, __shfl_xor(bs, o, kWave), __shfl_xor(bk, o, kWave));
  if (lane == 0) {
    w_s[wave] = bs;
    w_k[wave] = bk;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < NT / kWave; ++w) better_pair(bs, bk, w_s[w], w_k[w]);
  __syncthreads();  // w_s / w_k may be reused
}

// one workgroup per unplaced token: the best cluster after its last
// proposal in the token's own order (cosine desc, cluster id asc), then a
// slot in that cluster's proposal block.  A whole workgroup scans the row so
// that the late rounds, with few tokens left, are not one wave's chain of
// loads.
__global__ __launch_bounds__(kKmThreads) void propose_kernel(Round r) {
  __shared__ double w_s[kKmWaves];
  __shared__ int w_k[kKmWaves];
  const int32_t i = r.freel[blockIdx.x];  // grid = unplaced tokens
  double bs;
  int bk;
  best_after<kKmThreads>(r, i, r.last[i], w_s, w_k, bs, bk);
  if (threadIdx.x == 0) {
    if (bk < 0) {
      r.counters[kCtrBad] = 1;  // only with non-finite cosines
      r.last[i] = -2;
      return;
    }
    const int slot = atomicAdd(&r.pcnt[bk], 1);
    if (slot < kKmQ) {
      r.prop[(int64_t)bk * kKmQ + slot] = i;
      r.prop_s[(int64_t)bk * kKmQ + slot] = bs;
      r.last[i] = bk;
      if (slot == 0) r.act[atomicAdd(&r.counters[kCtrAct + r.par], 1)] = bk;
    } else {
      // the block is full: propose again next round (last is unchanged)
      r.freel_next[atomicAdd(&r.counters[kCtrFree + r.par], 1)] = i;
    }
  }
}

// the clusters with proposals, grid-strided over the workgroups: rank
// held + proposed tokens, keep the first b (written in rank order), send
// back the rest
__global__ __launch_bounds__(kKmThreads) void accept_kernel(Round r) {
  __shared__ int32_t sh_id[kMaxKmB];
  __shared__ double sh_s[kMaxKmB];
  const int nact = r.counters[kCtrAct + r.par];
  const int b = r.b;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // the next round's counters (the previous round's, already read)
    r.counters[kCtrFree + (r.par ^ 1)] = 0;
    r.counters[kCtrAct + (r.par ^ 1)] = 0;
  }
  for (int a = blockIdx.x; a < nact; a += gridDim.x) {
    const int k = r.act[a];
    const int pc = r.pcnt[k];
    const int np = pc < kKmQ ? pc : kKmQ;
    const int h = r.hn[k];
    const int m = h + np;
    // every wave has read pcnt[k] and hn[k] before they are rewritten, and
    // is done with the previous cluster's LDS copy
    __syncthreads();
    if (threadIdx.x == 0) r.pcnt[k] = 0;  // zero for the next round
    int32_t* hold = r.holds + (int64_t)k * b;
    double* hold_s = r.holds_s + (int64_t)k * b;
    const int32_t* pid = r.prop + (int64_t)k * kKmQ;
    const double* ps = r.prop_s + (int64_t)k * kKmQ;
    if (m <= b) {
      for (int j = threadIdx.x; j < np; j += kKmThreads) {
        hold[h + j] = pid[j];
        hold_s[h + j] = ps[j];
      }
      if (threadIdx.x == 0) r.hn[k] = m;
      continue;
    }
    for (int j = threadIdx.x; j < h; j += kKmThreads) {
      sh_id[j] = hold[j];
      sh_s[j] = hold_s[j];
    }
    __syncthreads();
    for (int j = threadIdx.x; j < m; j += kKmThreads) {
      const int32_t id = j < h ? sh_id[j] : pid[j - h];
      const double sj = j < h ? sh_s[j] : ps[j - h];
      int rank = 0;
      for (int l = 0; l < h; ++l) rank += before(sh_s[l], sh_id[l], sj, id);
      for (int l = 0; l < np; ++l) rank += before(ps[l], pid[l], sj, id);
      if (rank < b) {
        hold[rank] = id;
        hold_s[rank] = sj;
      } else {
        r.freel_next[atomicAdd(&r.counters[kCtrFree + r.par], 1)] = id;
      }
    }
    if (threadIdx.x == 0) r.hn[k] = b;
  }
}

// The last unplaced tokens, one workgroup, one proposal at a time (the
// order of proposals does not change where deferred acceptance ends): the
// token on top of the stack proposes to its best cluster after its last
// one; a cluster with room takes it; a full cluster takes it only over its
// weakest holder, which then takes its place on the stack.  Each token
// proposes to a cluster at most once, so the loop ends; a budget of v * c
// proposals guards it anyway.
constexpr int kTailMax = 1024;  // stack capacity of the tail
// Unplaced tokens at which the rounds hand over to the tail: a round costs
// about as much as 6 sequential proposals (two launches and a host round
// trip against one row scan each)
constexpr int kTailStart = 8;
constexpr int kTailThreads = 1024;  // one row scan per proposal: all loads at once
__global__ __launch_bounds__(kTailThreads) void tail_kernel(Round r) {
  __shared__ int32_t stack[kTailMax];
  __shared__ int32_t h_id[kMaxKmB];  // the proposed-to cluster's holders
  __shared__ double h_s[kMaxKmB];
  __shared__ int top, stop, s_k, s_h;
  __shared__ double s_s;
  __shared__ double w_s[kTailThreads / kWave];
  __shared__ int w_k[kTailThreads / kWave];
  for (int j = threadIdx.x; j < r.nfree; j += kTailThreads) stack[j] = r.freel[j];
  if (threadIdx.x == 0) {
    top = r.nfree;
    stop = 0;
  }
  const int b = r.b;
  int64_t budget = r.v * (int64_t)r.c;
  __syncthreads();
  while (top > 0 && !stop) {
    const int32_t i = stack[top - 1];
    double bs;
    int bk;
    best_after<kTailThreads>(r, i, r.last[i], w_s, w_k, bs, bk);
    if (threadIdx.x == 0) {
      if (bk < 0 || --budget < 0) {
        r.counters[kCtrBad] = 1;
        stop = 1;
      }
      s_k = bk;
      s_s = bs;
      s_h = bk >= 0 ? r.hn[bk] : 0;
    }
    __syncthreads();
    if (stop) break;
    const int k = s_k;
    const int h = s_h;
    int32_t* hold = r.holds + (int64_t)k * b;
    double* hold_s = r.holds_s + (int64_t)k * b;
    if (h == b) {  // full: its holders into LDS, all loads at once
      for (int j = threadIdx.x; j < b; j += kTailThreads) {
        h_id[j] = hold[j];
        h_s[j] = hold_s[j];
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      r.last[i] = k;
      if (h < b) {
        hold[h] = i;
        hold_s[h] = s_s;
        r.hn[k] = h + 1;
        --top;
      } else {
        int wpos = 0;  // the holder that ranks last
        for (int l = 1; l < b; ++l)
          if (before(h_s[wpos], h_id[wpos], h_s[l], h_id[l])) wpos = l;
        if (before(s_s, i, h_s[wpos], h_id[wpos])) {
          stack[top - 1] = h_id[wpos];
          hold[wpos] = i;
          hold_s[wpos] = s_s;
        }
        // else the token stays on top and proposes further down its list
      }
    }
    __syncthreads();  // top, the stack and the LDS copies as thread 0 left them
  }
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
  double *X, *C, *S, *prop_s, *holds_s;
  int32_t *init, *fa, *fb, *last, *pcnt, *prop, *holds, *hn, *prev, *ctr, *act;
  KM_TRY(buf.get(&X, (size_t)v * d));
  KM_TRY(buf.get(&C, (size_t)c * d));
  KM_TRY(buf.get(&S, (size_t)v * c));
  KM_TRY(buf.get(&prop_s, (size_t)c * kKmQ));
  KM_TRY(buf.get(&holds_s, (size_t)v));
  KM_TRY(buf.get(&init, (size_t)c));
  KM_TRY(buf.get(&fa, (size_t)v));
  KM_TRY(buf.get(&fb, (size_t)v));
  KM_TRY(buf.get(&last, (size_t)v));
  KM_TRY(buf.get(&pcnt, (size_t)c));
  KM_TRY(buf.get(&prop, (size_t)c * kKmQ));
  KM_TRY(buf.get(&holds, (size_t)v));
  KM_TRY(buf.get(&hn, (size_t)c));
  KM_TRY(buf.get(&prev, (size_t)v));
  KM_TRY(buf.get(&ctr, kCtrWords));
  KM_TRY(buf.get(&act, (size_t)c));
  int32_t* host_ctr = nullptr;
  KM_TRY(hipHostMalloc((void**)&host_ctr, kCtrWords * sizeof(int32_t), 0));
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
    KM_TRY(hipMemsetAsync(ctr, 0, kCtrWords * 4, s));
    KM_TRY(hipMemsetAsync(pcnt, 0, (size_t)c * 4, s));  // accept re-zeroes what it used
    hipLaunchKernelGGL(iota_kernel, dim3(blocks_for(v, 256)), dim3(256), 0, s, fa, v);
    KM_TRY(hipGetLastError());
    int32_t nfree = (int32_t)v;
    int64_t rounds = 0;
    while (nfree > 0) {
      const int par = (int)(rounds & 1);
      Round r{};
      r.S = S;
      r.v = v;
      r.c = c;
      r.b = b;
      r.par = par;
      r.freel = fa;
      r.nfree = nfree;
      r.last = last;
      r.pcnt = pcnt;
      r.prop = prop;
      r.prop_s = prop_s;
      r.act = act;
      r.holds = holds;
      r.holds_s = holds_s;
      r.hn = hn;
      r.freel_next = fb;
      r.counters = ctr;
      if (nfree <= kTailStart) {
        hipLaunchKernelGGL(tail_kernel, dim3(1), dim3(kTailThreads), 0, s, r);
        KM_TRY(hipGetLastError());
        KM_TRY(hipMemcpyAsync(host_ctr, ctr, kCtrWords * 4, hipMemcpyDeviceToHost, s));
        KM_TRY(hipStreamSynchronize(s));
        if (host_ctr[kCtrBad]) {
          *status = 1;  // a token found no cluster: non-finite cosines
          return hipSuccess;
        }
        break;
      }
      hipLaunchKernelGGL(propose_kernel, dim3(nfree), dim3(kKmThreads), 0, s, r);
      // at most one cluster with proposals per proposal
      hipLaunchKernelGGL(accept_kernel, dim3(nfree < c ? nfree : c), dim3(kKmThreads), 0, s, r);
      KM_TRY(hipGetLastError());
      KM_TRY(hipMemcpyAsync(host_ctr, ctr, kCtrWords * 4, hipMemcpyDeviceToHost, s));
      KM_TRY(hipStreamSynchronize(s));
      if (host_ctr[kCtrBad]) {
        *status = 1;  // a token found no cluster: non-finite cosines
        return hipSuccess;
      }
      nfree = host_ctr[kCtrFree + par];
      int32_t* t = fa;
      fa = fb;
      fb = t;
      // every round keeps at least one proposal (a full block keeps its
      // first kKmQ), and a token proposes to each cluster at most once
      if (++rounds > v * (int64_t)c) {
        *status = 1;
        return hipSuccess;
      }
    }
    hipLaunchKernelGGL(table_kernel, dim3(c), dim3(kKmThreads), 0, s, holds, b, a.c2t,
                       it > 0 ? prev : nullptr, ctr + kCtrChanged);
    KM_TRY(hipGetLastError());
    KM_TRY(hipMemcpyAsync(host_ctr, ctr, kCtrWords * 4, hipMemcpyDeviceToHost, s));
    KM_TRY(hipStreamSynchronize(s));
    *iters = it + 1;
    if (it > 0 && host_ctr[kCtrChanged] == 0) break;  // the centroids are already its means
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
