// C ABI of libflashhead: the prepared handle and its workspace, and the
// enqueue of each decode step (descriptor checks and the INT4 quantizer are
// host-only code in fh_host.cpp).
#include <math.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "fh_host.h"
#include "fh_internal.h"

using namespace fh;

struct fh_handle {
  int64_t v = 0;
  int d = 0, c = 0, b = 0, dtype = 0, quant = 0, max_batch = 0, max_p = 0;
  int esize = 0;
  int64_t row_bytes = 0;  // d * esize: rows of C and of the cluster-major copy
  int device = 0;
  void* C = nullptr;          // c x d
  int32_t* c2t = nullptr;     // c x b
  uint8_t* Ec = nullptr;      // cluster-major copy of E (v x d), unless borrowed
  // the rows stage 2 reads: the copy (row k*b + j = token C2T[k, j]) or, with
  // FH_FLAG_BORROW_E, the caller's E itself (row = token)
  const uint8_t* rows = nullptr;
  int64_t rows_stride = 0;    // bytes between rows of `rows`
  int borrowed = 0;
  uint8_t* q4 = nullptr;      // INT4 tiles
  uint16_t* q4s = nullptr;    // INT4 scales
  int ntiles = 0, groups = 0;
  // workspace (left zeroed / consistent by every call)
  float* keys = nullptr;      // max_batch x c
  int32_t* sel = nullptr;     // max_batch x max_p
  uint64_t* row_best = nullptr;  // max_batch x kMaxGrid partial best keys (GEMV stage 2)
  uint32_t* counters = nullptr;
  float2* lse_part = nullptr; // max_batch x kMaxGrid
  uint64_t* masks = nullptr;  // c
  uint32_t* error = nullptr;  // 1
  // batched path
  int32_t* ulist = nullptr;         // union of the selected clusters (c)
  int32_t* ucount = nullptr;
  uint64_t* part_best = nullptr;    // stage-2 partials, grid x max_batch
  float2* part_lse = nullptr;
  // all-cluster stream: one record per (16-row item, batch row)
  uint64_t* all_best = nullptr;     // (v / 16) x max_batch
  float2* all_lse = nullptr;
  int32_t* dbg_tokens = nullptr;    // max_batch: the debug gather's own tokens
  // single-launch batch-1 decode
  int num_cu = 0;
  int b1_blocks_per_cu = 0;         // decode workgroups one compute unit holds at once
  int flags = 0;                    // FH_FLAG_*
  float* b1_keys = nullptr;         // 2 x b1_key_stride(c), all bits set between launches
  float* b1_raw = nullptr;          // 2 x b1_key_stride(c) plain scores (adaptive sampling)
  uint64_t* b1_slots = nullptr;     // 2 x kDecodeB1SlotStride words, zero between launches
  float2* b1_lse = nullptr;         // kDecodeB1SlotStride words
  int32_t* b1_sel = nullptr;        // 2 x kDecodeB1MaxP, -1 between launches
  int last_path = 0;                // kernels of the last step (flashhead_query 10)
  uint32_t* b1_epoch = nullptr;     // launch counter (picks the buffer set)
  uint32_t* b1_go = nullptr;        // 2 words: all keys seen, per buffer set (0 between launches)
  int32_t* t2row = nullptr;         // v: row of each token in the cluster-major copy


  int64_t bytes = 0;
  std::vector<void*> allocs;
  // per-kernel timing (flashhead_profile_begin / _end)
  std::vector<hipEvent_t> prof_ev;  // 6 per recorded call
  int prof_cap = 0, prof_calls = 0;
};

namespace {

constexpr int kMaxGrid = 8192;       // largest grid.x of a decode launch
constexpr int kDenseMaxGrid = 8192;  // dense: partial slots of the batched kernel (2 x 4096)
constexpr double kStreamAllCover = 0.85;  // batched: expected selected share from which
                                          // every cluster is streamed

// selection keys of a batch row: c floats padded to a 16-byte multiple
int64_t key_stride(int c) { return ((int64_t)c + 3) & ~(int64_t)3; }
// the single launch's key buffers: padded to whole 128-byte lines, so that
// each workgroup's run of keys fills lines of its own
int64_t b1_key_stride(int c) { return ((int64_t)c + 31) & ~(int64_t)31; }


void drop_profile(fh_handle* h) {
  for (hipEvent_t e : h->prof_ev) (void)hipEventDestroy(e);
  h->prof_ev.clear();
  h->prof_cap = h->prof_calls = 0;
}

void free_handle(fh_handle* h) {
  if (!h) return;
  drop_profile(h);
  for (void* p : h->allocs) (void)hipFree(p);
  delete h;
}

template <typename T>
hipError_t alloc(fh_handle* h, T** p, size_t bytes) {
  void* q = nullptr;
  const hipError_t e = hipMalloc(&q, bytes < 16 ? 16 : bytes);
  if (e != hipSuccess) return e;
  h->allocs.push_back(q);
  h->bytes += (int64_t)bytes;
  *p = static_cast<T*>(q);
  return hipSuccess;
}

// the HIP error behind the last FH_ERR_HIP / FH_ERR_OOM of this thread
thread_local hipError_t g_last_hip = hipSuccess;

int hip_fail(hipError_t e) {
  g_last_hip = e;
  return e == hipErrorOutOfMemory ? FH_ERR_OOM : FH_ERR_HIP;
}

int check_device(const fh_handle* h) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  return dev == h->device ? FH_OK : FH_ERR_INVALID_ARG;
}

#define FH_TRY(expr)                                              \
  do {                                                            \
    const hipError_t e_ = (expr);                                 \
    if (e_ != hipSuccess) return hip_fail(e_);                   \
  } while (0)

int prepare_impl(const fh_desc* ds, fh_handle* h) {
  hipStream_t s = static_cast<hipStream_t>(ds->stream);
  FH_TRY(hipGetDevice(&h->device));
  FH_TRY(hipDeviceGetAttribute(&h->num_cu, hipDeviceAttributeMultiprocessorCount, h->device));
  FH_TRY(decode_b1_occupancy(h->dtype, h->quant != FH_QUANT_NONE, (int)(h->row_bytes / 16),
                             ds->c, &h->b1_blocks_per_cu));
  const int64_t v = ds->v;
  const int c = ds->c, b = ds->b, d = ds->d;
  FH_TRY(alloc(h, &h->c2t, (size_t)v * 4));
  FH_TRY(hipMemcpyAsync(h->c2t, ds->c2t, (size_t)v * 4, hipMemcpyHostToDevice, s));
  FH_TRY(alloc(h, &h->C, (size_t)c * h->row_bytes));
  const uint8_t* E = static_cast<const uint8_t*>(ds->E);
  const int64_t lde_bytes = ds->lde * h->esize;
  if (ds->C)
    FH_TRY(hipMemcpyAsync(h->C, ds->C, (size_t)c * h->row_bytes, hipMemcpyDeviceToDevice, s));
  else
    FH_TRY(launch_centroid_means(E, lde_bytes, h->dtype, d, h->c2t, c, b, h->C, s));
  if (h->borrowed) {
    h->rows = E;
    h->rows_stride = lde_bytes;
  } else {
    FH_TRY(alloc(h, &h->Ec, (size_t)v * h->row_bytes));
    FH_TRY(launch_cluster_major_copy(E, lde_bytes, h->c2t, v, h->row_bytes, h->Ec, s));
    h->rows = h->Ec;
    h->rows_stride = h->row_bytes;
  }
  {
    // token -> row of the cluster-major copy (the inverse of the table)
    std::vector<int32_t> inv((size_t)v);
    invert_permutation(ds->c2t, v, inv.data());
    FH_TRY(alloc(h, &h->t2row, (size_t)v * 4));
    FH_TRY(hipMemcpyAsync(h->t2row, inv.data(), (size_t)v * 4, hipMemcpyHostToDevice, s));
    FH_TRY(hipStreamSynchronize(s));  // the host vector dies at scope end
  }
  if (h->quant == FH_QUANT_INT4_G128 || h->quant == FH_QUANT_INT4_G128_MEAN) {
    std::vector<uint16_t> hostC((size_t)c * d);
    FH_TRY(hipMemcpyAsync(hostC.data(), h->C, hostC.size() * 2, hipMemcpyDeviceToHost, s));
    FH_TRY(hipStreamSynchronize(s));
    std::vector<double> mu;
    if (h->quant == FH_QUANT_INT4_G128_MEAN) column_mean_shift(hostC.data(), c, d, mu);
    std::vector<uint8_t> codes;
    std::vector<uint16_t> scales;
    quantize_int4(hostC.data(), mu.empty() ? nullptr : mu.data(), c, d, codes, scales,
                  &h->ntiles, &h->groups);
    FH_TRY(alloc(h, &h->q4, codes.size()));
    FH_TRY(alloc(h, &h->q4s, scales.size() * 2));
    FH_TRY(hipMemcpyAsync(h->q4, codes.data(), codes.size(), hipMemcpyHostToDevice, s));
    FH_TRY(hipMemcpyAsync(h->q4s, scales.data(), scales.size() * 2, hipMemcpyHostToDevice, s));
    FH_TRY(hipStreamSynchronize(s));  // host vectors die at scope end
  }
  const int mb = h->max_batch;
  FH_TRY(alloc(h, &h->keys, (size_t)kMaxKSplit * mb * key_stride(c) * 4));  // K-slice partials
  FH_TRY(alloc(h, &h->sel, (size_t)mb * h->max_p * 4));
  FH_TRY(alloc(h, &h->row_best, (size_t)mb * kMaxGrid * 8));
  FH_TRY(alloc(h, &h->counters, (size_t)mb * kArriveWords * 4));
  FH_TRY(alloc(h, &h->lse_part, (size_t)mb * kMaxGrid * 8));
  FH_TRY(alloc(h, &h->masks, (size_t)(c + 1) * 8));  // the select reads pairs
  FH_TRY(alloc(h, &h->error, 4));
  FH_TRY(hipMemsetAsync(h->sel, 0, (size_t)mb * h->max_p * 4, s));
  FH_TRY(hipMemsetAsync(h->counters, 0, (size_t)mb * kArriveWords * 4, s));
  FH_TRY(hipMemsetAsync(h->masks, 0, (size_t)(c + 1) * 8, s));
  FH_TRY(hipMemsetAsync(h->error, 0, 4, s));
  FH_TRY(alloc(h, &h->ulist, (size_t)c * 4));
  FH_TRY(alloc(h, &h->ucount, 4));
  FH_TRY(alloc(h, &h->part_best, (size_t)stage2_mfma_grid() * mb * 8));
  FH_TRY(alloc(h, &h->part_lse, (size_t)stage2_mfma_grid() * mb * 8));
  if (mb >= 2 && h->b % 16 == 0 && batched_supported(h->dtype, d, 2, false)) {
    FH_TRY(alloc(h, &h->all_best, (size_t)(v / 16) * mb * 8));
    FH_TRY(alloc(h, &h->all_lse, (size_t)(v / 16) * mb * 8));
    FH_TRY(alloc(h, &h->dbg_tokens, (size_t)mb * 4));
  }
  FH_TRY(alloc(h, &h->b1_keys, (size_t)2 * b1_key_stride(c) * 4));
  FH_TRY(hipMemsetAsync(h->b1_keys, 0xFF, (size_t)2 * b1_key_stride(c) * 4, s));
  FH_TRY(alloc(h, &h->b1_raw, (size_t)2 * b1_key_stride(c) * 4));
  FH_TRY(hipMemsetAsync(h->b1_raw, 0xFF, (size_t)2 * b1_key_stride(c) * 4, s));
  FH_TRY(alloc(h, &h->b1_slots, (size_t)2 * kDecodeB1SlotStride * 8));
  FH_TRY(hipMemsetAsync(h->b1_slots, 0, (size_t)2 * kDecodeB1SlotStride * 8, s));
  FH_TRY(alloc(h, &h->b1_lse, (size_t)kDecodeB1SlotStride * 8));
  FH_TRY(alloc(h, &h->b1_sel, (size_t)2 * kDecodeB1MaxP * 4));
  FH_TRY(hipMemsetAsync(h->b1_sel, 0xFF, (size_t)2 * kDecodeB1MaxP * 4, s));
  FH_TRY(alloc(h, &h->b1_epoch, 4));
  FH_TRY(hipMemsetAsync(h->b1_epoch, 0, 4, s));
  FH_TRY(alloc(h, &h->b1_go, 8));
  FH_TRY(hipMemsetAsync(h->b1_go, 0, 8, s));
  FH_TRY(hipMemsetAsync(h->ucount, 0, 4, s));
  FH_TRY(hipStreamSynchronize(s));
  return FH_OK;
}

// The kernels a step of this shape takes: 1 the single-launch batch-1 decode
// (*grid workgroups), 2 stage 1 and stage 2 as separate row-dot launches,
// 3 the batched matrix-core path.  The single launch's workgroups wait on
// one another, so it is taken only when every one of them can be resident
// at once.  The row-dot launches need no such guarantee: in each batch row
// one workgroup waits for the others, which never wait, so they progress as
// long as the device holds more than B workgroups.
int plan_path(int c, int b, int d, int64_t row_bytes, int dtype, bool int4, int B, int p,
              int num_cu, int blocks_per_cu, int flags, int* grid) {
  *grid = 0;
  if (B >= 2 && b % 16 == 0 && batched_supported(dtype, d, B, int4)) {
    if (flags & FH_FLAG_SELECT_FIRST) return 3;
    if (flags & FH_FLAG_STREAM_ALL) return 4;
    // expected share of clusters that at least one of B independent rows
    // selects: when most clusters are read anyway, reading all of them
    // without waiting for the selection costs less.  Measured crossover (cold
    // calls, one MI355X): about 0.85 at the Llama-3.2-1B head shape, whose
    // stream walks K in 256-wide chunks (d % 256 == 0); at the Gemma-3-1B
    // INT4 head shape (d = 1152, 128-wide chunks) selecting first was as
    // fast or faster at every batch from 8 to 64 rows
    const double cover = 1.0 - pow(1.0 - (double)p / c, (double)B);
    return (cover >= kStreamAllCover && d % 256 == 0) ? 4 : 3;
  }
  if (B == 1 && stage1_selects(c)) {
    const int g = decode_b1_grid(c, p, (int)(row_bytes / 16), (c + 15) / 16, (int64_t)p * b,
                                 int4, num_cu);
    if (g > 0 && g <= kMaxGrid && (int64_t)g <= (int64_t)num_cu * blocks_per_cu) {
      *grid = g;
      return 1;
    }
  }
  return 2;
}

// adaptive (nullable): p_min and eps of the adaptive probe count, p its upper
// clamp, and the per-row counts' output
struct AdaptiveCall {
  int p_min;
  float eps;
  int32_t* out_p;
};

int step_impl(fh_handle* h, const void* H, int B, int p, int mode, float tau,
              const uint64_t* seeds, int32_t* out, float* out_lse, const fh_debug* dbg,
              void* stream, const AdaptiveCall* adaptive = nullptr) {
  if (!h || !H || !out) return FH_ERR_INVALID_ARG;
  if (B < 1 || B > h->max_batch || p < 1 || p > h->max_p || p > h->c) return FH_ERR_INVALID_ARG;
  if (adaptive && (adaptive->p_min < 1 || adaptive->p_min > p || !(adaptive->eps > 0.0f) ||
                   !(adaptive->eps <= 1.0f)))
    return FH_ERR_INVALID_ARG;
  if (mode == FH_MODE_SAMPLE && (!seeds || !(tau > 0.0f) || !isfinite(tau)))
    return FH_ERR_INVALID_ARG;
  if (!aligned16(H)) return FH_ERR_UNSUPPORTED;
  if (dbg && ((dbg->cand_ids == nullptr) != (dbg->cand_logits == nullptr)))
    return FH_ERR_INVALID_ARG;
  {
    const int st = check_device(h);
    if (st != FH_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  Timing tm[3];
  const Timing* t1 = nullptr;
  const Timing* t2 = nullptr;
  const Timing* t3 = nullptr;
  if (h->prof_calls < h->prof_cap) {
    const size_t e = (size_t)h->prof_calls++ * 6;
    for (int i = 0; i < 3; ++i) tm[i] = Timing{h->prof_ev[e + 2 * i], h->prof_ev[e + 2 * i + 1]};
    t1 = &tm[0];
    t2 = &tm[1];
    t3 = &tm[2];
  }
  const bool sample = mode == FH_MODE_SAMPLE;
  const float inv_tau = sample ? 1.0f / tau : 1.0f;
  const int nchunk = (int)(h->row_bytes / 16);
  Adaptive ad{};
  if (adaptive) {
    ad.on = 1;
    ad.p_min = adaptive->p_min;
    ad.L = (float)log(1.0 / (double)adaptive->eps);
    ad.rt = sample ? inv_tau : 1.0f;  // greedy decoding reads the rule at tau = 1
    ad.out_p = adaptive->out_p;
  }
  // adaptive sampling counts on plain scores while the keys carry noise
  const bool raw_scores = adaptive && sample;


  const bool int4 = h->quant != FH_QUANT_NONE;
  int b1_grid = 0;
  int path = plan_path(h->c, h->b, h->d, h->row_bytes, h->dtype, int4, B, p, h->num_cu,
                       h->b1_blocks_per_cu, h->flags, &b1_grid);
  const bool batched = path == 3 || path == 4;

  // stage 1 (+ selection by each batch row's last block on the GEMV path)
  Stage1Args s1{};
  s1.C = static_cast<const uint8_t*>(h->C);
  s1.row_bytes = h->row_bytes;
  s1.nchunk = nchunk;
  s1.c = h->c;
  s1.d = h->d;
  s1.q4 = h->q4;
  s1.q4s = h->q4s;
  s1.ntiles = h->ntiles;
  s1.groups = h->groups;
  s1.H = static_cast<const uint8_t*>(H);
  s1.h_bytes = h->row_bytes;
  s1.keys = h->keys;
  s1.key_stride = key_stride(h->c);
  s1.part_stride = (int64_t)h->max_batch * key_stride(h->c);
  s1.dbg_scores = dbg ? dbg->scores : nullptr;
  s1.sample = sample;
  s1.inv_tau = inv_tau;
  s1.seeds = seeds;
  s1.select = (!batched && stage1_selects(h->c)) ? 1 : 0;  // path 1 selects inside its launch too
  s1.p = p;
  s1.zcut = select_zcut(h->c, p);
  s1.ad = ad;
  s1.raw = (raw_scores && !batched) ? h->keys + s1.part_stride : nullptr;  // slice 1
  s1.raw_keys = raw_scores && batched;
  s1.counters = h->counters;
  s1.sel = h->sel;
  s1.sel_stride = h->max_p;
  s1.masks = nullptr;
  s1.error = h->error;

  // stage-2 gather over the cluster-major copy (GEMV paths)
  auto gather_args = [&]() {
    RowdotArgs a{};
    a.base = h->rows;
    a.row_bytes = h->rows_stride;
    a.borrowed = h->borrowed;
    a.nchunk = nchunk;
    a.H = static_cast<const uint8_t*>(H);
    a.h_bytes = h->row_bytes;
    a.nrows = (int64_t)p * h->b;
    a.sel = h->sel;
    a.sel_stride = h->max_p;
    a.c2t = h->c2t;
    a.b = h->b;
    a.nclusters = h->c;
    a.part_best = h->row_best;
    a.counters = h->counters;
    a.lse_part = h->lse_part;
    a.out_tokens = out;
    a.out_lse = out_lse;
    a.dbg_ids = dbg ? dbg->cand_ids : nullptr;
    a.dbg_logits = dbg ? dbg->cand_logits : nullptr;
    a.dbg_stride = (int64_t)p * h->b;
    a.sample = sample;
    a.inv_tau = inv_tau;
    a.seeds = seeds;
    return a;
  };

  // batch 1: the whole step in one launch when the shape allows it
  if (path == 1) {
    DecodeB1Args f{};
    f.s1 = s1;
    f.s2 = gather_args();
    f.s1.keys = h->b1_keys;
    f.s1.key_stride = b1_key_stride(h->c);
    f.raw = h->b1_raw;
    f.s1.raw = raw_scores ? h->b1_raw : nullptr;  // a flag here: the kernel picks the set
    f.s2.part_best = h->b1_slots;
    f.s2.lse_part = h->b1_lse;
    f.sel = h->b1_sel;
    f.epoch = h->b1_epoch;
    f.go = h->b1_go;
    f.slot_stride = kDecodeB1SlotStride;
    {
      FH_TRY(launch_decode_b1(f, h->dtype, int4, b1_grid,
                              (h->flags & FH_FLAG_COOPERATIVE) != 0, s, t1));
      if (t2) {  // selection and stage 2 ran inside the one launch
        (void)hipEventRecord(t2->start, s);
        (void)hipEventRecord(t2->stop, s);
        (void)hipEventRecord(t3->start, s);
        (void)hipEventRecord(t3->stop, s);
      }
      if (dbg && dbg->clusters) {
        // the selection of this launch sits in the set its epoch picked
        FH_TRY(launch_b1_copy_sel(h->b1_epoch, h->b1_sel, kDecodeB1MaxP, dbg->clusters, p, s));
      }
      h->last_path = 1;
      return FH_OK;
    }
  }

  h->last_path = path;
  if (path == 4) {
    Stage2mArgs a{};
    a.base = h->rows;
    a.row_bytes = h->rows_stride;
    a.borrowed = h->borrowed;
    a.v = h->v;
    a.c = h->c;
    a.b = h->b;
    a.d = h->d;
    a.B = B;
    a.p = p;
    a.H = static_cast<const uint8_t*>(H);
    a.h_bytes = h->row_bytes;
    a.c2t = h->c2t;
    a.sample = sample;
    a.inv_tau = inv_tau;
    a.seeds = seeds;
    a.with_lse = out_lse != nullptr;
    a.part_best = h->all_best;
    a.part_lse = h->all_lse;
    a.keys = h->keys;
    a.key_stride = key_stride(h->c);
    a.dbg_scores = dbg ? dbg->scores : nullptr;
    a.raw_scores = raw_scores;
    a.ksplit = 1;
    a.cbase = static_cast<const uint8_t*>(h->C);
    a.c_row_bytes = h->row_bytes;
    a.n1 = int4 ? h->ntiles : (h->c + 15) / 16;
    a.q4 = int4 ? h->q4 : nullptr;
    a.q4s = int4 ? h->q4s : nullptr;
    a.groups = h->groups;
    SelectArgs sa{};
    sa.keys = h->keys;
    sa.key_stride = key_stride(h->c);
    sa.c = h->c;
    sa.p = p;
    sa.zcut = s1.zcut;
    sa.sel = h->sel;
    sa.sel_stride = h->max_p;
    sa.error = h->error;
    sa.nparts = 1;
    sa.part_stride = s1.part_stride;
    sa.sample = sample;
    sa.inv_tau = inv_tau;
    sa.seeds = seeds;
    sa.form_keys = raw_scores;
    sa.ad = ad;
    sa.dbg_scores = (raw_scores && dbg) ? dbg->scores : nullptr;
    sa.fold_best = h->all_best;
    sa.fold_lse = out_lse ? h->all_lse : nullptr;
    sa.fold_sub = h->b / 16;
    sa.fold_pitch = B;
    sa.out_tokens = out;
    sa.out_lse = out_lse;
    FH_TRY(launch_stream_all(a, sa, s, t1, t2));
    if (t3) {  // stage 2 ran inside the first launch
      (void)hipEventRecord(t3->start, s);
      (void)hipEventRecord(t3->stop, s);
    }
    if (dbg && dbg->cand_ids) {
      // the stream keeps one record per cluster, not the candidates: the
      // debug output gathers the selected clusters' rows again (row-dot
      // logits, which round apart from the stream's by the summation order)
      // and writes its own tokens aside; the step's tokens stay the fold's
      RowdotArgs g = gather_args();
      g.out_tokens = h->dbg_tokens;
      g.out_lse = nullptr;
      const int gx = rowdot_grid(g.nrows, nchunk, kRowGather);
      if (gx > kMaxGrid) return FH_ERR_UNSUPPORTED;
      FH_TRY(launch_rowdot(g, kRowGather, h->dtype, B, gx, s));
    }
    if (dbg && dbg->clusters) {
      FH_TRY(hipMemcpy2DAsync(dbg->clusters, (size_t)p * 4, h->sel, (size_t)h->max_p * 4,
                              (size_t)p * 4, B, hipMemcpyDeviceToDevice, s));
    }
    return FH_OK;
  }
  int ksplit = 1;
  if (batched) {
    FH_TRY(launch_stage1_mfma(s1, int4, B, s, t1, &ksplit));
  } else {
    FH_TRY(launch_stage1(s1, h->dtype, int4, B, s, t1));
  }
  if (!s1.select) {
    SelectArgs a{};
    a.keys = h->keys;
    a.key_stride = key_stride(h->c);
    a.c = h->c;
    a.p = p;
    a.zcut = s1.zcut;
    a.sel = h->sel;
    a.sel_stride = h->max_p;
    a.masks = batched ? h->masks : nullptr;
    a.error = h->error;
    a.nparts = ksplit;
    a.part_stride = s1.part_stride;
    a.sample = sample;
    a.inv_tau = inv_tau;
    a.seeds = seeds;
    a.form_keys = s1.raw_keys;
    a.raw = s1.raw;
    a.ad = ad;
    a.dbg_scores = (ksplit > 1 || a.form_keys) && dbg ? dbg->scores : nullptr;
    if (batched && B < kUnionMinRows) {
      a.ulist = h->ulist;
      a.ucount = h->ucount;
    }
    FH_TRY(launch_select(a, B, s, t2));
  } else if (t2) {  // selection ran inside stage 1
    (void)hipEventRecord(t2->start, s);
    (void)hipEventRecord(t2->stop, s);
  }
  if (dbg && dbg->clusters) {
    FH_TRY(hipMemcpy2DAsync(dbg->clusters, (size_t)p * 4, h->sel, (size_t)h->max_p * 4,
                            (size_t)p * 4, B, hipMemcpyDeviceToDevice, s));
  }
  // stage 2: candidate logits + decode
  if (batched) {
    Stage2mArgs a{};
    a.base = h->rows;
    a.row_bytes = h->rows_stride;
    a.borrowed = h->borrowed;
    a.v = h->v;
    a.c = h->c;
    a.b = h->b;
    a.d = h->d;
    a.B = B;
    a.p = p;
    a.H = static_cast<const uint8_t*>(H);
    a.h_bytes = h->row_bytes;
    // small batches select few clusters in all: stage 2 walks their list;
    // from kUnionMinRows rows on, the union covers most clusters and
    // stage 2 walks all of them, skipping the ones no row selected
    a.ulist = B < kUnionMinRows ? h->ulist : nullptr;
    a.ucount = B < kUnionMinRows ? h->ucount : nullptr;
    a.masks = h->masks;
    a.c2t = h->c2t;
    a.sel = h->sel;
    a.sel_stride = h->max_p;
    a.sample = sample;
    a.inv_tau = inv_tau;
    a.seeds = seeds;
    a.with_lse = out_lse != nullptr;
    a.part_best = h->part_best;
    a.part_lse = h->part_lse;
    a.out_tokens = out;
    a.out_lse = out_lse;
    a.dbg_ids = dbg ? dbg->cand_ids : nullptr;
    a.dbg_logits = dbg ? dbg->cand_logits : nullptr;
    a.dbg_stride = (int64_t)p * h->b;
    FH_TRY(launch_stage2_mfma(a, false, s, t3));
    return FH_OK;
  }
  {
    RowdotArgs a = gather_args();
    const int gx = rowdot_grid(a.nrows, nchunk, kRowGather);
    if (gx > kMaxGrid) return FH_ERR_UNSUPPORTED;
    FH_TRY(launch_rowdot(a, kRowGather, h->dtype, B, gx, s, t3));
  }
  return FH_OK;
}

}  // namespace

// Workspace of flashhead_mc_marginal: byte offsets of its parts, each
// 256-byte aligned.
struct McLayout {
  size_t sel, flags, cl, zq, qcl, contrib, total;
};
static McLayout mc_layout(int c, int n, int p, int q) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  McLayout L{};
  size_t o = 0;
  L.sel = o;
  o += up((size_t)n * p * 4);
  L.flags = o;
  o += up((size_t)c * 4);
  L.cl = o;
  o += up((size_t)c * 8);
  L.zq = o;
  o += up((size_t)q * 4);
  L.qcl = o;
  o += up((size_t)q * 4);
  L.contrib = o;
  o += up((size_t)n * q * 4);
  L.total = o;
  return L;
}

namespace {

int dense_impl(const void* E, int64_t v, int32_t d, int32_t dtype, int64_t lde, const void* H,
               int32_t B, int32_t mode, float tau, const uint64_t* seeds, int32_t* out_tokens,
               float* out_lse, void* workspace, bool clear_counters, void* stream);

// The workspace of dense_head_static: the layout of dense_head's workspace
// for FH_DENSE_STATIC_MAX_BATCH rows, one copy per device, held until the
// process ends.  Host code never uses this name as an address: each
// device's copy is found once through hipGetSymbolAddress.
constexpr size_t kStaticScratchBytes =
    (size_t)FH_DENSE_STATIC_MAX_BATCH * (kArriveWords * 4 + kDenseMaxGrid * 16);
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array (looked up on the first
// call on that device, with the device current).
int static_scratch(void** out) {
  int dev = -1;
  FH_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return FH_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    FH_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return FH_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FH_OK;
}

}  // namespace

extern "C" {

const char* flashhead_last_hip_error(void) { return hipGetErrorName(g_last_hip); }

int flashhead_plan_step(int32_t c, int32_t b, int32_t d, int32_t dtype, int32_t quant, int32_t B,
                        int32_t p, int32_t num_cu, int32_t blocks_per_cu, int32_t flags,
                        int32_t* grid) {
  if (!grid) return FH_ERR_INVALID_ARG;
  *grid = 0;
  const int es = esize_of(dtype);
  if (c < 1 || b < 1 || d < 1 || !es || B < 1 || B > FH_MAX_BATCH || p < 1 || p > c ||
      num_cu < 1 || blocks_per_cu < 0 || quant < FH_QUANT_NONE || quant > FH_QUANT_INT4_G128_MEAN)
    return FH_ERR_INVALID_ARG;
  if ((flags & FH_FLAG_STREAM_ALL) && (flags & FH_FLAG_SELECT_FIRST)) return FH_ERR_INVALID_ARG;
  int g = 0;
  const int path = plan_path(c, b, d, (int64_t)d * es, dtype, quant != FH_QUANT_NONE, B, p,
                             num_cu, blocks_per_cu, flags, &g);
  *grid = g;
  return path;
}

int flashhead_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 || !aligned16(buf)) return FH_ERR_INVALID_ARG;
  int dev = 0, ncu = 0;
  FH_TRY(hipGetDevice(&dev));
  FH_TRY(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  FH_TRY(launch_stream_read(buf, bytes, sink, ncu, static_cast<hipStream_t>(stream)));
  return FH_OK;
}

const char* flashhead_status_string(int status) {
  switch (status) {
    case FH_OK: return "ok";
    case FH_ERR_INVALID_ARG: return "invalid argument";
    case FH_ERR_NOT_PERMUTATION: return "C2T is not a permutation of [0, v)";
    case FH_ERR_UNSUPPORTED: return "unsupported dtype, alignment or shape";
    case FH_ERR_HIP: return "HIP runtime error";
    case FH_ERR_OOM: return "device out of memory";
    default: return "unknown status";
  }
}

int flashhead_prepare(const fh_desc* ds, fh_handle** out) {
  if (!out) return FH_ERR_INVALID_ARG;
  *out = nullptr;
  {
    const int st = validate_desc(ds);
    if (st != FH_OK) return st;
  }
  const int es = esize_of(ds->dtype);
  const int64_t row_bytes = (int64_t)ds->d * es;
  fh_handle* h = new (std::nothrow) fh_handle();
  if (!h) return FH_ERR_OOM;
  h->v = ds->v;
  h->d = ds->d;
  h->c = ds->c;
  h->b = ds->b;
  h->dtype = ds->dtype;
  h->quant = ds->quant;
  h->max_batch = ds->max_batch;
  h->max_p = ds->max_p;
  h->esize = es;
  h->row_bytes = row_bytes;
  h->flags = ds->flags;
  h->borrowed = (ds->flags & FH_FLAG_BORROW_E) != 0;
  const int st = prepare_impl(ds, h);
  if (st != FH_OK) {
    (void)hipStreamSynchronize(static_cast<hipStream_t>(ds->stream));
    free_handle(h);
    return st;
  }
  *out = h;
  return FH_OK;
}

void flashhead_destroy(fh_handle* h) { free_handle(h); }

int flashhead_greedy(fh_handle* h, const void* H, int32_t B, int32_t p, int32_t* out_tokens,
                     const fh_debug* dbg, void* stream) {
  return step_impl(h, H, B, p, FH_MODE_GREEDY, 1.0f, nullptr, out_tokens, nullptr, dbg, stream);
}

int flashhead_sample(fh_handle* h, const void* H, int32_t B, int32_t p, float tau,
                     const uint64_t* seeds, int32_t* out_tokens, float* out_lse,
                     const fh_debug* dbg, void* stream) {
  return step_impl(h, H, B, p, FH_MODE_SAMPLE, tau, seeds, out_tokens, out_lse, dbg, stream);
}

int flashhead_greedy_adaptive(fh_handle* h, const void* H, int32_t B, int32_t p_min,
                              int32_t p_max, float eps, int32_t* out_tokens, int32_t* out_p,
                              const fh_debug* dbg, void* stream) {
  const AdaptiveCall ad{p_min, eps, out_p};
  return step_impl(h, H, B, p_max, FH_MODE_GREEDY, 1.0f, nullptr, out_tokens, nullptr, dbg,
                   stream, &ad);
}

int flashhead_sample_adaptive(fh_handle* h, const void* H, int32_t B, int32_t p_min,
                              int32_t p_max, float eps, float tau, const uint64_t* seeds,
                              int32_t* out_tokens, float* out_lse, int32_t* out_p,
                              const fh_debug* dbg, void* stream) {
  const AdaptiveCall ad{p_min, eps, out_p};
  return step_impl(h, H, B, p_max, FH_MODE_SAMPLE, tau, seeds, out_tokens, out_lse, dbg, stream,
                   &ad);
}

size_t flashhead_mc_workspace_bytes(const fh_handle* h, int32_t n_draws, int32_t p,
                                    int32_t n_tokens) {
  if (!h || n_draws < 1 || p < 1 || n_tokens < 1) return 0;
  return mc_layout(h->c, n_draws, p, n_tokens).total;
}

int flashhead_mc_marginal(fh_handle* h, const void* H, int32_t p, float tau,
                          const uint64_t* seeds, int32_t n_draws, const int32_t* tokens,
                          int32_t n_tokens, float* out_prob, float* out_lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!h || !H || !seeds || !tokens || !out_prob || !workspace) return FH_ERR_INVALID_ARG;
  if (p < 1 || p > h->c || p > h->max_p || p > kMcMaxP) return FH_ERR_INVALID_ARG;
  if (!(tau > 0.0f) || !isfinite(tau)) return FH_ERR_INVALID_ARG;
  if (n_draws < 1 || n_draws > (1 << 20) || n_tokens < 1 || n_tokens > (1 << 16))
    return FH_ERR_INVALID_ARG;
  const McLayout L = mc_layout(h->c, n_draws, p, n_tokens);
  if (workspace_bytes < L.total) return FH_ERR_INVALID_ARG;
  if (!aligned16(H) || ((uintptr_t)workspace & 255u) != 0) return FH_ERR_UNSUPPORTED;
  {
    const int st = check_device(h);
    if (st != FH_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool int4 = h->quant != FH_QUANT_NONE;
  const int nchunk = (int)(h->row_bytes / 16);

  // stage 1 once: the plain scores of h into the handle's first key row
  Stage1Args s1{};
  s1.C = static_cast<const uint8_t*>(h->C);
  s1.row_bytes = h->row_bytes;
  s1.nchunk = nchunk;
  s1.c = h->c;
  s1.d = h->d;
  s1.q4 = h->q4;
  s1.q4s = h->q4s;
  s1.ntiles = h->ntiles;
  s1.groups = h->groups;
  s1.H = static_cast<const uint8_t*>(H);
  s1.h_bytes = h->row_bytes;
  s1.keys = h->keys;
  s1.key_stride = key_stride(h->c);
  s1.inv_tau = 1.0f;
  s1.error = h->error;
  FH_TRY(launch_stage1(s1, h->dtype, int4, 1, s));

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  McArgs a{};
  a.scores = h->keys;
  a.score_stride = key_stride(h->c);
  a.c = h->c;
  a.p = p;
  a.zcut = select_zcut(h->c, p);
  a.inv_tau = 1.0f / tau;
  a.seeds = seeds;
  a.n = n_draws;
  a.sel = reinterpret_cast<int32_t*>(ws + L.sel);
  a.flags = reinterpret_cast<uint32_t*>(ws + L.flags);
  a.cl = reinterpret_cast<float2*>(ws + L.cl);
  a.H = static_cast<const uint8_t*>(H);
  a.nchunk = nchunk;
  a.Ec = h->rows;
  a.row_bytes = h->rows_stride;
  a.borrowed = h->borrowed;
  a.b = h->b;
  a.t2row = h->t2row;
  a.v = h->v;
  a.tokens = tokens;
  a.q = n_tokens;
  a.zq = reinterpret_cast<float*>(ws + L.zq);
  a.qcl = reinterpret_cast<int32_t*>(ws + L.qcl);
  a.contrib = reinterpret_cast<float*>(ws + L.contrib);
  a.out_prob = out_prob;
  a.out_lse = out_lse;
  a.error = h->error;
  FH_TRY(hipMemsetAsync(a.flags, 0, (size_t)h->c * 4, s));

  // a cluster's rows in the cluster-major copy, folded into (max, sum)
  RowdotArgs ra{};
  ra.base = h->rows;
  ra.row_bytes = h->rows_stride;
  ra.borrowed = h->borrowed;
  ra.nchunk = nchunk;
  ra.nrows = h->b;
  ra.c2t = h->c2t;
  ra.b = h->b;
  ra.nclusters = h->c;
  ra.inv_tau = 1.0f / tau;
  ra.out_lse = out_prob;  // only marks that the rows' lse is folded; never written here
  FH_TRY(launch_mc(a, ra, h->dtype, s));
  return FH_OK;
}

size_t dense_head_workspace_bytes(int32_t B) {
  if (B < 1) return 0;
  const size_t nb = (size_t)B;
  return nb * kArriveWords * 4 + nb * kDenseMaxGrid * 16;
}

int dense_head(const void* E, int64_t v, int32_t d, int32_t dtype, int64_t lde, const void* H,
               int32_t B, int32_t mode, float tau, const uint64_t* seeds, int32_t* out_tokens,
               float* out_lse, void* workspace, void* stream) {
  if (!workspace) return FH_ERR_INVALID_ARG;
  return dense_impl(E, v, d, dtype, lde, H, B, mode, tau, seeds, out_tokens, out_lse,
                    workspace, false, stream);
}

int dense_head_static(const void* E, int64_t v, int32_t d, int32_t dtype, int64_t lde,
                      const void* H, int32_t B, int32_t mode, float tau, const uint64_t* seeds,
                      int32_t* out_tokens, float* out_lse, void* stream) {
  if (B > FH_DENSE_STATIC_MAX_BATCH) return FH_ERR_INVALID_ARG;
  void* ws = nullptr;
  const int st = static_scratch(&ws);
  if (st != FH_OK) return st;
  return dense_impl(E, v, d, dtype, lde, H, B, mode, tau, seeds, out_tokens, out_lse, ws, true,
                    stream);
}

}  // extern "C"

namespace {

int dense_impl(const void* E, int64_t v, int32_t d, int32_t dtype, int64_t lde, const void* H,
               int32_t B, int32_t mode, float tau, const uint64_t* seeds, int32_t* out_tokens,
               float* out_lse, void* workspace, bool clear_counters, void* stream) {
  if (!E || !H || !out_tokens || !workspace) return FH_ERR_INVALID_ARG;
  if (v < 1 || d < 1 || lde < d || B < 1 || B > FH_MAX_BATCH) return FH_ERR_INVALID_ARG;
  if (mode != FH_MODE_GREEDY && mode != FH_MODE_SAMPLE) return FH_ERR_INVALID_ARG;
  if (mode == FH_MODE_SAMPLE && (!seeds || !(tau > 0.0f) || !isfinite(tau)))
    return FH_ERR_INVALID_ARG;
  if (v > (int64_t)INT32_MAX) return FH_ERR_UNSUPPORTED;
  const int es = esize_of(dtype);
  if (!es) return FH_ERR_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)d * es;
  if (row_bytes % 16 || (lde * es) % 16 || row_bytes > FH_MAX_ROW_BYTES) return FH_ERR_UNSUPPORTED;
  if (!aligned16(E) || !aligned16(H) || !aligned16(workspace)) return FH_ERR_UNSUPPORTED;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t nb = (size_t)B;
  // workspace: arrival counters | partial best keys | partial lse pairs
  uint32_t* ws_ctr = reinterpret_cast<uint32_t*>(ws);
  uint64_t* ws_best = reinterpret_cast<uint64_t*>(ws + nb * kArriveWords * 4);
  float2* ws_lse = reinterpret_cast<float2*>(ws + nb * kArriveWords * 4 + nb * kDenseMaxGrid * 8);
  if (B >= 2 && batched_supported(dtype, d, B, false)) {
    Stage2mArgs m{};
    m.base = static_cast<const uint8_t*>(E);
    m.row_bytes = lde * es;
    m.v = v;
    m.b = 16;
    m.d = d;
    m.B = B;
    m.H = static_cast<const uint8_t*>(H);
    m.h_bytes = row_bytes;
    m.sample = mode == FH_MODE_SAMPLE;
    m.inv_tau = m.sample ? 1.0f / tau : 1.0f;
    m.seeds = seeds;
    m.with_lse = out_lse != nullptr;
    m.part_best = ws_best;
    m.part_lse = ws_lse;
    m.out_tokens = out_tokens;
    m.out_lse = out_lse;
    FH_TRY(launch_stage2_mfma(m, true, static_cast<hipStream_t>(stream)));
    return FH_OK;
  }
  RowdotArgs a{};
  a.base = static_cast<const uint8_t*>(E);
  a.row_bytes = lde * es;
  a.nchunk = (int)(row_bytes / 16);
  a.H = static_cast<const uint8_t*>(H);
  a.h_bytes = row_bytes;
  a.nrows = v;
  a.part_best = ws_best;
  a.counters = ws_ctr;
  a.lse_part = ws_lse;
  a.out_tokens = out_tokens;
  a.out_lse = out_lse;
  a.sample = mode == FH_MODE_SAMPLE;
  a.inv_tau = a.sample ? 1.0f / tau : 1.0f;
  a.seeds = seeds;
  const int gx = rowdot_grid(v, a.nchunk, kRowDense);
  if (gx > kDenseMaxGrid) return FH_ERR_UNSUPPORTED;
  // the shared array keeps the last call's contents: its arrival counters
  // are cleared before use (a fill kernel, which a graph may capture)
  if (clear_counters)
    FH_TRY(launch_fill_u32(ws_ctr, 0u, (int64_t)nb * kArriveWords,
                           static_cast<hipStream_t>(stream)));
  FH_TRY(launch_rowdot(a, kRowDense, dtype, B, gx, static_cast<hipStream_t>(stream)));
  return FH_OK;
}

}  // namespace

extern "C" {



int flashhead_kmeans(const void* E, int64_t v, int32_t d, int32_t dtype, int64_t lde, int32_t c,
                     const int32_t* init, int32_t max_iter, int32_t* c2t, double* centroids,
                     int32_t* iters_run, void* stream) {
  if (iters_run) *iters_run = 0;
  if (!E || !init || !c2t) return FH_ERR_INVALID_ARG;
  if (v < 1 || c < 1 || d < 1 || lde < d || max_iter < 1 || v % c) return FH_ERR_INVALID_ARG;
  const int es = esize_of(dtype);
  if (!es) return FH_ERR_UNSUPPORTED;
  if (v > (int64_t)INT32_MAX || c > FH_MAX_C || v / c > kMaxKmB) return FH_ERR_UNSUPPORTED;
  if ((uintptr_t)E % es) return FH_ERR_UNSUPPORTED;
  std::vector<char> seen((size_t)v, 0);
  for (int32_t k = 0; k < c; ++k) {
    if (init[k] < 0 || init[k] >= v || seen[init[k]]) return FH_ERR_INVALID_ARG;
    seen[init[k]] = 1;
  }
  KMeansArgs a{};
  a.E = static_cast<const uint8_t*>(E);
  a.lde_bytes = lde * es;
  a.dtype = dtype;
  a.v = v;
  a.d = d;
  a.c = c;
  a.init_host = init;
  a.max_iter = max_iter;
  a.c2t = c2t;
  a.centroids = centroids;
  int iters = 0, status = 0;
  FH_TRY(run_kmeans(a, static_cast<hipStream_t>(stream), &iters, &status));
  if (iters_run) *iters_run = iters;
  return status ? FH_ERR_INVALID_ARG : FH_OK;
}

int flashhead_export_centroids(const fh_handle* h, void* dst) {
  if (!h || !dst) return FH_ERR_INVALID_ARG;
  FH_TRY(hipMemcpy(dst, h->C, (size_t)h->c * h->row_bytes, hipMemcpyDeviceToHost));
  return FH_OK;
}

int flashhead_export_int4(const fh_handle* h, uint8_t* codes, uint16_t* scales) {
  if (!h || !codes || !scales) return FH_ERR_INVALID_ARG;
  if (h->quant == FH_QUANT_NONE) return FH_ERR_UNSUPPORTED;
  const size_t tiles = (size_t)h->ntiles * h->groups;
  FH_TRY(hipMemcpy(codes, h->q4, tiles * 1024, hipMemcpyDeviceToHost));
  FH_TRY(hipMemcpy(scales, h->q4s, tiles * 16 * 2, hipMemcpyDeviceToHost));
  return FH_OK;
}

int flashhead_profile_begin(fh_handle* h, int32_t max_calls) {
  if (!h || max_calls < 1 || max_calls > (1 << 20)) return FH_ERR_INVALID_ARG;
  drop_profile(h);
  h->prof_ev.resize((size_t)max_calls * 6, nullptr);
  for (auto& e : h->prof_ev) {
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      e = nullptr;
      drop_profile(h);
      return hip_fail(err);
    }
  }
  h->prof_cap = max_calls;
  h->prof_calls = 0;
  return FH_OK;
}

int flashhead_profile_end(fh_handle* h, double* stage_ms, int32_t* calls) {
  if (!h || !stage_ms || !calls) return FH_ERR_INVALID_ARG;
  double acc[3] = {0.0, 0.0, 0.0};
  const int n = h->prof_calls;
  int st = FH_OK;
  for (int i = 0; i < n && st == FH_OK; ++i) {
    for (int k = 0; k < 3; ++k) {
      hipEvent_t a = h->prof_ev[(size_t)i * 6 + 2 * k], b = h->prof_ev[(size_t)i * 6 + 2 * k + 1];
      float ms = 0.0f;
      hipError_t err = hipEventSynchronize(b);
      if (err == hipSuccess) err = hipEventElapsedTime(&ms, a, b);
      if (err != hipSuccess) {
        st = hip_fail(err);
        break;
      }
      acc[k] += ms;
    }
  }
  for (int k = 0; k < 3; ++k) stage_ms[k] = n ? acc[k] / n : 0.0;
  *calls = n;
  drop_profile(h);
  return st;
}

int flashhead_query(const fh_handle* h, int32_t what, int64_t* value) {
  if (!h || !value) return FH_ERR_INVALID_ARG;
  switch (what) {
    case 0: *value = h->v; break;
    case 1: *value = h->d; break;
    case 2: *value = h->c; break;
    case 3: *value = h->b; break;
    case 4: *value = h->dtype; break;
    case 5: *value = h->quant; break;
    case 6: *value = h->max_batch; break;
    case 7: *value = h->max_p; break;
    case 8: *value = h->bytes; break;
    case 10: *value = h->last_path; break;
    case 12: *value = h->b1_blocks_per_cu; break;
    case 13: *value = h->num_cu; break;
    case 14: *value = h->flags; break;
    case 11: {  // the single launch's buffer set for the next launch
      uint32_t ep = 0, go[2] = {0u, 0u};
      FH_TRY(hipMemcpy(&ep, h->b1_epoch, 4, hipMemcpyDeviceToHost));
      FH_TRY(hipMemcpy(go, h->b1_go, 8, hipMemcpyDeviceToHost));
      const int set = (int)(ep & 1u);
      const int64_t ks = b1_key_stride(h->c);
      std::vector<uint32_t> keys((size_t)ks);
      std::vector<int32_t> sel((size_t)kDecodeB1MaxP);
      std::vector<uint64_t> slots((size_t)kDecodeB1SlotStride);
      FH_TRY(hipMemcpy(keys.data(), h->b1_keys + set * ks, (size_t)ks * 4,
                       hipMemcpyDeviceToHost));
      FH_TRY(hipMemcpy(sel.data(), h->b1_sel + set * kDecodeB1MaxP, (size_t)kDecodeB1MaxP * 4,
                       hipMemcpyDeviceToHost));
      FH_TRY(hipMemcpy(slots.data(), h->b1_slots + set * kDecodeB1SlotStride,
                       (size_t)kDecodeB1SlotStride * 8, hipMemcpyDeviceToHost));
      int64_t bits = 0;
      for (int k = 0; k < h->c; ++k)
        if (keys[(size_t)k] != 0xFFFFFFFFu) bits |= 1;
      for (int i = 0; i < kDecodeB1MaxP; ++i)
        if (sel[(size_t)i] != -1) bits |= 2;
      for (int j = 0; j < kDecodeB1MaxGrid; ++j)
        if (slots[(size_t)j * 16] != 0ull) bits |= 4;
      if (go[set] != 0u) bits |= 8;
      FH_TRY(hipMemcpy(keys.data(), h->b1_raw + set * ks, (size_t)ks * 4, hipMemcpyDeviceToHost));
      for (int k = 0; k < h->c; ++k)
        if (keys[(size_t)k] != 0xFFFFFFFFu) bits |= 32;
      *value = bits;
      break;
    }
    case 9: {  // selection error flag (synchronous read and clear)
      uint32_t e = 0;
      FH_TRY(hipMemcpy(&e, h->error, 4, hipMemcpyDeviceToHost));
      if (e) FH_TRY(hipMemset(h->error, 0, 4));
      *value = e;
      break;
    }
    default: return FH_ERR_INVALID_ARG;
  }
  return FH_OK;
}

}  // extern "C"
