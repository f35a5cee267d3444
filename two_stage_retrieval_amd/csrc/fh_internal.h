// Host-side declarations shared by the translation units of libflashhead.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flashhead.h"

namespace fh {

// Arrival counters of one batch row (see wait_arrivals in fh_device.h).
constexpr int kArriveCounters = 32;
constexpr int kArriveStride = 32;  // uint32 per counter: one 128-byte line each
constexpr int kArriveWords = kArriveCounters * kArriveStride;

// Adaptive probe count (the selecting workgroup's rule, see adaptive_count in
// fh_select.h).  `on` = 0: the call's p probes every row.
struct Adaptive {
  int on;
  int p_min;          // the call's p is the upper clamp
  float L;            // ln(1 / eps)
  float rt;           // 1 / tau of the rule (1 for greedy decoding)
  int32_t* out_p;     // device, B probe counts, or null
};
// A selection entry past a row's probe count (never a cluster id).
constexpr int32_t kUnusedEntry = 0x7FFFFFFF;

// Which rows a row-dot launch visits and what it does with each dot product.
enum RowdotMode : int {
  kRowGather = 1,  // candidate rows C2T[sel[i / b], i % b]; decode epilogue
  kRowDense = 2,   // rows [0, nrows) of `base`; decode epilogue
};

struct RowdotArgs {
  const uint8_t* base;   // E (dense, or the caller's E when borrowed), C, or the
                         // cluster-major copy of E (gather)
  int64_t row_bytes;     // stride between rows of `base`
  int borrowed;          // gather: base is the caller's E, candidate rows are
                         // token rows C2T[k, j] (else rows k*b + j of the copy)
  int nchunk;            // 16-byte chunks per row
  const uint8_t* H;      // B x d, row stride h_bytes
  int64_t h_bytes;
  int64_t nrows;         // logical rows per batch row
  // gather
  const int32_t* sel;    // B x sel_stride, selected clusters (ascending)
  int sel_stride;
  const int32_t* c2t;    // c x b
  int b;
  int nclusters;         // c (selected ids are clamped to [0, c))
  // decode epilogue
  uint64_t* part_best;   // B x gridDim.x partial best decode keys
  uint32_t* counters;    // B x kArriveWords arrival counters (zero between calls)
  float2* lse_part;      // B x gridDim.x partial (max, sum)
  int32_t* out_tokens;
  float* out_lse;
  int32_t* dbg_ids;      // optional, B x dbg_stride
  float* dbg_logits;
  int64_t dbg_stride;
  // sampling
  int sample;
  float inv_tau;
  const uint64_t* seeds;
};

struct SelectArgs {
  const float* keys;     // B x key_stride
  int64_t key_stride;
  // nparts > 1: keys holds nparts partial-score blocks part_stride floats
  // apart; the select sums them in slice order and forms the keys (score, or
  // score / tau + Gumbel noise), writing the scores to dbg_scores if given
  int nparts;
  int64_t part_stride;
  int sample;
  float inv_tau;
  const uint64_t* seeds;
  float* dbg_scores;     // B x c
  int form_keys;         // keys holds plain scores (nparts == 1 too): form the keys here
  const float* raw;      // adaptive count on these plain scores (B x key_stride) when the
                         // keys already carry noise; null otherwise
  int c, p;
  float zcut;            // histogram range hint (select_zcut; 0: none)
  Adaptive ad;
  int32_t* sel;          // B x sel_stride, written ascending
  int sel_stride;
  uint64_t* masks;       // optional: per-cluster bitmask of selecting rows
  uint32_t* error;       // optional: set non-zero if a row selected != p
  // optional union of the rows' clusters, compacted by a second launch
  // (needs masks)
  int32_t* ulist;        // clusters with a non-zero mask, ascending
  int32_t* ucount;
  // select-and-fold (the all-cluster stream): after its selection, row r
  // folds the per-(16-row item, row) partials of its selected clusters
  const uint64_t* fold_best;  // items x fold_pitch best decode keys
  const float2* fold_lse;     // items x fold_pitch (max, sum) of z / tau, or null
  int fold_sub;               // items per cluster (b / 16)
  int fold_pitch;             // batch rows per item record
  int32_t* out_tokens;
  float* out_lse;
};

struct Stage2mArgs {
  const uint8_t* base;   // C (scores), cluster-major copy of E or the caller's E
                         // (flash, see borrowed) or E (dense)
  int64_t row_bytes;
  int borrowed;          // flash: base is the caller's E, rows C2T[k, j]
  int64_t v;             // rows of E (dense)
  int c;                 // rows of C (scores)
  int b, d, B, p;
  const uint8_t* H;      // B x d bf16
  int64_t h_bytes;
  const int32_t* ulist;  // flash: union of the selected clusters, ascending,
  const int32_t* ucount; // or null: every cluster, skipping zero masks
  uint64_t* masks;       // flash: rows that selected each cluster
  const int32_t* c2t;
  const int32_t* sel;    // flash debug: B x sel_stride ascending selections
  int sel_stride;
  int sample;
  float inv_tau;
  const uint64_t* seeds;
  int with_lse;
  uint64_t* part_best;   // per block x B
  float2* part_lse;
  int32_t* out_tokens;
  float* out_lse;
  int32_t* dbg_ids;
  float* dbg_logits;
  int64_t dbg_stride;
  // scores epilogue (stage 1)
  float* keys;
  int64_t key_stride;
  float* dbg_scores;
  int ksplit;            // K slices (scores); > 1: keys holds per-slice partial scores
  int64_t part_stride;   // floats between the slices' B x key_stride blocks
  int raw_scores;        // scores epilogue: plain scores even at one slice (the
                         // select then forms the keys)
  // the all-cluster stream (stage 1 and stage 2 in one launch): items
  // [0, n1) are stage-1 items (16 centroid rows of cbase, or INT4 tiles when
  // q4 is set), items from n1 on are the 16-row items of every cluster;
  // part_best / part_lse receive one record per (item, batch row), item-major
  const uint8_t* cbase;
  int64_t c_row_bytes;
  int64_t n1;
  const uint8_t* q4;
  const uint16_t* q4s;
  int groups;
};
constexpr int kMaxKSplit = 4;
// batched stage 2 walks the union list below this many rows, every cluster
// (skipping unselected ones) from it on
constexpr int kUnionMinRows = 16;

struct Stage1Args {
  const uint8_t* C;       // c x d centroids (bf16 / fp32)
  int64_t row_bytes;      // d * element size
  int nchunk;             // 16-byte chunks per row
  int c, d;
  const uint8_t* q4;      // INT4 tiles (see flashhead_export_int4)
  const uint16_t* q4s;
  int ntiles, groups;     // ceil(c / 16), d / 128
  const uint8_t* H;       // B x d
  int64_t h_bytes;
  float* keys;            // B x key_stride selection keys (stride: c rounded up to 4)
  int64_t key_stride;
  int64_t part_stride;    // batched stage 1: floats between K-slice partial blocks
  float* dbg_scores;      // optional raw scores, B x c
  float* raw;             // adaptive sampling: B x key_stride plain scores beside the
                          // keys (the rule counts on scores, the selection on keys)
  int raw_keys;           // batched INT4 stage 1: store plain scores as the keys
  int sample;
  float inv_tau;
  const uint64_t* seeds;
  // selection by the last block of each batch row (when select != 0)
  int select;
  int p;
  float zcut;             // histogram range hint (select_zcut; 0: none)
  Adaptive ad;
  uint32_t* counters;     // B x kArriveWords arrival counters (zero between calls)
  int32_t* sel;           // B x sel_stride, written ascending
  int sel_stride;
  uint64_t* masks;        // optional per-cluster row bitmask
  uint32_t* error;
};

// The single-launch batch-1 decode: stage 1 + selection (s1) and stage 2
// gather + decode (s2, kRowGather).  Two buffer sets, picked by the parity
// of the device word *epoch (advanced by every launch):
//   s1.keys       2 x key_stride floats, every key pending (all bits set)
//                 before the first launch;
//   sel           2 x kDecodeB1MaxP int32, all -1 before the first launch;
//   s2.part_best  2 x slot_stride u64 words of slots (slot j at word 16 j),
//                 zero before the first launch;
//   s2.lse_part   slot_stride u64 words of lse partials (same spacing).
//   go            2 words, zero before the first launch: workgroup 0 sets
//                 the current set's word once it holds every key (a hint
//                 that the other workgroups may now prefetch).
// Launches keep them consistent.  The selection of the launch is copied to
// s1.sel (plain) only for the debug output.
constexpr int kDecodeB1MaxP = 2048;
constexpr int kDecodeB1MaxGrid = 512;
constexpr int64_t kDecodeB1SlotStride = (int64_t)kDecodeB1MaxGrid * 16;  // u64 words
struct DecodeB1Args {
  Stage1Args s1;         // s1.raw non-null: this launch publishes plain scores
  RowdotArgs s2;
  float* raw;            // 2 x key_stride plain scores (adaptive sampling), every
                         // entry pending before the first launch; a launch that
                         // uses its set marks it pending again once it is read
  int32_t* sel;
  uint32_t* epoch;
  int64_t slot_stride;
  uint32_t* go;
};

// Monte Carlo marginal (Formula 7): n draws of the probed clusters from one
// row of stage-1 scores, per-cluster (max, sum) pairs of z / tau over the
// union of the draws, and the mean conditional probability of q query tokens.
constexpr int kMcMaxP = 4096;
struct McArgs {
  const float* scores;    // c stage-1 scores (one row)
  int64_t score_stride;   // floats the score row is read over (c rounded up to 4)
  int c, p;
  float zcut;             // histogram range hint (select_zcut)
  float inv_tau;
  const uint64_t* seeds;  // n Philox keys, one per draw
  int n;
  int32_t* sel;           // n x p, each draw's clusters ascending
  uint32_t* flags;        // c, zero between calls: clusters some draw selected
  float2* cl;             // c (max, sum of exp(x - max)) of z / tau over a cluster's rows
  const uint8_t* H;       // the hidden vector (d elements of E's type)
  int nchunk;             // 16-byte chunks per row
  const uint8_t* Ec;      // cluster-major copy of E, or the caller's E (borrowed)
  int64_t row_bytes;      // stride of Ec's rows
  int borrowed;
  int b;
  const int32_t* t2row;   // v: row of each token in the cluster-major copy
  int64_t v;
  const int32_t* tokens;  // q query tokens
  int q;
  float* zq;              // q exact logits
  int32_t* qcl;           // q clusters of the query tokens
  float* contrib;         // q x n conditional probabilities (token-major)
  float* out_prob;        // q estimates
  float* out_lse;         // optional: n lse of z / tau over each draw's candidates
  uint32_t* error;
};
hipError_t launch_mc(const McArgs& a, const RowdotArgs& ra, int dtype, hipStream_t s);

// Optional events recorded exactly around one kernel (hipExtLaunchKernel).
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
};

hipError_t launch_rowdot(const RowdotArgs& a, int mode, int dtype, int B, int grid_x,
                         hipStream_t s, const Timing* tm = nullptr);
int rowdot_grid(int64_t nrows, int nchunk, int mode);
hipError_t launch_select(const SelectArgs& a, int B, hipStream_t s, const Timing* tm = nullptr);
// Selection of each batch row, then the fold of the all-cluster stream's
// records over the row's selected clusters (the fold_* fields, out_*).
hipError_t launch_select_fold(const SelectArgs& a, int B, hipStream_t s,
                              const Timing* tm = nullptr);
// The selection's histogram range hint for p of c keys: z with an upper
// normal tail of min(1, 4 p / c), or 0 (no hint) when that tail is half or
// more, or c is small.
float select_zcut(int c, int p);
hipError_t launch_stage1(const Stage1Args& a, int dtype, bool int4, int B, hipStream_t s,
                         const Timing* tm = nullptr);
bool stage1_selects(int c);
// Workgroups of the single-launch batch-1 decode for a shape (0: the shape
// does not take it), one per compute unit at most: c clusters, p probes,
// nchunk 16-byte chunks per row, ntiles INT4 tiles, nrows = p * b candidate
// rows.  Pure host arithmetic.
int decode_b1_grid(int c, int p, int nchunk, int ntiles, int64_t nrows, bool int4, int num_cu);
// Workgroups of the decode kernel that the shape uses that one compute unit
// holds at once (the occupancy API), in *blocks.
hipError_t decode_b1_occupancy(int dtype, bool int4, int nchunk, int c, int* blocks);
// coop: through the cooperative launch API (all workgroups resident together)
hipError_t launch_decode_b1(const DecodeB1Args& a, int dtype, bool int4, int grid, bool coop,
                            hipStream_t s, const Timing* tm = nullptr);
// the variant with the adaptive probe count (fh_decode_b1_adapt.hip)
hipError_t launch_decode_b1_adaptive(const DecodeB1Args& a, int dtype, bool int4, int grid,
                                     bool coop, hipStream_t s, const Timing* tm);
hipError_t decode_b1_occupancy_adaptive(int dtype, bool int4, int nchunk, int c, int* blocks);
hipError_t launch_centroid_means(const uint8_t* E, int64_t row_bytes, int dtype, int d,
                                 const int32_t* c2t, int c, int b, void* C, hipStream_t s);
bool batched_supported(int dtype, int d, int B, bool int4);
// returns the K slices used (the select sums them) in *ksplit
hipError_t launch_stage1_mfma(const Stage1Args& a, bool int4, int B, hipStream_t s,
                              const Timing* tm, int* ksplit);
int stage2_mfma_grid();
// The all-cluster stream: one launch of stage 1 and the per-(item, row)
// partials of every cluster (a), then per batch row its selection and the
// fold of its selected clusters' partials (sa).  Events: t1 around the
// stream, t2 around the select-and-fold.
hipError_t launch_stream_all(const Stage2mArgs& a, const SelectArgs& sa, hipStream_t s,
                             const Timing* t1, const Timing* t2);
hipError_t launch_stage2_mfma(const Stage2mArgs& a, bool dense, hipStream_t s,
                              const Timing* tm = nullptr);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int num_cu,
                              hipStream_t s);
// n words of p set to value by a kernel on s
hipError_t launch_fill_u32(uint32_t* p, uint32_t value, int64_t n, hipStream_t s);
// The single launch's selection (the set below the epoch it left) into dst.
hipError_t launch_b1_copy_sel(const uint32_t* epoch, const int32_t* sets, int64_t set_stride,
                              int32_t* dst, int p, hipStream_t s);
// Equal-size spherical k-means (fh_kmeans.hip).  E device, init host
// (c distinct ids), c2t device out (c x b, rows ascending), centroids device
// out (c x d float64) or null.  Blocking: allocates its own workspace and
// synchronizes s.  *status = 1 when a token found no cluster (only with
// non-finite input).
constexpr int kMaxKmB = 1024;  // tokens per cluster
struct KMeansArgs {
  const uint8_t* E;
  int64_t lde_bytes;
  int dtype;
  int64_t v;
  int d, c;
  const int32_t* init_host;
  int max_iter;
  int32_t* c2t;
  double* centroids;
};
hipError_t run_kmeans(const KMeansArgs& a, hipStream_t s, int* iters, int* status);
hipError_t launch_cluster_major_copy(const uint8_t* E, int64_t lde_bytes, const int32_t* c2t,
                                     int64_t v, int64_t row_bytes, uint8_t* Ec, hipStream_t s);

}  // namespace fh
