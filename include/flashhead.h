/*
 * flashhead.h -- C ABI of the MI355X (gfx950) FlashHead two-stage retrieval
 * classification head.
 *
 * What the calls compute (sources are the FlashHead pages):
 *   - "FlashHead: Efficient Drop-In Replacement for the Classification Head
 *     in Language Model Inference", reading notes (dihengye.cn), sections
 *     "Overall architecture", "Module 1" .. "Module 4", "Key formulas" 1-7,
 *     "Figure 1";
 *   - the FlashHead paper page (thelatestinai.com, arXiv 2603.14591),
 *     abstract and Figure 1 caption.
 *
 * The head replaces the dense logits z = E h (Formula 1) at one decode step:
 *   stage 1  s = C h over c unit-norm centroids (Figure 1), optionally with
 *            INT4 centroids (Module 3);
 *   select   p clusters: the p largest s (greedy, Module 2) or p draws
 *            without replacement from softmax(s / tau) (sampling, Module 2);
 *   stage 2  the p*b candidate tokens C2T[S[i / b], i mod b] (Module 1: the
 *            dense equal-size c x b table), their exact logits E_t h, then an
 *            argmax (Formula 2) or a temperature sample over the candidates
 *            (Formula 3).
 * The head returns token ids, not a distribution over the vocabulary (the
 * notes' Module 4: the full distribution is only reachable by Monte Carlo).
 *
 * Conventions shared by every call
 *   - Device pointers are HIP device memory of the current device; host
 *     pointers are ordinary host memory.  `stream` is a hipStream_t (NULL =
 *     the default stream).
 *   - Matrices are row-major.  E is v x d with a row stride of `lde`
 *     elements; H is B x d, contiguous.  dtype FH_DTYPE_F32 means float32
 *     storage, FH_DTYPE_BF16 means bfloat16 storage (uint16 bit patterns);
 *     H always has E's dtype.  All arithmetic accumulates in fp32.
 *   - Alignment: E, C and H base addresses must be 16-byte aligned and a row
 *     (d * element size, and lde * element size) a multiple of 16 bytes.
 *   - Ties: a larger value wins, then the lower index (cluster or token id).
 *   - Random numbers: Philox4x32-10 keyed by a per-row 64-bit seed, counter
 *     (idx >> 2, stream, 0, 0), word idx & 3; stream 0 draws per cluster id,
 *     stream 1 per token id; Gumbel noise -log(-log u) with
 *     u = (2 * (x >> 9) + 1) * 2^-24.
 *   - Inputs must be finite; the library does not scan them.
 *   - Calls on one handle must not overlap in time (the handle owns the
 *     workspace); calls are asynchronous on `stream`, make no allocation and
 *     no host synchronisation, and leave the workspace ready for the next
 *     call.  Errors found at enqueue time return synchronously and enqueue
 *     nothing.
 */
#ifndef FLASHHEAD_H
#define FLASHHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes: 0 = success, negative = error. */
#define FH_OK 0
#define FH_ERR_INVALID_ARG (-1)     /* NULL pointer, size or range error     */
#define FH_ERR_NOT_PERMUTATION (-2) /* C2T is not a permutation of [0, v)    */
#define FH_ERR_UNSUPPORTED (-3)     /* dtype, alignment or shape not handled */
#define FH_ERR_HIP (-4)             /* a HIP runtime call failed             */
#define FH_ERR_OOM (-5)             /* device allocation failed (prepare)    */

#define FH_DTYPE_F32 0
#define FH_DTYPE_BF16 1

#define FH_QUANT_NONE 0
#define FH_QUANT_INT4_G128 1 /* stage-1 centroids as 4-bit codes, groups of
                                128 columns, one bf16 scale per group        */
#define FH_QUANT_INT4_G128_MEAN 2 /* the same codes of C minus mu, mu the bf16
                                of C's column means: every stage-1 score
                                moves by mu . h, which changes neither the top
                                p nor a Gumbel-top-p draw; the debug scores
                                are the shifted ones                         */

#define FH_MODE_GREEDY 0
#define FH_MODE_SAMPLE 1

/* fh_desc.flags */
#define FH_FLAG_COOPERATIVE 1 /* launch the single-launch batch-1 decode (see
                                flashhead_plan_step) through the cooperative
                                launch API, whose runtime guarantees that all
                                its workgroups are resident together, also
                                while other work shares the device.  Without
                                it prepare checks with the occupancy API that
                                they fit on the device at once, which holds
                                when nothing else occupies it.               */
#define FH_FLAG_BORROW_E 2    /* stage 2 reads the rows of the caller's E
                                through C2T (E is borrowed: it must stay
                                allocated and unchanged while the handle
                                lives) instead of a cluster-major copy that
                                prepare makes (v * d elements more device
                                memory; the handle then does not keep E)    */
#define FH_FLAG_STREAM_ALL 4  /* batched steps (B >= 2) always take the
                                all-cluster stream (flashhead_plan_step,
                                path 4)                                      */
#define FH_FLAG_SELECT_FIRST 8 /* batched steps always select first and then
                                stream only the selected clusters (path 3).
                                With neither flag the plan picks by the
                                expected share of clusters the batch selects;
                                setting both is FH_ERR_INVALID_ARG           */

/* Limits of this implementation. */
#define FH_MAX_BATCH 64     /* rows per call                               */
#define FH_MAX_C 32768      /* clusters                                    */
#define FH_MAX_ROW_BYTES 8192 /* d * element size (bf16: d <= 4096)        */

typedef struct fh_handle fh_handle;

/*
 * Description of a prepared head.  Stage-1 centroids C and the table C2T
 * come from the offline equal-size spherical k-means (notes, Module 1 and
 * Formulas 4-5); this library takes them as inputs, or computes C from E and
 * C2T by Formula 5 when C is NULL.
 */
typedef struct fh_desc {
  int64_t v;          /* vocabulary size; must equal c * b                 */
  int32_t d;          /* hidden size                                       */
  int32_t c;          /* number of clusters (1..FH_MAX_C)                  */
  int32_t b;          /* tokens per cluster                                */
  int32_t dtype;      /* FH_DTYPE_F32 or FH_DTYPE_BF16 (E, C, H)           */
  int64_t lde;        /* row stride of E in elements (>= d)                */
  const void* E;      /* device, v x lde.  Without FH_FLAG_BORROW_E it is
                         read during prepare only: the handle keeps its own
                         cluster-major copy (row k*b + j = E[C2T[k, j]],
                         v x d), so E may be freed or changed after prepare
                         returns.  With it, stage 2 reads E itself, which
                         must then outlive the handle unchanged            */
  const int32_t* c2t; /* host, c x b; must be a permutation of [0, v);
                         copied at prepare                                 */
  const void* C;      /* device, c x d contiguous in dtype, unit-norm rows,
                         or NULL to compute C = unit(mean of cluster rows)
                         (Formula 5; bf16 by round-to-nearest-even when
                         dtype is bf16); copied at prepare                 */
  int32_t quant;      /* FH_QUANT_NONE, FH_QUANT_INT4_G128 or
                         FH_QUANT_INT4_G128_MEAN (INT4: needs bf16, d a
                         multiple of 128)                                  */
  int32_t max_batch;  /* largest B passed to later calls (1..FH_MAX_BATCH) */
  int32_t max_p;      /* largest p passed to later calls (1..c)            */
  void* stream;       /* hipStream_t for prepare's own work                */
  int32_t flags;      /* FH_FLAG_* bits, 0 for the defaults                */
} fh_desc;

/*
 * Optional debug outputs (device pointers, each may be NULL).  They cost
 * extra writes and exist for tests and analysis.
 *   scores      B x c   stage-1 scores s = C h (before any noise)
 *   clusters    B x p   selected cluster ids per row: ascending, except
 *                       that the single-launch batch-1 decode lists first
 *                       the clusters whose keys lie in the selection
 *                       histogram's bins above its boundary bin (ascending;
 *                       they are published before the boundary bin is
 *                       resolved), then those taken from it (ascending)
 *   cand_ids    B x p*b candidate token ids; row r lists, for the j-th
 *                       entry of `clusters`, its b tokens C2T[k, 0..b) at
 *                       [j*b, j*b + b)
 *   cand_logits B x p*b exact logits of cand_ids (fp32)
 */
typedef struct fh_debug {
  float* scores;
  int32_t* clusters;
  int32_t* cand_ids;
  float* cand_logits;
} fh_debug;

/*
 * One-time preparation (notes: "Implementation details" -- the head stores
 * the centroid matrix and the C2T map).  Validates the description, checks
 * that C2T is a permutation of [0, v) (FH_ERR_NOT_PERMUTATION otherwise),
 * copies C2T and C to device memory owned by the handle (or computes C),
 * builds the INT4 codes when asked, allocates the workspace, and waits for
 * `stream` to finish.  On error *out is set to NULL and nothing is kept.
 */
int flashhead_prepare(const fh_desc* desc, fh_handle** out);

/* Frees everything the handle owns (not E).  NULL is accepted. */
void flashhead_destroy(fh_handle* h);

/*
 * Greedy decode step for B rows (notes, Module 2 greedy mode and Formula 2):
 * per row r, S = the p clusters with the largest C h_r, then
 * out_tokens[r] = argmax over the p*b candidates of E_t h_r.
 *   H          device, B x d in the handle's dtype
 *   B          1..max_batch;  p  1..max_p
 *   out_tokens device, B int32
 *   dbg        optional debug outputs (NULL for none)
 */
int flashhead_greedy(fh_handle* h, const void* H, int32_t B, int32_t p,
                     int32_t* out_tokens, const fh_debug* dbg, void* stream);

/*
 * Sampling decode step (notes, Module 2 sampling mode and Formula 3; the
 * paper's abstract, innovation 3).  Per row r with key seeds[r]:
 * S = the p largest s_k / tau + G0(k) (Gumbel-top-p: p successive draws
 * without replacement from softmax(s / tau)), then out_tokens[r] = the
 * candidate with the largest z_t / tau + G1(t) (Gumbel-max: one draw from
 * the softmax of z / tau over the candidates).
 *   tau        finite, > 0; the same temperature scales both stages
 *   seeds      device, B uint64 Philox keys (e.g. (step << 32) | row)
 *   out_lse    device, B fp32 log sum_{t in candidates} exp(z_t / tau), or
 *              NULL (the normaliser of p(t | h, S), the summand of
 *              Formula 7)
 */
int flashhead_sample(fh_handle* h, const void* H, int32_t B, int32_t p,
                     float tau, const uint64_t* seeds, int32_t* out_tokens,
                     float* out_lse, const fh_debug* dbg, void* stream);

/*
 * Adaptive probe count (the notes' "Potential improvements": fewer probes
 * for easy tokens, more for hard ones; the pages give no rule, the rule here
 * is this library's reading).  Per row r, p'_r = the number of clusters
 * whose stage-1 softmax weight at temperature tau is at least eps times the
 * largest weight, i.e. of k with s_k / tau >= max_j s_j / tau - ln(1 / eps),
 * clamped to [p_min, p_max]; greedy decoding reads the rule at tau = 1.  The
 * step then runs as flashhead_greedy / flashhead_sample with p = p'_r for
 * that row (the count uses the plain scores; in sampling mode the p'_r
 * clusters are the Gumbel-top-p'_r draws).
 *   p_min, p_max  1 <= p_min <= p_max <= max_p
 *   eps           0 < eps <= 1 (1: only the top score's ties; toward 0: p_max)
 *   out_p         device, B int32 counts p'_r, or NULL
 * The debug outputs hold p_max entries per row: entries [p'_r, p_max) of
 * `clusters` read 0x7FFFFFFF, and candidate entries past p'_r * b are not
 * written.  Other conventions as for flashhead_greedy / flashhead_sample.
 */
int flashhead_greedy_adaptive(fh_handle* h, const void* H, int32_t B, int32_t p_min,
                              int32_t p_max, float eps, int32_t* out_tokens,
                              int32_t* out_p, const fh_debug* dbg, void* stream);
int flashhead_sample_adaptive(fh_handle* h, const void* H, int32_t B, int32_t p_min,
                              int32_t p_max, float eps, float tau, const uint64_t* seeds,
                              int32_t* out_tokens, float* out_lse, int32_t* out_p,
                              const fh_debug* dbg, void* stream);

/*
 * Monte Carlo marginal (notes, Module 4 and Formula 7): the estimate of
 * p(v | h) for each query token v as the mean over n_draws independent
 * draws S_i of
 *   p(v | h, S_i) = exp(z_v / tau - lse_i)  if v's cluster is in S_i, else 0,
 * where lse_i = log sum over the candidates t of S_i of exp(z_t / tau).  S_i
 * is drawn as in flashhead_sample (Gumbel-top-p of the stage-1 scores over
 * tau with the Philox key seeds[i]), so draw i probes the clusters that
 * flashhead_sample with that key would, and lse_i is its out_lse.  Stage 1
 * runs once for all draws, and each cluster that any draw selects has its
 * candidate logits computed once.
 *   H          device, 1 x d in E's dtype, 16-byte aligned
 *   p          1 <= p <= min(c, max_p, 4096)
 *   tau        finite, > 0
 *   seeds      device, n_draws uint64 Philox keys; 1 <= n_draws <= 2^20
 *   tokens     device, n_tokens token ids in [0, v); 1 <= n_tokens <= 2^16.
 *              An id outside [0, v) is read as token 0 and sets bit 4 of
 *              the self-check word (flashhead_query 9).
 *   out_prob   device, n_tokens fp32 estimates
 *   out_lse    device, n_draws fp32 lse_i, or NULL
 *   workspace  device memory of at least
 *              flashhead_mc_workspace_bytes(h, n_draws, p, n_tokens) bytes,
 *              256-byte aligned, owned by the caller; its contents need no
 *              initialisation and one call is in flight per workspace (and,
 *              as for every call, per handle).
 * Asynchronous on `stream`; argument errors return before anything is
 * enqueued.  The sum over the draws runs in a fixed order, so a call is
 * reproducible bit for bit.
 */
size_t flashhead_mc_workspace_bytes(const fh_handle* h, int32_t n_draws, int32_t p,
                                    int32_t n_tokens);
int flashhead_mc_marginal(fh_handle* h, const void* H, int32_t p, float tau,
                          const uint64_t* seeds, int32_t n_draws, const int32_t* tokens,
                          int32_t n_tokens, float* out_prob, float* out_lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * The dense head it replaces (Formula 1 followed by Formula 2 or 3), as the
 * in-library comparison: z = E h_r over all v tokens, then argmax or the
 * Gumbel-max sample with stream-1 noise keyed by token id (so that
 * flashhead_sample with p = c returns the same ids).
 *   workspace  device memory of dense_head_workspace_bytes(B) bytes, 16-byte
 *              aligned.  Its first 4096 * B bytes (completion counters) must
 *              be zero before the first use; every call leaves them zero.
 *              The rest holds per-workgroup partials, rewritten each call.
 *              One call in flight per workspace.
 *   out_lse    optional, as for flashhead_sample (over all v tokens)
 */
size_t dense_head_workspace_bytes(int32_t B);
int dense_head(const void* E, int64_t v, int32_t d, int32_t dtype,
               int64_t lde, const void* H, int32_t B, int32_t mode,
               float tau, const uint64_t* seeds, int32_t* out_tokens,
               float* out_lse, void* workspace, void* stream);

/*
 * dense_head for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that forbid hipMalloc): the same kernels and
 * results, with the workspace in a fixed array inside the library instead
 * of a caller's buffer.  The array holds the workspace of
 * FH_DENSE_STATIC_MAX_BATCH rows (dense_head_workspace_bytes(16) bytes,
 * about 2.1 MB); each device the library runs on keeps its own copy until
 * the process ends.  The call allocates nothing; its arrival counters are
 * cleared by a kernel on `stream` before use.  All calls on one device
 * share that device's array, so calls that overlap in time on one device
 * (other streams, other threads) race and must not be made.
 *   B          1..FH_DENSE_STATIC_MAX_BATCH (FH_ERR_INVALID_ARG beyond)
 *   the other arguments as for dense_head
 */
#define FH_DENSE_STATIC_MAX_BATCH 16
int dense_head_static(const void* E, int64_t v, int32_t d, int32_t dtype,
                      int64_t lde, const void* H, int32_t B, int32_t mode,
                      float tau, const uint64_t* seeds, int32_t* out_tokens,
                      float* out_lse, void* stream);

/*
 * Equal-size spherical k-means (notes, Module 1; Formula 4, the summed
 * cosine of each token to its cluster's unit centroid; Formula 5, the
 * centroid is the unit-normalised mean of the cluster's rows): the offline
 * step that builds C2T from E, with every cluster holding exactly b = v / c
 * tokens.  The pages leave the size constraint's mechanism open; the
 * assignment here places tokens by cosine, pairs taken in descending order
 * (ties: lower token id, then lower cluster id), each into a cluster with
 * room: the unique stable capacity-b assignment.  Each iteration computes
 * the cosines of the unit rows of E to the centroids, the assignment, then
 * the Formula 5 update; it stops after max_iter assignments or when an
 * assignment repeats the previous one.  Cosines and centroids are float64.
 *   E          device, v x d, row stride lde elements, dtype F32 or BF16,
 *              aligned to its element size; finite (a zero row has cosine 0
 *              to every centroid)
 *   c          clusters, v % c == 0, c <= FH_MAX_C, v / c <= 1024
 *   init       host, c distinct token ids in [0, v): the initial centroids
 *              are their unit rows (the caller draws them)
 *   max_iter   >= 1
 *   c2t        device out, c x b int32, each row ascending; the result can
 *              be passed to flashhead_prepare (as fh_desc.c2t, after a copy
 *              to the host)
 *   centroids  device out, c x d float64 (Formula 5 of the returned c2t),
 *              or NULL
 *   iters_run  host out, assignments computed, or NULL
 * Blocking: allocates its own device workspace (about 8 * v * (d + c)
 * bytes), synchronizes `stream` and frees the workspace before returning.
 * FH_ERR_INVALID_ARG for bad sizes, repeated or out-of-range init ids, and
 * when a token finds no cluster (only with non-finite input); FH_ERR_OOM
 * when the workspace does not fit.
 */
int flashhead_kmeans(const void* E, int64_t v, int32_t d, int32_t dtype,
                     int64_t lde, int32_t c, const int32_t* init,
                     int32_t max_iter, int32_t* c2t, double* centroids,
                     int32_t* iters_run, void* stream);

/* Static text for a status code. */
const char* flashhead_status_string(int status);

/* Name of the HIP error (hipGetErrorName) behind the most recent
 * FH_ERR_HIP or FH_ERR_OOM returned to the calling thread; "hipSuccess" if
 * there was none.  The string is static. */
const char* flashhead_last_hip_error(void);

/*
 * Prepare-time data, copied to host memory (synchronous):
 *   flashhead_export_centroids  c x d in the handle's dtype
 *   flashhead_export_int4       codes: ceil(c/16) * (d/128) tiles of 1024
 *     bytes; tile (t, g) lane l (0..63) owns row 16t + (l mod 16) and
 *     columns 128g + 32(l div 16) + [0, 32); its 16 bytes hold those 32
 *     codes, byte j = column 2j (low nibble) and column 2j + 1 (high
 *     nibble), two's complement.  scales: ceil(c/16) * (d/128) * 16 bf16,
 *     scale of (row 16t + i, group g) at index (t * (d/128) + g) * 16 + i.
 *     Rows past c are zero.
 */
int flashhead_export_centroids(const fh_handle* h, void* dst_host);
int flashhead_export_int4(const fh_handle* h, uint8_t* codes_host,
                          uint16_t* scales_host);

/* Sizes of a prepared head: what = 0 v, 1 d, 2 c, 3 b, 4 dtype, 5 quant,
 * 6 max_batch, 7 max_p, 8 device bytes owned by the handle, 9 the
 * self-check word (reading it synchronises with the device and clears it;
 * bit 0: a selection produced a count other than p; bits 1-3: a bounded
 * wait between workgroups of one launch gave up, after about 0.4 s, and the
 * step's output is not to be trusted; bit 4: a query token outside [0, v)
 * in flashhead_mc_marginal), 10 the kernels the last step ran (0 none yet,
 * 1 the single-launch batch-1 decode, 2 stage 1 and stage 2 as separate
 * row-dot launches, 3 the batched matrix-core path that selects first,
 * 4 the batched all-cluster stream), 11 the state of the
 * single launch's buffer set that the next launch uses, read back
 * synchronously (0 when every key and plain score reads pending, every
 * selection entry -1, and every merge slot and the set's go word zero;
 * otherwise bit 0 keys, 1 selection, 2 slots, 3 go word, 5 plain scores;
 * bit 4 is not used), 12 the single-launch decode kernel's
 * workgroups that one compute unit holds at once (occupancy API, measured
 * at prepare), 13 the device's compute units, 14 fh_desc.flags.
 * The decode calls are asynchronous and cannot return what goes wrong
 * inside a kernel: a caller that must know checks the self-check word (9)
 * after synchronising, as the tests and the benchmark do. */
int flashhead_query(const fh_handle* h, int32_t what, int64_t* value);

/*
 * The kernels a decode step of a head of this shape takes, on the host
 * alone (no device call): returns 1 (the single-launch batch-1 decode:
 * stage 1, selection, stage 2 and decode in one launch of *grid
 * workgroups), 2 (stage 1 with the selection, then stage 2 with the decode,
 * as two row-dot launches; *grid = 0), 3 (the batched matrix-core path:
 * stage 1, the selection, then stage 2 over the clusters some row selected;
 * *grid = 0) or 4 (the batched all-cluster stream: one launch computes the
 * stage-1 keys and, for every cluster and batch row, the best decode key and
 * log-sum-exp of the cluster's candidates, while no selection exists yet;
 * then per row the selection and the fold of its selected clusters' records;
 * *grid = 0), or FH_ERR_INVALID_ARG for sizes no step accepts.  Paths 3 and
 * 4 give the same tokens for the same selections: path 4 reads every
 * cluster once instead of only the selected ones, and drops the wait for
 * the selection.  Without a path flag, batched steps take path 4 when the
 * expected share of clusters that at least one of B independent rows
 * selects, 1 - (1 - p / c)^B, is at least 0.85 and d is a multiple of 256
 * (the shapes where the stream was measured faster).  On path 4 the candidates'
 * debug logits (fh_debug.cand_ids / cand_logits) come from a second gather
 * of the selected rows after the step (debug only: it does not change the
 * step's tokens or lse).
 *   c, b, d, dtype, quant   as in fh_desc
 *   B, p                    as in flashhead_greedy / flashhead_sample
 *   num_cu                  compute units of the device (flashhead_query 13)
 *   blocks_per_cu           single-launch workgroups one compute unit holds
 *                           at once (flashhead_query 12)
 *   flags                   fh_desc.flags
 * The single launch's workgroups wait on one another (the selection waits
 * for every stage-1 key, stage 2 for the selection, the merge for every
 * partial), so it is taken only when grid <= num_cu * blocks_per_cu.  In the
 * two-launch path one workgroup per batch row waits for the others, which
 * never wait, so it progresses whenever the device holds more than B
 * workgroups.  flashhead_greedy and flashhead_sample follow this plan.
 */
int flashhead_plan_step(int32_t c, int32_t b, int32_t d, int32_t dtype, int32_t quant,
                        int32_t B, int32_t p, int32_t num_cu, int32_t blocks_per_cu,
                        int32_t flags, int32_t* grid);

/*
 * Measurement reference, not part of the method: reads `bytes` (a multiple
 * of 16, 16-byte aligned device memory) once with a plain streaming kernel
 * on the stream and may write one word to `sink` (device).  Timed by the
 * caller, it gives the read bandwidth this GPU achieves; it also evicts the
 * caches without leaving dirty lines.
 */
int flashhead_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/*
 * Per-kernel timing for measurement (not for the decode loop).
 * flashhead_profile_begin creates 6 HIP events per call for the next
 * max_calls decode calls on this handle; each of those calls records them
 * exactly around its stage-1, select and stage-2 kernels (on the call's
 * stream; when the selection runs inside the stage-1 kernel, as it does for
 * c <= 16384, stage 1 includes it and the select time is reported as zero).  flashhead_profile_end waits for the recorded events, writes the
 * average duration in milliseconds of each of the three kernels per call to
 * stage_ms[0..2] and the number of recorded calls to *calls, and releases
 * the events.
 */
int flashhead_profile_begin(fh_handle* h, int32_t max_calls);
int flashhead_profile_end(fh_handle* h, double* stage_ms, int32_t* calls);

/*
 * Timeline of the single-launch batch-1 decode, for measurement only.  The
 * library returns FH_ERR_UNSUPPORTED (and *words = 0); its measurement build
 * (libflashhead_trace.so, the same sources built with timeline hooks)
 * copies the timestamps its hooks stored during the launches since the
 * last read to host[0 .. *words) and clears them.  Layout (64-bit words):
 * 8 workgroup events x 512 workgroups, then 4 wave events x 8192 waves, then
 * 16 selection phases as (shader-clock cycles, device-clock time) pairs,
 * then 16 counters; *clock_khz is the device clock's rate.  A launch
 * overwrites the previous one's stamps; 0 means not recorded.
 */
int flashhead_trace_read(uint64_t* host, int64_t max_words, int64_t* words,
                         int64_t* clock_khz);

#ifdef __cplusplus
}
#endif
#endif /* FLASHHEAD_H */
