/*
 * cb.h - C ABI of the catalog-constrained beam-search library for AMD MI355X
 * (gfx950).
 *
 * One decoding step of beam search over a catalog of Semantic-ID token
 * sequences, filter first:
 *   (1) a per-step sliced prefix index gives every beam its valid next tokens
 *       and the row each extension maps to in the next step's table
 *       (ZeroGR summary, "Why slice the index by decoding step?");
 *   (2) only those tokens are scored against the beam's hidden vector, or the
 *       whole codebook is scored and the valid columns picked out, the choice
 *       made per step by a measurement taken in advance (ZeroGR summary, "Why
 *       fewer scores are not automatically faster");
 *   (3) log-softmax over the valid tokens only, added to the beam's
 *       accumulated log-probability (ZeroGR summary, "The pipeline", stage 4);
 *   (4) the K best candidates of each query become its next beams, each
 *       carrying its next-step row (same passage; STATIC sec. 4.3 BeamSearch and
 *       Gather).
 *
 * Conventions used by every entry point
 *   - Steps are numbered t = 0 .. L-1; step t extends prefixes of length t.
 *   - "Row" r of step t is the r-th smallest distinct length-t prefix of the
 *     catalog in lexicographic order (row 0 of step 0 is the empty prefix).
 *     The rows of step t+1 are the edges of step t in order, so an edge's
 *     position is its next row (ZeroGR: in sparse tables a token's position is
 *     its next-step row).  At the last step the next row is the item's rank in
 *     the sorted, duplicate-free catalog.
 *   - A query owns K consecutive beam slots; slot b = q*K + k.  A dead slot
 *     has row -1 and accumulated log-prob -inf.  At t = 0 the caller passes
 *     row 0 and 0.0 in slot k = 0 of each query and dead slots elsewhere.
 *   - Outputs of a step are, per query, the K best candidates best first by
 *     (new log-prob descending, parent slot ascending, token ascending);
 *     fewer than K valid candidates leave sentinel slots (token = parent =
 *     row = -1, log-prob = -inf).  `parent` is the slot k (0..K-1) within
 *     the same query.
 *   - Device pointers are HIP device addresses; `stream` is a hipStream_t
 *     (NULL = the default stream).  Calls on a stream are asynchronous and
 *     stream ordered; errors detected on the host are returned before any
 *     launch, device faults surface at the caller's next synchronisation.
 *   - Every function returns a cb_status; on failure cb_last_error() gives a
 *     message (thread local, valid until the next call on that thread).
 *   - Floating point: scores accumulate in float32 (bf16 x bf16 products are
 *     exact in float32); the softmax and the accumulated log-prob are float32.
 */
#ifndef CB_H
#define CB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CB_OK = 0,
    CB_EINVAL = -1,        /* an argument is out of range, misaligned or inconsistent */
    CB_ENOMEM = -2,        /* host or device allocation failed */
    CB_EHIP = -3,          /* a HIP runtime call failed */
    CB_EUNSUPPORTED = -4,  /* a shape this build does not handle (e.g. V > 65535) */
    CB_ECAPACITY = -5      /* beam width or step width beyond what the kernels hold */
} cb_status;

typedef enum { CB_F32 = 0, CB_BF16 = 1 } cb_dtype;

/* Scoring path of a step: full-codebook MFMA product then a gather of the
 * valid columns (DENSE), or a gather-dot over the valid tokens only (SPARSE).
 * SPARSE_SPLIT is SPARSE with the rows too wide for one wavefront scored
 * first by a separate pass spread over many workgroups (same results; it
 * differs from SPARSE only under the LDS selection).  AUTO uses the measured
 * choice of cb_tune, else a width rule. */
typedef enum { CB_PATH_AUTO = 0, CB_PATH_DENSE = 1, CB_PATH_SPARSE = 2, CB_PATH_SPARSE_SPLIT = 3 } cb_path;

/* Storage of a step table: CSR (row_ptr + tokens) for narrow steps, a per-row
 * bitmap (+ row_ptr) for wide steps (ZeroGR: dense tables where many tokens
 * are valid, sparse ones where few are; STATIC sec. 5.1 / App. B: dense masks
 * for the first levels, CSR below).  AUTO picks the smaller of the two. */
typedef enum { CB_STORE_AUTO = 0, CB_STORE_CSR = 1, CB_STORE_BITMAP = 2 } cb_store;

/* Decoding variant of a plan (ZeroGR, "Does filtering first change the
 * recommendations?"; the summary's unconstrained speed reference):
 *   CB_MODE_FILTER_FIRST   softmax over each beam's valid tokens (default);
 *   CB_MODE_SCORE_FIRST    softmax over the whole codebook, then only the
 *                          valid tokens are candidates;
 *   CB_MODE_UNCONSTRAINED  every token of the codebook is a candidate and
 *                          the softmax covers all of them; the index only
 *                          sets L and V, and every live beam's row is 0. */
typedef enum { CB_MODE_FILTER_FIRST = 0, CB_MODE_SCORE_FIRST = 1, CB_MODE_UNCONSTRAINED = 2 } cb_mode;

/* Per-query top-K of a step (the segmented top-K with the (score desc,
 * parent asc, token asc) tie-break; ZeroGR "The pipeline", FlashTrie App. D.3
 * block merge).  LDS: the query's best keys are kept by one wavefront in
 * registers and LDS, K <= 64, rows no wider than the fused kernels' LDS.
 * RADIX: every candidate's key is written to HBM and the K-th largest is
 * found by radix select over the whole GPU, K <= 1024, any row width.  AUTO
 * takes LDS where it applies, else RADIX.  Both give identical outputs. */
typedef enum { CB_SELECT_AUTO = 0, CB_SELECT_LDS = 1, CB_SELECT_RADIX = 2 } cb_select;

typedef struct cb_index cb_index; /* owns the device-resident step tables */
typedef struct cb_plan cb_plan;   /* owns the workspace for (Q_max, K, d, dtype) and the per-step path */

typedef struct {
    int64_t n_rows;      /* distinct length-t prefixes */
    int64_t n_edges;     /* distinct length-(t+1) prefixes (= rows of step t+1) */
    int32_t max_fanout;  /* the widest row: fixed slot count of the step (ZeroGR, fixed candidate slots) */
    int32_t storage;     /* CB_STORE_CSR or CB_STORE_BITMAP */
    int64_t bytes;       /* device bytes of this step's table */
} cb_step_info;

/* Build the step-sliced index of a catalog and upload it to `device`.
 *   sids      host int32 [n_items][L], row-major; tokens in [0, V).  Read only
 *             during the call.  Repeated items are removed (the catalog is a
 *             set: STATIC sec. 4.1).
 *   L >= 1, 2 <= V <= 65535, 1 <= n_items < 2^31.
 *   device    HIP device ordinal, or -1 to build host tables only (for
 *             inspection with cb_index_info / cb_index_row; such an index
 *             cannot be stepped).
 *   store     a cb_store policy applied to every step (AUTO per step).
 *   *out      receives the index; release with cb_free_index.
 * Errors: CB_EINVAL (shape, token out of range), CB_EUNSUPPORTED, CB_ENOMEM,
 * CB_EHIP.  Synchronous. */
cb_status cb_build_index(const int32_t* sids, int64_t n_items, int32_t L, int32_t V,
                         int32_t device, int32_t store, cb_index** out);

/* Shape of an index: L, V, distinct items and device (-1 = host only).
 * Any output pointer may be NULL. */
cb_status cb_index_shape(const cb_index* idx, int32_t* L, int32_t* V, int64_t* n_items, int32_t* device);

/* Per-step statistics of the table of step t (0 <= t < L): rows, edges, the
 * widest row (the step's fixed slot count: ZeroGR summary, "Why fewer scores
 * are not automatically faster", candidates padded to a fixed number of
 * slots; STATIC sec. 4.2, a static maximum branch factor per level), storage
 * and device bytes.  Errors: CB_EINVAL (NULL, t out of range). */
cb_status cb_index_info(const cb_index* idx, int32_t t, cb_step_info* out);

/* Host-side lookup of one row: its valid tokens (ascending) and their next
 * rows.  Writes at most `cap` entries to tokens / next_rows (either may be
 * NULL) and the row's full count to *n.  Synchronous (reads device tables
 * back when the host copy was released). */
cb_status cb_index_row(const cb_index* idx, int32_t t, int64_t row,
                       int32_t* tokens, int64_t* next_rows, int32_t cap, int32_t* n);

/* Release an index (frees device tables).  NULL is ignored.  Plans created
 * from it must not be used afterwards (destroying them is still allowed). */
void cb_free_index(cb_index* idx);

/* Write the index's tables to a file (host or device index; device tables
 * are read back).  The file holds the tables exactly as built, so loading it
 * skips the sort and deduplication of the catalog (ZeroGR summary: the index
 * is built on the CPU once and streamed to the GPU).  Format: tag
 * "CBINDEX1", int32 L, V, int64 n_items, per step int64 n_rows, n_edges,
 * int32 widest row, storage, then row_ptr u32 [n_rows+1] and either tok u16
 * [n_edges] + first token per row u16 [n_rows] (CSR) or bits u32 and rank u16
 * [n_rows][ceil(V/32)] (bitmap); last a 64-bit FNV-1a hash of all preceding
 * bytes; little-endian.  Errors: CB_EINVAL (NULL, cannot write), CB_EHIP. */
cb_status cb_index_save(const cb_index* idx, const char* path);

/* Read an index written by cb_index_save and upload it to `device` (-1: host
 * tables only).  Every structural invariant is checked on the host first
 * (row counts chained across steps, row pointers, ascending in-range tokens,
 * bitmap rank directory, hash), so a damaged file returns CB_EINVAL and
 * nothing reaches the device.  Errors: CB_EINVAL, CB_ENOMEM, CB_EHIP. */
cb_status cb_index_load(const char* path, int32_t device, cb_index** out);

/* Create a plan: allocates, once, every device buffer the step and decode
 * need for up to Q_max queries of beam width K, hidden width d (multiple of 8)
 * and element type dtype (of W and of the hidden vectors).  Nothing is
 * allocated later by cb_step / cb_decode (FlashTrie App. D: per-batch state
 * allocated once).  The index must stay alive while the plan exists.
 * Beam widths up to 64 use the LDS selection on every step whose rows fit
 * it; wider beams and wider rows use the radix selection, whose candidate
 * workspace (12 bytes per candidate slot: Q_max * K * widest row) is
 * allocated here when some step needs it, else on the first
 * cb_set_select(..., CB_SELECT_RADIX).  The fused per-query sparse step
 * holds up to 2048 elements of a hidden vector; wider plans take sparse steps
 * as a per-beam expansion + per-query merge (or the radix selection, whose
 * scoring loops over any width), and never the persistent decode.
 * Errors: CB_EINVAL, CB_ECAPACITY (K > 1024, d > 16384, or a candidate
 * workspace beyond 2^31 slots per query), CB_ENOMEM, CB_EHIP. */
cb_status cb_plan_create(cb_index* idx, int32_t Q_max, int32_t K, int32_t d, cb_dtype dtype, cb_plan** out);

/* Force the top-K selection of step t (tests run both ways).  CB_SELECT_LDS
 * where it does not apply returns CB_ECAPACITY; CB_SELECT_RADIX may allocate
 * the radix workspace (CB_ENOMEM).  CB_SELECT_AUTO restores the default.
 * Synchronous with respect to the host; do not call while steps of this plan
 * are being captured. */
cb_status cb_set_select(cb_plan* plan, int32_t t, cb_select select);

/* The selection step t will use (never CB_SELECT_AUTO). */
cb_status cb_get_select(const cb_plan* plan, int32_t t, cb_select* select);

/* Set the decoding variant (STATIC sec. 4.3: log-softmax over the whole
 * codebook, then the mask — score first; ZeroGR summary, "Does it actually
 * work better?": unconstrained decoding as the speed reference).  Both need
 * every step's full score row: all steps take the dense path (cb_get_path
 * reports CB_PATH_DENSE, cb_tune has nothing to choose, sparse paths return
 * CB_EUNSUPPORTED).  A step takes the LDS selection where it holds the
 * variant (K <= 64, rows that fit its LDS; unconstrained also a bf16 plan
 * with V <= 4096, V a multiple of 4), else the radix selection, whose
 * workspace is allocated here (unconstrained: K * V candidates per query).
 * Errors: CB_EINVAL (unknown mode); CB_EUNSUPPORTED for a bf16 plan with d
 * not a multiple of 64, a step forced to a sparse path or to an LDS
 * selection that cannot hold the variant; CB_ECAPACITY, CB_ENOMEM from the
 * radix workspace.  Synchronous with respect to the host. */
cb_status cb_set_mode(cb_plan* plan, cb_mode mode);

/* The plan's decoding variant. */
cb_status cb_get_mode(const cb_plan* plan, cb_mode* mode);

/* Force the scoring path of step t (tests run both ways).  CB_PATH_AUTO
 * restores the measured or default choice.  CB_PATH_SPARSE_SPLIT may allocate
 * the radix-selection workspace (CB_ENOMEM). */
cb_status cb_set_path(cb_plan* plan, int32_t t, cb_path path);

/* Per-step forms of the kernels, all with the same results (every sum is per
 * wavefront or over fixed slots, every selection exact); cb_tune measures the
 * forms that apply to the step's path and selection and keeps the fastest
 * (ZeroGR summary, "Why fewer scores are not automatically faster": the
 * choice is measured in advance), replacing what these calls forced before
 * it; these calls force one, and 0 restores the default.
 *   CB_OPT_STEP_THREADS   workgroup size of the per-query sparse step: 256,
 *                         512 or 1024 (default 1024 for K >= 16, else 512)
 *   CB_OPT_SPLIT_ROWS     split sparse path: rows of more than this many tokens
 *                         (1..64; default 16) are scored apart, across the GPU
 *   CB_OPT_SPARSE_FORM    sparse path: 0 one workgroup per query does the whole
 *                         step; 1 one workgroup per beam expands its row (scores,
 *                         log-softmax, its best min(K, n)), then one wavefront
 *                         per query merges (always 1 when d > 2048)
 *   CB_OPT_DENSE_ROWS     full-codebook product over the live beams (1) or over
 *                         every beam slot without a live list (2; bf16 plans);
 *                         default: the live beams at step 0, every slot after
 *   CB_OPT_RADIX_PREPASS  radix selection with (2, default) or without (1) the
 *                         pre-pass that finishes queries whose live rows all
 *                         hold one token
 *   CB_OPT_QUERY_SPLIT    workgroups per query of the per-query sparse step:
 *                         1 (default), 2, 4 or 8; each scores a share of the
 *                         query's rows and the last to finish completes the
 *                         step (ZeroGR summary, "Why fewer scores are not
 *                         automatically faster": beams read uneven numbers
 *                         of weight rows; this spreads a heavy query's reads)
 *   CB_OPT_TOKEN_MAJOR    sparse scoring on the radix selection: per beam (1,
 *                         default; the beam's hidden vector staged, one W_t
 *                         row gathered per candidate) or by token (2; the
 *                         candidates grouped by token so that each W_t row is
 *                         read once for every beam holding it; d <= 2048)
 * Errors: CB_EINVAL (unknown option or value), CB_ECAPACITY (the form does not
 * fit the LDS, or the token-major workspace would pass 2^31 candidates),
 * CB_EUNSUPPORTED (every-slot product of an f32 plan). */
typedef enum {
    CB_OPT_STEP_THREADS = 0,
    CB_OPT_SPLIT_ROWS = 1,
    CB_OPT_SPARSE_FORM = 2,
    CB_OPT_DENSE_ROWS = 3,
    CB_OPT_RADIX_PREPASS = 4,
    CB_OPT_QUERY_SPLIT = 5,
    CB_OPT_TOKEN_MAJOR = 6
} cb_step_option;
cb_status cb_set_step_option(cb_plan* plan, int32_t t, cb_step_option option, int32_t value);

/* The form step t will use for `option` (never 0 except CB_OPT_SPARSE_FORM). */
cb_status cb_get_step_option(const cb_plan* plan, int32_t t, cb_step_option option, int32_t* value);

/* The path step t will take (never CB_PATH_AUTO). */
cb_status cb_get_path(const cb_plan* plan, int32_t t, cb_path* path);

/* One decoding step (the hot path) for Q <= Q_max queries at step t, as
 * ZeroGR's summary states it ("The pipeline": look up each beam's valid next
 * tokens in the step's table, score them, log-softmax over the valid tokens
 * only, add to the beam's accumulated log-probability, keep the K best per
 * query, each carrying its next-step row) with STATIC's beam update (sec.
 * 4.3: top-K over the flattened candidates of a query, then a gather of the
 * parents' next states).
 *   hidden     device [Q*K][d] of dtype: each slot's hidden vector (ignored
 *              for dead slots).  bf16 plans take the vectors already rounded.
 *   W_t        device [V][d] of dtype: output layer of step t, row-major.
 *   beam_rows  device int32 [Q*K]: row of each slot in step t's table, -1 dead
 *              (a row outside the table is treated as dead).
 *   acc_logp   device float [Q*K]: accumulated log-prob, -inf dead.
 *   out_*      device [Q*K]: tokens, parent slots, next rows, new accumulated
 *              log-probs, best first per query, sentinel padded.  Must not
 *              alias the inputs.
 * hidden and W_t 16-byte aligned (d is a multiple of 8, so every row is);
 * the per-slot arrays 4-byte aligned.  Enqueued on `stream`; returns after
 * the launches.  Concurrent calls on one plan from different streams race.
 * Errors: CB_EINVAL (t, Q, NULL or misaligned pointers, an output sharing a
 * byte with an input or another output, host-only index), CB_EHIP. */
cb_status cb_step(cb_plan* plan, int32_t t, int32_t Q, const void* hidden, const void* W_t,
                  const int32_t* beam_rows, const float* acc_logp,
                  int32_t* out_tokens, int32_t* out_parents, int32_t* out_rows, float* out_logp,
                  void* stream);

/* One decoding step without a plan, allocating nothing: for callers that
 * cannot allocate device memory at call time (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same kernels and
 * results as cb_step with CB_SELECT_LDS on the given path (CB_PATH_AUTO:
 * dense for bitmap steps, sparse for CSR steps; CB_PATH_SPARSE_SPLIT is not
 * taken).  Arguments as cb_step, plus the plan's K, d and dtype.
 * Workspace: a static device array of 32 MiB per device (held by each GPU the
 * library runs on until the process ends), shared by every call on that
 * device; the fused sparse step needs none of it, the dense path needs
 * (Q*K*min(K, widest row)*8 + Q*K*V*4 [+ 2*256*V*4 for bf16] + Q*K*8) bytes.
 * Calls that overlap on one device (e.g. on two streams) race on it.
 * Errors: CB_EINVAL (as cb_step; t, Q, K, d, dtype, path out of range),
 * CB_EUNSUPPORTED (dense path with bf16 and d not a multiple of 64),
 * CB_ECAPACITY (K > 64, a row too wide for the LDS selection, or a workspace
 * above 32 MiB), CB_EHIP. */
cb_status cb_step_noalloc(const cb_index* idx, int32_t t, int32_t Q, int32_t K, int32_t d, cb_dtype dtype,
                          cb_path path, const void* hidden, const void* W_t, const int32_t* beam_rows,
                          const float* acc_logp, int32_t* out_tokens, int32_t* out_parents, int32_t* out_rows,
                          float* out_logp, void* stream);

/* Full decode of all L steps (the beam-search loop of FlashTrie, arXiv HTML,
 * Algorithm 1: expand, prune to the beam, carry the survivors, backtrace the
 * sequences at the end) with a stand-in model whose hidden vector before
 * step t is h = s / ||s||_2, s = q + sum_{j<t} P_j[token_j] (s in float32;
 * norm and division in double; rounded to float32 and then to bf16 for bf16
 * plans).  The stand-in is not from the pages; it only feeds each step a
 * hidden vector that depends on the path taken.  The hidden update runs
 * between steps on the device.
 *   q     device float [Q][d];  P  device float [L-1][V][d] (may be NULL when
 *         L == 1);  W  device [L][V][d] of dtype.
 *   out_seqs  device int32 [Q*K][L] (-1 rows for dead slots);
 *   out_logp  device float [Q*K];  out_rows device int32 [Q*K] (item rank).
 *   trace_hidden / trace_rows / trace_acc: optional (NULL) device buffers
 *   [L][Q*K][d] dtype, [L][Q*K] int32, [L][Q*K] float receiving the inputs
 *   of every step.
 * W 16-byte aligned, the other arrays 4-byte aligned.
 * Enqueued on `stream`; nothing is allocated.  Errors as cb_step. */
cb_status cb_decode(cb_plan* plan, int32_t Q, const float* q, const float* P, const void* W,
                    int32_t* out_seqs, float* out_logp, int32_t* out_rows,
                    void* trace_hidden, int32_t* trace_rows, float* trace_acc, void* stream);

/* The smallest record stride of the wire format below: 8 + 16 K + 4 K L
 * bytes rounded up to a multiple of 8, written to *bytes.
 * Errors: CB_EINVAL (NULL, K < 1, L < 1). */
cb_status cb_wire_bytes(int32_t K, int32_t L, int64_t* bytes);

/* Wire-format results (FlashTrie, arXiv HTML, App. D.3 "Output
 * serialization"; length normalisation from its App. E, eq. 2, after Wu et
 * al.): the decode's best-first slots of every query written as the page's
 * on-wire record, in ascending order of score.  Query q's record starts at
 * out + q * stride:
 *   uint64  n_o                       live beams (finite log-prob)
 *   float64 logp_norm[n_o]            logp * (6 / (5 + L))^alpha
 *   uint64  sent_offset[n_o]          end offsets into tokens
 *   uint32  tokens[n_o * L]           sequence i = tokens[sent_offset[i-1],
 *                                     sent_offset[i]) with sent_offset[-1] = 0
 * The live beam of best-first rank r goes to wire slot n_o - 1 - r (the worst
 * live beam first); dead slots are left out.  Little-endian, as the device
 * stores it.
 *   seqs      device int32 [Q*K][L] (cb_decode's out_seqs)
 *   logp      device float [Q*K] (cb_decode's out_logp)
 *   alpha     length-normalisation strength (0: logp unchanged)
 *   out       device, 8-byte aligned, [Q][stride] bytes
 *   stride    >= cb_wire_bytes(K, L), a multiple of 8
 *   out_bytes optional device int64 [Q]: bytes of each record
 * All pointers on the current device; enqueued on `stream`; nothing is
 * allocated.  Errors: CB_EINVAL (Q < 0, K outside [1, 1024], L < 1, alpha
 * not finite, NULL or misaligned pointers, stride too small, out overlapping
 * seqs or logp), CB_EHIP. */
cb_status cb_wire_results(int32_t Q, int32_t K, int32_t L, const int32_t* seqs, const float* logp, double alpha,
                          void* out, int64_t stride, int64_t* out_bytes, void* stream);

/* Persistent decode (FlashTrie, arXiv HTML, sections 2.2 and 4.2: every step
 * of a query in one launch, paying the launch cost once).  When enabled and
 * cb_decode is called without trace buffers, the trailing run of steps whose
 * path resolves to CB_PATH_SPARSE with CB_SELECT_LDS in the per-query form
 * (CB_OPT_SPARSE_FORM 0; at least two steps) runs as one launch: one workgroup per query performs each of those steps
 * and the hidden updates between them, so no workgroup waits for another.
 * Results equal the step-by-step decode bit for bit.  enable: 1 on, 0 off
 * (one launch per step), -1 (the default) automatic: cb_tune times the
 * decode both ways and keeps the faster (on until measured).  Synchronous
 * with respect to the host. */
cb_status cb_set_decode_fusion(cb_plan* plan, int32_t enable);

/* Whether the persistent decode is in effect (1) or not (0). */
cb_status cb_get_decode_fusion(const cb_plan* plan, int32_t* enabled);

/* Mean decode time (microseconds) with one launch per step and with the
 * persistent tail, from the last cb_tune (negative when not measured). */
cb_status cb_tune_decode_times(const cb_plan* plan, float* stepwise_us, float* persistent_us);

/* Pre-measured path switch (ZeroGR: warm-up requests try every option per
 * step and keep the fastest).  Runs one warm-up decode on the given inputs;
 * at every step whose path is AUTO it times the dense and the sparse path
 * (`reps` launches each, HIP events) and records the faster; the decode then
 * continues on the recorded path.  Then, when the persistent decode is
 * automatic, times `reps` whole decodes with and without it and keeps the
 * faster.  Synchronises `stream`.  Arguments as cb_decode. */
cb_status cb_tune(cb_plan* plan, int32_t Q, const float* q, const float* P, const void* W,
                  int32_t reps, void* stream);

/* Measured mean time (microseconds) of each path at step t from the last
 * cb_tune (negative when not measured). */
cb_status cb_tune_times(const cb_plan* plan, int32_t t, float* dense_us, float* sparse_us);

/* Kernel timing (measurement support).  While profiling is on, every step
 * attaches an event pair to the dispatch of each kernel it launches
 * (hipExtLaunchKernel: the events take the kernel's own start and end times
 * as the GPU records them, the figures a kernel trace shows, without the
 * host's enqueue); cb_profile_stop synchronises those events and reports one
 * record per launch.  `kernel` is one of CB_KERNEL_*; `threads` the
 * workgroup size. */
typedef enum {
    CB_KERNEL_GEMM_BF16 = 0,      /* full-codebook scores, bf16 MFMA */
    CB_KERNEL_GEMM_F32 = 1,       /* full-codebook scores, float32 */
    CB_KERNEL_EXPAND_SPARSE = 2,  /* slot fill + gather-dot + softmax + per-beam top-K */
    CB_KERNEL_EXPAND_DENSE = 3,   /* slot fill + column gather + softmax + per-beam top-K */
    CB_KERNEL_MERGE = 4,          /* per-query top-K and next rows (after the dense expansion) */
    CB_KERNEL_STEP_QUERY = 5,     /* the whole sparse step, one workgroup per query */
    CB_KERNEL_LIVE_ROWS = 6,      /* list of live beams for the full-codebook scores */
    CB_KERNEL_RADIX_SCORE_SPARSE = 7, /* radix selection: offsets, slot fill, gather-dot of every candidate */
    CB_KERNEL_RADIX_SCORE_DENSE = 8,  /* radix selection: offsets, slot fill, column gather of every candidate */
    CB_KERNEL_RADIX_KEYS = 9,     /* radix selection: softmax, keys, first digit */
    CB_KERNEL_RADIX_REFINE = 10,  /* radix selection: second digit */
    CB_KERNEL_RADIX_COLLECT = 11, /* radix selection: survivors */
    CB_KERNEL_RADIX_SORT = 12,    /* radix selection: survivors sorted, outputs and next rows */
    CB_KERNEL_DECODE_TAIL = 13,   /* persistent decode of the trailing sparse steps (step = first one) */
    CB_KERNEL_RADIX_SMALL = 14,   /* radix selection: pre-pass finishing the queries whose rows hold one token */
    CB_KERNEL_ROW_LSE = 15,       /* radix selection: log-sum-exp of every beam in a pass of its own (score
                                     first: over the whole score row; unconstrained, and filter first where the
                                     step's rows hold more than 2,048 tokens on average: over the candidates'
                                     chunk pairs) */
    CB_KERNEL_TOKEN_LISTS = 16,   /* scores by token: candidates counted, offsets, lists (three launches) */
    CB_KERNEL_TOKEN_SCORE = 17    /* scores by token: each W_t row dotted with the hidden vectors of its beams,
                                     then the chunk softmax pairs (two launches) */
} cb_kernel;

typedef struct {
    int32_t step;     /* decoding step t */
    int32_t kernel;   /* cb_kernel */
    int32_t threads;  /* workgroup size */
    int32_t blocks;   /* workgroups launched */
    float us;         /* duration between the events around the launch */
} cb_kernel_time;

/* Start recording up to `capacity` launches (creates 2*capacity events;
 * launches beyond capacity are not recorded).  Restarting discards records. */
cb_status cb_profile_start(cb_plan* plan, int32_t capacity);

/* Stop recording, synchronise the recorded events and copy up to `cap`
 * records to `out` (may be NULL); *n receives the number recorded.  Releases
 * the events. */
cb_status cb_profile_stop(cb_plan* plan, cb_kernel_time* out, int32_t cap, int32_t* n);

/* Phase clock of the persistent decode (FlashTrie, arXiv HTML, section 4.3
 * and appendix D.4: per-phase device timestamps).  While profiling is on, a
 * persistent decode also records the device wall clock in every workgroup at
 * the start of each step and once the step's outputs are written.  After
 * cb_profile_stop this reports, for each step of the last such decode, the
 * mean over queries of the selection phase (step start to outputs written:
 * lookup, scoring, softmax, top-K) and of the hidden update that follows it
 * (outputs written to the next step's start; 0 for the last step).  *n
 * receives the number of steps recorded (0 when no persistent decode ran
 * while profiling was on); up to `cap` are copied to `out`. */
typedef struct {
    int32_t step;
    float select_us;
    float update_us;
} cb_phase_time;
cb_status cb_profile_phases(const cb_plan* plan, cb_phase_time* out, int32_t cap, int32_t* n);

/* Overhead floor (FlashTrie, arXiv HTML, App. K "GPU Overhead Floor": the
 * fixed cost of launches, barriers and selection passes below which a pass
 * cannot go however little work it does): n launches of an empty kernel of
 * `blocks` workgroups of `threads` threads on `stream` (current device).
 * With us == NULL they are only enqueued (a caller may capture them in a
 * graph and time the replays).  Otherwise each dispatch carries its own event
 * pair, the call synchronises, and us[0] receives the mean dispatch duration
 * (start to end of the kernel as the GPU records it), us[1] the mean time per
 * launch of the whole back-to-back sequence (microseconds).
 * Errors: CB_EINVAL (1 <= blocks <= 2^20, threads a multiple of 64 in
 * [64, 1024], 1 <= n <= 4096), CB_EHIP. */
cb_status cb_floor_probe(int32_t blocks, int32_t threads, int32_t n, float* us, void* stream);

/* Release a plan and its workspace.  NULL is ignored. */
void cb_plan_destroy(cb_plan* plan);

/* Message of the last failure on the calling thread ("" if none). */
const char* cb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CB_H */
