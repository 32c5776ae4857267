// Internal types of the constrained beam-search library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <condition_variable>
#include <cstdint>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "cb.h"

namespace cb {

// Thread-local error message behind cb_last_error().
void set_error(const std::string& msg);
void clear_error();

// Make `dev` current for the scope, restoring the caller's device after
// (dev < 0: host-only work, the runtime is left alone).
struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (dev < 0) return;
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
    DeviceGuard(const DeviceGuard&) = delete;
    DeviceGuard& operator=(const DeviceGuard&) = delete;
};

// Events the next kernel launch of this thread attaches to its dispatch
// (hipExtLaunchKernel: the events take the dispatch's own start and end
// times).  Set by the kernel-timing support around one launcher call; both
// null otherwise.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

// Device view of one step table.  Rows are the distinct length-t prefixes in
// lexicographic order; row r's edges are row_ptr[r] .. row_ptr[r+1]-1, ascending
// token, and edge e leads to row e of the next step.
struct StepDev {
    const uint32_t* row_ptr;  // [n_rows + 1]
    const uint16_t* tok;      // CSR: token of every edge [n_edges]; nullptr for bitmap steps
    const uint32_t* bits;     // bitmap: [n_rows][words], bit v of a row set iff token v is valid
    const uint16_t* rank;     // bitmap: [n_rows][words], set bits of the row in the words before
    int64_t n_rows;
    int32_t words;            // 32-bit words per bitmap row = ceil(V / 32)
    int32_t store;            // CB_STORE_CSR or CB_STORE_BITMAP
    int32_t S;                // widest row (fixed slot count of the step)
    const uint16_t* tok0;     // CSR: first token of every row [n_rows] (read with row_ptr); else nullptr
};

struct StepTable {
    int64_t n_rows = 0, n_edges = 0;
    int32_t S = 0;
    int32_t store = CB_STORE_CSR;
    int64_t bytes = 0;
    // host copies (kept for host-only indexes; released after upload otherwise)
    std::vector<uint32_t> row_ptr;
    std::vector<uint16_t> tok;
    std::vector<uint32_t> bits;
    std::vector<uint16_t> rank;
    std::vector<uint16_t> tok0;
    // device copies
    uint32_t* d_row_ptr = nullptr;
    uint16_t* d_tok = nullptr;
    uint32_t* d_bits = nullptr;
    uint16_t* d_rank = nullptr;
    uint16_t* d_tok0 = nullptr;

    StepDev dev(int32_t words) const {
        return StepDev{d_row_ptr, d_tok, d_bits, d_rank, n_rows, words, store, S, d_tok0};
    }
};

}  // namespace cb

struct cb_index {
    int32_t L = 0, V = 0, device = -1, words = 0;
    int64_t n_items = 0;
    std::vector<cb::StepTable> steps;
    cb::StepDev* d_steps = nullptr;  // device copy of every step's descriptor [L]
};

// Limits of the kernels in this build.
namespace cb {
constexpr int kMaxK = 64;            // beam width held by the per-query selection (one wave)
constexpr int kQueryMaxD = 2048;     // hidden width the fused per-query sparse step holds in registers
                                     // (wider: per-beam expansion + per-query merge, or the radix path)
constexpr int kMaxKRadix = 1024;     // beam width of the radix-select path (10-bit parent field of a key)
constexpr int kChunkLseTokens = 2048;  // radix path: steps whose rows hold more tokens on average get each
                                       // beam's log-sum-exp in a pass of its own (else the keys kernel
                                       // combines a beam's chunk pairs again for every chunk)
constexpr int kMaxLds = 65536;       // LDS one workgroup may use
constexpr int kPreMin = 16;          // split sparse path: rows above this many tokens scored apart, unless measured
constexpr int kExpandThreads = 256;  // per-beam expansion workgroup
constexpr int kMergeThreads = 256;   // per-query merge workgroup (dense path)
}

namespace cb {
// Workspace of the radix-select path (device pointers; sizes per query).
struct WideDev {
    int32_t* cand_off = nullptr;   // [Q_max][K+1] first candidate of each slot within its query
    int32_t* chunk_off = nullptr;  // [Q_max][K+1] first chunk of each slot within its query
    uint64_t* cand = nullptr;      // [Q_max][cap] candidates: z bits | ~index, then keys
    uint64_t* info = nullptr;      // [Q_max][cap] per candidate: next row | token | parent slot
    float* cms = nullptr;          // [Q_max][chunk_cap][2] (max z, sum exp(z - max)) per chunk
    uint32_t* hist = nullptr;      // [Q_max][2][radix bins] digit histograms of the two GPU-wide passes
    void* sel = nullptr;           // [Q_max] selection state
    int32_t* surv_n = nullptr;     // [Q_max] survivors collected
    uint64_t* surv = nullptr;      // [Q_max][survivor cap]
    int32_t* done = nullptr;       // [Q_max] 1: the pre-pass (k_wide_small) wrote the query's outputs
    int32_t use_done = 0;          // the kernels skip the queries marked done (set when the pre-pass ran)
    int32_t unc_v = 0;             // unconstrained decoding: every one of the unc_v tokens is a candidate
    const float* lse_row = nullptr;  // variants: [R] log-sum-exp of each beam's whole score row
    int64_t cap = 0, chunk_cap = 0;
};

// Workspace of the token-major scoring of the radix path's sparse steps (the
// candidates grouped by token: a counting sort per step).
struct TokDev {
    int32_t* count = nullptr;    // [V] candidates per token (zero between steps)
    int32_t* off = nullptr;      // [V + 1] first entry of each token
    int2* units = nullptr;       // [unit cap] (token | entries << 16, first entry): at most 16 entries of one token
    int32_t* n_units = nullptr;  // [1]
    int32_t* rank = nullptr;     // [Q_max][cap] rank among the token's entries (-1: not scored)
    uint2* list = nullptr;       // [Q_max * cap] (candidate, beam) grouped by token
};
}  // namespace cb

struct cb_plan {
    cb_index* idx = nullptr;
    int32_t device = -1;          // device of the workspace (destroy needs no index)
    int32_t Q_max = 0, K = 0, d = 0;
    cb_dtype dtype = CB_F32;
    int32_t Kc_max = 0;           // per-beam survivors kept: min(K, widest step)
    std::vector<int32_t> forced;  // per step: CB_PATH_* set by the caller
    std::vector<int32_t> tuned;   // per step: measured choice (0 = none)
    std::vector<int32_t> query_nt;  // per step: workgroup size of the per-query sparse step (0 = default), measured
    std::vector<int32_t> gemm_rows; // per step: product over live beams (1), every slot (2), or 0 = default
    std::vector<int32_t> radix_pre; // per step: radix selection with (2) or without (1) the one-token pre-pass, 0 = default
    std::vector<int32_t> split_min; // per step: split sparse path scores apart the rows above this many tokens (0 = 16)
    std::vector<int32_t> sparse_form; // per step: sparse step as one kernel per query (0) or per-beam expansion + merge (1)
    std::vector<int32_t> query_split; // per step: workgroups per query of the per-query sparse step (0 = 1), measured
    std::vector<float> tune_dense_us, tune_sparse_us;
    // workspace (allocated once)
    uint64_t* keys = nullptr;     // [Q_max*K][Kc_max] per-beam survivors (dense path, per-beam sparse form)
    uint64_t* side = nullptr;     // [Q_max*K][Kc_max] their next row << 16 | token (per-beam expansion)
    float* qz = nullptr;          // [Q_max][K*64 + S_max] scores handed between a query's workgroups
    float* lse_row = nullptr;     // [Q_max*K] whole-row log-sum-exp (the variants on the radix path)
    int32_t* qcnt = nullptr;      // [Q_max] their arrival counts (zero between launches)
    float* Z = nullptr;           // [Q_max*K][V] full-codebook scores (dense path)
    float* Zp = nullptr;          // [k-slices][rows][V] partial scores (dense path, few live beams)
    int32_t* live = nullptr;      // [Q_max*K] live beam slots (dense path)
    int32_t* ci_of = nullptr;     // [Q_max*K] compact index of each slot, -1 dead
    int32_t* n_live = nullptr;    // [1]
    std::vector<int32_t> select;  // per step: CB_SELECT_* set by the caller
    std::vector<int32_t> tuned_select;  // per step: measured choice (0 = none)
    cb::WideDev wide;             // radix-select workspace (allocated when a step may use it)
    cb::TokDev tok;               // token-major scoring workspace (allocated when a step may use it)
    int64_t tok_n = 0;            // candidates the token-major workspace holds (Q_max * cap)
    bool tok_dirty = false;       // per-token counts possibly left nonzero (a step stopped between its kernels)
    std::vector<int32_t> radix_tm; // per step: radix sparse scoring per chunk (1, default) or by token (2), 0 = default
    int32_t wide_S = 0;           // widest row the radix workspace was sized for
    // decode state
    float* s[2] = {nullptr, nullptr};    // [R][d] float32 state vectors
    void* h = nullptr;                    // [R][d] dtype hidden vectors
    int32_t* rows[2] = {nullptr, nullptr};
    float* acc[2] = {nullptr, nullptr};
    int32_t* hist_tok = nullptr;          // [L][R]
    int32_t* hist_par = nullptr;          // [L][R]
    int32_t* scratch_rows = nullptr;      // [R] (tuning)
    float* scratch_logp = nullptr;        // [R]
    int32_t* scratch_tok = nullptr;       // [R]
    int32_t* scratch_par = nullptr;       // [R]
    // persistent decode of the trailing sparse steps: mode -1 measured by
    // cb_tune (fuse_tuned, on until measured), 0 off, 1 on
    int32_t fuse_mode = -1;
    bool fuse_tuned = true;
    int32_t mode = CB_MODE_FILTER_FIRST;  // softmax support / constraint (cb_set_mode)
    float fuse_us[2] = {-1.f, -1.f};      // measured decode time without / with it
    // kernel timing (cb_profile_start / cb_profile_stop)
    bool prof_on = false;
    int32_t prof_cap = 0;
    std::vector<hipEvent_t> prof_ev;      // 2 per record
    std::vector<cb_kernel_time> prof_rec;
    uint64_t* phase_clk = nullptr;        // [Q_max][L][2] ticks of the persistent decode (while profiling)
    int32_t phase_t0 = -1, phase_Q = 0;   // its first step and query count (-1: none recorded)
    std::vector<cb_phase_time> phases;    // results at the last cb_profile_stop
};

namespace cb {

// Kernel launchers (kernels.hip).  All enqueue on `stream`; return hipError_t of the launch.
// Workgroup sizes and LDS bytes of the step kernels.
int expand_threads(const StepDev& st);
int query_threads(int K);
bool query_threads_ok(int nt);
size_t expand_lds_bytes(int S, int d, bool dense);
int expand_bitmap_max_v();
// LDS of the per-query sparse step at workgroup size nt (0: the default size).
size_t query_lds_bytes(int S, int K, int Kc, int d, int nt = 0);
int tail_threads(int K);
size_t tail_lds_bytes(int S, int K, int Kc, int d);
int gemm_blocks(cb_dtype dt, int R, int V, bool full);

// Sparse path: the whole step in one launch, one workgroup per query.
// pre / pre_off / pre_cap: scores of the wide rows from launch_wide_score(...,
// wide_only = pre_min, ...) (candidate z bits in the high half, per-query offsets
// [K+1], per-query capacity), or null to score them in the step kernel.
// nt: workgroup size (256, 512 or 1024; 0 = query_threads(K)); every size gives the same bits.
// pre_min: rows of more than pre_min tokens (and bitmap rows) read their scores from pre.
// G: workgroups per query (1, 2 or 4; 1 when gz or gcnt is null): each scores
// a share of the query's rows and the last to finish completes the step.
// gz: [Q][query_scores_floats(K, S)] scores; gcnt: [Q] arrival counts, zero
// before the first launch and left at zero by every launch.
hipError_t launch_step_query(const StepDev& st, cb_dtype dt, int Q, int K, int Kc, int d, int nt, const void* hidden,
                             const void* W, const int32_t* beam_rows, const float* acc, const uint64_t* pre,
                             const int32_t* pre_off, int64_t pre_cap, int pre_min, int32_t* tok, int32_t* par,
                             int32_t* rows, float* logp, int G, float* gz, int* gcnt, hipStream_t s);
int64_t query_scores_floats(int K, int S);
// Dense path: live-beam list, full-codebook scores, per-beam expansion, per-query merge.
hipError_t launch_live_rows(const StepDev& st, int R, const int32_t* beam_rows, const float* acc, int32_t* live,
                            int32_t* n_live, int32_t* ci_of, hipStream_t s);
// Whether the bf16 product finds the live beams itself (no k_live_rows).
bool gemm_finds_live(cb_dtype dt, int R);
// Whether the product can run over every beam slot (full = true: no live
// list, scores indexed by slot; the consumers learn it from n_live = -1).
bool gemm_full_ok(cb_dtype dt);
hipError_t launch_gemm_scores(cb_dtype dt, int R, int V, int d, const int32_t* live, int32_t* n_live,
                              const void* H, const void* W, float* Z, float* Zp, const StepDev& st,
                              const int32_t* beam_rows, const float* acc, int32_t* ci_of, bool full,
                              hipStream_t s);
size_t split_scores_floats(int V);
// Per-beam expansion (keys [R][Kc]); *sided tells whether the keys carry
// list places with side information [R][Kc] (then the merge takes `side`).
hipError_t launch_beam_expand(const StepDev& st, bool dense, cb_dtype dt, int R, int K, int Kc, int d,
                              const void* hidden, const void* W, const float* Z, const float* Zp, int64_t ldz,
                              const int32_t* n_live, const int32_t* ci_of, const int32_t* beam_rows,
                              const float* acc, uint64_t* keys, uint64_t* side, bool* sided, int mode,
                              hipStream_t s, int32_t* tok = nullptr, int32_t* par = nullptr,
                              int32_t* orows = nullptr, float* logp = nullptr, bool* solo_done = nullptr);
hipError_t launch_query_merge(const StepDev& st, int Q, int K, int Kc, const uint64_t* keys, const uint64_t* side,
                              const int32_t* beam_rows, int32_t* tok, int32_t* par, int32_t* rows, float* logp,
                              int mode, hipStream_t s, bool solo_done = false);
hipError_t launch_decode_init(int Q, int K, int d, cb_dtype dt, const float* q, float* s_out, void* h_out,
                              int32_t* rows, float* acc, hipStream_t st);
hipError_t launch_hidden_update(int R, int K, int d, cb_dtype dt, const float* s_old, const float* P_t,
                                const int32_t* tok, const int32_t* par, float* s_new, void* h_out,
                                hipStream_t st);
hipError_t launch_empty(int blocks, int threads, hipStream_t s);
hipError_t launch_backtrace(int R, int K, int L, const int32_t* hist_tok, const int32_t* hist_par,
                            int32_t* seqs, hipStream_t s);
// Wire-format results of Q queries (one workgroup each) at out + q * stride.
hipError_t launch_wire(int Q, int K, int L, const int32_t* seqs, const float* logp, double norm, void* out,
                       int64_t stride, int64_t* nbytes, hipStream_t s);
// Steps t0..L-1 of a decode (sparse, LDS selection) with the hidden updates
// in between, one persistent workgroup per query.  d_steps: device array [L];
// clk: NULL, or [Q][L][2] device wall-clock ticks (step start, outputs written).
hipError_t launch_decode_tail(const StepDev* d_steps, size_t lds, int t0, int L, int Q, int K, int d, int V,
                              cb_dtype dt, const void* W, const float* P, float* s0, float* s1, void* h,
                              int32_t* rows0, int32_t* rows1, float* acc0, float* acc1, int32_t* hist_tok,
                              int32_t* hist_par, uint64_t* clk, hipStream_t s);

// Radix-select path (any beam width up to kMaxKRadix): slot offsets and
// scores of every candidate (sparse dot or full-codebook gather), keys and the
// first digit, the second digit, survivor collection, and the survivors' sort
// with the outputs.
int wide_chunk();
int wide_bins();
int wide_surv_cap();
size_t wide_sel_bytes();
int wide_blocks_per_query(int Q);
int wide_hist_blocks_per_query(int Q);
// Workgroups launched per query by the histogram kernels, for queries of up to
// keys_bound candidates (each kernel uses as many as its actual count needs).
int wide_hist_blocks(int Q, int64_t keys_bound);
size_t wide_score_lds_bytes(int d, bool dense);
hipError_t launch_wide_score(const StepDev& st, bool dense, cb_dtype dt, int Q, int K, int d, const void* hidden,
                             const void* W, const float* Z, const float* Zp, int64_t ldz, const int32_t* n_live,
                             const int32_t* ci_of, const int32_t* beam_rows, const float* acc, int wide_only,
                             const WideDev& w, hipStream_t s);
// Token-major scoring (sparse steps on the radix selection, d <= 2048): the
// candidates' tokens and ranks per token, the per-token offsets and work units,
// the lists, the scores by token, then the chunk pairs of the scores.
hipError_t launch_tm_count(const StepDev& st, int Q, int K, const int32_t* beam_rows, const float* acc,
                           const WideDev& w, const TokDev& tk, hipStream_t s);
hipError_t launch_tm_scan(int V, const TokDev& tk, hipStream_t s);
hipError_t launch_tm_scatter(int Q, int K, const WideDev& w, const TokDev& tk, hipStream_t s);
hipError_t launch_tm_score(cb_dtype dt, int K, int d, const void* hidden, const void* W, const WideDev& w,
                           const TokDev& tk, hipStream_t s);
hipError_t launch_tm_pairs(int Q, int K, int64_t keys_bound, const WideDev& w, hipStream_t s);
hipError_t launch_tm_clear(int V, const TokDev& tk, hipStream_t s);
int tm_score_blocks();
int64_t tm_unit_cap(int64_t n, int V);

// Pre-pass of the radix selection: one workgroup per query finishes every
// query whose live rows all hold one token (outputs written, done[q] = 1)
// and leaves the others to the radix kernels (done[q] = 0).
hipError_t launch_wide_small(const StepDev& st, int Q, int K, const int32_t* beam_rows, const float* acc,
                             const WideDev& w, int32_t* tok, int32_t* par, int32_t* rows, float* logp, hipStream_t s);
hipError_t launch_wide_keys(int Q, int K, int64_t keys_bound, const float* acc, const WideDev& w, hipStream_t s);
// Score first on the radix path: the log-sum-exp of each live beam's whole
// score row (the softmax support of the variant), one workgroup per beam.
hipError_t launch_row_lse(const StepDev& st, cb_dtype dt, int R, int V, int d, const float* Z, const float* Zp,
                          const int32_t* n_live, const int32_t* ci_of, const int32_t* beam_rows, const float* acc,
                          float* lse_row, hipStream_t s);
// Unconstrained decoding on the radix path: each live beam's log-sum-exp over
// all its candidates, once per beam from the chunk pairs of the score pass.
hipError_t launch_chunk_lse(int Q, int K, const WideDev& w, float* lse_row, hipStream_t s);
hipError_t launch_wide_refine(int Q, int K, int64_t keys_bound, const WideDev& w, hipStream_t s);
hipError_t launch_wide_collect(int Q, int K, int64_t keys_bound, const WideDev& w, hipStream_t s);
hipError_t launch_wide_sort(const StepDev& st, int Q, int K, const int32_t* beam_rows, const WideDev& w,
                            int32_t* tok, int32_t* par, int32_t* rows, float* logp, hipStream_t s);

// One step on the given plan's workspace and path / selection (api.cpp; no
// validation).  The allocation-free step passes a plan whose workspace
// pointers lie in its static device array.
cb_status enqueue_step(cb_plan* p, int t, int Q, int32_t path, int32_t sel, const void* hidden, const void* Wt,
                       const int32_t* rows, const float* acc, int32_t* ot, int32_t* op, int32_t* orow, float* ol,
                       hipStream_t s);
// Whether a step's four outputs overlap one another or its inputs.
bool step_args_alias(size_t R, size_t d, size_t V, cb_dtype dt, const void* hidden, const void* W_t, const void* rows,
                     const void* acc, void* const outs[4]);
// Streams finished step tables of an index to its device (upload.cpp): a
// host thread of its own copies each pushed step in batches through two
// alternating pinned staging buffers on a copy stream of its own, then
// releases the step's host arrays.  Copies only, no kernels.
class StepUploader {
   public:
    explicit StepUploader(cb_index* idx);
    ~StepUploader();
    StepUploader(const StepUploader&) = delete;
    StepUploader& operator=(const StepUploader&) = delete;
    cb_status start();
    // step t's host tables are complete: queue them for upload
    void push(int t);
    // wait for every queued step; on failure cb_last_error() tells why (the
    // caller frees the index, whose device arrays may be partly allocated)
    cb_status finish();

   private:
    void run();
    void release();
    void fail(const std::string& m);
    bool stream_copy(void* dst, const void* src, size_t n);
    template <class T>
    bool upload_array(std::vector<T>& host, T** dev, const char* what);
    cb_index* idx_;
    hipStream_t stream_ = nullptr;
    void* stage_[2] = {nullptr, nullptr};
    hipEvent_t ev_[2] = {nullptr, nullptr};
    int cur_ = 0;
    std::thread thread_;
    bool started_ = false;
    std::mutex mu_;
    std::condition_variable cv_;
    std::deque<int> queue_;
    bool closed_ = false;
    cb_status status_ = CB_OK;  // written by the upload thread; read after the join
    std::string msg_;
};

// Index construction (index_build.cpp).
// Upload the host tables of idx to idx->device (release the host copies) and
// the step descriptors; frees idx on failure.
cb_status upload_index(cb_index* idx);
// Sort and deduplicate the catalog and build every step's host tables; each
// finished step is pushed to `up` (NULL: host tables only).
cb_status build_host_tables(const int32_t* sids, int64_t n_items, int32_t L, int32_t V, int32_t store,
                            cb_index* idx, StepUploader* up);
// Upload the step descriptors of an index whose tables are on the device.
cb_status upload_descriptors(cb_index* idx);

}  // namespace cb
