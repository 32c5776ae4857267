// C-ABI entry points of the constrained beam-search library.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "cb_internal.h"

namespace cb {

namespace {
thread_local std::string g_err;
}

thread_local LaunchEvents g_launch_events;
LaunchEvents& launch_events() { return g_launch_events; }

void set_error(const std::string& msg) { g_err = msg; }
void clear_error() { g_err.clear(); }


namespace {

cb_status hip_fail(const char* where, hipError_t e) {
    set_error(std::string(where) + ": " + hipGetErrorString(e));
    return CB_EHIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

// The step's outputs must be four distinct arrays that share no byte with
// its inputs (the kernels read inputs after other workgroups wrote outputs).
bool step_outputs_alias(size_t R, size_t d, size_t V, size_t es, const void* hidden, const void* W_t,
                        const void* rows, const void* acc, void* const outs[4]) {
    const void* in[4] = {hidden, W_t, rows, acc};
    const size_t in_n[4] = {R * d * es, V * d * es, R * 4, R * 4};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 4; ++j)
            if (overlaps(outs[i], R * 4, in[j], in_n[j])) return true;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], R * 4, outs[j], R * 4)) return true;
    }
    return false;
}
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t dtype_size(cb_dtype dt) { return dt == CB_BF16 ? 2 : 4; }

template <class T>
cb_status dev_alloc(T** p, size_t count, const char* what) {
    *p = nullptr;
    if (count == 0) return CB_OK;
    hipError_t e = hipMalloc(reinterpret_cast<void**>(p), count * sizeof(T));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        set_error(std::string("device allocation failed: ") + what);
        return CB_ENOMEM;
    }
    return CB_OK;
}

void dev_free(void* p) {
    if (p) (void)hipFree(p);
}

bool dense_available(const cb_plan* p) { return p->dtype == CB_F32 || (p->d % 64) == 0; }

int32_t resolve_path(const cb_plan* p, int t) {
    if (p->mode != CB_MODE_FILTER_FIRST) return CB_PATH_DENSE;  // the variants need full score rows
    int32_t f = p->forced[(size_t)t];
    if (f == CB_PATH_DENSE || f == CB_PATH_SPARSE || f == CB_PATH_SPARSE_SPLIT) return f;
    int32_t tu = p->tuned[(size_t)t];
    if (tu == CB_PATH_DENSE || tu == CB_PATH_SPARSE || tu == CB_PATH_SPARSE_SPLIT) return tu;
    const cb::StepTable& T = p->idx->steps[(size_t)t];
    return (T.store == CB_STORE_BITMAP && dense_available(p)) ? CB_PATH_DENSE : CB_PATH_SPARSE;
}

// Per-step option value (0 when the plan keeps none, as the allocation-free step's).
int32_t opt(const std::vector<int32_t>& v, int t) { return (size_t)t < v.size() ? v[(size_t)t] : 0; }

// Whether the full-codebook product of step t runs over every beam slot (no
// live list) rather than the compact list of live beams: measured by cb_tune,
// else over every slot after step 0 (beams fill their slots once a query has
// K candidates) and compact at step 0 (one live slot per query).
bool gemm_full(const cb_plan* p, int t) {
    if (!gemm_full_ok(p->dtype)) return false;
    const int32_t v = opt(p->gemm_rows, t);
    if (v == 1 || v == 2) return v == 2;
    return t > 0;
}

// Whether the LDS selection (fused sparse step, or dense expansion + merge)
// holds step t of this plan.
// Hidden widths above kQueryMaxD take the sparse step as a per-beam
// expansion (whose scoring loops over the whole width) + per-query merge
// instead of the fused per-query kernel, which keeps at most kQueryMaxD
// elements of a hidden vector in registers.
bool lds_select_ok(const cb_plan* p, int t) {
    if (p->K > kMaxK) return false;
    const cb::StepTable& T = p->idx->steps[(size_t)t];
    const int Kc = std::min(p->K, std::max(T.S, 1));
    const bool sparse_ok = p->d <= kQueryMaxD ? query_lds_bytes(T.S, p->K, Kc, p->d) <= (size_t)kMaxLds
                                              : expand_lds_bytes(T.S, p->d, false) <= (size_t)kMaxLds;
    return sparse_ok && expand_lds_bytes(T.S, p->d, true) <= (size_t)kMaxLds;
}

// Whether a decoding variant can take the LDS selection at step t: the
// dense expansion of every token (without a constraint) is the bitmap kernel,
// which needs a bf16 plan, V <= 4096 and V a multiple of 4.
bool variant_lds_ok(const cb_plan* p, int t) {
    if (!lds_select_ok(p, t)) return false;
    if (p->mode != CB_MODE_UNCONSTRAINED) return true;
    const int V = p->idx->V;
    return p->dtype == CB_BF16 && V <= expand_bitmap_max_v() && V % 4 == 0 && std::min(p->K, V) <= p->Kc_max;
}

int32_t resolve_select(const cb_plan* p, int t) {
    if (p->mode != CB_MODE_FILTER_FIRST) {
        const int32_t f = p->select[(size_t)t];
        if (f == CB_SELECT_RADIX || (f == CB_SELECT_LDS && variant_lds_ok(p, t))) return f;
        return variant_lds_ok(p, t) ? CB_SELECT_LDS : CB_SELECT_RADIX;
    }
    const int32_t f = p->select[(size_t)t];
    if (f == CB_SELECT_LDS || f == CB_SELECT_RADIX) return f;
    const int32_t tu = p->tuned_select[(size_t)t];
    if (tu == CB_SELECT_RADIX || (tu == CB_SELECT_LDS && lds_select_ok(p, t))) return tu;
    return lds_select_ok(p, t) ? CB_SELECT_LDS : CB_SELECT_RADIX;
}

void wide_release(cb_plan* p) {
    WideDev& w = p->wide;
    dev_free(w.cand_off);
    dev_free(w.chunk_off);
    dev_free(w.cand);
    dev_free(w.info);
    dev_free(w.cms);
    dev_free(w.hist);
    dev_free(w.sel);
    dev_free(w.surv_n);
    dev_free(w.surv);
    dev_free(w.done);
    w = WideDev();
    p->wide_S = 0;
    cb::TokDev& tk = p->tok;
    dev_free(tk.count);
    dev_free(tk.off);
    dev_free(tk.units);
    dev_free(tk.n_units);
    dev_free(tk.rank);
    dev_free(tk.list);
    tk = cb::TokDev();
    p->tok_n = 0;
    p->tok_dirty = false;
}

// Token-major workspace for the radix workspace's capacity (which must exist).
cb_status tok_alloc(cb_plan* p) {
    const int64_t n = (int64_t)p->Q_max * p->wide.cap;
    if (p->tok.list && p->tok_n >= n) return CB_OK;
    if (n >= (int64_t(1) << 31)) {
        set_error("token-major scoring: Q_max * K * widest row exceeds 2^31 candidates");
        return CB_ECAPACITY;
    }
    const int V = p->idx->V;
    cb::TokDev& tk = p->tok;
    dev_free(tk.count);
    dev_free(tk.off);
    dev_free(tk.units);
    dev_free(tk.n_units);
    dev_free(tk.rank);
    dev_free(tk.list);
    tk = cb::TokDev();
    p->tok_n = 0;
    cb_status st = dev_alloc(&tk.count, (size_t)V, "token counts");
    if (st == CB_OK) st = dev_alloc(&tk.off, (size_t)V + 1, "token offsets");
    if (st == CB_OK) st = dev_alloc(&tk.units, (size_t)tm_unit_cap(n, V), "token units");
    if (st == CB_OK) st = dev_alloc(&tk.n_units, 1, "token unit count");
    if (st == CB_OK) st = dev_alloc(&tk.rank, (size_t)n, "token ranks");
    if (st == CB_OK) st = dev_alloc(&tk.list, (size_t)n, "token lists");
    if (st == CB_OK) {
        const hipError_t e = hipMemset(tk.count, 0, (size_t)V * sizeof(int32_t));
        if (e != hipSuccess) st = hip_fail("token counts", e);
    }
    if (st != CB_OK) {
        dev_free(tk.count);
        dev_free(tk.off);
        dev_free(tk.units);
        dev_free(tk.n_units);
        dev_free(tk.rank);
        dev_free(tk.list);
        tk = cb::TokDev();
        return st;
    }
    p->tok_n = n;
    p->tok_dirty = false;
    return CB_OK;
}

// Radix-selection workspace sized for the plan's widest row.
cb_status wide_alloc(cb_plan* p) {
    int32_t S = 1;
    for (const auto& T : p->idx->steps) S = std::max(S, T.S);
    // without a constraint every token of the codebook is a candidate
    if (p->mode == CB_MODE_UNCONSTRAINED) S = std::max(S, p->idx->V);
    if (p->wide.cand && p->wide_S >= S) return CB_OK;
    if (p->wide.cand) wide_release(p);
    const int64_t cap = (int64_t)p->K * S;
    const int64_t chunk_cap = (int64_t)p->K * ((S + wide_chunk() - 1) / wide_chunk());
    if (cap >= (int64_t(1) << 31)) {
        set_error("radix selection: K * widest row exceeds 2^31 candidates per query");
        return CB_ECAPACITY;
    }
    const size_t Q = (size_t)p->Q_max;
    WideDev& w = p->wide;
    w.cap = cap;
    w.chunk_cap = chunk_cap;
    cb_status st = dev_alloc(&w.cand_off, Q * (p->K + 1), "radix offsets");
    if (st == CB_OK) st = dev_alloc(&w.chunk_off, Q * (p->K + 1), "radix chunk offsets");
    if (st == CB_OK) st = dev_alloc(&w.cand, Q * (size_t)cap, "radix candidates");
    if (st == CB_OK) st = dev_alloc(&w.info, Q * (size_t)cap, "radix candidate rows");
    if (st == CB_OK) st = dev_alloc(&w.cms, Q * (size_t)chunk_cap * 2, "radix chunk softmax");
    if (st == CB_OK) st = dev_alloc(&w.hist, Q * 2 * (size_t)wide_bins(), "radix histograms");
    if (st == CB_OK) {
        unsigned char* sel = nullptr;
        st = dev_alloc(&sel, Q * wide_sel_bytes(), "radix state");
        w.sel = sel;
    }
    if (st == CB_OK) st = dev_alloc(&w.surv_n, Q, "radix survivor counts");
    if (st == CB_OK) st = dev_alloc(&w.surv, Q * (size_t)wide_surv_cap(), "radix survivors");
    if (st == CB_OK) st = dev_alloc(&w.done, Q, "radix pre-pass flags");
    if (st != CB_OK) {
        wide_release(p);
        return st;
    }
    p->wide_S = S;
    // a step set to score by token keeps its workspace sized with this one
    for (const int32_t v : p->radix_tm)
        if (v == 2) return tok_alloc(p);
    return CB_OK;
}

// While profiling is on, attaches an event pair to the dispatch of the one
// kernel the next launcher call enqueues (its start and end as the GPU
// records them, not the host's enqueue).
struct ProfMark {
    cb_plan* p;
    int idx = -1;
    ProfMark(cb_plan* p_, hipStream_t, int t, int kernel, int threads, int blocks) : p(p_) {
        if (!p->prof_on || (int)p->prof_rec.size() >= p->prof_cap) return;
        idx = (int)p->prof_rec.size();
        p->prof_rec.push_back(cb_kernel_time{t, kernel, threads, blocks, 0.f});
        launch_events() = LaunchEvents{p->prof_ev[(size_t)idx * 2], p->prof_ev[(size_t)idx * 2 + 1]};
    }
    void done() { launch_events() = LaunchEvents{}; }
    ~ProfMark() { launch_events() = LaunchEvents{}; }
};

// Enqueue one step on the radix selection (no validation).
cb_status run_step_radix(cb_plan* p, int t, int Q, int32_t path, const void* hidden, const void* Wt,
                         const int32_t* rows, const float* acc, int32_t* ot, int32_t* op, int32_t* orow, float* ol,
                         hipStream_t s) {
    const cb_index* idx = p->idx;
    const cb::StepDev sd = idx->steps[(size_t)t].dev(idx->words);
    const int R = Q * p->K;
    if (!p->wide.cand) {
        set_error("cb_step: radix workspace missing");
        return CB_EINVAL;
    }
    // candidates a query can hold: K rows of the widest row (every token without a constraint)
    const int64_t kb = (int64_t)p->K * (p->mode == CB_MODE_UNCONSTRAINED ? idx->V : std::max(idx->steps[(size_t)t].S, 1));
    const int GS = wide_blocks_per_query(Q) * Q, GH = wide_hist_blocks(Q, kb) * Q;
    const bool dense = path == CB_PATH_DENSE;
    hipError_t e;
    // the one-token pre-pass (sparse scoring only): queries whose live rows
    // all hold one token are finished there and skipped by the kernels below
    WideDev w = p->wide;
    const int32_t pre_v = opt(p->radix_pre, t);
    w.use_done = !dense && pre_v != 1 ? 1 : 0;
    if (w.use_done) {
        ProfMark m(p, s, t, CB_KERNEL_RADIX_SMALL, 1024, Q);
        e = launch_wide_small(sd, Q, p->K, rows, acc, w, ot, op, orow, ol, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: radix pre-pass", e);
    }
    if (dense) {
        const bool full = gemm_full(p, t);
        if (!full && !gemm_finds_live(p->dtype, R)) {
            ProfMark m(p, s, t, CB_KERNEL_LIVE_ROWS, 1024, 1);
            e = launch_live_rows(sd, R, rows, acc, p->live, p->n_live, p->ci_of, s);
            m.done();
            if (e != hipSuccess) return hip_fail("cb_step: live beams", e);
        }
        const bool bf = p->dtype == CB_BF16;
        ProfMark m(p, s, t, bf ? CB_KERNEL_GEMM_BF16 : CB_KERNEL_GEMM_F32, bf ? 512 : 256,
                   gemm_blocks(p->dtype, R, idx->V, full));
        e = launch_gemm_scores(p->dtype, R, idx->V, p->d, p->live, p->n_live, hidden, Wt, p->Z, p->Zp, sd, rows, acc,
                               p->ci_of, full, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: full-codebook scores", e);
    }
    // the variants (dense scoring only): every token a candidate, or the
    // softmax over each beam's whole score row
    if (p->mode == CB_MODE_UNCONSTRAINED) w.unc_v = idx->V;
    if (p->mode == CB_MODE_SCORE_FIRST) {
        ProfMark m(p, s, t, CB_KERNEL_ROW_LSE, 256, R);
        e = launch_row_lse(sd, p->dtype, R, idx->V, p->d, p->Z, p->Zp, p->n_live, p->ci_of, rows, acc, p->lse_row, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: row log-sum-exp", e);
        w.lse_row = p->lse_row;
    }
    const cb::StepTable& T = idx->steps[(size_t)t];
    if (!dense && opt(p->radix_tm, t) == 2 && p->d <= kQueryMaxD) {
        // scores by token: each W_t row read once for all the beams that hold it
        cb_status st = tok_alloc(p);
        if (st != CB_OK) return st;
        const cb::TokDev& tk = p->tok;
        if (p->tok_dirty) {
            e = launch_tm_clear(idx->V, tk, s);
            if (e != hipSuccess) return hip_fail("cb_step: token counts", e);
        }
        p->tok_dirty = true;
        {
            ProfMark m(p, s, t, CB_KERNEL_TOKEN_LISTS, 256, GS);
            e = launch_tm_count(sd, Q, p->K, rows, acc, w, tk, s);
            m.done();
            if (e != hipSuccess) return hip_fail("cb_step: token counts", e);
        }
        {
            ProfMark m(p, s, t, CB_KERNEL_TOKEN_LISTS, 1024, 1);
            e = launch_tm_scan(idx->V, tk, s);
            m.done();
            if (e != hipSuccess) return hip_fail("cb_step: token offsets", e);
        }
        p->tok_dirty = false;
        {
            ProfMark m(p, s, t, CB_KERNEL_TOKEN_LISTS, 256, GS);
            e = launch_tm_scatter(Q, p->K, w, tk, s);
            m.done();
            if (e != hipSuccess) return hip_fail("cb_step: token lists", e);
        }
        {
            ProfMark m(p, s, t, CB_KERNEL_TOKEN_SCORE, 256, tm_score_blocks());
            e = launch_tm_score(p->dtype, p->K, p->d, hidden, Wt, w, tk, s);
            m.done();
            if (e != hipSuccess) return hip_fail("cb_step: scores by token", e);
        }
        {
            ProfMark m(p, s, t, CB_KERNEL_TOKEN_SCORE, 256, GH);
            e = launch_tm_pairs(Q, p->K, kb, w, s);
            m.done();
            if (e != hipSuccess) return hip_fail("cb_step: chunk softmax pairs", e);
        }
    } else {
        ProfMark m(p, s, t, dense ? CB_KERNEL_RADIX_SCORE_DENSE : CB_KERNEL_RADIX_SCORE_SPARSE, 256, GS);
        e = launch_wide_score(sd, dense, p->dtype, Q, p->K, p->d, hidden, Wt, p->Z, p->Zp, idx->V, p->n_live,
                              p->ci_of, rows, acc, 0, w, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: radix scores", e);
    }
    if (!w.lse_row && (p->mode == CB_MODE_UNCONSTRAINED ||
                       (p->mode == CB_MODE_FILTER_FIRST &&
                        T.n_edges > (int64_t)kChunkLseTokens * std::max<int64_t>(T.n_rows, 1)))) {
        // rows of many chunks on average (every token without a constraint,
        // or wide rows): each beam's log-sum-exp once, from its chunk pairs,
        // not again for each of its chunks
        ProfMark m(p, s, t, CB_KERNEL_ROW_LSE, 256, (R + 3) / 4);
        e = launch_chunk_lse(Q, p->K, w, p->lse_row, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: row log-sum-exp", e);
        w.lse_row = p->lse_row;
    }
    {
        ProfMark m(p, s, t, CB_KERNEL_RADIX_KEYS, 256, GH);
        e = launch_wide_keys(Q, p->K, kb, acc, w, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: radix keys", e);
    }
    {
        ProfMark m(p, s, t, CB_KERNEL_RADIX_REFINE, 256, GH);
        e = launch_wide_refine(Q, p->K, kb, w, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: radix refine", e);
    }
    {
        ProfMark m(p, s, t, CB_KERNEL_RADIX_COLLECT, 256, GH);
        e = launch_wide_collect(Q, p->K, kb, w, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: radix collect", e);
    }
    {
        ProfMark m(p, s, t, CB_KERNEL_RADIX_SORT, 1024, Q);
        e = launch_wide_sort(sd, Q, p->K, rows, w, ot, op, orow, ol, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: radix sort", e);
    }
    return CB_OK;
}

// Enqueue one step (no validation).
cb_status run_step(cb_plan* p, int t, int Q, int32_t path, int32_t sel, const void* hidden, const void* Wt,
                   const int32_t* rows, const float* acc, int32_t* ot, int32_t* op, int32_t* orow, float* ol,
                   hipStream_t s) {
    const cb_index* idx = p->idx;
    const cb::StepTable& T = idx->steps[(size_t)t];
    const cb::StepDev sd = T.dev(idx->words);
    const int R = Q * p->K;
    // survivors per beam: every token is a candidate without a constraint
    const int Kc = std::min(p->K, p->mode == CB_MODE_UNCONSTRAINED ? idx->V : std::max(T.S, 1));
    hipError_t e;
    if (sel == CB_SELECT_RADIX) return run_step_radix(p, t, Q, path, hidden, Wt, rows, acc, ot, op, orow, ol, s);
    const bool per_beam = p->d > kQueryMaxD || opt(p->sparse_form, t) == 1;
    if ((path == CB_PATH_SPARSE || path == CB_PATH_SPARSE_SPLIT) && per_beam) {
        // per-beam gather-dot expansion over the whole GPU, then the per-query
        // merge (wide hidden vectors, or the measured choice for the step)
        bool sided = false;
        {
            ProfMark m(p, s, t, CB_KERNEL_EXPAND_SPARSE, expand_threads(sd), R);
            e = launch_beam_expand(sd, false, p->dtype, R, p->K, Kc, p->d, hidden, Wt, nullptr, nullptr, idx->V,
                                   nullptr, nullptr, rows, acc, p->keys, p->side, &sided, p->mode, s);
            m.done();
            if (e != hipSuccess) return hip_fail("cb_step: sparse beam expansion", e);
        }
        ProfMark m(p, s, t, CB_KERNEL_MERGE, kMergeThreads, Q);
        e = launch_query_merge(sd, Q, p->K, Kc, p->keys, sided ? p->side : nullptr, rows, ot, op, orow, ol, p->mode,
                               s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: query merge", e);
        return CB_OK;
    }
    if (path == CB_PATH_SPARSE || path == CB_PATH_SPARSE_SPLIT) {
        const WideDev& w = p->wide;
        const bool split = path == CB_PATH_SPARSE_SPLIT && w.cand;
        // rows above pre_min tokens scored across many workgroups first (16 unless measured)
        const int pre_min = opt(p->split_min, t) > 0 ? opt(p->split_min, t) : kPreMin;
        if (split) {
            ProfMark m(p, s, t, CB_KERNEL_RADIX_SCORE_SPARSE, 256, wide_blocks_per_query(Q) * Q);
            e = launch_wide_score(sd, false, p->dtype, Q, p->K, p->d, hidden, Wt, nullptr, nullptr, idx->V, nullptr,
                                  nullptr, rows, acc, pre_min, w, s);
            m.done();
            if (e != hipSuccess) return hip_fail("cb_step: wide-row scores", e);
        }
        const int nt = query_threads_ok(opt(p->query_nt, t)) ? opt(p->query_nt, t) : query_threads(p->K);
        const int G = p->qz && p->qcnt && opt(p->query_split, t) > 1 ? opt(p->query_split, t) : 1;
        ProfMark m(p, s, t, CB_KERNEL_STEP_QUERY, nt, Q * G);
        e = launch_step_query(sd, p->dtype, Q, p->K, Kc, p->d, nt, hidden, Wt, rows, acc, split ? w.cand : nullptr,
                              split ? w.cand_off : nullptr, split ? w.cap : 0, pre_min, ot, op, orow, ol, G, p->qz,
                              p->qcnt, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: sparse step", e);
        return CB_OK;
    }
    const bool full = gemm_full(p, t);
    if (!full && !gemm_finds_live(p->dtype, R)) {
        ProfMark m(p, s, t, CB_KERNEL_LIVE_ROWS, 1024, 1);
        e = launch_live_rows(sd, R, rows, acc, p->live, p->n_live, p->ci_of, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: live beams", e);
    }
    {
        const bool bf = p->dtype == CB_BF16;
        ProfMark m(p, s, t, bf ? CB_KERNEL_GEMM_BF16 : CB_KERNEL_GEMM_F32, bf ? 512 : 256,
                   gemm_blocks(p->dtype, R, idx->V, full));
        e = launch_gemm_scores(p->dtype, R, idx->V, p->d, p->live, p->n_live, hidden, Wt, p->Z, p->Zp, sd, rows, acc,
                               p->ci_of, full, s);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: full-codebook scores", e);
    }
    bool sided = false, solo = false;
    {
        ProfMark m(p, s, t, CB_KERNEL_EXPAND_DENSE, expand_threads(sd), R);
        e = launch_beam_expand(sd, true, p->dtype, R, p->K, Kc, p->d, hidden, Wt, p->Z, p->Zp, idx->V, p->n_live,
                               p->ci_of, rows, acc, p->keys, p->side, &sided, p->mode, s, ot, op, orow, ol, &solo);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: beam expansion", e);
    }
    {
        ProfMark m(p, s, t, CB_KERNEL_MERGE, kMergeThreads, Q);
        e = launch_query_merge(sd, Q, p->K, Kc, p->keys, sided ? p->side : nullptr, rows, ot, op, orow, ol, p->mode,
                               s, solo);
        m.done();
        if (e != hipSuccess) return hip_fail("cb_step: query merge", e);
    }
    return CB_OK;
}

void profile_release(cb_plan* p) {
    for (hipEvent_t ev : p->prof_ev)
        if (ev) (void)hipEventDestroy(ev);
    dev_free(p->phase_clk);
    p->phase_clk = nullptr;
    p->phase_t0 = -1;
    p->prof_ev.clear();
    p->prof_rec.clear();
    p->prof_on = false;
    p->prof_cap = 0;
}

cb_status check_plan(const cb_plan* p, int32_t Q, const char* fn) {
    if (!p) {
        set_error(std::string(fn) + ": plan is NULL");
        return CB_EINVAL;
    }
    if (Q < 0 || Q > p->Q_max) {
        set_error(std::string(fn) + ": Q out of [0, Q_max]");
        return CB_EINVAL;
    }
    if (p->idx->device < 0) {
        set_error(std::string(fn) + ": index was built host-only (device -1)");
        return CB_EINVAL;
    }
    return CB_OK;
}

}  // namespace

// Entry points shared with the allocation-free step (noalloc.hip).
cb_status enqueue_step(cb_plan* p, int t, int Q, int32_t path, int32_t sel, const void* hidden, const void* Wt,
                       const int32_t* rows, const float* acc, int32_t* ot, int32_t* op, int32_t* orow, float* ol,
                       hipStream_t s) {
    return run_step(p, t, Q, path, sel, hidden, Wt, rows, acc, ot, op, orow, ol, s);
}

bool step_args_alias(size_t R, size_t d, size_t V, cb_dtype dt, const void* hidden, const void* W_t, const void* rows,
                     const void* acc, void* const outs[4]) {
    return step_outputs_alias(R, d, V, dtype_size(dt), hidden, W_t, rows, acc, outs);
}

// Device copy of every step's descriptor (read by the persistent decode).
cb_status upload_descriptors(cb_index* idx) {
    DeviceGuard g(idx->device);
    std::vector<cb::StepDev> descs;
    for (const auto& T : idx->steps) descs.push_back(T.dev(idx->words));
    cb_status st = dev_alloc(&idx->d_steps, descs.size(), "step descriptors");
    if (st == CB_OK) {
        hipError_t e = hipMemcpy(idx->d_steps, descs.data(), descs.size() * sizeof(cb::StepDev), hipMemcpyHostToDevice);
        if (e != hipSuccess) st = hip_fail("cb_build_index: upload", e);
    }
    return st;
}

// Stream the host tables of idx to idx->device (releasing the host copies)
// and upload the step descriptors.  On failure idx is freed.
cb_status upload_index(cb_index* idx) {
    StepUploader up(idx);
    cb_status st = up.start();
    if (st == CB_OK) {
        for (int t = 0; t < idx->L; ++t) up.push(t);
        st = up.finish();
    }
    if (st == CB_OK) st = upload_descriptors(idx);
    if (st != CB_OK) cb_free_index(idx);
    return st;
}

}  // namespace cb

using namespace cb;

extern "C" {

const char* cb_last_error(void) { return g_err.c_str(); }

cb_status cb_build_index(const int32_t* sids, int64_t n_items, int32_t L, int32_t V, int32_t device, int32_t store,
                         cb_index** out) {
    clear_error();
    if (!out) {
        set_error("cb_build_index: out is NULL");
        return CB_EINVAL;
    }
    *out = nullptr;
    if (!sids || n_items < 1 || n_items >= (int64_t(1) << 31) || L < 1 || L > 64 || V < 2) {
        set_error("cb_build_index: need sids != NULL, 1 <= n_items < 2^31, 1 <= L <= 64, V >= 2");
        return CB_EINVAL;
    }
    if (V > 65535) {
        set_error("cb_build_index: V > 65535 is not supported (tokens are stored as 16-bit)");
        return CB_EUNSUPPORTED;
    }
    if (store < CB_STORE_AUTO || store > CB_STORE_BITMAP) {
        set_error("cb_build_index: unknown storage policy");
        return CB_EINVAL;
    }
    for (int64_t i = 0; i < n_items * L; ++i)
        if (sids[i] < 0 || sids[i] >= V) {
            set_error("cb_build_index: token out of [0, V) at item " + std::to_string(i / L));
            return CB_EINVAL;
        }
    cb_index* idx = new (std::nothrow) cb_index();
    if (!idx) {
        set_error("cb_build_index: host allocation failed");
        return CB_ENOMEM;
    }
    idx->device = device;
    if (device < 0) {
        cb_status st = build_host_tables(sids, n_items, L, V, store, idx, nullptr);
        if (st != CB_OK) {
            delete idx;
            return st;
        }
        *out = idx;
        return CB_OK;
    }
    // each finished step streams to the device while the next one is built
    StepUploader up(idx);
    cb_status st = up.start();
    if (st == CB_OK) {
        st = build_host_tables(sids, n_items, L, V, store, idx, &up);
        const cb_status su = up.finish();  // joins the upload thread before anything is freed
        if (st == CB_OK) st = su;
    }
    if (st == CB_OK) st = upload_descriptors(idx);
    if (st != CB_OK) {
        cb_free_index(idx);
        return st;
    }
    *out = idx;
    return CB_OK;
}

cb_status cb_index_shape(const cb_index* idx, int32_t* L, int32_t* V, int64_t* n_items, int32_t* device) {
    clear_error();
    if (!idx) {
        set_error("cb_index_shape: index is NULL");
        return CB_EINVAL;
    }
    if (L) *L = idx->L;
    if (V) *V = idx->V;
    if (n_items) *n_items = idx->n_items;
    if (device) *device = idx->device;
    return CB_OK;
}

cb_status cb_index_info(const cb_index* idx, int32_t t, cb_step_info* out) {
    clear_error();
    if (!idx || !out || t < 0 || t >= idx->L) {
        set_error("cb_index_info: bad index, step or output");
        return CB_EINVAL;
    }
    const auto& T = idx->steps[(size_t)t];
    out->n_rows = T.n_rows;
    out->n_edges = T.n_edges;
    out->max_fanout = T.S;
    out->storage = T.store;
    out->bytes = T.bytes;
    return CB_OK;
}

cb_status cb_index_row(const cb_index* idx, int32_t t, int64_t row, int32_t* tokens, int64_t* next_rows, int32_t cap,
                       int32_t* n) {
    clear_error();
    if (!idx || !n || t < 0 || t >= idx->L) {
        set_error("cb_index_row: bad index, step or output");
        return CB_EINVAL;
    }
    const auto& T = idx->steps[(size_t)t];
    if (row < 0 || row >= T.n_rows) {
        set_error("cb_index_row: row out of range");
        return CB_EINVAL;
    }
    uint32_t rp[2];
    std::vector<uint16_t> tk;
    std::vector<uint32_t> bits;
    const bool host = !T.row_ptr.empty();
    if (!host && idx->device < 0) {
        set_error("cb_index_row: index holds no tables");
        return CB_EINVAL;
    }
    DeviceGuard g(host ? -1 : idx->device);
    if (host) {
        rp[0] = T.row_ptr[(size_t)row];
        rp[1] = T.row_ptr[(size_t)row + 1];
    } else {
        hipError_t e = hipMemcpy(rp, T.d_row_ptr + row, 8, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail("cb_index_row", e);
    }
    const uint32_t cnt = rp[1] - rp[0];
    if (T.store == CB_STORE_CSR) {
        tk.resize(cnt);
        if (host) {
            std::copy(T.tok.begin() + rp[0], T.tok.begin() + rp[1], tk.begin());
        } else if (cnt) {
            hipError_t e = hipMemcpy(tk.data(), T.d_tok + rp[0], cnt * 2, hipMemcpyDeviceToHost);
            if (e != hipSuccess) return hip_fail("cb_index_row", e);
        }
    } else {
        bits.resize((size_t)idx->words);
        if (host) {
            std::copy(T.bits.begin() + row * idx->words, T.bits.begin() + (row + 1) * idx->words, bits.begin());
        } else {
            hipError_t e = hipMemcpy(bits.data(), T.d_bits + row * idx->words, (size_t)idx->words * 4,
                                     hipMemcpyDeviceToHost);
            if (e != hipSuccess) return hip_fail("cb_index_row", e);
        }
        for (int w = 0; w < idx->words; ++w)
            for (int b = 0; b < 32; ++b)
                if (bits[(size_t)w] >> b & 1u) tk.push_back((uint16_t)(w * 32 + b));
    }
    *n = (int32_t)tk.size();
    for (int32_t j = 0; j < (int32_t)tk.size() && j < cap; ++j) {
        if (tokens) tokens[j] = tk[(size_t)j];
        if (next_rows) next_rows[j] = (int64_t)rp[0] + j;
    }
    return CB_OK;
}

void cb_free_index(cb_index* idx) {
    if (!idx) return;
    if (idx->device >= 0) {
        DeviceGuard g(idx->device);
        for (auto& T : idx->steps) {
            dev_free(T.d_row_ptr);
            dev_free(T.d_tok);
            dev_free(T.d_bits);
            dev_free(T.d_rank);
            dev_free(T.d_tok0);
        }
        dev_free(idx->d_steps);
    }
    delete idx;
}

cb_status cb_plan_create(cb_index* idx, int32_t Q_max, int32_t K, int32_t d, cb_dtype dtype, cb_plan** out) {
    clear_error();
    if (!out) {
        set_error("cb_plan_create: out is NULL");
        return CB_EINVAL;
    }
    *out = nullptr;
    if (!idx || Q_max < 1 || K < 1 || d < 8 || (d % 8) != 0 || (dtype != CB_F32 && dtype != CB_BF16)) {
        set_error("cb_plan_create: need an index, Q_max >= 1, K >= 1, d a positive multiple of 8, dtype F32/BF16");
        return CB_EINVAL;
    }
    if (idx->device < 0) {
        set_error("cb_plan_create: index was built host-only (device -1)");
        return CB_EINVAL;
    }
    if (K > kMaxKRadix) {
        set_error("cb_plan_create: K > " + std::to_string(kMaxKRadix) + " is not supported");
        return CB_ECAPACITY;
    }
    if (d > 16384) {
        set_error("cb_plan_create: d > 16384 is not supported (hidden vector staged in LDS)");
        return CB_ECAPACITY;
    }
    int32_t Smax = 1;
    for (const auto& T : idx->steps) Smax = std::max(Smax, T.S);
    const int32_t Kc = std::min(K, Smax);
    DeviceGuard g(idx->device);
    if (!g.ok) {
        set_error("cb_plan_create: cannot select the index's device");
        return CB_EHIP;
    }
    cb_plan* p = new (std::nothrow) cb_plan();
    if (!p) {
        set_error("cb_plan_create: host allocation failed");
        return CB_ENOMEM;
    }
    p->idx = idx;
    p->device = idx->device;
    p->Q_max = Q_max;
    p->K = K;
    p->d = d;
    p->dtype = dtype;
    p->Kc_max = Kc;
    p->forced.assign((size_t)idx->L, CB_PATH_AUTO);
    p->tuned.assign((size_t)idx->L, 0);
    p->query_nt.assign((size_t)idx->L, 0);
    p->gemm_rows.assign((size_t)idx->L, 0);
    p->radix_pre.assign((size_t)idx->L, 0);
    p->radix_tm.assign((size_t)idx->L, 0);
    p->split_min.assign((size_t)idx->L, 0);
    p->sparse_form.assign((size_t)idx->L, 0);
    p->query_split.assign((size_t)idx->L, 0);
    p->tune_dense_us.assign((size_t)idx->L, -1.f);
    p->tune_sparse_us.assign((size_t)idx->L, -1.f);
    p->select.assign((size_t)idx->L, CB_SELECT_AUTO);
    p->tuned_select.assign((size_t)idx->L, 0);
    const size_t R = (size_t)Q_max * K;
    cb_status st = dev_alloc(&p->keys, R * Kc, "candidate keys");
    if (st == CB_OK) st = dev_alloc(&p->side, R * Kc, "candidate side information");
    if (st == CB_OK) {
        int S_max = 1;
        for (int t = 0; t < idx->L; ++t) S_max = std::max(S_max, idx->steps[(size_t)t].S);
        st = dev_alloc(&p->qz, (size_t)Q_max * (size_t)query_scores_floats(K, S_max), "per-query score hand-off");
    }
    if (st == CB_OK) st = dev_alloc(&p->qcnt, (size_t)Q_max, "per-query arrival counts");
    if (st == CB_OK) st = dev_alloc(&p->lse_row, R, "row log-sum-exp");
    if (st == CB_OK && hipMemset(p->qcnt, 0, (size_t)Q_max * 4) != hipSuccess) {
        (void)hipGetLastError();
        set_error("cb_plan_create: clearing the arrival counts failed");
        st = CB_EHIP;
    }
    if (st == CB_OK) st = dev_alloc(&p->Z, R * (size_t)idx->V, "full-codebook scores");
    if (st == CB_OK && dtype == CB_BF16) st = dev_alloc(&p->Zp, split_scores_floats(idx->V), "partial scores");
    if (st == CB_OK) st = dev_alloc(&p->live, R, "live beams");
    if (st == CB_OK) st = dev_alloc(&p->ci_of, R, "compact index");
    if (st == CB_OK) st = dev_alloc(&p->n_live, 1, "live count");
    for (int i = 0; i < 2 && st == CB_OK; ++i) {
        st = dev_alloc(&p->s[i], R * d, "state");
        if (st == CB_OK) st = dev_alloc(&p->rows[i], R, "rows");
        if (st == CB_OK) st = dev_alloc(&p->acc[i], R, "acc");
    }
    if (st == CB_OK) {
        unsigned char* h = nullptr;
        st = dev_alloc(&h, R * d * dtype_size(dtype), "hidden");
        p->h = h;
    }
    if (st == CB_OK) st = dev_alloc(&p->hist_tok, R * idx->L, "token history");
    if (st == CB_OK) st = dev_alloc(&p->hist_par, R * idx->L, "parent history");
    if (st == CB_OK) st = dev_alloc(&p->scratch_rows, R, "scratch");
    if (st == CB_OK) st = dev_alloc(&p->scratch_logp, R, "scratch");
    if (st == CB_OK) st = dev_alloc(&p->scratch_tok, R, "scratch");
    if (st == CB_OK) st = dev_alloc(&p->scratch_par, R, "scratch");
    bool need_radix = false;
    for (int t = 0; t < idx->L; ++t) need_radix = need_radix || !lds_select_ok(p, t);
    if (st == CB_OK && need_radix) st = wide_alloc(p);
    if (st != CB_OK) {
        cb_plan_destroy(p);
        return st;
    }
    *out = p;
    return CB_OK;
}

cb_status cb_set_path(cb_plan* p, int32_t t, cb_path path) {
    clear_error();
    if (!p || t < 0 || t >= p->idx->L || path < CB_PATH_AUTO || path > CB_PATH_SPARSE_SPLIT) {
        set_error("cb_set_path: bad plan, step or path");
        return CB_EINVAL;
    }
    if (path == CB_PATH_SPARSE_SPLIT) {
        DeviceGuard g(p->device);
        cb_status st = wide_alloc(p);
        if (st != CB_OK) return st;
    }
    if (path == CB_PATH_DENSE && !dense_available(p)) {
        set_error("cb_set_path: the dense path needs d to be a multiple of 64 for bf16");
        return CB_EUNSUPPORTED;
    }
    if (p->mode != CB_MODE_FILTER_FIRST && path != CB_PATH_AUTO && path != CB_PATH_DENSE) {
        set_error("cb_set_path: the score-first and unconstrained variants take the dense path only");
        return CB_EUNSUPPORTED;
    }
    p->forced[(size_t)t] = path;
    return CB_OK;
}

cb_status cb_set_mode(cb_plan* p, cb_mode mode) {
    clear_error();
    if (!p || mode < CB_MODE_FILTER_FIRST || mode > CB_MODE_UNCONSTRAINED) {
        set_error("cb_set_mode: bad plan or mode");
        return CB_EINVAL;
    }
    if (mode != CB_MODE_FILTER_FIRST) {
        const cb_index* idx = p->idx;
        if (!dense_available(p)) {
            set_error("cb_set_mode: the variant needs the dense path (bf16: d a multiple of 64)");
            return CB_EUNSUPPORTED;
        }
        for (int t = 0; t < idx->L; ++t)
            if (p->forced[(size_t)t] != CB_PATH_AUTO && p->forced[(size_t)t] != CB_PATH_DENSE) {
                set_error("cb_set_mode: a step is forced to a sparse path");
                return CB_EUNSUPPORTED;
            }
        // each step takes the LDS selection where it holds the variant, else
        // the radix selection (beam widths above 64, rows too wide for the
        // LDS, every token of a codebook above 4,096 tokens as candidates)
        const int32_t old = p->mode;
        p->mode = mode;
        bool radix = false;
        for (int t = 0; t < idx->L; ++t) {
            if (p->select[(size_t)t] == CB_SELECT_LDS && !variant_lds_ok(p, t)) {
                p->mode = old;
                set_error("cb_set_mode: a step is forced to the LDS selection, which cannot hold the variant");
                return CB_EUNSUPPORTED;
            }
            radix = radix || resolve_select(p, t) == CB_SELECT_RADIX;
        }
        if (radix) {
            DeviceGuard g(p->idx->device);
            const cb_status st = wide_alloc(p);
            if (st != CB_OK) {
                p->mode = old;
                return st;
            }
        }
        return CB_OK;
    }
    p->mode = mode;
    return CB_OK;
}

cb_status cb_get_mode(const cb_plan* p, cb_mode* mode) {
    clear_error();
    if (!p || !mode) {
        set_error("cb_get_mode: plan or output is NULL");
        return CB_EINVAL;
    }
    *mode = (cb_mode)p->mode;
    return CB_OK;
}

cb_status cb_set_select(cb_plan* p, int32_t t, cb_select sel) {
    clear_error();
    if (!p || t < 0 || t >= p->idx->L || sel < CB_SELECT_AUTO || sel > CB_SELECT_RADIX) {
        set_error("cb_set_select: bad plan, step or selection");
        return CB_EINVAL;
    }
    if (sel == CB_SELECT_LDS && !(p->mode == CB_MODE_FILTER_FIRST ? lds_select_ok(p, t) : variant_lds_ok(p, t))) {
        set_error("cb_set_select: the LDS selection holds K <= 64 and rows that fit its LDS (unconstrained: "
                  "also a bf16 plan with V <= 4096, V a multiple of 4)");
        return CB_ECAPACITY;
    }
    if (sel == CB_SELECT_RADIX) {
        DeviceGuard g(p->idx->device);
        cb_status st = wide_alloc(p);
        if (st != CB_OK) return st;
    }
    p->select[(size_t)t] = sel;
    return CB_OK;
}

cb_status cb_get_select(const cb_plan* p, int32_t t, cb_select* sel) {
    clear_error();
    if (!p || !sel || t < 0 || t >= p->idx->L) {
        set_error("cb_get_select: bad plan, step or output");
        return CB_EINVAL;
    }
    *sel = (cb_select)resolve_select(p, t);
    return CB_OK;
}

cb_status cb_set_step_option(cb_plan* p, int32_t t, cb_step_option o, int32_t value) {
    clear_error();
    if (!p || t < 0 || t >= p->idx->L) {
        set_error("cb_set_step_option: bad plan or step");
        return CB_EINVAL;
    }
    const cb::StepTable& T = p->idx->steps[(size_t)t];
    switch (o) {
        case CB_OPT_STEP_THREADS: {
            if (value != 0 && !query_threads_ok(value)) {
                set_error("cb_set_step_option: step threads must be 0, 256, 512 or 1024");
                return CB_EINVAL;
            }
            const int Kc = std::min(p->K, std::max(T.S, 1));
            if (query_lds_bytes(T.S, p->K, Kc, p->d, value) > (size_t)kMaxLds) {
                set_error("cb_set_step_option: the step's LDS does not fit that workgroup size");
                return CB_ECAPACITY;
            }
            p->query_nt[(size_t)t] = value;
            return CB_OK;
        }
        case CB_OPT_SPLIT_ROWS:
            if (value < 0 || value > 64) break;
            p->split_min[(size_t)t] = value;
            return CB_OK;
        case CB_OPT_SPARSE_FORM:
            if (value < 0 || value > 1) break;
            if (value == 1 && expand_lds_bytes(T.S, p->d, false) > (size_t)kMaxLds) {
                set_error("cb_set_step_option: the per-beam expansion of this step does not fit the LDS");
                return CB_ECAPACITY;
            }
            p->sparse_form[(size_t)t] = value;
            return CB_OK;
        case CB_OPT_DENSE_ROWS:
            if (value < 0 || value > 2) break;
            if (value == 2 && !gemm_full_ok(p->dtype)) {
                set_error("cb_set_step_option: the product over every slot needs a bf16 plan");
                return CB_EUNSUPPORTED;
            }
            p->gemm_rows[(size_t)t] = value;
            return CB_OK;
        case CB_OPT_RADIX_PREPASS:
            if (value < 0 || value > 2) break;
            p->radix_pre[(size_t)t] = value;
            return CB_OK;
        case CB_OPT_QUERY_SPLIT:
            if (value != 0 && value != 1 && value != 2 && value != 4 && value != 8) break;
            p->query_split[(size_t)t] = value;
            return CB_OK;
        case CB_OPT_TOKEN_MAJOR: {
            if (value < 0 || value > 2) break;
            if (value == 2) {
                if (p->d > kQueryMaxD) {
                    set_error("cb_set_step_option: scores by token hold W_t rows of at most 2048 elements");
                    return CB_EINVAL;
                }
                DeviceGuard g(p->idx->device);
                cb_status st = wide_alloc(p);
                if (st == CB_OK) st = tok_alloc(p);
                if (st != CB_OK) return st;
            }
            p->radix_tm[(size_t)t] = value;
            return CB_OK;
        }
    }
    set_error("cb_set_step_option: unknown option or value out of range");
    return CB_EINVAL;
}

cb_status cb_get_step_option(const cb_plan* p, int32_t t, cb_step_option o, int32_t* value) {
    clear_error();
    if (!p || !value || t < 0 || t >= p->idx->L) {
        set_error("cb_get_step_option: bad plan, step or output");
        return CB_EINVAL;
    }
    switch (o) {
        case CB_OPT_STEP_THREADS: {
            const int32_t v = p->query_nt[(size_t)t];
            *value = query_threads_ok(v) ? v : query_threads(p->K);
            return CB_OK;
        }
        case CB_OPT_SPLIT_ROWS: *value = p->split_min[(size_t)t] > 0 ? p->split_min[(size_t)t] : kPreMin; return CB_OK;
        case CB_OPT_SPARSE_FORM: *value = (p->d > kQueryMaxD || p->sparse_form[(size_t)t] == 1) ? 1 : 0; return CB_OK;
        case CB_OPT_DENSE_ROWS: *value = gemm_full(p, t) ? 2 : 1; return CB_OK;
        case CB_OPT_RADIX_PREPASS: *value = p->radix_pre[(size_t)t] == 1 ? 1 : 2; return CB_OK;
        case CB_OPT_QUERY_SPLIT: *value = p->query_split[(size_t)t] > 1 ? p->query_split[(size_t)t] : 1; return CB_OK;
        case CB_OPT_TOKEN_MAJOR: *value = p->radix_tm[(size_t)t] == 2 ? 2 : 1; return CB_OK;
    }
    set_error("cb_get_step_option: unknown option");
    return CB_EINVAL;
}

cb_status cb_get_path(const cb_plan* p, int32_t t, cb_path* path) {
    clear_error();
    if (!p || !path || t < 0 || t >= p->idx->L) {
        set_error("cb_get_path: bad plan, step or output");
        return CB_EINVAL;
    }
    *path = (cb_path)resolve_path(p, t);
    return CB_OK;
}

cb_status cb_step(cb_plan* p, int32_t t, int32_t Q, const void* hidden, const void* W_t, const int32_t* beam_rows,
                  const float* acc_logp, int32_t* out_tokens, int32_t* out_parents, int32_t* out_rows,
                  float* out_logp, void* stream) {
    clear_error();
    cb_status st = check_plan(p, Q, "cb_step");
    if (st != CB_OK) return st;
    if (t < 0 || t >= p->idx->L) {
        set_error("cb_step: t out of [0, L)");
        return CB_EINVAL;
    }
    if (Q == 0) return CB_OK;
    // hidden vectors and W_t rows are read 16 bytes at a time; the per-slot arrays element-wise
    const void* vec[] = {hidden, W_t};
    const void* ptrs[] = {beam_rows, acc_logp, out_tokens, out_parents, out_rows, out_logp};
    for (const void* x : vec)
        if (!x || !aligned16(x)) {
            set_error("cb_step: hidden or W_t is NULL or not 16-byte aligned");
            return CB_EINVAL;
        }
    for (const void* x : ptrs)
        if (!x || !aligned4(x)) {
            set_error("cb_step: a per-slot array is NULL or not 4-byte aligned");
            return CB_EINVAL;
        }
    void* const outs[4] = {out_tokens, out_parents, out_rows, out_logp};
    if (step_outputs_alias((size_t)Q * p->K, (size_t)p->d, (size_t)p->idx->V, dtype_size(p->dtype), hidden, W_t,
                           beam_rows, acc_logp, outs)) {
        set_error("cb_step: an output array overlaps an input or another output");
        return CB_EINVAL;
    }
    DeviceGuard g(p->idx->device);
    return run_step(p, t, Q, resolve_path(p, t), resolve_select(p, t), hidden, W_t, beam_rows, acc_logp, out_tokens,
                    out_parents, out_rows, out_logp, (hipStream_t)stream);
}

static cb_status decode_impl(cb_plan* p, int32_t Q, const float* q, const float* P, const void* W, int32_t* out_seqs,
                             float* out_logp, int32_t* out_rows, void* tr_h, int32_t* tr_rows, float* tr_acc,
                             hipStream_t s, int reps) {
    const cb_index* idx = p->idx;
    const int L = idx->L, K = p->K, d = p->d, V = idx->V;
    const int R = Q * K;
    const size_t es = dtype_size(p->dtype);
    hipError_t e = launch_decode_init(Q, K, d, p->dtype, q, p->s[0], p->h, p->rows[0], p->acc[0], s);
    if (e != hipSuccess) return hip_fail("cb_decode: init", e);
    int cur = 0;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    if (reps > 0) {
        if ((e = hipEventCreate(&ev0)) != hipSuccess || (e = hipEventCreate(&ev1)) != hipSuccess)
            return hip_fail("cb_tune: events", e);
    }
    // persistent tail: the trailing steps on the fused per-query sparse step
    // with LDS selection run in one launch (untraced, untuned decodes only);
    // a step in the per-beam form ends the run, since the tail runs the
    // per-query form and must give the same bits as the step-by-step decode
    int t_fuse = L;
    const bool fuse = p->fuse_mode == 1 || (p->fuse_mode == -1 && p->fuse_tuned);
    if (fuse && reps == 0 && !tr_h && !tr_rows && !tr_acc && idx->d_steps && d <= kQueryMaxD) {
        while (t_fuse > 0 && resolve_path(p, t_fuse - 1) == CB_PATH_SPARSE &&
               resolve_select(p, t_fuse - 1) == CB_SELECT_LDS && opt(p->sparse_form, t_fuse - 1) != 1)
            --t_fuse;
        if (L - t_fuse < 2) t_fuse = L;
    }
    cb_status st = CB_OK;
    for (int t = 0; t < t_fuse && st == CB_OK; ++t) {
        const void* Wt = static_cast<const unsigned char*>(W) + (size_t)t * V * d * es;
        if (tr_h) {
            e = hipMemcpyAsync(static_cast<unsigned char*>(tr_h) + (size_t)t * R * d * es, p->h, (size_t)R * d * es,
                               hipMemcpyDeviceToDevice, s);
            if (e == hipSuccess && tr_rows)
                e = hipMemcpyAsync(tr_rows + (size_t)t * R, p->rows[cur], (size_t)R * 4, hipMemcpyDeviceToDevice, s);
            if (e == hipSuccess && tr_acc)
                e = hipMemcpyAsync(tr_acc + (size_t)t * R, p->acc[cur], (size_t)R * 4, hipMemcpyDeviceToDevice, s);
            if (e != hipSuccess) {
                st = hip_fail("cb_decode: trace copy", e);
                break;
            }
        } else if (tr_rows || tr_acc) {
            if (tr_rows) e = hipMemcpyAsync(tr_rows + (size_t)t * R, p->rows[cur], (size_t)R * 4, hipMemcpyDeviceToDevice, s);
            if (e == hipSuccess && tr_acc)
                e = hipMemcpyAsync(tr_acc + (size_t)t * R, p->acc[cur], (size_t)R * 4, hipMemcpyDeviceToDevice, s);
            if (e != hipSuccess) {
                st = hip_fail("cb_decode: trace copy", e);
                break;
            }
        }
        const bool path_free = p->forced[(size_t)t] == CB_PATH_AUTO;
        const bool sel_free = p->select[(size_t)t] == CB_SELECT_AUTO;
        if (reps > 0 && p->mode == CB_MODE_FILTER_FIRST && (path_free || sel_free)) {
            // time every allowed (scoring path, selection) pair on this step's inputs, outputs to scratch
            float best_us[2] = {-1.f, -1.f};  // dense, sparse (either variant): best over the selections
            float best = -1.f;
            int32_t best_path = 0, best_sel = 0, best_nt = 0, best_rows = 0, best_pre = 0, best_min = 0, best_form = 0,
                    best_split = 0, best_tm = 0;
            const int32_t paths[3] = {CB_PATH_DENSE, CB_PATH_SPARSE, CB_PATH_SPARSE_SPLIT};
            const int32_t sels[2] = {CB_SELECT_LDS, CB_SELECT_RADIX};
            const cb::StepTable& T = idx->steps[(size_t)t];
            // the split variant scores rows apart (it differs from plain sparse on any step with multi-token rows)
            const bool has_wide = T.store == CB_STORE_BITMAP || T.S > 1;
            for (int k = 0; k < 3 && st == CB_OK; ++k) {
                if (!path_free && paths[k] != resolve_path(p, t)) continue;
                if (paths[k] == CB_PATH_DENSE && !dense_available(p)) continue;
                for (int m = 0; m < 2 && st == CB_OK; ++m) {
                    if (!sel_free && sels[m] != p->select[(size_t)t]) continue;
                    if (sels[m] == CB_SELECT_LDS && !lds_select_ok(p, t)) continue;
                    if (paths[k] == CB_PATH_SPARSE_SPLIT && (sels[m] != CB_SELECT_LDS || !has_wide)) continue;
                    if ((paths[k] == CB_PATH_SPARSE_SPLIT || sels[m] == CB_SELECT_RADIX) && wide_alloc(p) != CB_OK) {
                        (void)hipGetLastError();
                        clear_error();
                        continue;
                    }
                    // variants with the same results: the per-query sparse step at its default
                    // workgroup size and at 256 threads (a step of few multi-token rows starts
                    // faster on the smaller); the full-codebook product over the live beams or
                    // over every slot (no live list)
                    const bool per_query = paths[k] != CB_PATH_DENSE && sels[m] == CB_SELECT_LDS && p->d <= kQueryMaxD;
                    const bool rows_var = paths[k] == CB_PATH_DENSE && gemm_full_ok(p->dtype);
                    // the radix selection with and without its one-token pre-pass (sparse scoring)
                    const bool pre_var = paths[k] != CB_PATH_DENSE && sels[m] == CB_SELECT_RADIX;
                    // the split path scoring apart the rows above 16 tokens, or every multi-token row
                    const bool split_var = paths[k] == CB_PATH_SPARSE_SPLIT && per_query;
                    // the plain sparse path also in its per-beam form (expansion over the whole
                    // GPU, then the per-query merge)
                    const bool form_var = paths[k] == CB_PATH_SPARSE && per_query &&
                                          expand_lds_bytes(T.S, p->d, false) <= (size_t)kMaxLds;
                    const int nts[4] = {0, 256, 0, 256};
                    const int mins[4] = {kPreMin, kPreMin, 1, 1};
                    // and the plain sparse path with two, four and eight workgroups per query
                    const bool qsplit_var = paths[k] == CB_PATH_SPARSE && per_query;
                    // and the radix selection's sparse scoring by token (with the pre-pass)
                    bool tm_var = pre_var && p->d <= kQueryMaxD;
                    if (tm_var && tok_alloc(p) != CB_OK) {
                        (void)hipGetLastError();
                        clear_error();
                        tm_var = false;
                    }
                    const int nv0 = split_var ? 4 : per_query || rows_var || pre_var ? 2 : 1;
                    const int nv1 = nv0 + (form_var ? 1 : 0);
                    const int nv2 = nv1 + (qsplit_var ? 3 : 0);
                    const int nv = nv2 + (tm_var ? 1 : 0);
                    for (int v = 0; v < nv && st == CB_OK; ++v) {
                        const bool beam_form = form_var && v == nv0;
                        const bool by_token = tm_var && v == nv2;
                        const int qs = v >= nv1 && v < nv2 ? 2 << (v - nv1) : 0;
                        p->sparse_form[(size_t)t] = beam_form ? 1 : 0;
                        p->query_split[(size_t)t] = qs;
                        p->query_nt[(size_t)t] = per_query && !beam_form && v < nv0 ? nts[v] : 0;
                        p->split_min[(size_t)t] = split_var ? mins[v] : 0;
                        p->gemm_rows[(size_t)t] = rows_var ? 1 + v : 0;
                        p->radix_pre[(size_t)t] = by_token ? 2 : pre_var && !beam_form ? 1 + v : 0;
                        p->radix_tm[(size_t)t] = by_token ? 2 : 0;
                        st = run_step(p, t, Q, paths[k], sels[m], p->h, Wt, p->rows[cur], p->acc[cur],
                                      p->scratch_tok, p->scratch_par, p->scratch_rows, p->scratch_logp, s);
                        if (st != CB_OK) break;
                        (void)hipEventRecord(ev0, s);
                        for (int r = 0; r < reps && st == CB_OK; ++r)
                            st = run_step(p, t, Q, paths[k], sels[m], p->h, Wt, p->rows[cur], p->acc[cur],
                                          p->scratch_tok, p->scratch_par, p->scratch_rows, p->scratch_logp, s);
                        (void)hipEventRecord(ev1, s);
                        if ((e = hipEventSynchronize(ev1)) != hipSuccess) {
                            st = hip_fail("cb_tune: synchronise", e);
                            break;
                        }
                        float ms = 0.f;
                        (void)hipEventElapsedTime(&ms, ev0, ev1);
                        const float us = ms * 1000.f / (float)reps;
                        const int slot = paths[k] == CB_PATH_DENSE ? 0 : 1;
                        if (best_us[slot] < 0.f || us < best_us[slot]) best_us[slot] = us;
                        if (best < 0.f || us < best) {
                            best = us;
                            best_path = paths[k];
                            best_sel = sels[m];
                            best_nt = p->query_nt[(size_t)t];
                            best_rows = p->gemm_rows[(size_t)t];
                            best_pre = p->radix_pre[(size_t)t];
                            best_min = p->split_min[(size_t)t];
                            best_form = p->sparse_form[(size_t)t];
                            best_split = p->query_split[(size_t)t];
                            best_tm = p->radix_tm[(size_t)t];
                        }
                    }
                    p->radix_tm[(size_t)t] = 0;
                    p->query_nt[(size_t)t] = 0;
                    p->split_min[(size_t)t] = 0;
                    p->gemm_rows[(size_t)t] = 0;
                    p->radix_pre[(size_t)t] = 0;
                    p->sparse_form[(size_t)t] = 0;
                    p->query_split[(size_t)t] = 0;
                }
            }
            if (st != CB_OK) break;
            p->tune_dense_us[(size_t)t] = best_us[0];
            p->tune_sparse_us[(size_t)t] = best_us[1];
            if (best_path) p->tuned[(size_t)t] = best_path;
            if (best_sel) p->tuned_select[(size_t)t] = best_sel;
            p->query_nt[(size_t)t] = best_nt;
            p->gemm_rows[(size_t)t] = best_rows;
            p->radix_pre[(size_t)t] = best_pre;
            p->split_min[(size_t)t] = best_min;
            p->sparse_form[(size_t)t] = best_form;
            p->query_split[(size_t)t] = best_split;
            p->radix_tm[(size_t)t] = best_tm;
        }
        st = run_step(p, t, Q, resolve_path(p, t), resolve_select(p, t), p->h, Wt, p->rows[cur], p->acc[cur],
                      p->hist_tok + (size_t)t * R, p->hist_par + (size_t)t * R, p->rows[1 - cur], p->acc[1 - cur], s);
        if (st != CB_OK) break;
        if (t + 1 < L) {
            e = launch_hidden_update(R, K, d, p->dtype, p->s[cur], P + (size_t)t * V * d, p->hist_tok + (size_t)t * R,
                                     p->hist_par + (size_t)t * R, p->s[1 - cur], p->h, s);
            if (e != hipSuccess) st = hip_fail("cb_decode: hidden update", e);
        }
        cur = 1 - cur;
    }
    if (ev0) (void)hipEventDestroy(ev0);
    if (ev1) (void)hipEventDestroy(ev1);
    if (st != CB_OK) return st;
    if (t_fuse < L) {
        size_t lds = 0;
        for (int t = t_fuse; t < L; ++t) {
            const cb::StepTable& T = idx->steps[(size_t)t];
            lds = std::max(lds, tail_lds_bytes(T.S, K, std::min(K, std::max(T.S, 1)), d));
        }
        ProfMark m(p, s, t_fuse, CB_KERNEL_DECODE_TAIL, tail_threads(K), Q);
        uint64_t* clk = p->prof_on ? p->phase_clk : nullptr;
        e = launch_decode_tail(idx->d_steps, lds, t_fuse, L, Q, K, d, V, p->dtype, W, P, p->s[cur], p->s[1 - cur],
                               p->h, p->rows[cur], p->rows[1 - cur], p->acc[cur], p->acc[1 - cur], p->hist_tok,
                               p->hist_par, clk, s);
        m.done();
        if (clk) {
            p->phase_t0 = t_fuse;
            p->phase_Q = Q;
        }
        if (e != hipSuccess) return hip_fail("cb_decode: persistent steps", e);
        if ((L - t_fuse) & 1) cur = 1 - cur;
    }
    if (out_seqs) {
        e = launch_backtrace(R, K, L, p->hist_tok, p->hist_par, out_seqs, s);
        if (e != hipSuccess) return hip_fail("cb_decode: backtrace", e);
    }
    if (out_rows && (e = hipMemcpyAsync(out_rows, p->rows[cur], (size_t)R * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return hip_fail("cb_decode: output copy", e);
    if (out_logp && (e = hipMemcpyAsync(out_logp, p->acc[cur], (size_t)R * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return hip_fail("cb_decode: output copy", e);
    return CB_OK;
}

cb_status cb_set_decode_fusion(cb_plan* p, int32_t enable) {
    clear_error();
    if (!p || enable < -1 || enable > 1) {
        set_error("cb_set_decode_fusion: plan is NULL or enable not in {-1, 0, 1}");
        return CB_EINVAL;
    }
    p->fuse_mode = enable;
    return CB_OK;
}

cb_status cb_get_decode_fusion(const cb_plan* p, int32_t* enabled) {
    clear_error();
    if (!p || !enabled) {
        set_error("cb_get_decode_fusion: plan or output is NULL");
        return CB_EINVAL;
    }
    *enabled = (p->fuse_mode == 1 || (p->fuse_mode == -1 && p->fuse_tuned)) ? 1 : 0;
    return CB_OK;
}

cb_status cb_tune_decode_times(const cb_plan* p, float* stepwise_us, float* persistent_us) {
    clear_error();
    if (!p) {
        set_error("cb_tune_decode_times: plan is NULL");
        return CB_EINVAL;
    }
    if (stepwise_us) *stepwise_us = p->fuse_us[0];
    if (persistent_us) *persistent_us = p->fuse_us[1];
    return CB_OK;
}

cb_status cb_decode(cb_plan* p, int32_t Q, const float* q, const float* P, const void* W, int32_t* out_seqs,
                    float* out_logp, int32_t* out_rows, void* trace_hidden, int32_t* trace_rows, float* trace_acc,
                    void* stream) {
    clear_error();
    cb_status st = check_plan(p, Q, "cb_decode");
    if (st != CB_OK) return st;
    if (Q == 0) return CB_OK;
    if (!q || !W || (p->idx->L > 1 && !P) || !out_seqs || !out_logp || !out_rows) {
        set_error("cb_decode: q, W, out_* (and P when L > 1) must be device pointers");
        return CB_EINVAL;
    }
    const void* ptrs[] = {q, P, out_seqs, out_logp, out_rows, trace_hidden, trace_rows, trace_acc};
    if (!aligned16(W)) {
        set_error("cb_decode: W is not 16-byte aligned");
        return CB_EINVAL;
    }
    for (const void* x : ptrs)
        if (x && !aligned4(x)) {
            set_error("cb_decode: a device pointer is not 4-byte aligned");
            return CB_EINVAL;
        }
    DeviceGuard g(p->idx->device);
    return decode_impl(p, Q, q, P, W, out_seqs, out_logp, out_rows, trace_hidden, trace_rows, trace_acc,
                       (hipStream_t)stream, 0);
}

cb_status cb_tune(cb_plan* p, int32_t Q, const float* q, const float* P, const void* W, int32_t reps, void* stream) {
    clear_error();
    cb_status st = check_plan(p, Q, "cb_tune");
    if (st != CB_OK) return st;
    if (!q || !W || (p->idx->L > 1 && !P) || reps < 1 || Q < 1) {
        set_error("cb_tune: need q, W, P (L > 1), Q >= 1 and reps >= 1");
        return CB_EINVAL;
    }
    DeviceGuard g(p->idx->device);
    st = decode_impl(p, Q, q, P, W, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, (hipStream_t)stream, reps);
    if (st != CB_OK) return st;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("cb_tune: synchronise", e);
    // the persistent decode against one launch per step, on the chosen paths
    const hipStream_t s = (hipStream_t)stream;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    if ((e = hipEventCreate(&ev0)) != hipSuccess || (e = hipEventCreate(&ev1)) != hipSuccess) {
        if (ev0) (void)hipEventDestroy(ev0);
        return hip_fail("cb_tune: events", e);
    }
    const int32_t mode = p->fuse_mode;
    p->fuse_us[0] = p->fuse_us[1] = -1.f;
    for (int f = 0; f < 2 && st == CB_OK; ++f) {
        p->fuse_mode = f;
        st = decode_impl(p, Q, q, P, W, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, s, 0);  // warm
        if (st == CB_OK) (void)hipEventRecord(ev0, s);
        for (int r = 0; r < reps && st == CB_OK; ++r)
            st = decode_impl(p, Q, q, P, W, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, s, 0);
        if (st != CB_OK) break;
        (void)hipEventRecord(ev1, s);
        if ((e = hipEventSynchronize(ev1)) != hipSuccess) {
            st = hip_fail("cb_tune: synchronise", e);
            break;
        }
        float ms = 0.f;
        (void)hipEventElapsedTime(&ms, ev0, ev1);
        p->fuse_us[f] = ms * 1000.f / (float)reps;
    }
    p->fuse_mode = mode;
    (void)hipEventDestroy(ev0);
    (void)hipEventDestroy(ev1);
    if (st != CB_OK) return st;
    p->fuse_tuned = p->fuse_us[1] <= p->fuse_us[0];
    return CB_OK;
}

cb_status cb_tune_times(const cb_plan* p, int32_t t, float* dense_us, float* sparse_us) {
    clear_error();
    if (!p || t < 0 || t >= p->idx->L) {
        set_error("cb_tune_times: bad plan or step");
        return CB_EINVAL;
    }
    if (dense_us) *dense_us = p->tune_dense_us[(size_t)t];
    if (sparse_us) *sparse_us = p->tune_sparse_us[(size_t)t];
    return CB_OK;
}

cb_status cb_profile_start(cb_plan* p, int32_t capacity) {
    clear_error();
    if (!p || capacity < 1 || p->idx->device < 0) {
        set_error("cb_profile_start: need a device plan and capacity >= 1");
        return CB_EINVAL;
    }
    DeviceGuard g(p->idx->device);
    profile_release(p);
    p->prof_ev.assign((size_t)capacity * 2, nullptr);
    for (auto& ev : p->prof_ev) {
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) {
            profile_release(p);
            return hip_fail("cb_profile_start: events", e);
        }
    }
    p->prof_rec.reserve((size_t)capacity);
    p->prof_cap = capacity;
    cb_status st = dev_alloc(&p->phase_clk, (size_t)p->Q_max * p->idx->L * 2, "phase clock");
    if (st != CB_OK) {
        profile_release(p);
        return st;
    }
    p->phase_t0 = -1;
    p->phases.clear();
    p->prof_on = true;
    return CB_OK;
}

cb_status cb_profile_stop(cb_plan* p, cb_kernel_time* out, int32_t cap, int32_t* n) {
    clear_error();
    if (!p || !n) {
        set_error("cb_profile_stop: bad plan or output");
        return CB_EINVAL;
    }
    DeviceGuard g(p->idx->device);
    cb_status st = CB_OK;
    for (size_t i = 0; i < p->prof_rec.size(); ++i) {
        hipError_t e = hipEventSynchronize(p->prof_ev[i * 2 + 1]);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, p->prof_ev[i * 2], p->prof_ev[i * 2 + 1]);
        if (e != hipSuccess) {
            st = hip_fail("cb_profile_stop", e);
            break;
        }
        p->prof_rec[i].us = ms * 1000.f;
    }
    *n = (int32_t)p->prof_rec.size();
    if (out)
        for (int32_t i = 0; i < *n && i < cap; ++i) out[i] = p->prof_rec[(size_t)i];
    p->phases.clear();
    if (st == CB_OK && p->phase_t0 >= 0 && p->phase_clk) {
        const int L = p->idx->L, t0 = p->phase_t0, Q = p->phase_Q;
        std::vector<uint64_t> clk((size_t)Q * L * 2);
        int rate_khz = 0;
        hipError_t e = hipDeviceSynchronize();  // the decode may sit on any stream
        if (e == hipSuccess) e = hipMemcpy(clk.data(), p->phase_clk, clk.size() * 8, hipMemcpyDeviceToHost);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, p->idx->device);
        if (e != hipSuccess || rate_khz <= 0) {
            st = hip_fail("cb_profile_stop: phase clock", e == hipSuccess ? hipErrorUnknown : e);
        } else {
            const double us_per_tick = 1000.0 / rate_khz;
            for (int t = t0; t < L; ++t) {
                double sel = 0.0, upd = 0.0;
                for (int q = 0; q < Q; ++q) {
                    const uint64_t* c = clk.data() + ((size_t)q * L + t) * 2;
                    sel += (double)(int64_t)(c[1] - c[0]);
                    if (t + 1 < L) upd += (double)(int64_t)(c[2] - c[1]);
                }
                p->phases.push_back(cb_phase_time{t, (float)(sel / Q * us_per_tick), (float)(upd / Q * us_per_tick)});
            }
        }
    }
    profile_release(p);
    return st;
}

cb_status cb_profile_phases(const cb_plan* p, cb_phase_time* out, int32_t cap, int32_t* n) {
    clear_error();
    if (!p || !n) {
        set_error("cb_profile_phases: bad plan or output");
        return CB_EINVAL;
    }
    *n = (int32_t)p->phases.size();
    if (out)
        for (int32_t i = 0; i < *n && i < cap; ++i) out[i] = p->phases[(size_t)i];
    return CB_OK;
}

cb_status cb_wire_bytes(int32_t K, int32_t L, int64_t* bytes) {
    clear_error();
    if (!bytes || K < 1 || L < 1) {
        set_error("cb_wire_bytes: need K >= 1, L >= 1 and an output");
        return CB_EINVAL;
    }
    *bytes = (8 + 16 * (int64_t)K + 4 * (int64_t)K * L + 7) & ~int64_t(7);
    return CB_OK;
}

cb_status cb_wire_results(int32_t Q, int32_t K, int32_t L, const int32_t* seqs, const float* logp, double alpha,
                          void* out, int64_t stride, int64_t* out_bytes, void* stream) {
    clear_error();
    if (Q < 0 || K < 1 || K > kMaxKRadix || L < 1 || !std::isfinite(alpha)) {
        set_error("cb_wire_results: need Q >= 0, 1 <= K <= 1024, L >= 1 and a finite alpha");
        return CB_EINVAL;
    }
    const int64_t need = 8 + 16 * (int64_t)K + 4 * (int64_t)K * L;
    if (stride < need || stride % 8) {
        set_error("cb_wire_results: stride must be a multiple of 8 and at least " + std::to_string(need));
        return CB_EINVAL;
    }
    if (Q == 0) return CB_OK;
    if (!seqs || !logp || !out || !aligned4(seqs) || !aligned4(logp) ||
        (reinterpret_cast<uintptr_t>(out) & 7) || (out_bytes && (reinterpret_cast<uintptr_t>(out_bytes) & 7))) {
        set_error("cb_wire_results: seqs / logp must be 4-byte aligned, out / out_bytes 8-byte aligned, none NULL "
                  "(out_bytes may be NULL)");
        return CB_EINVAL;
    }
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + (uintptr_t)(stride * Q);
    auto overlaps = [&](const void* p, size_t n) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        return a < o1 && o0 < a + n;
    };
    const size_t R = (size_t)Q * K;
    if (overlaps(seqs, R * L * 4) || overlaps(logp, R * 4) || (out_bytes && overlaps(out_bytes, (size_t)Q * 8))) {
        set_error("cb_wire_results: out overlaps seqs, logp or out_bytes");
        return CB_EINVAL;
    }
    const double norm = std::pow(6.0 / (5.0 + (double)L), alpha);
    const hipError_t e = launch_wire(Q, K, L, seqs, logp, norm, out, stride, out_bytes, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("cb_wire_results", e);
    return CB_OK;
}

cb_status cb_floor_probe(int32_t blocks, int32_t threads, int32_t n, float* us, void* stream) {
    clear_error();
    if (blocks < 1 || blocks > (1 << 20) || threads < 64 || threads > 1024 || threads % 64 || n < 1 || n > 4096) {
        set_error("cb_floor_probe: need 1 <= blocks <= 2^20, threads a multiple of 64 in [64, 1024], 1 <= n <= 4096");
        return CB_EINVAL;
    }
    const hipStream_t s = (hipStream_t)stream;
    if (!us) {
        for (int i = 0; i < n; ++i) {
            hipError_t e = launch_empty(blocks, threads, s);
            if (e != hipSuccess) return hip_fail("cb_floor_probe", e);
        }
        return CB_OK;
    }
    std::vector<hipEvent_t> ev((size_t)n * 2, nullptr);
    cb_status st = CB_OK;
    hipError_t e = hipSuccess;
    for (auto& x : ev)
        if ((e = hipEventCreate(&x)) != hipSuccess) {
            st = hip_fail("cb_floor_probe: events", e);
            break;
        }
    for (int i = 0; i < n && st == CB_OK; ++i) {
        launch_events() = LaunchEvents{ev[(size_t)i * 2], ev[(size_t)i * 2 + 1]};
        e = launch_empty(blocks, threads, s);
        launch_events() = LaunchEvents{};
        if (e != hipSuccess) st = hip_fail("cb_floor_probe", e);
    }
    if (st == CB_OK && (e = hipEventSynchronize(ev[(size_t)n * 2 - 1])) != hipSuccess)
        st = hip_fail("cb_floor_probe: synchronise", e);
    if (st == CB_OK) {
        double sum = 0.0;
        for (int i = 0; i < n && st == CB_OK; ++i) {
            float ms = 0.f;
            if ((e = hipEventElapsedTime(&ms, ev[(size_t)i * 2], ev[(size_t)i * 2 + 1])) != hipSuccess)
                st = hip_fail("cb_floor_probe: elapsed", e);
            sum += ms;
        }
        float all = 0.f;
        if (st == CB_OK && (e = hipEventElapsedTime(&all, ev[0], ev[(size_t)n * 2 - 1])) != hipSuccess)
            st = hip_fail("cb_floor_probe: elapsed", e);
        us[0] = (float)(sum * 1000.0 / n);
        us[1] = all * 1000.f / (float)n;
    }
    for (auto x : ev)
        if (x) (void)hipEventDestroy(x);
    return st;
}

void cb_plan_destroy(cb_plan* p) {
    if (!p) return;
    DeviceGuard g(p->device);  // the index may already be freed
    profile_release(p);
    wide_release(p);
    dev_free(p->keys);
    dev_free(p->side);
    dev_free(p->qz);
    dev_free(p->qcnt);
    dev_free(p->lse_row);
    dev_free(p->Z);
    dev_free(p->Zp);
    dev_free(p->live);
    dev_free(p->ci_of);
    dev_free(p->n_live);
    for (int i = 0; i < 2; ++i) {
        dev_free(p->s[i]);
        dev_free(p->rows[i]);
        dev_free(p->acc[i]);
    }
    dev_free(p->h);
    dev_free(p->hist_tok);
    dev_free(p->hist_par);
    dev_free(p->scratch_rows);
    dev_free(p->scratch_logp);
    dev_free(p->scratch_tok);
    dev_free(p->scratch_par);
    delete p;
}

}  // extern "C"
