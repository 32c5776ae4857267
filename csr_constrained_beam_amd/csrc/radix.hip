// Radix-select path of one constrained beam-search step (gfx950, wave64):
// beam widths up to 1024 and rows of any width.
//
// The per-query selection of kernels.hip holds a query's best keys in one
// wavefront, which bounds K by 64.  For wider beams (FlashTrie's beam widths
// of 100 to 1000, sec. 4.2) every candidate of a query is written to HBM as
// its 64-bit key and the query's K-th largest key is found by radix select on
// the high bits: 12-bit digits counted across the whole GPU (LDS histograms
// per workgroup, added into the query's global histogram; the next kernel's
// workgroups each read the finished histogram and pick the digit), after
// which the survivors (keys >= the threshold) are sorted by one workgroup and
// emitted.  Keys are distinct
// within a query (parent, token), so the selection is exact and the order is
// the (score desc, parent asc, token asc) order of the key.  If more than
// kSurvCap keys still share the two digits (massive exact score ties), the
// sort workgroup finishes the radix select on its own, 8 bits a pass.
//
// A query's candidates are laid out slot by slot, each slot's in ascending
// token order, so a candidate's index within its query orders exactly as
// (parent asc, token asc).  The radix keys therefore carry [63:32] the
// order-preserving score bits and [31:0] the complement of that index (unique,
// and descending key order is the tie-break); the candidate's token, parent
// and next row (the edge position row_ptr[r] + j of its j-th valid token) sit
// in a parallel array written when it is scored, so the outputs need one load.
//
// Work is cut into chunks of kWCH consecutive valid tokens of one beam; a
// beam's log-sum-exp is combined from its chunks' (max, sum exp) pairs.
//
// k_wide_score also serves the per-query (LDS) sparse step: with wide_only it
// scores just the rows of more than wide_only tokens (and bitmap rows), spread
// over many workgroups, and the step kernel then reads their scores instead of
// computing them one wavefront or one workgroup per row.
//
// Kernels per step: k_wide_score (slot offsets, scores, chunk softmax
// partials), k_wide_keys (keys, first-digit histogram), k_wide_refine (first
// digit, second-digit histogram), k_wide_collect (digits, survivors),
// k_wide_sort (sort, outputs, next rows).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "cb_internal.h"
#include "device.h"

namespace cb {
namespace {

constexpr int kWCH = 64;
constexpr int kWThreads = 256;
constexpr int kRBits = 12;
constexpr int kRBins = 1 << kRBits;
constexpr int kSurvCap = 8192;   // survivors the sort workgroup holds
constexpr int kSurvCap1 = 2048;  // stop after the first digit only below this
constexpr int kSortThreads = 1024;

enum : int32_t { kSelPending = 0, kSelThreshold = 1, kSelUnresolved = 2, kSelAll = 3 };

// Workgroups of a histogram kernel that take part for a query of n keys: the
// base count, more (up to the G launched) where each would hold more than
// kHistKeys keys; the others leave at once.
constexpr int kHistKeys = 16384;
__device__ __forceinline__ int hist_blocks_used(int G, int Gb, int n) {
    return min(G, max(Gb, (n + kHistKeys - 1) / kHistKeys));
}

// Per query, written by the scoring kernel (n_cand, state) and by the collect
// kernel (the resolved selection) for the sort kernel.
struct WideSel {
    uint64_t prefix;  // decided high bits of the query's K-th largest key
    int32_t need;     // keys still to take among those sharing `prefix`
    int32_t state;    // kSelAll: no more candidates than K, all survive
    int32_t n_cand;   // candidates of the query
    int32_t pad;
};

// j-th valid token (ascending) of row r.
__device__ int nth_token(const StepDev& st, int32_t r, uint32_t e0, int j) {
    if (st.store == CB_STORE_CSR) return st.tok[e0 + j];
    const uint16_t* rk = st.rank + (int64_t)r * st.words;
    int lo = 0, hi = st.words;  // last word whose preceding count is <= j
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int)rk[mid] <= j) lo = mid; else hi = mid;
    }
    uint32_t x = st.bits[(int64_t)r * st.words + lo];
    for (int m = j - (int)rk[lo]; m > 0; --m) x &= x - 1u;
    return lo * 32 + __ffs(x) - 1;
}

// Slot whose chunks contain chunk c (offs[0] <= c < offs[K]).
__device__ __forceinline__ int slot_of_chunk(const int32_t* offs, int K, int c) {
    int lo = 0, hi = K;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= c) lo = mid; else hi = mid;
    }
    return lo;
}

// Candidate and chunk offsets of the query's K slots into co_s / ho_s [K+1]
// (exclusive prefix sums of the slots' valid-token counts and chunk counts).
// All threads call.
template <int NT>
__device__ void slot_offsets(const StepDev& st, int q, int K, const int32_t* __restrict__ beam_rows,
                             const float* __restrict__ acc, int wide_only, int32_t* co_s, int32_t* ho_s, int* red_i,
                             int unc_v = 0) {
    constexpr int PER = (kMaxKRadix + NT - 1) / NT;
    const int k0 = threadIdx.x * PER;
    int n[PER];
    int sc = 0, sh = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int k = k0 + u;
        int x = 0;
        if (k < K) {
            const int64_t b = (int64_t)q * K + k;
            const int32_t r = beam_rows[b];
            // a live beam's candidates: its row's valid tokens, or (no
            // constraint) every token of the codebook
            if (beam_live(st, r, acc[b])) x = unc_v ? unc_v : (int)(st.row_ptr[r + 1] - st.row_ptr[r]);
            // wide_only > 0: only the rows the per-query kernel reads scores for
            // (more than wide_only tokens, and every bitmap row)
            if (wide_only && st.store == CB_STORE_CSR && x <= wide_only) x = 0;
        }
        n[u] = x;
        sc += x;
        sh += (x + kWCH - 1) / kWCH;
    }
    int tc, th;
    int oc = block_exclusive_scan<NT>(sc, red_i, &tc);
    int oh = block_exclusive_scan<NT>(sh, red_i, &th);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int k = k0 + u;
        if (k < K) {
            co_s[k] = oc;
            ho_s[k] = oh;
        }
        oc += n[u];
        oh += (n[u] + kWCH - 1) / kWCH;
    }
    if (threadIdx.x == 0) {
        co_s[K] = tc;
        ho_s[K] = th;
    }
    __syncthreads();
}


// Digit (bin) holding the need-th largest key, from the LDS counts h of
// nbins digits (bin index = digit value).  pick[0] = digit, pick[1] = keys in
// higher bins, pick[2] = keys in the bin.  All threads call.
template <int NT>
__device__ void block_pick(const uint32_t* h, int nbins, int need, int* red_i, int* pick) {
    const int per = (nbins + NT - 1) / NT;
    const int top = nbins - 1 - (int)threadIdx.x * per;  // this thread's bins: top, top-1, ... (highest first)
    int s = 0;
    for (int i = 0; i < per; ++i)
        if (top - i >= 0) s += (int)h[top - i];
    int tot;
    int above = block_exclusive_scan<NT>(s, red_i, &tot);
    if (above < need && above + s >= need) {
        for (int i = 0; i < per; ++i) {
            const int c = (int)h[top - i];
            if (above + c >= need) {
                pick[0] = top - i;
                pick[1] = above;
                pick[2] = c;
                break;
            }
            above += c;
        }
    }
    __syncthreads();
}

// Selection of a query as far as its digit histograms decide it, recomputed
// by every workgroup that needs it (the histograms are complete when the
// kernel that reads them starts, so no workgroup waits for another).  Digits
// are resolved one after the other; after each, the survivors if we stopped
// there are the keys above the boundary bin plus the whole bin.
struct SelView {
    uint64_t prefix;  // decided high bits of the K-th largest key
    int need;         // keys still to take among those sharing `prefix`
    int state;
};

template <int NT>
__device__ SelView resolve_digits(const WideDev& w, int q, int K, int n_cand, int passes, uint32_t* hs, int* red_i,
                                  int* pick) {
    SelView v;
    v.prefix = 0;
    v.need = min(K, n_cand);
    v.state = n_cand <= K ? kSelAll : kSelPending;
    if (v.state == kSelAll) return v;
    const int kt = v.need;
    for (int p = 0; p < passes; ++p) {
        const uint4* src = reinterpret_cast<const uint4*>(w.hist + ((int64_t)q * 2 + p) * kRBins);
        uint4* dst = reinterpret_cast<uint4*>(hs);
        for (int i = threadIdx.x; i < kRBins / 4; i += NT) dst[i] = src[i];
        __syncthreads();
        block_pick<NT>(hs, kRBins, v.need, red_i, pick);
        v.need -= pick[1];
        v.prefix |= (uint64_t)pick[0] << (64 - (p + 1) * kRBits);
        const int surv = kt - v.need + pick[2];
        __syncthreads();  // pick and hs are reused
        if (surv <= (p == 0 ? kSurvCap1 : kSurvCap)) {
            v.state = kSelThreshold;
            return v;
        }
    }
    v.state = passes == 2 ? kSelUnresolved : kSelPending;
    return v;
}

// Start of a scoring pass over query q (every workgroup g of the query): the
// slot offsets into co_s / ho_s; the query's first workgroup also publishes
// them and resets the query's selection state for the kernels that follow.
__device__ void wide_prologue(const StepDev& st, int q, int g, int K, const int32_t* __restrict__ beam_rows,
                              const float* __restrict__ acc, int wide_only, const WideDev& w, int32_t* co_s,
                              int32_t* ho_s, int* red_i) {
    const int tid = threadIdx.x;
    slot_offsets<kWThreads>(st, q, K, beam_rows, acc, wide_only, co_s, ho_s, red_i, w.unc_v);
    if (g == 0 && wide_only) {
        int32_t* co = w.cand_off + (int64_t)q * (K + 1);
        for (int k = tid; k <= K; k += kWThreads) co[k] = co_s[k];
    } else if (g == 0) {
        int32_t* co = w.cand_off + (int64_t)q * (K + 1);
        int32_t* ho = w.chunk_off + (int64_t)q * (K + 1);
        for (int k = tid; k <= K; k += kWThreads) {
            co[k] = co_s[k];
            ho[k] = ho_s[k];
        }
        uint32_t* hq = w.hist + (int64_t)q * 2 * kRBins;
        for (int i = tid; i < 2 * kRBins; i += kWThreads) hq[i] = 0;
        if (tid == 0) {
            const int tc = co_s[K];
            WideSel* sel = reinterpret_cast<WideSel*>(w.sel) + q;
            sel->prefix = 0;
            sel->need = min(K, tc);
            sel->n_cand = tc;
            sel->pad = 0;
            sel->state = tc <= K ? kSelAll : kSelPending;
            w.surv_n[q] = 0;
        }
    }
}

// Scores of every candidate, one chunk per workgroup iteration: z (sparse
// gather-dot against the beam's hidden vector staged in LDS, or the
// full-codebook score of the column), stored as z's bits over the key's low
// half (parent, token), and the chunk's (max, sum exp).  Every workgroup
// derives the slot offsets itself; the query's first one also publishes them
// and resets the query's selection state for the kernels that follow.
// CH: hidden width in 512-element chunks held in registers by the scoring
// loop (1, 2 or 4: d <= 512 * CH), or 0 for any width (one chunk at a time).
template <typename DT, bool DENSE, int CH>
__global__ __launch_bounds__(kWThreads) void k_wide_score(StepDev st, int K, int d, const DT* __restrict__ hidden,
                                                          const DT* __restrict__ W, const float* __restrict__ Z,
                                                          const float* __restrict__ Zp, int64_t ldz,
                                                          const int32_t* __restrict__ n_live,
                                                          const int32_t* __restrict__ ci_of, int split_ok,
                                                          const int32_t* __restrict__ beam_rows,
                                                          const float* __restrict__ acc, int wide_only, WideDev w,
                                                          int G) {
    extern __shared__ __align__(16) float h_s[];  // [d], sparse scoring only
    __shared__ float z_s[kWCH];
    __shared__ uint16_t tok_s[kWCH];
    __shared__ int32_t co_s[kMaxKRadix + 1], ho_s[kMaxKRadix + 1];
    __shared__ int red_i[kWThreads / kWave];
    const int q = blockIdx.x / G, g = blockIdx.x % G, tid = threadIdx.x;
    if (w.use_done && w.done[q]) return;  // finished by the pre-pass (uniform over the workgroup)
    wide_prologue(st, q, g, K, beam_rows, acc, wide_only, w, co_s, ho_s, red_i);
    const int nch = ho_s[K];
    if constexpr (DENSE) {
        // full-codebook scores: one chunk per wavefront, each lane reading its
        // token's column of the score row (no staging, no workgroup barrier)
        const int split = split_ok ? gemm_split(*n_live, (int)ldz, d) : 1;
        const int lane = tid & (kWave - 1);
        constexpr int NWV = kWThreads / kWave;
        for (int c = g * NWV + tid / kWave; c < nch; c += G * NWV) {
            const int k = slot_of_chunk(ho_s, K, c);
            const int64_t b = (int64_t)q * K + k;
            int32_t r = 0;
            uint32_t e0 = 0;
            if (!w.unc_v) {  // without a constraint the tokens are the columns
                r = beam_rows[b];
                e0 = st.row_ptr[r];
            }
            const int j0 = (c - ho_s[k]) * kWCH;
            const int cnt = min(kWCH, co_s[k + 1] - co_s[k] - j0);
            int v = 0;
            float z = -INFINITY;
            if (lane < cnt) {
                v = w.unc_v ? j0 + lane : nth_token(st, r, e0, j0 + lane);
                if (split == 1) {
                    z = Z[b * ldz + v];
                } else {
                    const float* zb = Zp + (int64_t)ci_of[b] * ldz + v;
                    z = 0.f;
                    for (int x = 0; x < split; ++x) z += zb[(int64_t)x * kSplitRows * ldz];
                }
            }
            const float m = wave_max(z);
            const float sm = wave_sum(lane < cnt ? exp_sm(z - m) : 0.f);
            if (lane == 0) {
                float* p = w.cms + ((int64_t)q * w.chunk_cap + c) * 2;
                p[0] = m;
                p[1] = sm;
            }
            if (lane < cnt) {
                const uint32_t c_ix = (uint32_t)(co_s[k] + j0 + lane);
                const int64_t o = (int64_t)q * w.cap + c_ix;
                w.cand[o] = ((uint64_t)__float_as_uint(z) << 32) | (uint64_t)(0xFFFFFFFFu - c_ix);
                const uint32_t nxt = w.unc_v ? 0u : e0 + (uint32_t)(j0 + lane);
                w.info[o] = ((uint64_t)nxt << 32) | ((uint64_t)v << 16) | (uint64_t)k;
            }
        }
        return;
    }
    int staged = -1;
    for (int c = g; c < nch; c += G) {
        const int k = slot_of_chunk(ho_s, K, c);
        const int64_t b = (int64_t)q * K + k;
        const int32_t r = beam_rows[b];
        const uint32_t e0 = st.row_ptr[r];
        const int n = co_s[k + 1] - co_s[k];
        const int j0 = (c - ho_s[k]) * kWCH;
        const int cnt = min(kWCH, n - j0);
        if (tid < cnt) tok_s[tid] = (uint16_t)(w.unc_v ? j0 + tid : nth_token(st, r, e0, j0 + tid));
        if (staged != k && n > 1) {
            for (int i = tid; i < d; i += kWThreads) h_s[i] = to_f32(hidden[b * d + i]);
            staged = k;
        }
        __syncthreads();
        if (n == 1) {
            // one valid token: log-softmax 0 whatever the score (no reads)
            if (tid == 0) z_s[0] = 0.f;
        } else if constexpr (CH > 0) {
            // every W_t row chunk of 16 tokens per wave in flight at once (the
            // chunk's 64 tokens in one round trip at d <= 1024 bf16)
            block_scores_ch<DT, kWThreads, CH, 128>(h_s, W, d, tok_s, cnt, z_s);
        } else {
            block_scores<DT, kWThreads>(h_s, W, d, tok_s, cnt, z_s);
        }
        __syncthreads();
        if (tid < kWave) {
            const float z = tid < cnt ? z_s[tid] : -INFINITY;
            const float m = wave_max(z);
            const float s = wave_sum(tid < cnt ? exp_sm(z - m) : 0.f);
            if (tid == 0) {
                float* p = w.cms + ((int64_t)q * w.chunk_cap + c) * 2;
                p[0] = m;
                p[1] = s;
            }
            if (tid < cnt) {
                const uint32_t c_ix = (uint32_t)(co_s[k] + j0 + tid);
                const int64_t o = (int64_t)q * w.cap + c_ix;
                w.cand[o] = ((uint64_t)__float_as_uint(z) << 32) | (uint64_t)(0xFFFFFFFFu - c_ix);
                // next row: the edge position, or row 0 of the next table without a constraint
                const uint32_t nxt = w.unc_v ? 0u : e0 + (uint32_t)(j0 + tid);
                w.info[o] = ((uint64_t)nxt << 32) | ((uint64_t)tok_s[tid] << 16) | (uint64_t)k;
            }
        }
        __syncthreads();
    }
}

// Token-major scoring of a sparse step.  The per-chunk scoring above stages a
// beam's hidden vector and gathers one W_t row per candidate, so a token held
// by many beams has its row fetched once per beam.  Here the candidates are
// grouped by token (a counting sort: count, scan, scatter), and each token's
// row is read once into registers and dotted with the hidden vectors of the
// beams that hold it (2 KB each at d = 1024 bf16, hit in L2 across the beam's
// tokens).  The work is cut into units of up to kTmUnit entries of one token,
// so that a token held by every beam does not serialise one wavefront.
constexpr int kTmUnit = 16;

// Slot offsets (published as by k_wide_score), every candidate's token, next
// row and parent slot, and its rank among its token's candidates (one atomic
// on the token's count); the candidate of a one-token row has log-softmax 0
// whatever its score, so it is written at once (z = 0) and takes no rank.
__global__ __launch_bounds__(kWThreads) void k_tm_count(StepDev st, int K, const int32_t* __restrict__ beam_rows,
                                                        const float* __restrict__ acc, WideDev w, TokDev tk, int G) {
    __shared__ int32_t co_s[kMaxKRadix + 1], ho_s[kMaxKRadix + 1];
    __shared__ int red_i[kWThreads / kWave];
    const int q = blockIdx.x / G, g = blockIdx.x % G, tid = threadIdx.x;
    if (w.use_done && w.done[q]) return;  // uniform over the workgroup
    wide_prologue(st, q, g, K, beam_rows, acc, 0, w, co_s, ho_s, red_i);
    const int nch = ho_s[K];
    const int lane = tid & (kWave - 1);
    constexpr int NWV = kWThreads / kWave;
    for (int c = g * NWV + tid / kWave; c < nch; c += G * NWV) {
        const int k = slot_of_chunk(ho_s, K, c);
        const int32_t r = beam_rows[(int64_t)q * K + k];
        const uint32_t e0 = st.row_ptr[r];
        const int n = co_s[k + 1] - co_s[k];
        const int j0 = (c - ho_s[k]) * kWCH;
        if (lane < min(kWCH, n - j0)) {
            const int v = nth_token(st, r, e0, j0 + lane);
            const uint32_t c_ix = (uint32_t)(co_s[k] + j0 + lane);
            const int64_t o = (int64_t)q * w.cap + c_ix;
            w.info[o] = ((uint64_t)(e0 + (uint32_t)(j0 + lane)) << 32) | ((uint64_t)v << 16) | (uint64_t)k;
            if (n == 1) {
                w.cand[o] = (uint64_t)(0xFFFFFFFFu - c_ix);  // z = +0.0
                tk.rank[o] = -1;
            } else {
                tk.rank[o] = atomicAdd(&tk.count[v], 1);
            }
        }
    }
}

// Exclusive prefix sums of the per-token counts (first list entry of each
// token) and of their units; the unit table (token and entry count in .x,
// first entry in .y) and the number of units; the counts are cleared for the
// next step.  One workgroup; thread i takes the PER tokens from i * PER on,
// loaded 4 at a time, all loads in flight before any is used.
template <int PER>
__global__ __launch_bounds__(1024) void k_tm_scan(int V, TokDev tk) {
    __shared__ int red_i[1024 / kWave];
    const int v0 = (int)threadIdx.x * PER;
    int c[PER];
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
        if (v0 + i + 4 <= V) {
            const int4 x = *reinterpret_cast<const int4*>(tk.count + v0 + i);
            c[i] = x.x;
            c[i + 1] = x.y;
            c[i + 2] = x.z;
            c[i + 3] = x.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) c[i + e] = v0 + i + e < V ? tk.count[v0 + i + e] : 0;
        }
    }
    int se = 0, su = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        se += c[i];
        su += (c[i] + kTmUnit - 1) / kTmUnit;
    }
    int te, tu;
    int oe = block_exclusive_scan<1024>(se, red_i, &te);
    int ou = block_exclusive_scan<1024>(su, red_i, &tu);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int v = v0 + i;
        if (v < V) {
            tk.off[v] = oe;
            tk.count[v] = 0;
            for (int x = 0; x < c[i]; x += kTmUnit) tk.units[ou++] = make_int2(v | (min(kTmUnit, c[i] - x) << 16), oe + x);
            oe += c[i];
        }
    }
    if (threadIdx.x == 0) {
        tk.off[V] = te;
        *tk.n_units = tu;
    }
}

// Every candidate that takes a rank into its token's entries: entry
// off[v] + rank = (candidate, beam).
__global__ __launch_bounds__(kWThreads) void k_tm_scatter(int K, WideDev w, TokDev tk, int G) {
    const int q = blockIdx.x / G, g = blockIdx.x % G;
    if (w.use_done && w.done[q]) return;
    const int n = reinterpret_cast<const WideSel*>(w.sel)[q].n_cand;
    const int64_t base = (int64_t)q * w.cap;
    for (int i = g * kWThreads + (int)threadIdx.x; i < n; i += G * kWThreads) {
        const int rk = tk.rank[base + i];
        if (rk < 0) continue;
        const uint64_t inf = w.info[base + i];
        const int v = (int)((inf >> 16) & 0xFFFFu), k = (int)(inf & 0xFFFFu);
        tk.list[tk.off[v] + rk] = make_uint2((uint32_t)(base + i), (uint32_t)(q * K + k));
    }
}

// Scores by token: one wavefront per unit holds the token's W_t row in
// registers (lane l: elements 512 c + 8 l ... + 7), loads the unit's entries
// one per lane, and takes them eight at a time (their hidden rows all in
// flight), each a dot product with the entry's beam's hidden vector (fp32
// products and sums, the wavefront's butterfly last); the candidate's key
// half gets z's bits.
template <typename DT, int CH>
__global__ __launch_bounds__(kWThreads) void k_tm_score(int K, int d, const DT* __restrict__ hidden,
                                                        const DT* __restrict__ W, WideDev w, TokDev tk) {
    constexpr int NWV = kWThreads / kWave;
    constexpr int U = 8;
    static_assert(kTmUnit <= kWave, "a unit's entries are held one per lane");
    const int lane = threadIdx.x & (kWave - 1);
    const int nu = *tk.n_units;
    for (int u = blockIdx.x * NWV + (int)threadIdx.x / kWave; u < nu; u += gridDim.x * NWV) {
        const int2 un = tk.units[u];
        const int v = un.x & 0xFFFF, cnt = un.x >> 16, e0 = un.y;
        const uint2 mine = tk.list[e0 + min(lane, cnt - 1)];
        float wr[CH][8];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i = c * kWave * 8 + lane * 8;
            if (i < d) load8(W + (int64_t)v * d + i, wr[c]);
            else
#pragma unroll
                for (int x = 0; x < 8; ++x) wr[c][x] = 0.f;
        }
        for (int j = 0; j < cnt; j += U) {
            uint32_t ex[U], eb[U];
#pragma unroll
            for (int x = 0; x < U; ++x) {
                const int jj = min(j + x, cnt - 1);  // uniform over the wavefront
                ex[x] = (uint32_t)__builtin_amdgcn_readlane((int)mine.x, jj);
                eb[x] = (uint32_t)__builtin_amdgcn_readlane((int)mine.y, jj);
            }
            Raw8<DT> h[U][CH];
#pragma unroll
            for (int x = 0; x < U; ++x)
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const int i = c * kWave * 8 + lane * 8;
                    if (i < d) h[x][c].load(hidden + (int64_t)eb[x] * d + i);
                    else h[x][c].zero();
                }
#pragma unroll
            for (int x = 0; x < U; ++x) {
                float sv = 0.f;
#pragma unroll
                for (int c = 0; c < CH; ++c) sv = h[x][c].dot(wr[c], sv);
                const float z = wave_sum(sv);
                if (lane == 0 && j + x < cnt) {
                    const int64_t qc = (int64_t)(eb[x] / (uint32_t)K) * w.cap;
                    const uint32_t c_ix = (uint32_t)((int64_t)ex[x] - qc);
                    w.cand[ex[x]] = ((uint64_t)__float_as_uint(z) << 32) | (uint64_t)(0xFFFFFFFFu - c_ix);
                }
            }
        }
    }
}

// Chunk pairs (max z, sum exp(z - max)) of every chunk of candidates, one
// wavefront per chunk, from the key halves the token-major scoring wrote; the
// keys kernel then combines them into each beam's log-sum-exp as after the
// per-chunk scoring.
__global__ __launch_bounds__(kWThreads) void k_tm_pairs(int K, WideDev w, int G, int Gb) {
    __shared__ int32_t co_s[kMaxKRadix + 1], ho_s[kMaxKRadix + 1];
    const int q = blockIdx.x / G, g = blockIdx.x % G, tid = threadIdx.x;
    if (w.use_done && w.done[q]) return;
    const int GE = hist_blocks_used(G, Gb, reinterpret_cast<const WideSel*>(w.sel)[q].n_cand);
    if (g >= GE) return;  // uniform over the workgroup
    const int lane = tid & (kWave - 1);
    constexpr int NWV = kWThreads / kWave;
    const int32_t* co = w.cand_off + (int64_t)q * (K + 1);
    const int32_t* ho = w.chunk_off + (int64_t)q * (K + 1);
    for (int k = tid; k <= K; k += kWThreads) {
        co_s[k] = co[k];
        ho_s[k] = ho[k];
    }
    __syncthreads();
    const int nch = ho_s[K];
    const uint64_t* cq = w.cand + (int64_t)q * w.cap;
    for (int c = g * NWV + tid / kWave; c < nch; c += GE * NWV) {
        const int k = slot_of_chunk(ho_s, K, c);
        const int j0 = (c - ho_s[k]) * kWCH;
        const int cnt = min(kWCH, co_s[k + 1] - co_s[k] - j0);
        const float z = lane < cnt ? __uint_as_float((uint32_t)(cq[co_s[k] + j0 + lane] >> 32)) : -INFINITY;
        const float m = wave_max(z);
        const float sm = wave_sum(lane < cnt ? exp_sm(z - m) : 0.f);
        if (lane == 0) {
            float* p = w.cms + ((int64_t)q * w.chunk_cap + c) * 2;
            p[0] = m;
            p[1] = sm;
        }
    }
}

// Log-sum-exp of every live beam's whole score row, one workgroup of 256 per
// beam.  Thread tid keeps a running (max, sum of exps) over the columns
// tid + 256 i, taken eight columns at a time (summed over the k-slices, if
// any, in slice order) so that eight loads are in flight per thread; the 256
// pairs are then combined in thread order.  Score first takes its softmax over
// the whole codebook.
template <bool SPLIT>
__device__ __forceinline__ void row_lse_scan(const float* __restrict__ zb, int V, int split, int64_t sstride,
                                             int tid, float& m, float& sm) {
    constexpr int U = 8;
    for (int c0 = tid; c0 < V; c0 += 256 * U) {
        float z[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + 256 * u;
            z[u] = -INFINITY;
            if (c < V) z[u] = zb[c];
        }
        if (SPLIT) {
            for (int x = 1; x < split; ++x) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + 256 * u;
                    if (c < V) z[u] += zb[x * sstride + c];
                }
            }
        }
        float mx = z[0];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, z[u]);
        const float mn = fmaxf(m, mx);  // finite: column c0 < V is in range
        float s = sm * exp_sm(m - mn);
#pragma unroll
        for (int u = 0; u < U; ++u) s += exp_sm(z[u] - mn);  // columns past V add exp(-inf) = 0
        m = mn;
        sm = s;
    }
}

__global__ __launch_bounds__(256) void k_row_lse(StepDev st, int R, int V, int d, const float* __restrict__ Z,
                                                 const float* __restrict__ Zp, const int32_t* __restrict__ n_live,
                                                 const int32_t* __restrict__ ci_of, int split_ok,
                                                 const int32_t* __restrict__ beam_rows,
                                                 const float* __restrict__ acc, float* __restrict__ lse_row) {
    __shared__ float pm[256], ps[256];
    const int b = blockIdx.x, tid = threadIdx.x;
    if (!beam_live(st, beam_rows[b], acc[b])) {  // uniform over the workgroup
        if (tid == 0) lse_row[b] = -INFINITY;
        return;
    }
    const int split = split_ok ? gemm_split(*n_live, V, d) : 1;
    const float* zb = split == 1 ? Z + (int64_t)b * V : Zp + (int64_t)ci_of[b] * V;
    float m = -INFINITY, sm = 0.f;
    if (split == 1)
        row_lse_scan<false>(zb, V, 1, 0, tid, m, sm);
    else
        row_lse_scan<true>(zb, V, split, (int64_t)kSplitRows * V, tid, m, sm);
    pm[tid] = m;
    ps[tid] = sm;
    __syncthreads();
    if (tid < kWave) {
        // lane l combines the pairs l, l + 64, l + 128, l + 192, then the wave
        float M = pm[tid];
        for (int x = 1; x < 4; ++x) M = fmaxf(M, pm[tid + 64 * x]);
        float S = 0.f;
        for (int x = 0; x < 4; ++x) {
            const float mx = pm[tid + 64 * x];
            S += mx == -INFINITY ? 0.f : ps[tid + 64 * x] * exp_sm(mx - M);
        }
        const float MM = wave_max(M);
        S = wave_sum(M == -INFINITY ? 0.f : S * exp_sm(M - MM));
        if (tid == 0) lse_row[b] = MM + logf(S);
    }
}

// LDS histogram increment by the lanes in `on`, one atomic per distinct bin
// of the wavefront (keys of one chunk mostly share their top digit).  All
// lanes of the wavefront call.
__device__ __forceinline__ void wave_hist_add(uint32_t* hs, uint32_t bin, bool on) {
    uint64_t todo = __ballot(on);
    while (todo) {
        const int lead = __ffsll((unsigned long long)todo) - 1;
        const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, lead);
        const uint64_t same = __ballot(on && bin == lb);
        if ((int)(threadIdx.x & (kWave - 1)) == lead) atomicAdd(&hs[lb], (uint32_t)__popcll(same));
        todo &= ~same;
    }
}

// Running (max, sum of exps) over the chunk pairs x, x + 64, ... below end.
__device__ __forceinline__ void chunk_pairs(const float* __restrict__ cms, int x, int end, float& m, float& s) {
    for (; x < end; x += kWave) {
        const float cm = cms[2 * x], cs = cms[2 * x + 1];
        if (cm > m) {
            s = s * exp_sm(m - cm) + cs;
            m = cm;
        } else {
            s += cs * exp_sm(cm - m);
        }
    }
}

// Unconstrained decoding: each live beam's log-sum-exp over its candidates
// (the whole codebook row), combined once from its chunks' pairs, one
// wavefront per beam; dead beams (no chunks) get -inf.
__global__ __launch_bounds__(256) void k_chunk_lse(int Q, int K, WideDev w, float* __restrict__ lse_row) {
    const int lane = threadIdx.x & (kWave - 1);
    const int b = blockIdx.x * (256 / kWave) + (int)threadIdx.x / kWave;
    if (b >= Q * K) return;  // uniform over the wavefront
    const int q = b / K, k = b - q * K;
    if (w.use_done && w.done[q]) return;
    const int32_t* ho = w.chunk_off + (int64_t)q * (K + 1);
    const int h0 = ho[k], h1 = ho[k + 1];
    float m = -INFINITY, s = 0.f;
    chunk_pairs(w.cms + (int64_t)q * w.chunk_cap * 2, h0 + lane, h1, m, s);
    const float M = wave_max(m);
    const float S = wave_sum(m == -INFINITY ? 0.f : s * exp_sm(m - M));
    if (lane == 0) lse_row[b] = h1 > h0 ? M + logf(S) : -INFINITY;
}

// Keys of every candidate (one chunk per wavefront): the beam's log-sum-exp
// from its chunks, score = acc + (z - lse) in float32, and the histogram of
// the keys' top digit.
__global__ __launch_bounds__(kWThreads) void k_wide_keys(int K, const float* __restrict__ acc, WideDev w, int G,
                                                         int Gb) {
    __shared__ __align__(16) uint32_t hs[kRBins];
    __shared__ int32_t co_s[kMaxKRadix + 1], ho_s[kMaxKRadix + 1];
    const int q = blockIdx.x / G, g = blockIdx.x % G, tid = threadIdx.x;
    if (w.use_done && w.done[q]) return;
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    constexpr int NWV = kWThreads / kWave;
    const WideSel* sel = reinterpret_cast<const WideSel*>(w.sel) + q;
    const int GE = hist_blocks_used(G, Gb, sel->n_cand);
    if (g >= GE) return;  // uniform over the workgroup
    const bool pending = sel->state == kSelPending;  // uniform over the query's workgroups
    for (int i = tid; i < kRBins; i += kWThreads) hs[i] = 0;
    const int32_t* co = w.cand_off + (int64_t)q * (K + 1);
    const int32_t* ho = w.chunk_off + (int64_t)q * (K + 1);
    for (int k = tid; k <= K; k += kWThreads) {
        co_s[k] = co[k];
        ho_s[k] = ho[k];
    }
    __syncthreads();
    const int nch = ho_s[K];
    const float* cms = w.cms + (int64_t)q * w.chunk_cap * 2;
    uint64_t* cq = w.cand + (int64_t)q * w.cap;
    for (int c = g * NWV + wv; c < nch; c += GE * NWV) {
        const int k = slot_of_chunk(ho_s, K, c);
        // the softmax support: the candidates (their chunks' pairs), or the
        // per-beam value of the variants (the whole row)
        float lse;
        if (w.lse_row) {
            lse = w.lse_row[(int64_t)q * K + k];
        } else {
            float m = -INFINITY, s = 0.f;
            chunk_pairs(cms, ho_s[k] + lane, ho_s[k + 1], m, s);
            const float M = wave_max(m);
            lse = M + logf(wave_sum(m == -INFINITY ? 0.f : s * exp_sm(m - M)));
        }
        const float a = acc[(int64_t)q * K + k];
        const int j0 = (c - ho_s[k]) * kWCH;
        const int cnt = min(kWCH, co_s[k + 1] - co_s[k] - j0);
        uint64_t key = 0;
        if (lane < cnt) {
            uint64_t* p = cq + co_s[k] + j0 + lane;
            const uint64_t v = *p;
            const float z = __uint_as_float((uint32_t)(v >> 32));
            key = ((uint64_t)score_order_bits(a + (z - lse)) << 32) | (v & 0xFFFFFFFFull);
            *p = key;
        }
        if (pending) wave_hist_add(hs, (uint32_t)(key >> (64 - kRBits)), lane < cnt);
    }
    if (!pending) return;
    __syncthreads();
    uint32_t* h1 = w.hist + (int64_t)q * 2 * kRBins;
    for (int i = tid; i < kRBins; i += kWThreads)
        if (hs[i]) atomicAdd(&h1[i], hs[i]);
}

// Second digit, over the keys that share the first (queries the first digit
// left open).
__global__ __launch_bounds__(kWThreads) void k_wide_refine(int K, WideDev w, int G, int Gb) {
    __shared__ __align__(16) uint32_t hs[kRBins];
    __shared__ int red_i[kWThreads / kWave];
    __shared__ int pick[3];
    const int q = blockIdx.x / G, g = blockIdx.x % G, tid = threadIdx.x;
    if (w.use_done && w.done[q]) return;
    const WideSel* sel = reinterpret_cast<const WideSel*>(w.sel) + q;
    if (sel->state != kSelPending) return;  // uniform over the query's workgroups
    const int n = sel->n_cand;
    const int GE = hist_blocks_used(G, Gb, n);
    if (g >= GE) return;
    const SelView v = resolve_digits<kWThreads>(w, q, K, n, 1, hs, red_i, pick);
    if (v.state != kSelPending) return;
    for (int i = tid; i < kRBins; i += kWThreads) hs[i] = 0;
    __syncthreads();
    const uint64_t pre = v.prefix >> (64 - kRBits);
    const uint64_t* cq = w.cand + (int64_t)q * w.cap;
    // four keys per thread in flight
    const int stride = GE * kWThreads;
    for (int i0 = g * kWThreads + tid; i0 < n; i0 += 4 * stride) {
        uint64_t k4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * stride;
            k4[u] = i < n ? cq[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + u * stride < n && (k4[u] >> (64 - kRBits)) == pre)
                atomicAdd(&hs[(k4[u] >> (64 - 2 * kRBits)) & (kRBins - 1)], 1u);
    }
    __syncthreads();
    uint32_t* h2 = w.hist + (int64_t)q * 2 * kRBins + kRBins;
    for (int i = tid; i < kRBins; i += kWThreads)
        if (hs[i]) atomicAdd(&h2[i], hs[i]);
}

// Survivors (keys >= the query's threshold) appended to the query's list;
// the query's first workgroup records the resolved selection for the sort.
__global__ __launch_bounds__(kWThreads) void k_wide_collect(int K, WideDev w, int G, int Gb) {
    __shared__ __align__(16) uint32_t hs[kRBins];
    __shared__ int red_i[kWThreads / kWave];
    __shared__ int pick[3];
    const int q = blockIdx.x / G, g = blockIdx.x % G, tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    if (w.use_done && w.done[q]) return;
    WideSel* sel = reinterpret_cast<WideSel*>(w.sel) + q;
    const int n = sel->n_cand;
    if (n <= K) return;  // every candidate survives (sel->state is rewritten below, so not read here)
    const int GE = hist_blocks_used(G, Gb, n);
    if (g >= GE) return;
    const SelView v = resolve_digits<kWThreads>(w, q, K, n, 2, hs, red_i, pick);
    if (g == 0 && tid == 0) {
        sel->prefix = v.prefix;
        sel->need = v.need;
        sel->state = v.state;
    }
    if (v.state != kSelThreshold) return;
    const uint64_t thr = v.prefix;  // every key >= the prefix with zero low bits survives
    const uint64_t* cq = w.cand + (int64_t)q * w.cap;
    uint64_t* out = w.surv + (int64_t)q * kSurvCap;
    // four keys per thread in flight; i0 is uniform over the workgroup
    const int stride = GE * kWThreads;
    for (int i0 = g * kWThreads; i0 < n; i0 += 4 * stride) {
        uint64_t k4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * stride + tid;
            k4[u] = i < n ? cq[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool take = i0 + u * stride + tid < n && k4[u] >= thr;
            const uint64_t mask = __ballot(take);
            int base = 0;
            if (lane == 0 && mask) base = atomicAdd(&w.surv_n[q], (int)__popcll(mask));
            base = lane_bcast(base, 0);
            if (take) {
                const int pos = base + (int)__popcll(mask & ((1ull << lane) - 1ull));
                if (pos < kSurvCap) out[pos] = k4[u];
            }
        }
    }
}

// In-register stage of the block bitonic sort: registers r and r ^ RJ hold
// the partners (element i = r * kSortThreads + thread).
template <int E, int RJ>
__device__ __forceinline__ void sort_reg_stage(uint64_t (&v)[E], int k) {
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int r2 = r ^ RJ;
        if (r2 > r && r2 < E) {
            const bool desc = ((r * kSortThreads) & k) == 0;
            const uint64_t a = v[r], b = v[r2];
            const bool sw = desc ? a < b : a > b;
            v[r] = sw ? b : a;
            v[r2] = sw ? a : b;
        }
    }
}

// Bitonic sort, descending, of the E * kSortThreads keys held as v[r] =
// element r * kSortThreads + thread.  Partners closer than a wavefront are
// exchanged by lane shuffles, partners in other wavefronts through LDS (xch:
// E * kSortThreads keys), partners in other registers of the same thread in
// place.  All threads call.
template <int E>
__device__ void block_sort_desc(uint64_t (&v)[E], uint64_t* xch) {
    constexpr int NT = kSortThreads;
    constexpr int P = NT * E;
    const int tid = threadIdx.x;
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= NT) {
                const int rj = j / NT;
                if (rj == 1) sort_reg_stage<E, 1>(v, k);
                else if (rj == 2) sort_reg_stage<E, 2>(v, k);
                else sort_reg_stage<E, 4>(v, k);
            } else if (j >= kWave) {
#pragma unroll
                for (int r = 0; r < E; ++r) xch[r * NT + tid] = v[r];
                __syncthreads();
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const uint64_t o = xch[r * NT + (tid ^ j)];
                    const int i = r * NT + tid;
                    const bool take_max = ((i & j) == 0) == ((i & k) == 0);
                    v[r] = take_max ? umax64(v[r], o) : umin64(v[r], o);
                }
                __syncthreads();
            } else {
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const uint64_t o = shfl_xor64(v[r], j);
                    const int i = r * NT + tid;
                    const bool take_max = ((i & j) == 0) == ((i & k) == 0);
                    v[r] = take_max ? umax64(v[r], o) : umin64(v[r], o);
                }
            }
        }
    }
}

// Output slot i of query q from a radix key (0 = sentinel).
__device__ void emit_radix(const WideDev& w, int q, int K, int i, uint64_t key, int32_t* out_tok, int32_t* out_par,
                           int32_t* out_rows, float* out_logp) {
    const int64_t o = (int64_t)q * K + i;
    if (key == 0ull) {
        out_tok[o] = -1;
        out_par[o] = -1;
        out_rows[o] = -1;
        out_logp[o] = -INFINITY;
        return;
    }
    const uint32_t c_ix = 0xFFFFFFFFu - (uint32_t)key;
    const uint64_t inf = w.info[(int64_t)q * w.cap + c_ix];
    out_tok[o] = (int32_t)((inf >> 16) & 0xFFFFu);
    out_par[o] = (int32_t)(inf & 0xFFFFu);
    out_rows[o] = (int32_t)(uint32_t)(inf >> 32);
    out_logp[o] = score_from_order_bits((uint32_t)(key >> 32));
}

// Survivors src[0..n) (n <= E * kSortThreads) sorted; the best K emitted.
template <int E>
__device__ void sort_and_emit(const WideDev& w, int q, int K, const uint64_t* src, int n, uint64_t* xch,
                              int32_t* out_tok, int32_t* out_par, int32_t* out_rows, float* out_logp) {
    const int tid = threadIdx.x;
    uint64_t v[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int i = r * kSortThreads + tid;
        v[r] = i < n ? src[i] : 0ull;
    }
    __syncthreads();  // src may alias xch
    block_sort_desc<E>(v, xch);
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int i = r * kSortThreads + tid;
        if (i < K) emit_radix(w, q, K, i, v[r], out_tok, out_par, out_rows, out_logp);
    }
}

// Per query: the survivors sorted descending, the best K emitted.  A query
// whose threshold is still open after the two GPU-wide digits finishes the
// radix select here, 8 bits a pass.
__global__ __launch_bounds__(kSortThreads) void k_wide_sort(int K, WideDev w, int32_t* __restrict__ out_tok,
                                                            int32_t* __restrict__ out_par,
                                                            int32_t* __restrict__ out_rows,
                                                            float* __restrict__ out_logp) {
    extern __shared__ __align__(16) uint64_t ks[];  // [kSurvCap]
    __shared__ uint32_t h8[256];
    __shared__ int red_i[kSortThreads / kWave];
    __shared__ int pick[3];
    __shared__ int cnt_s;
    const int q = blockIdx.x, tid = threadIdx.x;
    if (w.use_done && w.done[q]) return;
    const WideSel* sel = reinterpret_cast<const WideSel*>(w.sel) + q;
    const int n_cand = sel->n_cand;
    const int state = sel->state;
    const uint64_t* cq = w.cand + (int64_t)q * w.cap;
    const uint64_t* src;
    int n;
    if (state == kSelUnresolved) {
        uint64_t prefix = sel->prefix;
        int need = sel->need;
        const int kt = min(K, n_cand);
        for (int shift = 64 - 2 * kRBits - 8;; shift -= 8) {
            for (int i = tid; i < 256; i += kSortThreads) h8[i] = 0;
            __syncthreads();
            for (int i = tid; i < n_cand; i += kSortThreads) {
                const uint64_t key = cq[i];
                if ((key >> (shift + 8)) == (prefix >> (shift + 8))) atomicAdd(&h8[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            block_pick<kSortThreads>(h8, 256, need, red_i, pick);
            need -= pick[1];
            prefix |= (uint64_t)pick[0] << shift;
            const bool done = kt - need + pick[2] <= kSurvCap || shift == 0;
            __syncthreads();
            if (done) break;
        }
        if (tid == 0) cnt_s = 0;
        __syncthreads();
        for (int i = tid; i < n_cand; i += kSortThreads) {
            const uint64_t key = cq[i];
            if (key >= prefix) {
                const int pos = atomicAdd(&cnt_s, 1);
                if (pos < kSurvCap) ks[pos] = key;
            }
        }
        __syncthreads();
        n = min(cnt_s, kSurvCap);
        src = ks;
    } else if (state == kSelAll) {
        n = n_cand;  // <= K <= kSortThreads
        src = cq;
    } else {
        n = min(w.surv_n[q], kSurvCap);
        src = w.surv + (int64_t)q * kSurvCap;
    }
    if (n <= kSortThreads)
        sort_and_emit<1>(w, q, K, src, n, ks, out_tok, out_par, out_rows, out_logp);
    else if (n <= 2 * kSortThreads)
        sort_and_emit<2>(w, q, K, src, n, ks, out_tok, out_par, out_rows, out_logp);
    else if (n <= 4 * kSortThreads)
        sort_and_emit<4>(w, q, K, src, n, ks, out_tok, out_par, out_rows, out_logp);
    else
        sort_and_emit<8>(w, q, K, src, n, ks, out_tok, out_par, out_rows, out_logp);
}

// Pre-pass, one workgroup of kSortThreads threads per query, one thread per
// beam slot (K <= kSortThreads).  A row with one valid token has log-softmax
// exactly 0 whatever its score, so when every live row of the query has one
// token (CSR) its K candidates are (acc_k, k, token) and no score is needed:
// if the live slots come first and their log-probs do not increase the
// outputs are the inputs in place (slot i = beam i); otherwise the K keys are
// sorted (score desc, parent asc).  The query is then marked done for the
// radix kernels that follow; any other query is left to them (done = 0, so
// the array needs no clearing between steps).
__global__ __launch_bounds__(kSortThreads) void k_wide_small(StepDev st, int K, const int32_t* __restrict__ beam_rows,
                                                             const float* __restrict__ acc, WideDev w,
                                                             int32_t* __restrict__ out_tok,
                                                             int32_t* __restrict__ out_par,
                                                             int32_t* __restrict__ out_rows,
                                                             float* __restrict__ out_logp) {
    __shared__ uint64_t xch[kSortThreads];
    __shared__ float a_s[kSortThreads];
    __shared__ uint32_t e0_s[kSortThreads];
    __shared__ uint16_t t_s[kSortThreads];
    const int q = blockIdx.x, k = threadIdx.x;
    const int32_t r = k < K ? beam_rows[(int64_t)q * K + k] : -1;
    const float a = k < K ? acc[(int64_t)q * K + k] : -INFINITY;
    const bool live = k < K && beam_live(st, r, a);
    const uint32_t e0 = live ? st.row_ptr[r] : 0u;
    const int n = live ? (int)(st.row_ptr[r + 1] - e0) : 0;
    const int f0 = live && st.tok0 ? (int)st.tok0[r] : 0;  // in flight with row_ptr
    const bool one = live && st.store == CB_STORE_CSR && n == 1 && st.tok0;
    a_s[k] = live ? a : -INFINITY;
    e0_s[k] = e0;
    t_s[k] = (uint16_t)f0;
    __syncthreads();
    // a slot that breaks the in-place order: live after a dead slot, or a
    // log-prob above the previous slot's
    const bool viol = live && k > 0 && !(a_s[k - 1] >= a);
    const int n_other = __syncthreads_count(live && !one);
    const int n_viol = __syncthreads_count(viol);
    if (n_other > 0) {
        if (k == 0) w.done[q] = 0;
        return;  // uniform: the radix kernels take this query
    }
    const int64_t base = (int64_t)q * K;
    if (n_viol == 0) {
        if (k < K) {
            out_tok[base + k] = live ? f0 : -1;
            out_par[base + k] = live ? k : -1;
            out_rows[base + k] = live ? (int32_t)e0 : -1;
            out_logp[base + k] = live ? a + 0.f : -INFINITY;
        }
    } else {
        // one key per slot: score bits, then the complement of the slot (so
        // that equal scores order by parent ascending); 0 = no candidate
        uint64_t v[1] = {live ? ((uint64_t)score_order_bits(a + 0.f) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)k)
                              : 0ull};
        block_sort_desc<1>(v, xch);
        if (k < K) {
            const uint64_t key = v[0];
            const int p = key ? (int)(0xFFFFFFFFu - (uint32_t)key) : -1;
            out_tok[base + k] = key ? (int32_t)t_s[p] : -1;
            out_par[base + k] = key ? p : -1;
            out_rows[base + k] = key ? (int32_t)e0_s[p] : -1;
            out_logp[base + k] = key ? score_from_order_bits((uint32_t)(key >> 32)) : -INFINITY;
        }
    }
    if (k == 0) w.done[q] = 1;
}

}  // namespace

// ---- launchers -----------------------------------------------------------------

int wide_chunk() { return kWCH; }
int wide_bins() { return kRBins; }
int wide_surv_cap() { return kSurvCap; }
size_t wide_sel_bytes() { return sizeof(WideSel); }
// Workgroups per query: the scoring kernel spreads a query's chunks over up
// to 1024 workgroups; the histogram kernels use up to 256 (one per CU).
int wide_blocks_per_query(int Q) { return Q >= 2048 ? 1 : (2048 / (Q > 0 ? Q : 1) > 1024 ? 1024 : 2048 / Q); }
int wide_hist_blocks_per_query(int Q) { return Q >= 256 ? 1 : 256 / (Q > 0 ? Q : 1); }
int wide_hist_blocks(int Q, int64_t keys_bound) {
    const int base = wide_hist_blocks_per_query(Q);
    const int cap = std::max(base, 2048 / std::max(Q, 1));
    const int64_t want = (keys_bound + kHistKeys - 1) / kHistKeys;
    return (int)std::min<int64_t>(cap, std::max<int64_t>(base, want));
}
size_t wide_score_lds_bytes(int d, bool dense) { return dense ? 0 : (size_t)d * 4; }

hipError_t launch_wide_score(const StepDev& st, bool dense, cb_dtype dt, int Q, int K, int d, const void* hidden,
                             const void* W, const float* Z, const float* Zp, int64_t ldz, const int32_t* n_live,
                             const int32_t* ci_of, const int32_t* beam_rows, const float* acc, int wide_only,
                             const WideDev& w, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int G = wide_blocks_per_query(Q);
    const dim3 grid(Q * G);
    const size_t lds = wide_score_lds_bytes(d, dense);
    const int split_ok = dt == CB_BF16 ? 1 : 0;
#define CB_WSCORE(DT, DENSE, CHV)                                                                        \
    CB_LAUNCH((k_wide_score<DT, DENSE, CHV>), grid, dim3(kWThreads), lds, s, st, K, d, (const DT*)hidden, \
              (const DT*)W, Z, Zp, ldz, n_live, ci_of, split_ok, beam_rows, acc, wide_only, w, G)
#define CB_WSCORE_CH(DT)                                     \
    do {                                                     \
        if (d <= 512) CB_WSCORE(DT, false, 1);               \
        else if (d <= 1024) CB_WSCORE(DT, false, 2);         \
        else if (d <= 2048) CB_WSCORE(DT, false, 4);         \
        else CB_WSCORE(DT, false, 0);                        \
    } while (0)
    if (dt == CB_BF16) {
        if (dense) CB_WSCORE(uint16_t, true, 0); else CB_WSCORE_CH(uint16_t);
    } else {
        if (dense) CB_WSCORE(float, true, 0); else CB_WSCORE_CH(float);
    }
#undef CB_WSCORE_CH
#undef CB_WSCORE
    return hipGetLastError();
}

hipError_t launch_tm_count(const StepDev& st, int Q, int K, const int32_t* beam_rows, const float* acc,
                           const WideDev& w, const TokDev& tk, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int G = wide_blocks_per_query(Q);
    CB_LAUNCH(k_tm_count, dim3(Q * G), dim3(kWThreads), 0, s, st, K, beam_rows, acc, w, tk, G);
    return hipGetLastError();
}

hipError_t launch_tm_scan(int V, const TokDev& tk, hipStream_t s) {
    if (V <= 4096) CB_LAUNCH(k_tm_scan<4>, dim3(1), dim3(1024), 0, s, V, tk);
    else if (V <= 8192) CB_LAUNCH(k_tm_scan<8>, dim3(1), dim3(1024), 0, s, V, tk);
    else if (V <= 16384) CB_LAUNCH(k_tm_scan<16>, dim3(1), dim3(1024), 0, s, V, tk);
    else if (V <= 32768) CB_LAUNCH(k_tm_scan<32>, dim3(1), dim3(1024), 0, s, V, tk);
    else CB_LAUNCH(k_tm_scan<64>, dim3(1), dim3(1024), 0, s, V, tk);
    return hipGetLastError();
}

hipError_t launch_tm_scatter(int Q, int K, const WideDev& w, const TokDev& tk, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int G = wide_blocks_per_query(Q);
    CB_LAUNCH(k_tm_scatter, dim3(Q * G), dim3(kWThreads), 0, s, K, w, tk, G);
    return hipGetLastError();
}

int tm_score_blocks() { return 2048; }

// Units of n entries over V tokens: each token's entries in runs of at most
// kTmUnit, so at most n / kTmUnit + V.
int64_t tm_unit_cap(int64_t n, int V) { return n / kTmUnit + V + 1; }

__global__ __launch_bounds__(256) void k_tm_clear(int V, TokDev tk) {
    const int v = blockIdx.x * 256 + (int)threadIdx.x;
    if (v < V) tk.count[v] = 0;
}

hipError_t launch_tm_clear(int V, const TokDev& tk, hipStream_t s) {
    CB_LAUNCH(k_tm_clear, dim3((V + 255) / 256), dim3(256), 0, s, V, tk);
    return hipGetLastError();
}

hipError_t launch_tm_score(cb_dtype dt, int K, int d, const void* hidden, const void* W, const WideDev& w,
                           const TokDev& tk, hipStream_t s) {
    const dim3 grid(tm_score_blocks());
#define CB_TMS(DT, CHV) \
    CB_LAUNCH((k_tm_score<DT, CHV>), grid, dim3(kWThreads), 0, s, K, d, (const DT*)hidden, (const DT*)W, w, tk)
#define CB_TMS_CH(DT)                          \
    do {                                       \
        if (d <= 512) CB_TMS(DT, 1);           \
        else if (d <= 1024) CB_TMS(DT, 2);     \
        else CB_TMS(DT, 4);                    \
    } while (0)
    if (d > 2048) return hipErrorInvalidValue;
    if (dt == CB_BF16) CB_TMS_CH(uint16_t); else CB_TMS_CH(float);
#undef CB_TMS_CH
#undef CB_TMS
    return hipGetLastError();
}

hipError_t launch_tm_pairs(int Q, int K, int64_t keys_bound, const WideDev& w, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int G = wide_hist_blocks(Q, keys_bound), Gb = wide_hist_blocks_per_query(Q);
    CB_LAUNCH(k_tm_pairs, dim3(Q * G), dim3(kWThreads), 0, s, K, w, G, Gb);
    return hipGetLastError();
}

hipError_t launch_wide_small(const StepDev& st, int Q, int K, const int32_t* beam_rows, const float* acc,
                             const WideDev& w, int32_t* tok, int32_t* par, int32_t* rows, float* logp, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    CB_LAUNCH(k_wide_small, dim3(Q), dim3(kSortThreads), 0, s, st, K, beam_rows, acc, w, tok, par, rows, logp);
    return hipGetLastError();
}

hipError_t launch_row_lse(const StepDev& st, cb_dtype dt, int R, int V, int d, const float* Z, const float* Zp,
                          const int32_t* n_live, const int32_t* ci_of, const int32_t* beam_rows, const float* acc,
                          float* lse_row, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    CB_LAUNCH(k_row_lse, dim3(R), dim3(256), 0, s, st, R, V, d, Z, Zp, n_live, ci_of, dt == CB_BF16 ? 1 : 0,
              beam_rows, acc, lse_row);
    return hipGetLastError();
}

hipError_t launch_chunk_lse(int Q, int K, const WideDev& w, float* lse_row, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    CB_LAUNCH(k_chunk_lse, dim3((Q * K + 3) / 4), dim3(256), 0, s, Q, K, w, lse_row);
    return hipGetLastError();
}

hipError_t launch_wide_keys(int Q, int K, int64_t keys_bound, const float* acc, const WideDev& w,
                            hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int G = wide_hist_blocks(Q, keys_bound), Gb = wide_hist_blocks_per_query(Q);
    CB_LAUNCH(k_wide_keys, dim3(Q * G), dim3(kWThreads), 0, s, K, acc, w, G, Gb);
    return hipGetLastError();
}

hipError_t launch_wide_refine(int Q, int K, int64_t keys_bound, const WideDev& w, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int G = wide_hist_blocks(Q, keys_bound), Gb = wide_hist_blocks_per_query(Q);
    CB_LAUNCH(k_wide_refine, dim3(Q * G), dim3(kWThreads), 0, s, K, w, G, Gb);
    return hipGetLastError();
}

hipError_t launch_wide_collect(int Q, int K, int64_t keys_bound, const WideDev& w, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int G = wide_hist_blocks(Q, keys_bound), Gb = wide_hist_blocks_per_query(Q);
    CB_LAUNCH(k_wide_collect, dim3(Q * G), dim3(kWThreads), 0, s, K, w, G, Gb);
    return hipGetLastError();
}

hipError_t launch_wide_sort(const StepDev& st, int Q, int K, const int32_t* beam_rows, const WideDev& w,
                            int32_t* tok, int32_t* par, int32_t* rows, float* logp, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int lds = kSurvCap * 8;
    static const hipError_t lds_ok =
        hipFuncSetAttribute((const void*)k_wide_sort, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (lds_ok != hipSuccess) return lds_ok;
    CB_LAUNCH(k_wide_sort, dim3(Q), dim3(kSortThreads), lds, s, K, w, tok, par, rows, logp);
    return hipGetLastError();
}

}  // namespace cb
