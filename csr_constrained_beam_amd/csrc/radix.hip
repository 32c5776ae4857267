// Radix-select path of one constrained beam-search step (gfx950, wave64):
// beam widths up to 1024 and rows of any width.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "cb_internal.h"
#include "device.h"

namespace cb {
namespace {
// ---- radix-select path: beam widths up to 1024 -----------------------------
//
// The per-query selection above holds a query's best keys in one wavefront,
// which bounds K by 64.  For wider beams (FlashTrie's beam widths of 100 to
// 1000, sec. 4.2) every candidate of a query is written to HBM as its 64-bit
// key and the query's K-th largest key is found by radix select on the high
// bits: two 12-bit digits counted across the whole GPU (LDS histograms per
// workgroup, added into the query's global histogram; the last workgroup of
// the query to finish picks the digit), after which the survivors (keys >=
// the threshold, at most kSurvCap) are sorted in LDS and emitted.  Keys are
// distinct within a query (parent, token), so the selection is exact and the
// order is the (score desc, parent asc, token asc) order of the key.  If more
// than kSurvCap keys still share the two digits (massive exact score ties),
// the sort workgroup finishes the radix select on its own, 8 bits a pass.
//
// Work is cut into chunks of kWCH consecutive valid tokens of one beam; a
// beam's log-sum-exp is combined from its chunks' (max, sum exp) pairs.

constexpr int kWCH = 64;
constexpr int kWThreads = 256;
constexpr int kRBits = 12;
constexpr int kRBins = 1 << kRBits;
constexpr int kSurvCap = 8192;
constexpr int kSortThreads = 1024;

enum : int32_t { kSelPending = 0, kSelThreshold = 1, kSelUnresolved = 2 };

struct WideSel {
    uint64_t prefix;  // decided high bits of the query's K-th largest key
    uint64_t thr;     // state kSelThreshold: the survivors are the keys >= thr
    int32_t need;     // keys still to take among those sharing `prefix`
    int32_t state;
    int32_t n_cand;   // candidates of the query
    uint32_t done;    // workgroups of the query finished with the current pass
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

// Slot of the query whose chunks contain chunk c (offs[0] <= c < offs[K]).
__device__ __forceinline__ int slot_of_chunk(const int32_t* offs, int K, int c) {
    int lo = 0, hi = K;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= c) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ uint32_t load_count(const uint32_t* p, bool coherent) {
    return coherent ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
}

// Digit (bin) holding the need-th largest key, from the counts of nbins
// digits (bin index = digit value).  pick[0] = digit, pick[1] = keys in
// higher bins, pick[2] = keys in the bin.  All threads call.
template <int NT>
__device__ void block_pick(const uint32_t* h, int nbins, bool coherent, int need, int* red_i, int* pick) {
    const int per = (nbins + NT - 1) / NT;
    const int top = nbins - 1 - (int)threadIdx.x * per;  // this thread's bins: top, top-1, ... (highest first)
    int s = 0;
    for (int i = 0; i < per; ++i)
        if (top - i >= 0) s += (int)load_count(h + top - i, coherent);
    int tot;
    int above = block_exclusive_scan<NT>(s, red_i, &tot);
    if (above < need && above + s >= need) {
        for (int i = 0; i < per; ++i) {
            const int c = (int)load_count(h + top - i, coherent);
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

// After a digit at bit `shift` is picked: survivors if we stopped here are the
// keys above the boundary bin plus the whole bin.
__device__ void sel_advance(WideSel* sel, int K, const int* pick, int shift, bool last_pass) {
    const int kt = min(K, sel->n_cand);
    const int need = sel->need - pick[1];
    const uint64_t prefix = sel->prefix | ((uint64_t)pick[0] << shift);
    sel->prefix = prefix;
    sel->need = need;
    if (kt - need + pick[2] <= kSurvCap) {
        sel->thr = prefix;
        sel->state = kSelThreshold;
    } else if (last_pass) {
        sel->state = kSelUnresolved;
    }
}

// True in the last workgroup of the query to reach this point (its earlier
// global atomics are then visible to it).
__device__ bool last_of_query(WideSel* sel, int G, int* flag) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(&sel->done, 1u);
        *flag = prev == (uint32_t)(G - 1);
        if (*flag) sel->done = 0;  // ready for the next pass
    }
    __syncthreads();
    if (*flag) __threadfence();
    return *flag != 0;
}

// Per query: candidate and chunk offsets of every slot, selection state, and
// cleared histograms.  One workgroup per query, one thread per slot.
__global__ __launch_bounds__(1024) void k_wide_plan(StepDev st, int K, const int32_t* __restrict__ beam_rows,
                                                    const float* __restrict__ acc, WideDev w) {
    __shared__ int red_i[1024 / kWave];
    const int q = blockIdx.x, k = threadIdx.x;
    int n = 0;
    if (k < K) {
        const int64_t b = (int64_t)q * K + k;
        const int32_t r = beam_rows[b];
        if (beam_live(st, r, acc[b])) n = (int)(st.row_ptr[r + 1] - st.row_ptr[r]);
    }
    int tc, th;
    const int oc = block_exclusive_scan<1024>(n, red_i, &tc);
    const int oh = block_exclusive_scan<1024>((n + kWCH - 1) / kWCH, red_i, &th);
    int32_t* co = w.cand_off + (int64_t)q * (K + 1);
    int32_t* ho = w.chunk_off + (int64_t)q * (K + 1);
    if (k < K) {
        co[k] = oc;
        ho[k] = oh;
    }
    if (k == 0) {
        co[K] = tc;
        ho[K] = th;
        WideSel* sel = reinterpret_cast<WideSel*>(w.sel) + q;
        sel->prefix = 0;
        sel->need = min(K, tc);
        sel->n_cand = tc;
        sel->done = 0;
        sel->state = tc <= K ? kSelThreshold : kSelPending;
        sel->thr = 1;  // every candidate key is nonzero
        w.surv_n[q] = 0;
    }
    uint32_t* hq = w.hist + (int64_t)q * 2 * kRBins;
    for (int i = k; i < 2 * kRBins; i += 1024) hq[i] = 0;
}

// Scores of every candidate, one chunk per workgroup iteration: z (sparse
// gather-dot against the beam's hidden vector staged in LDS, or the
// full-codebook score of the column), stored as z's bits over the key's low
// half (parent, token), and the chunk's (max, sum exp).
template <typename DT, bool DENSE>
__global__ __launch_bounds__(kWThreads) void k_wide_score(StepDev st, int K, int d, const DT* __restrict__ hidden,
                                                          const DT* __restrict__ W, const float* __restrict__ Z,
                                                          const float* __restrict__ Zp, int64_t ldz,
                                                          const int32_t* __restrict__ n_live,
                                                          const int32_t* __restrict__ ci_of, int split_ok,
                                                          const int32_t* __restrict__ beam_rows, WideDev w) {
    extern __shared__ __align__(16) float h_s[];  // [d], sparse scoring only
    __shared__ float z_s[kWCH];
    __shared__ uint16_t tok_s[kWCH];
    const int q = blockIdx.x / w.G, g = blockIdx.x % w.G, tid = threadIdx.x;
    const int32_t* co = w.cand_off + (int64_t)q * (K + 1);
    const int32_t* ho = w.chunk_off + (int64_t)q * (K + 1);
    const int nch = ho[K];
    int split = 1;
    if (DENSE && split_ok) split = gemm_split(*n_live, (int)ldz, d);
    int staged = -1;
    for (int c = g; c < nch; c += w.G) {
        const int k = slot_of_chunk(ho, K, c);
        const int64_t b = (int64_t)q * K + k;
        const int32_t r = beam_rows[b];
        const uint32_t e0 = st.row_ptr[r];
        const int n = co[k + 1] - co[k];
        const int j0 = (c - ho[k]) * kWCH;
        const int cnt = min(kWCH, n - j0);
        if (tid < cnt) tok_s[tid] = (uint16_t)nth_token(st, r, e0, j0 + tid);
        if (!DENSE && staged != k) {
            for (int i = tid; i < d; i += kWThreads) h_s[i] = to_f32(hidden[b * d + i]);
            staged = k;
        }
        __syncthreads();
        if (DENSE) {
            if (tid < cnt) {
                const int v = tok_s[tid];
                float z = 0.f;
                if (split == 1) {
                    z = Z[b * ldz + v];
                } else {
                    const float* zb = Zp + (int64_t)ci_of[b] * ldz + v;
                    for (int x = 0; x < split; ++x) z += zb[(int64_t)x * kSplitRows * ldz];
                }
                z_s[tid] = z;
            }
        } else {
            block_scores<DT, kWThreads>(h_s, W, d, tok_s, cnt, z_s);
        }
        __syncthreads();
        if (tid < kWave) {
            const float z = tid < cnt ? z_s[tid] : -INFINITY;
            const float m = wave_max(z);
            const float s = wave_sum(tid < cnt ? expf(z - m) : 0.f);
            if (tid == 0) {
                float* p = w.cms + ((int64_t)q * w.chunk_cap + c) * 2;
                p[0] = m;
                p[1] = s;
            }
            if (tid < cnt)
                w.cand[(int64_t)q * w.cap + co[k] + j0 + tid] = ((uint64_t)__float_as_uint(z) << 32) |
                                                                 ((uint64_t)(1023 - k) << 16) |
                                                                 (uint64_t)(65535 - tok_s[tid]);
        }
        __syncthreads();
    }
}

// Keys of every candidate (one chunk per wavefront): the beam's log-sum-exp
// from its chunks, score = acc + (z - lse) in float32, and the histogram of
// the keys' top digit; the query's last workgroup picks that digit.
__global__ __launch_bounds__(kWThreads) void k_wide_keys(int K, const float* __restrict__ acc, WideDev w) {
    __shared__ uint32_t hs[kRBins];
    __shared__ int red_i[kWThreads / kWave];
    __shared__ int pick[3];
    __shared__ int flag;
    const int q = blockIdx.x / w.G, g = blockIdx.x % w.G, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    constexpr int NWV = kWThreads / kWave;
    for (int i = tid; i < kRBins; i += kWThreads) hs[i] = 0;
    __syncthreads();
    const int32_t* co = w.cand_off + (int64_t)q * (K + 1);
    const int32_t* ho = w.chunk_off + (int64_t)q * (K + 1);
    const int nch = ho[K];
    const float* cms = w.cms + (int64_t)q * w.chunk_cap * 2;
    uint64_t* cq = w.cand + (int64_t)q * w.cap;
    for (int c = g * NWV + wv; c < nch; c += w.G * NWV) {
        const int k = slot_of_chunk(ho, K, c);
        float m = -INFINITY, s = 0.f;
        for (int x = ho[k] + lane; x < ho[k + 1]; x += kWave) {
            const float cm = cms[2 * x], cs = cms[2 * x + 1];
            if (cm > m) {
                s = s * expf(m - cm) + cs;
                m = cm;
            } else {
                s += cs * expf(cm - m);
            }
        }
        const float M = wave_max(m);
        const float S = wave_sum(m == -INFINITY ? 0.f : s * expf(m - M));
        const float lse = M + logf(S);
        const float a = acc[(int64_t)q * K + k];
        const int j0 = (c - ho[k]) * kWCH;
        const int cnt = min(kWCH, co[k + 1] - co[k] - j0);
        if (lane < cnt) {
            uint64_t* p = cq + co[k] + j0 + lane;
            const uint64_t v = *p;
            const float z = __uint_as_float((uint32_t)(v >> 32));
            const uint64_t key = ((uint64_t)score_order_bits(a + (z - lse)) << 32) | (v & 0xFFFFFFFFull);
            *p = key;
            atomicAdd(&hs[key >> (64 - kRBits)], 1u);
        }
    }
    __syncthreads();
    WideSel* sel = reinterpret_cast<WideSel*>(w.sel) + q;
    if (sel->state != kSelPending) return;  // uniform over the query's workgroups
    uint32_t* h1 = w.hist + (int64_t)q * 2 * kRBins;
    for (int i = tid; i < kRBins; i += kWThreads)
        if (hs[i]) atomicAdd(&h1[i], hs[i]);
    if (!last_of_query(sel, w.G, &flag)) return;
    block_pick<kWThreads>(h1, kRBins, true, sel->need, red_i, pick);
    if (tid == 0) sel_advance(sel, K, pick, 64 - kRBits, false);
}

// Second digit, over the keys that share the first.
__global__ __launch_bounds__(kWThreads) void k_wide_refine(int K, WideDev w) {
    __shared__ uint32_t hs[kRBins];
    __shared__ int red_i[kWThreads / kWave];
    __shared__ int pick[3];
    __shared__ int flag;
    const int q = blockIdx.x / w.G, g = blockIdx.x % w.G, tid = threadIdx.x;
    WideSel* sel = reinterpret_cast<WideSel*>(w.sel) + q;
    if (sel->state != kSelPending) return;  // uniform over the query's workgroups
    for (int i = tid; i < kRBins; i += kWThreads) hs[i] = 0;
    __syncthreads();
    const uint64_t pre = sel->prefix >> (64 - kRBits);
    const int n = sel->n_cand;
    const uint64_t* cq = w.cand + (int64_t)q * w.cap;
    for (int i = g * kWThreads + tid; i < n; i += w.G * kWThreads) {
        const uint64_t key = cq[i];
        if ((key >> (64 - kRBits)) == pre) atomicAdd(&hs[(key >> (64 - 2 * kRBits)) & (kRBins - 1)], 1u);
    }
    __syncthreads();
    uint32_t* h2 = w.hist + (int64_t)q * 2 * kRBins + kRBins;
    for (int i = tid; i < kRBins; i += kWThreads)
        if (hs[i]) atomicAdd(&h2[i], hs[i]);
    if (!last_of_query(sel, w.G, &flag)) return;
    block_pick<kWThreads>(h2, kRBins, true, sel->need, red_i, pick);
    if (tid == 0) sel_advance(sel, K, pick, 64 - 2 * kRBits, true);
}

// Survivors (keys >= the query's threshold) appended to the query's list.
__global__ __launch_bounds__(kWThreads) void k_wide_collect(WideDev w) {
    const int q = blockIdx.x / w.G, g = blockIdx.x % w.G, tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const WideSel* sel = reinterpret_cast<const WideSel*>(w.sel) + q;
    if (sel->state != kSelThreshold) return;
    const uint64_t thr = sel->thr;
    const int n = sel->n_cand;
    const uint64_t* cq = w.cand + (int64_t)q * w.cap;
    uint64_t* out = w.surv + (int64_t)q * kSurvCap;
    for (int i0 = g * kWThreads; i0 < n; i0 += w.G * kWThreads) {
        const int i = i0 + tid;
        const uint64_t key = i < n ? cq[i] : 0ull;
        const bool take = i < n && key >= thr;
        const uint64_t mask = __ballot(take);
        int base = 0;
        if (lane == 0 && mask) base = atomicAdd(&w.surv_n[q], (int)__popcll(mask));
        base = __shfl(base, 0);
        if (take) {
            const int pos = base + (int)__popcll(mask & ((1ull << lane) - 1ull));
            if (pos < kSurvCap) out[pos] = key;
        }
    }
}

// Per query: the survivors sorted descending in LDS (bitonic), the best K
// emitted.  A query whose threshold is still open after the two GPU-wide
// digits finishes the radix select here, 8 bits a pass.
__global__ __launch_bounds__(kSortThreads) void k_wide_sort(StepDev st, int K, const int32_t* __restrict__ beam_rows,
                                                            WideDev w, int32_t* __restrict__ out_tok,
                                                            int32_t* __restrict__ out_par,
                                                            int32_t* __restrict__ out_rows,
                                                            float* __restrict__ out_logp) {
    extern __shared__ __align__(16) uint64_t ks[];  // [kSurvCap]
    __shared__ uint32_t h8[256];
    __shared__ int red_i[kSortThreads / kWave];
    __shared__ int pick[3];
    __shared__ int cnt_s;
    __shared__ uint64_t thr_s;
    const int q = blockIdx.x, tid = threadIdx.x;
    const WideSel* sel = reinterpret_cast<const WideSel*>(w.sel) + q;
    const int n_cand = sel->n_cand;
    const uint64_t* cq = w.cand + (int64_t)q * w.cap;
    int n;
    if (sel->state == kSelUnresolved) {
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
            block_pick<kSortThreads>(h8, 256, false, need, red_i, pick);
            need -= pick[1];
            prefix |= (uint64_t)pick[0] << shift;
            const bool done = kt - need + pick[2] <= kSurvCap || shift == 0;
            __syncthreads();
            if (done) break;
        }
        if (tid == 0) {
            thr_s = prefix;
            cnt_s = 0;
        }
        __syncthreads();
        const uint64_t thr = thr_s;
        for (int i = tid; i < n_cand; i += kSortThreads) {
            const uint64_t key = cq[i];
            if (key >= thr) {
                const int pos = atomicAdd(&cnt_s, 1);
                if (pos < kSurvCap) ks[pos] = key;
            }
        }
        __syncthreads();
        n = min(cnt_s, kSurvCap);
    } else {
        n = min(w.surv_n[q], kSurvCap);
        const uint64_t* src = w.surv + (int64_t)q * kSurvCap;
        for (int i = tid; i < n; i += kSortThreads) ks[i] = src[i];
    }
    int P = kWave;
    while (P < n) P <<= 1;
    for (int i = n + tid; i < P; i += kSortThreads) ks[i] = 0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < P; i += kSortThreads) {
                const int o = i ^ j;
                if (o > i) {
                    const uint64_t a = ks[i], b = ks[o];
                    const bool desc = (i & k) == 0;
                    if (desc ? a < b : a > b) {
                        ks[i] = b;
                        ks[o] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < K; i += kSortThreads)
        emit(st, q, K, i, i < n ? ks[i] : 0ull, beam_rows, out_tok, out_par, out_rows, out_logp);
}

}  // namespace

// ---- launchers -----------------------------------------------------------------

int wide_chunk() { return kWCH; }
int wide_bins() { return kRBins; }
int wide_surv_cap() { return kSurvCap; }
size_t wide_sel_bytes() { return sizeof(WideSel); }
int wide_blocks_per_query(int Q) { return Q >= 2048 ? 1 : (2048 / (Q > 0 ? Q : 1) > 1024 ? 1024 : 2048 / Q); }
size_t wide_score_lds_bytes(int d, bool dense) { return dense ? 0 : (size_t)d * 4; }

hipError_t launch_wide_plan(const StepDev& st, int Q, int K, const int32_t* beam_rows, const float* acc,
                            const WideDev& w, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_wide_plan, dim3(Q), dim3(1024), 0, s, st, K, beam_rows, acc, w);
    return hipGetLastError();
}

hipError_t launch_wide_score(const StepDev& st, bool dense, cb_dtype dt, int Q, int K, int d, const void* hidden,
                             const void* W, const float* Z, const float* Zp, int64_t ldz, const int32_t* n_live,
                             const int32_t* ci_of, const int32_t* beam_rows, const WideDev& w, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const dim3 grid(Q * w.G);
    const size_t lds = wide_score_lds_bytes(d, dense);
    const int split_ok = dt == CB_BF16 ? 1 : 0;
#define CB_WSCORE(DT, DENSE)                                                                                  \
    hipLaunchKernelGGL((k_wide_score<DT, DENSE>), grid, dim3(kWThreads), lds, s, st, K, d, (const DT*)hidden, \
                       (const DT*)W, Z, Zp, ldz, n_live, ci_of, split_ok, beam_rows, w)
    if (dt == CB_BF16) {
        if (dense) CB_WSCORE(uint16_t, true); else CB_WSCORE(uint16_t, false);
    } else {
        if (dense) CB_WSCORE(float, true); else CB_WSCORE(float, false);
    }
#undef CB_WSCORE
    return hipGetLastError();
}

hipError_t launch_wide_keys(int Q, int K, const float* acc, const WideDev& w, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_wide_keys, dim3(Q * w.G), dim3(kWThreads), 0, s, K, acc, w);
    return hipGetLastError();
}

hipError_t launch_wide_refine(int Q, int K, const WideDev& w, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_wide_refine, dim3(Q * w.G), dim3(kWThreads), 0, s, K, w);
    return hipGetLastError();
}

hipError_t launch_wide_collect(int Q, const WideDev& w, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_wide_collect, dim3(Q * w.G), dim3(kWThreads), 0, s, w);
    return hipGetLastError();
}

hipError_t launch_wide_sort(const StepDev& st, int Q, int K, const int32_t* beam_rows, const WideDev& w,
                            int32_t* tok, int32_t* par, int32_t* rows, float* logp, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int lds = kSurvCap * 8;
    static const hipError_t lds_ok =
        hipFuncSetAttribute((const void*)k_wide_sort, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (lds_ok != hipSuccess) return lds_ok;
    hipLaunchKernelGGL(k_wide_sort, dim3(Q), dim3(kSortThreads), lds, s, st, K, beam_rows, w, tok, par, rows, logp);
    return hipGetLastError();
}

}  // namespace cb
