// Device kernels of one constrained beam-search step on gfx950 (wave64).
//
// Sparse path (one launch per step), k_step_query: one workgroup per query.
//   Phase 1, one wavefront per beam whose row has <= 64 valid tokens:
//     a1 slot fill  - lane j holds the row's j-th token (CSR rows, ascending);
//     a2 scores     - for each token the whole wave reads its W_t row in place
//                     (16-byte coalesced lanes) against the hidden vector held in
//                     registers, fixed-order butterfly sum; lane j keeps z_j;
//     a3 softmax    - wave max / sum over the valid lanes only (ZeroGR "The
//                     pipeline", stage 4: log-softmax over valid tokens, added to
//                     the accumulated log-prob);
//     a4 (beam)     - the beam's best min(K, n) candidate keys, written to the
//                     beam's fixed slots in LDS (ZeroGR: fixed candidate slots;
//                     a beam cannot place more than K candidates among its
//                     query's K best).
//   Phase 2, rows with more than 64 tokens (and bitmap rows): the whole
//     workgroup per beam (tokens, hidden vector and scores staged in LDS).
//   Phase 3 (a4 query): the K best keys of the query, their next rows.
//
// Dense path: k_live_rows (compact list of live beams), k_gemm_bf16 / k_gemm_f32
// (scores of the live beams against the whole codebook; ZeroGR "full
// scoring"), k_beam_expand (one workgroup per beam: gather of the valid
// columns, softmax, best min(K, n) keys) and k_query_merge (per query K best).
//
// Candidate key: [63:32] order-preserving bits of the float32 score,
// [25:16] 1023 - parent slot, [15:0] 65535 - token.  Keys are unique within a
// query; descending key order is (score desc, parent asc, token asc); 0 marks
// an empty slot.
//
// Beam widths beyond 64 (and rows too wide for these kernels' LDS) take the
// radix-select path in radix.hip.
//
// Selection of the best Kc (<= 64) of n keys in a workgroup: tau = the Kc-th
// largest of the per-thread maxima is a lower bound of the true Kc-th largest
// key (the maxima are a subset of the keys), so the keys >= tau contain the
// answer; usually only about Kc of them survive, and those are sorted with
// register-resident wave64 bitonic networks.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "cb_internal.h"
#include "device.h"

namespace cb {
namespace {

// Next-step row of `token` in row r: its edge position.
__device__ int32_t edge_of(const StepDev& st, int32_t r, int token) {
    const uint32_t e0 = st.row_ptr[r];
    if (st.store == CB_STORE_CSR) {
        uint32_t lo = 0, hi = st.row_ptr[r + 1] - e0;
        while (lo < hi) {
            uint32_t mid = (lo + hi) >> 1;
            if ((int)st.tok[e0 + mid] < token) lo = mid + 1; else hi = mid;
        }
        return (int32_t)(e0 + lo);
    }
    const int64_t x = (int64_t)r * st.words + (token >> 5);
    return (int32_t)(e0 + st.rank[x] + __popc(st.bits[x] & ((1u << (token & 31)) - 1u)));
}

// Output slot i of query q from its key.
__device__ __forceinline__ void emit(const StepDev& st, int q, int K, int i, uint64_t key, const int32_t* __restrict__ beam_rows,
                     int32_t* out_tok, int32_t* out_par, int32_t* out_rows, float* out_logp) {
    const int64_t o = (int64_t)q * K + i;
    if (key == 0ull) {
        out_tok[o] = -1;
        out_par[o] = -1;
        out_rows[o] = -1;
        out_logp[o] = -INFINITY;
        return;
    }
    const int parent = 1023 - (int)((key >> 16) & 1023u);
    const int token = 65535 - (int)(key & 0xFFFFu);
    out_tok[o] = token;
    out_par[o] = parent;
    out_rows[o] = edge_of(st, beam_rows[(int64_t)q * K + parent], token);
    out_logp[o] = score_from_order_bits((uint32_t)(key >> 32));
}

// Output slot i of query q from its key, in the fused sparse step: the
// parent's row start, width and tokens were kept in LDS when the row was
// read, so the next row needs no global reads.  n_s[p] >= 0: narrow row of
// n_s[p] tokens, sorted, in tokq[p * 64 ...]; otherwise a wide row of
// -1 - n_s[p] tokens whose best min(Kc, n) candidates left their tokens in
// tokq[p * 64 ...] and their positions in the row in jq[p * 64 ...].  nrows /
// nacc (may be NULL): LDS copies of the next rows and log-probs, per slot.
__device__ void emit_query(int q, int K, int Kc, int i, uint64_t key, const uint32_t* e0_s, const int* n_s,
                           const uint16_t* tokq, const int* jq, int32_t* out_tok, int32_t* out_par, int32_t* out_rows,
                           float* out_logp, int32_t* nrows, float* nacc) {
    const int64_t o = (int64_t)q * K + i;
    if (key == 0ull) {
        out_tok[o] = -1;
        out_par[o] = -1;
        out_rows[o] = -1;
        out_logp[o] = -INFINITY;
        if (nrows) {
            nrows[i] = -1;
            nacc[i] = -INFINITY;
        }
        return;
    }
    const int parent = 1023 - (int)((key >> 16) & 1023u);
    const int token = 65535 - (int)(key & 0xFFFFu);
    const uint32_t e0 = e0_s[parent];
    const int nn = n_s[parent];
    int32_t row;
    if (nn >= 0) {
        const uint16_t* tq = tokq + parent * kWave;
        int lo = 0, hi = nn;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if ((int)tq[mid] < token) lo = mid + 1; else hi = mid;
        }
        row = (int32_t)(e0 + lo);
    } else {
        const int m = min(Kc, -1 - nn);
        const uint16_t* tq = tokq + parent * kWave;
        int j = 0;
        for (int x = 0; x < m; ++x)
            if ((int)tq[x] == token) j = jq[parent * kWave + x];
        row = (int32_t)(e0 + j);
    }
    const float lp = score_from_order_bits((uint32_t)(key >> 32));
    out_tok[o] = token;
    out_par[o] = parent;
    out_rows[o] = row;
    out_logp[o] = lp;
    if (nrows) {
        nrows[i] = row;
        nacc[i] = lp;
    }
}

// ---- LDS layouts (shared by launchers and kernels) --------------------------

struct ExpandLds {
    int z, h, tok, list, stage, total;
};
__host__ __device__ inline ExpandLds expand_lds(int S, int d, bool dense, int NT) {
    ExpandLds l;
    l.stage = 0;
    l.z = l.stage + NT * 8;
    l.list = l.z + ((S * 4 + 15) & ~15);
    l.h = l.list + ((S * 4 + 15) & ~15);
    l.tok = l.h + (dense ? 0 : ((d * 4 + 15) & ~15));
    l.total = l.tok + ((S * 2 + 15) & ~15);
    return l;
}

struct QueryLds {
    int qkeys, stage, list, z, h, tok, tokq, zmid, total;
};
__host__ __device__ inline QueryLds query_lds(int S, int K, int Kc, int d, int NT) {
    QueryLds l;
    const int M = K * Kc;
    l.qkeys = 0;
    l.stage = l.qkeys + M * 8;
    l.list = l.stage + NT * 8;
    l.z = l.list + (((S > M ? S : M) * 4 + 15) & ~15);
    l.h = l.z + ((S * 4 + 15) & ~15);
    l.tok = l.h + ((d * 4 + 15) & ~15);
    l.tokq = l.tok + ((S * 2 + 15) & ~15);
    l.zmid = l.tokq + ((K * kWave * 2 + 15) & ~15);
    l.total = l.zmid + (S > 1 ? K * kWave * 4 : 0);
    return l;
}

// ---- sparse step: one workgroup per query ----------------------------------

// Tokens per scoring task of the per-query step (phase 1b), within a register
// budget: the task's W_t row chunks plus the beam's hidden-vector chunks.
template <typename DT, int CH>
__host__ __device__ constexpr int kTaskTokens() {
    constexpr int kRw = sizeof(DT) == 2 ? 4 : 8;
    return 4 * CH * kRw + CH * 8 <= 96 ? 4 : (2 * CH * kRw + CH * 8 <= 96 ? 2 : 1);
}

// The whole sparse step of query q by one workgroup (body of k_step_query and
// of each step of k_decode_tail).  rows_q / acc_q: the query's K beam rows
// and accumulated log-probs (global or LDS).  smem: the query_lds layout of
// this step; best: LDS [64], left holding the query's K winning keys;
// nrows / nacc: NULL, or LDS [K] receiving the next rows and log-probs.
// Every sum is per wave or over fixed slots, so any workgroup size (a
// multiple of 64) gives the same bits.
//
// G > 1 workgroups per query (g = 0..G-1): each scores its share of the
// query's scoring tasks (phase 1b) and writes the scores to gz [K * 64 + S]
// as well; the workgroup that finishes last (a per-query arrival count in
// *gcnt, which it resets) reads the others' scores back and completes the
// step.  No workgroup waits for another.
template <typename DT, int NT, int CH>
__device__ void step_query_block(const StepDev& st, int q, int K, int Kc, int d, const DT* __restrict__ hidden,
                                 const DT* __restrict__ W, const int32_t* __restrict__ rows_q,
                                 const float* __restrict__ acc_q, const uint64_t* __restrict__ pre,
                                 const int32_t* __restrict__ pre_off, int64_t pre_cap, int pre_min,
                                 int32_t* __restrict__ out_tok, int32_t* __restrict__ out_par,
                                 int32_t* __restrict__ out_rows, float* __restrict__ out_logp, unsigned char* smem,
                                 uint64_t* best, int32_t* nrows, float* nacc, int G = 1, int g = 0,
                                 float* __restrict__ gz = nullptr, int* __restrict__ gcnt = nullptr) {
    __shared__ float red_f[red_slots<NT>()];
    __shared__ int red_i[NT / kWave];
    __shared__ uint64_t bcast;
    // per beam, from its row: row, accumulated log-prob, row start, width
    // (negative: -1 - width of a row too wide for phases 1 / 1b)
    __shared__ int32_t r_s[kWave];
    __shared__ float a_s[kWave];
    __shared__ uint32_t e0_s[kWave];
    __shared__ int n_s[kWave];
    __shared__ int nbig;
    __shared__ int big[kWave];
    __shared__ int nsm;               // rows scored in phases 1 - 1c: 2..kSmallRow tokens, and wider
    __shared__ int sml[kWave];        // CSR rows whose tokens fit the flat buffer tok_s / z_s together
    __shared__ int sn[kWave];         // their widths
    __shared__ int mbase[kWave];      // -1: fixed slots tokq / zmid; else the row's start in tok_s / z_s
    __shared__ int nmed;              // rows with mbase >= 0
    __shared__ int moff[kWave + 1];   // their first scoring task
    __shared__ int ncand;             // keys in the candidate list qkeys
    __shared__ int ident;             // the step is the identity (see the prologue)
    __shared__ int last;              // G > 1: this workgroup completes the step
    __shared__ uint64_t slot[kWave];  // survivors of one wide row
    const QueryLds lay = query_lds(st.S, K, Kc, d, NT);
    uint64_t* qkeys = reinterpret_cast<uint64_t*>(smem + lay.qkeys);
    uint64_t* stage = reinterpret_cast<uint64_t*>(smem + lay.stage);
    int* list = reinterpret_cast<int*>(smem + lay.list);
    float* z_s = reinterpret_cast<float*>(smem + lay.z);
    float* h_s = reinterpret_cast<float*>(smem + lay.h);
    uint16_t* tok_s = reinterpret_cast<uint16_t*>(smem + lay.tok);
    uint16_t* tokq = reinterpret_cast<uint16_t*>(smem + lay.tokq);
    float* zmid = reinterpret_cast<float*>(smem + lay.zmid);
    int* jmid = reinterpret_cast<int*>(smem + lay.zmid);  // wide rows: positions of their survivors

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    constexpr int NW = NT / kWave;

    // prologue, one lane per beam (wave 0; K <= 64): the beam's row and
    // accumulated log-prob, then its row pointers and first token, all beams'
    // loads in flight together.  A row with one valid token needs nothing
    // more: its log-softmax is exactly 0 whatever its score (z - (z + log 1)),
    // so neither its hidden vector nor its W_t row is read and its candidate
    // key is the beam's accumulated log-prob.  Rows of 2..64 tokens (CSR) go
    // to phase 1, and so do wider CSR rows while their tokens fit the S slots
    // of the flat buffer; the rest and bitmap rows go to phase 2.
    if (wv == 0) {
        const int k = lane;
        const int32_t r = k < K ? rows_q[k] : -1;
        const float a = k < K ? acc_q[k] : -INFINITY;
        const bool live = k < K && beam_live(st, r, a);
        const uint32_t e0 = live ? st.row_ptr[r] : 0u;
        const int n = live ? (int)(st.row_ptr[r + 1] - e0) : 0;
        const int f0 = live && st.tok0 ? (int)st.tok0[r] : 0;  // in flight with row_ptr
        const bool csr = st.store == CB_STORE_CSR;
        const bool one = live && csr && n == 1 && st.tok0;
        const bool narrow = live && csr && !one && n <= kSmallRow;
        // wider CSR rows, in slot order while their tokens fit the S slots of
        // tok_s / z_s (free until phase 2): scored with the narrow rows
        const bool mcand = live && csr && n > kSmallRow;
        const int mincl = wave_inclusive_scan(mcand ? n : 0);
        const bool medium = mcand && mincl <= st.S;
        const bool wide = live && !one && !narrow && !medium;
        if (live) {
            r_s[k] = r;
            a_s[k] = a;
            e0_s[k] = e0;
            n_s[k] = (one || narrow) ? n : -1 - n;  // negative: survivors listed in tokq / jmid
        }
        if (one) tokq[k * kWave] = (uint16_t)f0;
        const uint64_t key = one ? make_key(a + 0.f, k, f0) : 0ull;
        const uint64_t m_one = __ballot(one), m_nar = __ballot(narrow || medium), m_wide = __ballot(wide),
                       m_live = __ballot(live), m_med = __ballot(medium);
        const uint64_t below = (1ull << lane) - 1ull;
        if (one) qkeys[__popcll(m_one & below)] = key;
        if (narrow || medium) {
            const int i = __popcll(m_nar & below);
            sml[i] = k;
            sn[i] = n;
            mbase[i] = medium ? mincl - n : -1;
        }
        if (wide) big[__popcll(m_wide & below)] = k;
        // identity: every live row has one token, the live slots come first
        // and their log-probs do not increase, so the K candidates (acc_k,
        // k, token) are already in (score desc, parent asc) order and slot i
        // of the output is beam i
        const float a_prev = __shfl(a, lane > 0 ? lane - 1 : 0);
        const bool viol = live && lane > 0 && !(a_prev >= a);
        const bool id = m_live == m_one && (m_live & (m_live + 1ull)) == 0ull && __ballot(viol) == 0ull;
        if (id && g == 0) {
            best[lane] = key;
            if (k < K) {
                const int64_t o = (int64_t)q * K + k;
                out_tok[o] = one ? f0 : -1;
                out_par[o] = one ? k : -1;
                out_rows[o] = one ? (int32_t)e0 : -1;
                out_logp[o] = one ? a + 0.f : -INFINITY;
                if (nrows) {
                    nrows[k] = one ? (int32_t)e0 : -1;
                    nacc[k] = one ? a + 0.f : -INFINITY;
                }
            }
        }
        if (lane == 0) {
            ncand = __popcll(m_one);
            nsm = __popcll(m_nar);
            nmed = __popcll(m_med);
            nbig = __popcll(m_wide);
            ident = id;
        }
    }
    __syncthreads();
    if (ident) return;  // uniform over the workgroup

    // phase 1: the tokens of every row of 2..64 tokens (CSR) into the
    // query's fixed slots tokq[k * 64 + j], all rows at once (one global round
    // trip); rows whose scores were computed apart get them here too
    const int ns = nsm;
    for (int x = tid; x < ns * kWave; x += NT) {
        const int i = x / kWave, k = sml[i], j = x % kWave, n = sn[i];
        if (j < n && mbase[i] < 0) {
            tokq[k * kWave + j] = st.tok[e0_s[k] + j];
            if (pre && n > pre_min)
                zmid[k * kWave + j] =
                    __uint_as_float((uint32_t)(pre[(int64_t)q * pre_cap + pre_off[(int64_t)q * (K + 1) + k] + j] >> 32));
        }
    }
    for (int i = 0; nmed && i < ns; ++i) {  // the wider rows: every token of one row per pass
        const int base = mbase[i];
        if (base < 0) continue;
        const int k = sml[i], n = sn[i];
        for (int j = tid; j < n; j += NT) {
            tok_s[base + j] = st.tok[e0_s[k] + j];
            if (pre && n > pre_min)
                z_s[base + j] =
                    __uint_as_float((uint32_t)(pre[(int64_t)q * pre_cap + pre_off[(int64_t)q * (K + 1) + k] + j] >> 32));
        }
    }
    if (wv == 0) {
        // tasks of MT consecutive tokens of one row, over every row still to score
        const int n = lane < ns ? sn[lane] : 0;
        const int c = lane < ns && !(pre && n > pre_min) ? (n + kTaskTokens<DT, CH>() - 1) / kTaskTokens<DT, CH>() : 0;
        const int incl = wave_inclusive_scan(c);
        if (lane < ns) moff[lane + 1] = incl;
        if (lane == 0) moff[0] = 0;
    }
    __syncthreads();

    // phase 1b: scores of those rows, by the whole block.  Their tokens form
    // a flat list of tasks of MT consecutive tokens of one row; each wave
    // takes TPW tasks at a time, so that every wave has TPW * MT W_t rows in
    // flight and all the rows of the query are scored in as few global round
    // trips as the block's width allows.  Per token the products are summed
    // chunk by chunk, then by the wave butterfly.
    constexpr int kRw = sizeof(DT) == 2 ? 4 : 8;  // VGPRs per 8 elements of a W_t row
    constexpr int MT = kTaskTokens<DT, CH>();
    constexpr int TPW = 2 * (MT * CH * kRw + CH * 8) <= 96 ? 2 : 1;
    const int ntask = moff[ns];
    if (G > 1 && ntask == 0 && g != 0) return;  // nothing to share: workgroup 0 does the step alone
    const bool handoff = G > 1 && ntask > 0;
    // this workgroup's share of the tasks
    const int tb = handoff ? (int)((int64_t)ntask * g / G) : 0;
    const int te = handoff ? (int)((int64_t)ntask * (g + 1) / G) : ntask;
    for (int t0 = tb + wv; t0 < te; t0 += TPW * NW) {
        int kq[TPW], j0[TPW], nn[TPW], mb[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int task = t0 + u * NW;
            int lo = 0;
            if (task < te) {  // the row whose tasks hold this one: last i with moff[i] <= task
                int hi = ns;
                while (hi - lo > 1) {
                    const int md = (lo + hi) >> 1;
                    if (moff[md] <= task) lo = md; else hi = md;
                }
            }
            kq[u] = task < te ? sml[lo] : 0;
            j0[u] = task < te ? (task - moff[lo]) * MT : 0;
            nn[u] = task < te ? min(MT, sn[lo] - j0[u]) : 0;
            mb[u] = task < te ? mbase[lo] : -1;
        }
        Raw8<DT> hr[TPW][CH];
        Raw8<DT> w8[TPW][MT][CH];
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int i2 = c * kWave * 8 + lane * 8;
                if (nn[u] > 0 && i2 < d) hr[u][c].load(hidden + ((int64_t)q * K + kq[u]) * d + i2);
                else hr[u][c].zero();
            }
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int jj = 0; jj < MT; ++jj) {
                const bool on = jj < nn[u];
                const int tkn = !on ? 0 : mb[u] < 0 ? (int)tokq[kq[u] * kWave + j0[u] + jj]
                                                    : (int)tok_s[mb[u] + j0[u] + jj];
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const int i2 = c * kWave * 8 + lane * 8;
                    if (on && i2 < d) w8[u][jj][c].load(W + (int64_t)tkn * d + i2);
                    else w8[u][jj][c].zero();
                }
            }
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int jj = 0; jj < MT; ++jj) {
                float sv = 0.f;
#pragma unroll
                for (int c = 0; c < CH; ++c) sv = w8[u][jj][c].dot_raw(hr[u][c], sv);
                const float t = wave_sum(sv);
                if (lane == 0 && jj < nn[u]) {
                    const int zi = mb[u] < 0 ? kq[u] * kWave + j0[u] + jj : K * kWave + mb[u] + j0[u] + jj;
                    if (mb[u] < 0) zmid[zi] = t;
                    else z_s[mb[u] + j0[u] + jj] = t;
                    // device-coherent store (no cache write-back needed before the hand-off)
                    if (handoff) __hip_atomic_store(gz + zi, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
    }
    __syncthreads();
    if (handoff) {
        // hand-off: the scores went out as device-coherent stores; every
        // wave waits until its stores are acknowledged, then one arrival per
        // workgroup on the query's count (a device-coherent atomic); the
        // last to arrive resets the count and reads the others' scores with
        // device-coherent loads, the rest stop
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(gcnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = prev == G - 1;
            if (last) __hip_atomic_store(gcnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!last) return;  // uniform over the workgroup
        for (int x = tid; x < ns * kWave; x += NT) {
            const int i = x / kWave, k = sml[i], j = x % kWave, n = sn[i];
            if (j < n && mbase[i] < 0 && !(pre && n > pre_min))
                zmid[k * kWave + j] = __hip_atomic_load(gz + k * kWave + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        for (int i = 0; nmed && i < ns; ++i) {
            const int base = mbase[i], n = sn[i];
            if (base < 0 || (pre && n > pre_min)) continue;
            for (int j = tid; j < n; j += NT)
                z_s[base + j] = __hip_atomic_load(gz + K * kWave + base + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    }
    // phase 1c: softmax and the beam's best min(n, Kc) keys, one wave per row
    // (the reductions only over the lanes the row occupies)
    for (int i = wv; i < ns; i += NW) {
        const int k = sml[i], n = sn[i], base = mbase[i];
        if (base >= 0) {
            // a wider row, 64 tokens at a time: max, then the sum of exps, then
            // its best min(n, Kc) keys by sorting each 64 and merging
            const float* zr = z_s + base;
            const uint16_t* tr = tok_s + base;
            float m = -INFINITY;
            for (int c0 = 0; c0 < n; c0 += kWave) m = fmaxf(m, c0 + lane < n ? zr[c0 + lane] : -INFINITY);
            m = wave_max(m);
            float se = 0.f;
            for (int c0 = 0; c0 < n; c0 += kWave) se += c0 + lane < n ? exp_sm(zr[c0 + lane] - m) : 0.f;
            const float lse = m + logf(wave_sum(se));
            auto keyj = [&](int j) { return j < n ? make_key(a_s[k] + (zr[j] - lse), k, (int)tr[j]) : 0ull; };
            uint64_t top = 0ull;
            if (n <= 4 * kWave) {
                // up to 4 keys per lane: the threshold selection, ranked in one
                // window of the wave's 64 stage slots when it holds <= 64 keys
                uint64_t kv[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) kv[x] = keyj(lane + x * kWave);
                auto sc = [&](int x) { return (uint32_t)(kv[x] >> 32); };
                auto kf = [&](int x) { return kv[x]; };
                if (n <= 2 * kWave) top = wave_top<2, kWave>(Kc, sc, kf, stage + wv * kWave);
                else top = wave_top<4, kWave>(Kc, sc, kf, stage + wv * kWave);
            } else {
                for (int c0 = 0; c0 < n; c0 += kWave) {
                    const uint64_t key = wave_sort_desc(keyj(c0 + lane));
                    top = c0 == 0 ? key : wave_merge_top(top, key);
                }
            }
            const bool sv = lane < Kc && top != 0ull;
            if (sv) {
                // the survivor's token and its position in the row (ascending tokens)
                const int tkn = 65535 - (int)(top & 0xFFFFu);
                int lo = 0, hi = n;
                while (lo < hi) {
                    const int md = (lo + hi) >> 1;
                    if ((int)tr[md] < tkn) lo = md + 1; else hi = md;
                }
                tokq[k * kWave + lane] = (uint16_t)tkn;
                jmid[k * kWave + lane] = lo;
            }
            wave_append(sv, top, qkeys, &ncand);
            continue;
        }
        const bool on = lane < n;
        const float z = on ? zmid[k * kWave + lane] : -INFINITY;
        const int tk = on ? (int)tokq[k * kWave + lane] : 0;
        const int w = pow2_at_least(n);
        const float m = wave_max_w(z, w);
        const float se = wave_sum_w(on ? exp_sm(z - m) : 0.f, w);
        const float lse = m + logf(se);
        uint64_t key = on ? make_key(a_s[k] + (z - lse), k, tk) : 0ull;
        if (n > Kc)  // the row's Kc best (one key per lane: one window of at most 64 to rank)
            key = wave_top<1, kWave>(Kc, [&](int) { return (uint32_t)(key >> 32); }, [&](int) { return key; },
                                     stage + wv * kWave);
        wave_append(lane < min(n, Kc), key, qkeys, &ncand);
    }
    __syncthreads();

    // phase 2: wide rows left over and bitmap rows, the whole block per beam
    const int nb = nbig;
    for (int i = 0; i < nb; ++i) {
        const int k = big[i];
        const int64_t b = (int64_t)q * K + k;
        const int32_t r = r_s[k];
        const float a = a_s[k];
        const uint32_t e0 = e0_s[k];
        const int n = -1 - n_s[k];
        block_fill_tokens<NT>(st, r, e0, n, tok_s, red_i);
        if (pre) {  // scored apart, across many workgroups
            const uint64_t* zp = pre + (int64_t)q * pre_cap + pre_off[(int64_t)q * (K + 1) + k];
            for (int j = tid; j < n; j += NT) z_s[j] = __uint_as_float((uint32_t)(zp[j] >> 32));
            __syncthreads();
        } else {
            for (int x = tid; x < d; x += NT) h_s[x] = to_f32(hidden[b * d + x]);
            __syncthreads();
            block_scores_ch<DT, NT, CH>(h_s, W, d, tok_s, n, z_s);
            __syncthreads();
        }
        const float lse = block_lse<NT>(z_s, n, red_f);
        auto keyf = [&](int j) { return make_key(a + (z_s[j] - lse), k, (int)tok_s[j]); };
        if (n <= Kc) {
            for (int j = tid; j < Kc; j += NT) slot[j] = j < n ? keyf(j) : 0ull;
        } else {
            block_select_top<NT>(n, Kc, keyf, slot, stage, list, red_i, &bcast);
        }
        __syncthreads();
        if (wv == 0) {
            const uint64_t v = lane < Kc ? slot[lane] : 0ull;
            if (v) {
                // the survivor's token and its position in the row (tok_s is
                // ascending), kept for the next row at emission
                const int tkn = 65535 - (int)(v & 0xFFFFu);
                int lo = 0, hi = n;
                while (lo < hi) {
                    const int md = (lo + hi) >> 1;
                    if ((int)tok_s[md] < tkn) lo = md + 1; else hi = md;
                }
                tokq[k * kWave + lane] = (uint16_t)tkn;
                jmid[k * kWave + lane] = lo;
            }
            wave_append(v != 0ull, v, qkeys, &ncand);
        }
        __syncthreads();
    }

    // phase 3: the query's K best of its candidate list
    block_select_list<NT>(ncand, K, qkeys, best, stage, list, red_i, &bcast);
    __syncthreads();
    for (int i = tid; i < K; i += NT)
        emit_query(q, K, Kc, i, best[i], e0_s, n_s, tokq, jmid, out_tok, out_par, out_rows, out_logp, nrows, nacc);
}

template <typename DT, int NT, int CH>
__global__ __launch_bounds__(NT) void k_step_query(StepDev st, int K, int Kc, int d,
                                                   const DT* __restrict__ hidden, const DT* __restrict__ W,
                                                   const int32_t* __restrict__ beam_rows,
                                                   const float* __restrict__ acc, const uint64_t* __restrict__ pre,
                                                   const int32_t* __restrict__ pre_off, int64_t pre_cap, int pre_min,
                                                   int32_t* __restrict__ out_tok,
                                                   int32_t* __restrict__ out_par, int32_t* __restrict__ out_rows,
                                                   float* __restrict__ out_logp, int G, float* __restrict__ gz,
                                                   int64_t gz_stride, int* __restrict__ gcnt) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ uint64_t best[kWave];
    const int q = blockIdx.x / G, g = blockIdx.x % G;
    step_query_block<DT, NT, CH>(st, q, K, Kc, d, hidden, W, beam_rows + (int64_t)q * K, acc + (int64_t)q * K, pre,
                                 pre_off, pre_cap, pre_min, out_tok, out_par, out_rows, out_logp, smem, best, nullptr,
                                 nullptr, G, g, G > 1 ? gz + (int64_t)q * gz_stride : nullptr,
                                 G > 1 ? gcnt + q : nullptr);
}

// ---- dense step: per-beam expansion and per-query merge --------------------

// One workgroup per beam: the row's valid tokens, their scores (gather-dot
// against the hidden vector, or columns of the full-codebook scores), the
// log-softmax over them and the beam's best min(K, n) candidate keys.  The
// keys carry the candidate's place i in the beam's list (low 16 bits 65535 -
// i; within a beam the list is in (score desc, token asc) order, so the key
// order across beams is still (score desc, parent asc, token asc)); side[b *
// Kc + i] holds its next row << 16 | token, so that the merge emits without
// looking anything up in the index.  CH: hidden width in 512-element chunks
// kept in registers by the scoring loop (0: any width, one chunk at a time).
template <typename DT, bool DENSE, int NT, int CH>
__global__ __launch_bounds__(NT) void k_beam_expand(StepDev st, int K, int Kc, int d,
                                                    const DT* __restrict__ hidden, const DT* __restrict__ W,
                                                    const float* __restrict__ Z, const float* __restrict__ Zp,
                                                    int64_t ldz, const int32_t* __restrict__ n_live,
                                                    const int32_t* __restrict__ ci_of, int split_ok,
                                                    const int32_t* __restrict__ beam_rows,
                                                    const float* __restrict__ acc, uint64_t* __restrict__ keys_out,
                                                    uint64_t* __restrict__ side, int mode) {
    auto split_of = [&](const int32_t* nl) { return split_ok ? gemm_split(*nl, (int)ldz, d) : 1; };
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red_f[red_slots<NT>()];
    __shared__ int red_i[NT / kWave];
    __shared__ uint64_t bcast;
    const ExpandLds lay = expand_lds(st.S, d, DENSE, NT);
    uint64_t* stage = reinterpret_cast<uint64_t*>(smem + lay.stage);
    float* z_s = reinterpret_cast<float*>(smem + lay.z);
    int* list = reinterpret_cast<int*>(smem + lay.list);
    float* h_s = reinterpret_cast<float*>(smem + lay.h);
    uint16_t* tok_s = reinterpret_cast<uint16_t*>(smem + lay.tok);

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    uint64_t* out = keys_out + (int64_t)b * Kc;
    const int32_t r = beam_rows[b];
    const float a = acc[b];
    if (!beam_live(st, r, a)) {
        for (int j = tid; j < Kc; j += NT) out[j] = 0;
        return;
    }
    const uint32_t e0 = st.row_ptr[r];
    const int n = (int)(st.row_ptr[r + 1] - e0);
    block_fill_tokens<NT>(st, r, e0, n, tok_s, red_i);
    if (!DENSE && n > 1)
        for (int i = tid; i < d; i += NT) h_s[i] = to_f32(hidden[(int64_t)b * d + i]);
    __syncthreads();
    if (!DENSE && n == 1) {
        // one valid token: log-softmax 0 whatever the score (no reads)
        if (tid == 0) z_s[0] = 0.f;
    } else if (DENSE) {
        const int split = split_of(n_live);
        if (split == 1) {
            const float* zb = Z + (int64_t)b * ldz;
            for (int j = tid; j < n; j += NT) z_s[j] = zb[tok_s[j]];
        } else {
            const float* zb = Zp + (int64_t)ci_of[b] * ldz;
            for (int j = tid; j < n; j += NT) {
                float z = 0.f;
                for (int x = 0; x < split; ++x) z += zb[(int64_t)x * kSplitRows * ldz + tok_s[j]];
                z_s[j] = z;
            }
        }
    } else if constexpr (CH > 0) {
        // 16 tokens per wave with all their W_t row chunks in flight
        block_scores_ch<DT, NT, CH, 128>(h_s, W, d, tok_s, n, z_s);
    } else {
        block_scores<DT, NT>(h_s, W, d, tok_s, n, z_s);
    }
    __syncthreads();
    float lse;
    if (DENSE && mode == CB_MODE_SCORE_FIRST) {
        // score first: the denominator covers every column of the score row
        const int split = split_of(n_live);
        const float* zb = split == 1 ? Z + (int64_t)b * ldz : Zp + (int64_t)ci_of[b] * ldz;
        auto zc = [&](int c) {
            float z = 0.f;
            for (int x = 0; x < split; ++x) z += zb[(int64_t)x * kSplitRows * ldz + c];
            return z;
        };
        float m = -INFINITY;
        for (int c = tid; c < (int)ldz; c += NT) m = fmaxf(m, zc(c));
        m = block_max<NT>(m, red_f);
        float se = 0.f;
        for (int c = tid; c < (int)ldz; c += NT) se += exp_sm(zc(c) - m);
        lse = m + logf(block_sum<NT>(se, red_f));
    } else {
        lse = block_lse<NT>(z_s, n, red_f);
    }
    const int parent = b % K;
    // selected by the candidate's position j in the row (the same order as by
    // token: a row's tokens ascend), then re-keyed by its place in the list
    __shared__ uint64_t sel_s[kWave];
    auto keyf = [&](int j) { return make_key(a + (z_s[j] - lse), parent, j); };
    if (n <= Kc) {
        for (int j = tid; j < Kc; j += NT) sel_s[j] = j < n ? keyf(j) : 0ull;
    } else {
        block_select_top<NT>(n, Kc, keyf, sel_s, stage, list, red_i, &bcast);
    }
    __syncthreads();
    for (int i = tid; i < Kc; i += NT) {
        uint64_t key = sel_s[i];
        if (key) {
            const int j = 65535 - (int)(key & 0xFFFFu);
            side[(int64_t)b * Kc + i] = ((uint64_t)(e0 + (uint32_t)j) << 16) | tok_s[j];
            key = (key & ~0xFFFFull) | (uint64_t)(65535 - i);
        }
        out[i] = key;
    }
}

// Outputs of a query's merge.
struct MergeOut {
    int32_t* tok;
    int32_t* par;
    int32_t* rows;
    float* logp;
};

// The query's K best of its K * Kc candidate keys, one wavefront: lane l
// owns keys l + 64 i (i < M).  side: NULL when the keys carry tokens (the
// bitmap expansion; the next row comes from the step table), else the
// per-beam side information of k_beam_expand (keys carry list places).
template <int M>
__device__ __forceinline__ void merge_query_wave(const StepDev& st, int q, int K, int Kc,
                                                 const uint64_t* __restrict__ keys,
                                                 const uint64_t* __restrict__ side,
                                                 const int32_t* __restrict__ beam_rows, const MergeOut& mo, int mode,
                                                 uint64_t* wl, int solo_done = 0) {
    const int lane = threadIdx.x & (kWave - 1);
    const int n = K * Kc;
    const uint64_t* src = keys + (int64_t)q * n;
    uint64_t kv[M];
    // branch-free loads (indices past the list re-read its last key, then
    // masked), so that all M loads are in flight together
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int c = lane + kWave * i;
        const uint64_t v = src[min(c, n - 1)];
        kv[i] = c < n ? v : 0ull;
    }
    if (solo_done) {
        // keys of one parent only: the query's one live beam wrote its outputs
        float pmin = 2048.f, pmax = -1.f;
#pragma unroll
        for (int i = 0; i < M; ++i)
            if (kv[i]) {
                const float pf = (float)((kv[i] >> 16) & 1023u);
                pmin = fminf(pmin, pf);
                pmax = fmaxf(pmax, pf);
            }
        pmin = -wave_max(-pmin);
        pmax = wave_max(pmax);
        if (pmax >= 0.f && pmin == pmax) return;  // uniform over the wavefront
    }
    const uint64_t best = wave_top<M>(K, [&](int i) { return (uint32_t)(kv[i] >> 32); }, [&](int i) { return kv[i]; },
                                      wl);
    if (lane < K && side) {
        const int64_t o = (int64_t)q * K + lane;
        if (!best) {
            mo.tok[o] = -1;
            mo.par[o] = -1;
            mo.rows[o] = -1;
            mo.logp[o] = -INFINITY;
        } else {
            const int parent = 1023 - (int)((best >> 16) & 1023u);
            const int i = 65535 - (int)(best & 0xFFFFu);
            const uint64_t info = side[((int64_t)q * K + parent) * Kc + i];
            mo.tok[o] = (int32_t)(info & 0xFFFFu);
            mo.par[o] = parent;
            mo.rows[o] = (int32_t)(info >> 16);
            mo.logp[o] = score_from_order_bits((uint32_t)(best >> 32));
        }
    } else if (lane < K) {
        if (mode == CB_MODE_UNCONSTRAINED) {
            // no catalog: every live beam sits at row 0 of the next table
            const int64_t o = (int64_t)q * K + lane;
            mo.tok[o] = best ? 65535 - (int)(best & 0xFFFFu) : -1;
            mo.par[o] = best ? 1023 - (int)((best >> 16) & 1023u) : -1;
            mo.rows[o] = best ? 0 : -1;
            mo.logp[o] = best ? score_from_order_bits((uint32_t)(best >> 32)) : -INFINITY;
        } else {
            emit(st, q, K, lane, best, beam_rows, mo.tok, mo.par, mo.rows, mo.logp);
        }
    }
}

// Dense path on a bitmap step: one wavefront per beam, four beams per
// workgroup.  Lane l owns the M columns g*256 + 4l .. g*256 + 4l + 3
// (g < M/4), so that every 16-byte load of the wave reads 1 KB of the score
// row contiguously; their scores (summed over the k-slices, if any) and
// validity bits stay in registers; softmax and the beam's best min(K, n) keys
// use wave reductions only.  Requires V <= 64*M and V % 4 == 0.  MODE: the
// decoding variant (a template argument, so that the per-column tests are
// the variant's own and nothing else: this kernel is bound by the issue of
// its per-column instructions, four cycles each for a 64-lane wave).
template <int M, int MODE>
__global__ __launch_bounds__(256) void k_expand_bitmap(StepDev st, int R, int K, int Kc, int V, int d,
                                                       const float* __restrict__ Z, const float* __restrict__ Zp,
                                                       const int32_t* __restrict__ n_live,
                                                       const int32_t* __restrict__ ci_of,
                                                       const int32_t* __restrict__ beam_rows,
                                                       const float* __restrict__ acc, uint64_t* __restrict__ keys_out,
                                                       MergeOut mo) {
    static_assert(M % 4 == 0 && M <= 64, "columns are read 4 at a time, at most 64 per lane");
    constexpr int G = M / 4;
    __shared__ uint64_t wl_all[4][kWaveListCap + kWave];
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int b = blockIdx.x * 4 + wv;
    if (b >= R) return;
    uint64_t* out = keys_out + (int64_t)b * Kc;
    const int32_t r = beam_rows[b];
    const float a = acc[b];
    if (!beam_live(st, r, a)) {
        if (lane < Kc) out[lane] = 0;
        return;
    }
    // the beam alone in its query (the root step of a decode): its best keys
    // are the query's outputs, written here (the merge then skips the query)
    const int qb = b / K, parent = b - qb * K;
    bool solo = false;
    uint32_t e0 = 0u;
    if (MODE != CB_MODE_UNCONSTRAINED && mo.tok) {
        const int32_t rk = lane < K ? beam_rows[(int64_t)qb * K + lane] : -1;
        const float ak = lane < K ? acc[(int64_t)qb * K + lane] : -INFINITY;
        solo = __ballot(lane < K && beam_live(st, rk, ak)) == (1ull << parent);
        e0 = st.row_ptr[r];
    }
    auto col = [&](int i) { return (i >> 2) * (kWave * 4) + lane * 4 + (i & 3); };
    const uint32_t* rb = MODE == CB_MODE_UNCONSTRAINED ? nullptr : st.bits + (int64_t)r * st.words;
    const int split = gemm_split(*n_live, V, d);
    const float* zb = split == 1 ? Z + (int64_t)b * V : Zp + (int64_t)ci_of[b] * V;
    float z[M];
#pragma unroll
    for (int i = 0; i < M; ++i) z[i] = 0.f;
#pragma unroll
    for (int x = 0; x < kSplitMax; ++x) {
        if (x < split) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                // columns past the row re-read its last four (in bounds, no
                // branch around the loads); their validity bits are 0
                const int c = min(col(4 * g), V - 4);
                const float4 v4 = *reinterpret_cast<const float4*>(zb + (int64_t)x * kSplitRows * V + c);
                z[4 * g] += v4.x;
                z[4 * g + 1] += v4.y;
                z[4 * g + 2] += v4.z;
                z[4 * g + 3] += v4.w;
            }
        }
    }
    // validity of this lane's columns: the row's bitmap read once (lane l
    // holds words l and l + 64), then group g's four bits, which lie in word
    // 8g + l/8 at bit 4(l%8), fetched from the lane holding that word
    uint32_t vb[G];
    uint32_t w0 = 0u, w1 = 0u;
    const int words = (V + 31) >> 5;
    if constexpr (MODE != CB_MODE_UNCONSTRAINED) {
        w0 = rb[min(lane, words - 1)];
        w1 = G > 8 ? rb[min(lane + kWave, words - 1)] : 0u;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int src = (g * 8 + (lane >> 3)) & (kWave - 1);
            const uint32_t w = (uint32_t)__shfl((int)(g < 8 ? w0 : w1), src);
            vb[g] = col(4 * g) < V ? (w >> ((lane & 7) * 4)) & 0xFu : 0u;
        }
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) vb[g] = col(4 * g) < V ? 0xFu : 0u;
    }
    // candidates: the row's valid tokens, or (no constraint) every column
    auto valid = [&](int i) { return ((vb[i >> 2] >> (i & 3)) & 1u) != 0; };
    // softmax support: the candidates, or (score first) every column
    // (columns past V have validity 0, so that filter first needs no bound test)
    auto in_lse = [&](int i) { return MODE == CB_MODE_FILTER_FIRST ? valid(i) : col(i) < V; };
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < M; ++i) m = fmaxf(m, in_lse(i) ? z[i] : -INFINITY);
    m = wave_max(m);
    float se = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i) se += in_lse(i) ? exp_sm(z[i] - m) : 0.f;
    const float lse = m + logf(wave_sum(se));
    uint32_t sc[M];
#pragma unroll
    for (int i = 0; i < M; ++i) sc[i] = valid(i) ? score_order_bits(a + (z[i] - lse)) : 0u;
    const uint64_t best = wave_top<M>(
        Kc, [&](int i) { return sc[i]; },
        [&](int i) { return ((uint64_t)sc[i] << 32) | ((uint64_t)(1023 - parent) << 16) | (uint64_t)(65535 - col(i)); },
        wl_all[wv]);
    if (lane < Kc) out[lane] = best;
    if (solo) {  // uniform over the wavefront
        // next row of the lane's survivor: the row's first edge plus the set
        // bits of the row below its column (prefix counts of the words lane l
        // holds, l and l + 64)
        const int p0 = lane < words ? __popc(w0) : 0;
        const int p1 = lane + kWave < words ? __popc(w1) : 0;
        const int x0 = wave_inclusive_scan(p0) - p0;
        const int x1 = wave_inclusive_scan(p1) - p1 + lane_bcast(x0 + p0, kWave - 1);
        const int c = best ? 65535 - (int)(best & 0xFFFFu) : 0;
        const int wd = c >> 5, src = wd & (kWave - 1);
        const int pre0 = __shfl(x0, src), pre1 = __shfl(x1, src);
        const uint32_t bw0 = (uint32_t)__shfl((int)w0, src), bw1 = (uint32_t)__shfl((int)w1, src);
        const uint32_t bits = wd < kWave ? bw0 : bw1;
        const int nxt = (int)(e0 + (uint32_t)(wd < kWave ? pre0 : pre1) + (uint32_t)__popc(bits & ((1u << (c & 31)) - 1u)));
        if (lane < K) {
            const int64_t o = (int64_t)qb * K + lane;
            const bool on = lane < Kc && best != 0ull;
            mo.tok[o] = on ? c : -1;
            mo.par[o] = on ? parent : -1;
            mo.rows[o] = on ? nxt : -1;
            mo.logp[o] = on ? score_from_order_bits((uint32_t)(best >> 32)) : -INFINITY;
        }
    }
}

// Dense path on a CSR step (filter first): one wavefront per beam, four
// beams per workgroup.  The row's tokens and their score columns are gathered
// a window of 64 * U at a time (U per lane, all loads in flight); a first
// pass takes the log-sum-exp over the row (running max and sum of exps), a
// second the beam's best min(Kc, n) keys, each window's merged with the best
// so far (rows of one window keep their scores in registers between the
// passes).  Keys re-keyed by their place in the beam's list, with side
// information (next row << 16 | token), as k_beam_expand writes them.
template <int U>
__global__ __launch_bounds__(256) void k_expand_csr_wave(StepDev st, int R, int K, int Kc, int d, int64_t ldz,
                                                         const float* __restrict__ Z, const float* __restrict__ Zp,
                                                         const int32_t* __restrict__ n_live,
                                                         const int32_t* __restrict__ ci_of, int split_ok,
                                                         const int32_t* __restrict__ beam_rows,
                                                         const float* __restrict__ acc,
                                                         uint64_t* __restrict__ keys_out,
                                                         uint64_t* __restrict__ side) {
    __shared__ uint64_t wl_all[4][kWaveListCap + kWave];
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int b = blockIdx.x * 4 + wv;
    if (b >= R) return;  // uniform over the wavefront
    uint64_t* out = keys_out + (int64_t)b * Kc;
    const int32_t r = beam_rows[b];
    const float a = acc[b];
    if (!beam_live(st, r, a)) {
        if (lane < Kc) out[lane] = 0;
        return;
    }
    const uint32_t e0 = st.row_ptr[r];
    const int n = (int)(st.row_ptr[r + 1] - e0);  // >= 1: every row of a table has a child
    const int split = split_ok ? gemm_split(*n_live, (int)ldz, d) : 1;
    const float* zb = split == 1 ? Z + (int64_t)b * ldz : Zp + (int64_t)ci_of[b] * ldz;
    constexpr int WIN = kWave * U;
    // positions past the row re-read its last token (in bounds, no branch
    // around the loads) and are masked
    auto window = [&](int c0, float (&z)[U]) {
        int tk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) tk[u] = st.tok[e0 + min(c0 + u * kWave + lane, n - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v = 0.f;
            for (int x = 0; x < split; ++x) v += zb[(int64_t)x * kSplitRows * ldz + tk[u]];
            z[u] = c0 + u * kWave + lane < n ? v : -INFINITY;
        }
    };
    float z0[U];
    float m = -INFINITY, sm = 0.f;
    for (int c0 = 0; c0 < n; c0 += WIN) {
        float z[U];
        window(c0, z);
        if (c0 == 0)
#pragma unroll
            for (int u = 0; u < U; ++u) z0[u] = z[u];
        float wmx = z[0];
#pragma unroll
        for (int u = 1; u < U; ++u) wmx = fmaxf(wmx, z[u]);
        const float mn = fmaxf(m, wave_max(wmx));  // finite: the window holds a token of the row
        float ws = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) ws += exp_sm(z[u] - mn);  // masked positions add exp(-inf) = 0
        sm = sm * exp_sm(m - mn) + wave_sum(ws);
        m = mn;
    }
    const float lse = m + logf(sm);
    const int parent = b % K;
    uint64_t best = 0;
    for (int c0 = 0; c0 < n; c0 += WIN) {
        float z[U];
        if (c0 == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) z[u] = z0[u];
        } else {
            window(c0, z);
        }
        uint32_t sc[U + 1];
#pragma unroll
        for (int u = 0; u < U; ++u) sc[u] = c0 + u * kWave + lane < n ? score_order_bits(a + (z[u] - lse)) : 0u;
        sc[U] = (uint32_t)(best >> 32);
        const uint64_t prev = best;
        best = wave_top<U + 1>(
            Kc, [&](int i) { return sc[i]; },
            [&](int i) {
                return i < U ? ((uint64_t)sc[i] << 32) | ((uint64_t)(1023 - parent) << 16) |
                                   (uint64_t)(65535 - (c0 + i * kWave + lane))
                             : prev;
            },
            wl_all[wv]);
    }
    if (lane < Kc) {
        uint64_t key = best;
        if (key) {
            const int j = 65535 - (int)(key & 0xFFFFu);
            side[(int64_t)b * Kc + lane] = ((uint64_t)(e0 + (uint32_t)j) << 16) | st.tok[e0 + j];
            key = (key & ~0xFFFFull) | (uint64_t)(65535 - lane);
        }
        out[lane] = key;
    }
}

// Dense path, per query: one wavefront per query, four queries per workgroup.
template <int M>
__global__ __launch_bounds__(256) void k_query_merge_w(StepDev st, int Q, int K, int Kc,
                                                       const uint64_t* __restrict__ keys,
                                                       const uint64_t* __restrict__ side,
                                                       const int32_t* __restrict__ beam_rows, MergeOut mo, int mode,
                                                       int solo_done) {
    __shared__ uint64_t wl_all[4][kWaveListCap + kWave];
    const int wv = threadIdx.x / kWave;
    const int q = blockIdx.x * 4 + wv;
    if (q >= Q) return;
    merge_query_wave<M>(st, q, K, Kc, keys, side, beam_rows, mo, mode, wl_all[wv], solo_done);
}

// ---- full-codebook scores of the live beams (dense path) ------------------

// Compact list of the live beam slots (ascending), their count, and the
// compact index of every slot (-1 when dead).
template <int NT>
__global__ __launch_bounds__(NT) void k_live_rows(StepDev st, int R, const int32_t* __restrict__ beam_rows,
                                                  const float* __restrict__ acc, int32_t* __restrict__ live,
                                                  int32_t* __restrict__ n_live, int32_t* __restrict__ ci_of) {
    // rounds of U * NT slots: slot r0 + u * NT + tid for u < U (coalesced, all
    // loads in flight at once); each wavefront's count per u by a ballot, then
    // one scan over the (u, wavefront) counts in slot order
    constexpr int U = 8, NW = NT / kWave;
    static_assert(U * NW <= NT, "one thread per (u, wavefront) count");
    __shared__ int wc[U * NW];
    __shared__ int red_i[NW];
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const uint64_t below = (1ull << lane) - 1ull;
    int base = 0;
    for (int r0 = 0; r0 < R; r0 += U * NT) {
        bool x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = r0 + u * NT + (int)threadIdx.x;
            x[u] = b < R && beam_live(st, beam_rows[b], acc[b]);
        }
        uint64_t m[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            m[u] = __ballot(x[u]);
            if (lane == 0) wc[u * NW + wv] = __popcll(m[u]);
        }
        __syncthreads();
        const int c = (int)threadIdx.x < U * NW ? wc[threadIdx.x] : 0;
        int tot;
        const int o = block_exclusive_scan<NT>(c, red_i, &tot);
        __syncthreads();  // every count read before it is overwritten
        if ((int)threadIdx.x < U * NW) wc[threadIdx.x] = o;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = r0 + u * NT + (int)threadIdx.x;
            if (b < R) {
                const int pos = base + wc[u * NW + wv] + __popcll(m[u] & below);
                if (x[u]) live[pos] = b;
                ci_of[b] = x[u] ? pos : -1;
            }
        }
        base += tot;
        __syncthreads();  // wc is rewritten by the next round
    }
    if (threadIdx.x == 0) *n_live = base;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Scores of the live beams against the whole codebook, bf16 in, float32
// accumulate on MFMA 32x32x16: one 128x128 tile of one k-slice per workgroup,
// 8 waves of 32x64; LDS double buffered (dynamic, 72 KiB) with the next k-tile
// prefetched into registers (native vector types, so the staging stays in
// VGPRs).  With one slice, Z[beam][v]; with several, Zp[slice][compact
// row][v].  Consecutive tiles on one XCD share W columns.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Rows of the product, three ways:
//  - every slot (all_slots = 1, R slots): tile rows are the beam slots, dead
//    ones included (their scores are never read); no prologue.  Workgroup 0
//    writes n_live = -1, which tells the consumers that the scores are one
//    slice indexed by slot.
//  - live beams found in the prologue (all_slots = 0, 0 < R <= kFoldSlots): every
//    workgroup marks the live slots (each thread a run of consecutive slots),
//    one block scan gives their compact positions, and the workgroup keeps
//    the slots of its own tile; workgroup 0 also writes n_live and ci_of.
//  - otherwise (R == 0) the compact list comes from k_live_rows.
constexpr int kFoldSlots = 4 * kGemmThreads;

__global__ __launch_bounds__(kGemmThreads) void k_gemm_bf16(int V, int d, const int32_t* __restrict__ live,
                                                            int32_t* __restrict__ n_live,
                                                            const uint16_t* __restrict__ H,
                                                            const uint16_t* __restrict__ W, float* __restrict__ Z,
                                                            float* __restrict__ Zp, int64_t ldz, StepDev st, int R,
                                                            const int32_t* __restrict__ beam_rows,
                                                            const float* __restrict__ beam_acc,
                                                            int32_t* __restrict__ ci_of, int all_slots) {
    extern __shared__ __align__(16) uint16_t gsm[];
    uint16_t* As = gsm;                     // [2][kBM * kLDP]
    uint16_t* Bs = gsm + 2 * kBM * kLDP;    // [2][kBN * kLDP]
    __shared__ int rows_s[kBM];
    __shared__ int red_i[kGemmThreads / kWave];
    constexpr int NT = kGemmThreads;
    constexpr int CA = kBM * kBK / 8 / NT, CB = kBN * kBK / 8 / NT;  // 16-byte chunks per thread
    constexpr int TJ = kWN / 32;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int L = blockIdx.x;
    int nl;
    uint32_t onmask = 0;
    int pos0 = 0, run = 0, b0 = 0;
    if (all_slots) {
        nl = -R;  // one slice over every slot (tiles from R below)
        if (L == 0 && tid == 0) *n_live = -1;
    } else if (R > 0) {
        run = (R + NT - 1) / NT;
        b0 = tid * run;
        int c = 0;
        for (int j = 0; j < run; ++j) {
            const int b = b0 + j;
            const bool on = b < R && beam_live(st, beam_rows[b], beam_acc[b]);
            onmask |= (uint32_t)on << j;
            c += on;
        }
        pos0 = block_exclusive_scan<NT>(c, red_i, &nl);
        if (L == 0) {
            int p = pos0;
            for (int j = 0; j < run; ++j)
                if (b0 + j < R) ci_of[b0 + j] = (onmask >> j & 1u) ? p++ : -1;
            if (tid == 0) *n_live = nl;
        }
    } else {
        nl = *n_live;
    }
    const int split = gemm_split(nl, V, d);
    if (all_slots) nl = R;
    const int mt = (nl + kBM - 1) / kBM, nt = (V + kBN - 1) / kBN;
    const int N = mt * nt * split;
    if (L >= N) return;  // uniform over the workgroup
    const int full = (N / 8) * 8;
    const int lin = L < full ? (L % 8) * (full / 8) + L / 8 : L;
    const int zs = lin % split, tile = lin / split;
    const int m0 = (tile % mt) * kBM, n0 = (tile / mt) * kBN;
    const int klen = d / split, kbeg = zs * klen;

    if (all_slots) {
        if (tid < kBM) rows_s[tid] = m0 + tid < R ? m0 + tid : -1;
    } else if (R > 0) {
        if (tid < kBM) rows_s[tid] = -1;
        __syncthreads();
        int p = pos0;
        for (int j = 0; j < run; ++j)
            if (onmask >> j & 1u) {
                if (p >= m0 && p < m0 + kBM) rows_s[p - m0] = b0 + j;
                ++p;
            }
    } else if (tid < kBM) {
        rows_s[tid] = m0 + tid < nl ? live[m0 + tid] : -1;
    }
    __syncthreads();
    const int wm = (wv / (kBN / kWN)) * kWM, wn = (wv % (kBN / kWN)) * kWN;

    // Rows past the live list or the codebook read a valid row instead (the
    // tile's first live beam, the last codebook row): their products are
    // never stored, and unconditional loads keep the prefetch ring free of
    // branches, so the compiler waits only for the tile it stashes.
    const uint16_t* pa[CA];
    const uint16_t* pb[CB];
    int oa[CA], ob[CB];
#pragma unroll
    for (int u = 0; u < CA; ++u) {
        const int c = tid + u * NT, r = c / (kBK / 8), cc = (c % (kBK / 8)) * 8;
        const int hb = rows_s[r] >= 0 ? rows_s[r] : rows_s[0];
        pa[u] = H + (int64_t)hb * d + kbeg + cc;
        oa[u] = r * kLDP + cc;
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
        const int c = tid + u * NT, r = c / (kBK / 8), cc = (c % (kBK / 8)) * 8;
        pb[u] = W + (int64_t)min(n0 + r, V - 1) * d + kbeg + cc;
        ob[u] = r * kLDP + cc;
    }
    // Register ring of kPF k-tiles: tile kt+kPF is requested while tile kt is
    // computed, so kPF-1 global round trips are always in flight (the loop is
    // otherwise bound by one global latency per k-tile).
    constexpr int kPF = 4;
    u32x4_t ra[kPF][CA], rb[kPF][CB];
#define CB_GEMM_FETCH(slot, k0)                                                                   \
    _Pragma("unroll") for (int x_ = 0; x_ < CA; ++x_) ra[slot][x_] =                              \
        *reinterpret_cast<const u32x4_t*>(pa[x_] + (k0));                                          \
    _Pragma("unroll") for (int x_ = 0; x_ < CB; ++x_) rb[slot][x_] =                              \
        *reinterpret_cast<const u32x4_t*>(pb[x_] + (k0));
#define CB_GEMM_STASH(slot, buf)                                                                  \
    _Pragma("unroll") for (int x_ = 0; x_ < CA; ++x_)                                             \
        *reinterpret_cast<u32x4_t*>(&As[(buf) * kBM * kLDP + oa[x_]]) = ra[slot][x_];             \
    _Pragma("unroll") for (int x_ = 0; x_ < CB; ++x_)                                             \
        *reinterpret_cast<u32x4_t*>(&Bs[(buf) * kBN * kLDP + ob[x_]]) = rb[slot][x_];

    f32x16_t acc[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

    const int nk = klen / kBK;
    // all fragments of the LDS k-tile first, then the MFMAs back to back
    auto compute = [&](int buf) {
        const uint16_t* Ab = As + buf * kBM * kLDP;
        const uint16_t* Bb = Bs + buf * kBN * kLDP;
        constexpr int NKK = kBK / 16;
        u32x4_t af[NKK], bf[NKK][TJ];
#pragma unroll
        for (int x = 0; x < NKK; ++x) {
            af[x] = *reinterpret_cast<const u32x4_t*>(&Ab[(wm + (lane & 31)) * kLDP + x * 16 + (lane >> 5) * 8]);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                bf[x][j] = *reinterpret_cast<const u32x4_t*>(
                    &Bb[(wn + j * 32 + (lane & 31)) * kLDP + x * 16 + (lane >> 5) * 8]);
        }
#pragma unroll
        for (int x = 0; x < NKK; ++x)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[x]),
                                                                 __builtin_bit_cast(bf16x8_t, bf[x][j]), acc[j],
                                                                 0, 0, 0);
    };
    if (nk % kPF == 0) {
        // Every fetch and stash unconditional (tiles past the end re-read the
        // last one, and the final stash fills an unused buffer), so the waits
        // the compiler inserts cover only the tile being stashed.
#pragma unroll
        for (int u = 0; u < kPF; ++u) {
            CB_GEMM_FETCH(u, u * kBK)
        }
        CB_GEMM_STASH(0, 0)
        __syncthreads();
        for (int kt0 = 0; kt0 < nk; kt0 += kPF) {
#pragma unroll
            for (int u = 0; u < kPF; ++u) {
                const int kt = kt0 + u;  // tile kt is in LDS buffer kt & 1; its register slot u is free
                compute(kt & 1);
                CB_GEMM_STASH((u + 1) % kPF, (kt & 1) ^ 1)
                CB_GEMM_FETCH(u, min(kt + kPF, nk - 1) * kBK)
                __syncthreads();
            }
        }
    } else {
        CB_GEMM_FETCH(0, 0)
        CB_GEMM_STASH(0, 0)
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + 1 < nk) {
                CB_GEMM_FETCH(0, (kt + 1) * kBK)
            }
            compute(kt & 1);
            if (kt + 1 < nk) {
                CB_GEMM_STASH(0, (kt & 1) ^ 1)
            }
            __syncthreads();
        }
    }
#undef CB_GEMM_FETCH
#undef CB_GEMM_STASH
    if ((V & 3) == 0 && (ldz & 3) == 0) {
        // the tile through LDS (the k loop left it free after its last
        // barrier), then out in 16-byte stores along whole rows: 2 rows of the
        // tile per wave instruction instead of 2 partial rows of 32 columns
        constexpr int LDC = kBN + 4;
        static_assert(kBM * LDC * 4 <= kGemmLds, "the output tile fits the LDS of the A and B tiles");
        float* Cs = reinterpret_cast<float*>(gsm);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int rr = wm + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
#pragma unroll
            for (int j = 0; j < TJ; ++j) Cs[rr * LDC + wn + j * 32 + (lane & 31)] = acc[j][e];
        }
        __syncthreads();
        constexpr int C4 = kBN / 4;
#pragma unroll
        for (int x = tid; x < kBM * C4; x += NT) {
            const int rr = x / C4, c = (x % C4) * 4, col = n0 + c;
            const int hb = rows_s[rr];
            if (hb < 0 || col >= V) continue;
            float* dst = split == 1 ? Z + (int64_t)hb * ldz : Zp + ((int64_t)zs * kSplitRows + m0 + rr) * ldz;
            *reinterpret_cast<float4*>(dst + col) = *reinterpret_cast<const float4*>(&Cs[rr * LDC + c]);
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int rr = wm + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        const int hb = rows_s[rr];
        if (hb < 0) continue;
        float* dst = split == 1 ? Z + (int64_t)hb * ldz : Zp + ((int64_t)zs * kSplitRows + m0 + rr) * ldz;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int col = n0 + wn + j * 32 + (lane & 31);
            if (col < V) dst[col] = acc[j][e];
        }
    }
}

// float32 full-codebook scores of the live beams: 16x16 output tile per
// workgroup, one output per thread, the k loop in ascending order.
__global__ __launch_bounds__(256) void k_gemm_f32(int V, int d, const int32_t* __restrict__ live,
                                                  const int32_t* __restrict__ n_live, const float* __restrict__ H,
                                                  const float* __restrict__ W, float* __restrict__ Z, int64_t ldz) {
    __shared__ float As[16][17], Bs[16][17];
    const int nl = *n_live;
    if ((int)blockIdx.y * 16 >= nl) return;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int ri = blockIdx.y * 16 + ty, col = blockIdx.x * 16 + tx;
    const int ar = blockIdx.y * 16 + ty < nl ? live[blockIdx.y * 16 + ty] : -1;
    const int bc = blockIdx.x * 16 + ty;
    float s = 0.f;
    for (int k0 = 0; k0 < d; k0 += 16) {
        As[ty][tx] = (ar >= 0 && k0 + tx < d) ? H[(int64_t)ar * d + k0 + tx] : 0.f;
        Bs[ty][tx] = (bc < V && k0 + tx < d) ? W[(int64_t)bc * d + k0 + tx] : 0.f;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) s = fmaf(As[ty][k], Bs[tx][k], s);
        __syncthreads();
    }
    if (ri < nl && col < V) Z[(int64_t)live[ri] * ldz + col] = s;
}

// ---- stand-in model between steps (decode only) ---------------------------

__device__ __forceinline__ void store_h(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }
__device__ __forceinline__ void store_h(float* p, float v) { *p = v; }

// h = s / ||s||_2: norm and division in double, rounded to float32 (then bf16).
template <typename DT, int NT>
__device__ void normalise_into(const float* sb, int d, DT* hb, double* red) {
    double ss = 0.0;
    for (int i = threadIdx.x; i < d; i += NT) ss += (double)sb[i] * (double)sb[i];
    ss = block_sum<NT>(ss, red);
    const double nrm = sqrt(ss);
    for (int i = threadIdx.x; i < d; i += NT) store_h(hb + i, (float)((double)sb[i] / nrm));
}

template <typename DT, int NT>
__global__ __launch_bounds__(NT) void k_decode_init(int K, int d, const float* __restrict__ q,
                                                    float* __restrict__ s_out, DT* __restrict__ h_out,
                                                    int32_t* __restrict__ rows, float* __restrict__ acc) {
    __shared__ double red[NT / kWave];
    const int b = blockIdx.x, k = b % K, qi = b / K;
    DT* hb = h_out + (int64_t)b * d;
    if (threadIdx.x == 0) {
        rows[b] = k == 0 ? 0 : -1;
        acc[b] = k == 0 ? 0.f : -INFINITY;
    }
    if (k != 0) {
        for (int i = threadIdx.x; i < d; i += NT) store_h(hb + i, 0.f);
        return;
    }
    float* sb = s_out + (int64_t)b * d;
    for (int i = threadIdx.x; i < d; i += NT) sb[i] = q[(int64_t)qi * d + i];
    __syncthreads();
    normalise_into<DT, NT>(sb, d, hb, red);
}

__device__ __forceinline__ void store_h4(uint16_t* p, float a, float b, float c, float e) {
    uint2 v;
    v.x = (uint32_t)f32_to_bf16_rne(a) | (uint32_t)f32_to_bf16_rne(b) << 16;
    v.y = (uint32_t)f32_to_bf16_rne(c) | (uint32_t)f32_to_bf16_rne(e) << 16;
    *reinterpret_cast<uint2*>(p) = v;
}
__device__ __forceinline__ void store_h4(float* p, float a, float b, float c, float e) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, e);
}

// Stand-in model update by one wavefront, of NB slots at once (their loads
// in flight together): s_new = s_old[parent slot] + P_t[token] in float32,
// h = s_new / ||s_new||_2 with the squares summed in double (fused
// multiply-adds in element order per lane, then a butterfly), rounded to
// float32 (then bf16).  Dead slots (token < 0) get h = 0; slots b < 0 are
// skipped.  REG: d a multiple of 256 and at most 256 * NV, P_t 16-byte
// aligned; every lane keeps 4 consecutive elements per 256 in registers.
// Otherwise lane-strided single elements, re-read from s_new.  Both launch
// forms make the same choice for a given (d, P), so they agree bit for bit.
template <typename DT, bool REG, int NV, int NB>
__device__ void hidden_update_wave(const int (&b)[NB], const int (&tk)[NB], const int (&par)[NB], int K, int d,
                                   const float* __restrict__ s_old, const float* __restrict__ P_t,
                                   float* __restrict__ s_new, DT* __restrict__ h_out) {
    const int lane = lane_id();
    if constexpr (REG) {
        float4 v[NB][NV];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (b[u] < 0 || tk[u] < 0) continue;  // uniform over the wavefront
            const float* sp = s_old + (int64_t)((b[u] / K) * K + par[u]) * d;
            const float* pv = P_t + (int64_t)tk[u] * d;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if (j * kWave * 4 >= d) break;
                const int i = lane * 4 + j * kWave * 4;
                const float4 x = *reinterpret_cast<const float4*>(sp + i);
                const float4 y = *reinterpret_cast<const float4*>(pv + i);
                v[u][j] = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
            }
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (b[u] < 0) continue;
            DT* hb = h_out + (int64_t)b[u] * d;
            if (tk[u] < 0) {
                for (int i = lane; i < d; i += kWave) store_h(hb + i, 0.f);
                continue;
            }
            float* sn = s_new + (int64_t)b[u] * d;
            double ss = 0.0;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if (j * kWave * 4 >= d) break;
                const float4 x = v[u][j];
                *reinterpret_cast<float4*>(sn + lane * 4 + j * kWave * 4) = x;
                ss = fma((double)x.x, (double)x.x, ss);
                ss = fma((double)x.y, (double)x.y, ss);
                ss = fma((double)x.z, (double)x.z, ss);
                ss = fma((double)x.w, (double)x.w, ss);
            }
            const double nrm = sqrt(wave_sum(ss));
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if (j * kWave * 4 >= d) break;
                const float4 x = v[u][j];
                store_h4(hb + lane * 4 + j * kWave * 4, (float)((double)x.x / nrm), (float)((double)x.y / nrm),
                         (float)((double)x.z / nrm), (float)((double)x.w / nrm));
            }
        }
    } else {
        for (int u = 0; u < NB; ++u) {
            if (b[u] < 0) continue;
            DT* hb = h_out + (int64_t)b[u] * d;
            if (tk[u] < 0) {
                for (int i = lane; i < d; i += kWave) store_h(hb + i, 0.f);
                continue;
            }
            const float* sp = s_old + (int64_t)((b[u] / K) * K + par[u]) * d;
            const float* pv = P_t + (int64_t)tk[u] * d;
            float* sn = s_new + (int64_t)b[u] * d;
            double ss = 0.0;
            for (int i = lane; i < d; i += kWave) {
                const float x = sp[i] + pv[i];
                sn[i] = x;
                ss = fma((double)x, (double)x, ss);
            }
            const double nrm = sqrt(wave_sum(ss));
            for (int i = lane; i < d; i += kWave) store_h(hb + i, (float)((double)sn[i] / nrm));
        }
    }
}

// Largest d the register-resident update takes.
constexpr int kRegMaxD = 2048;

template <typename DT, bool REG>
__global__ __launch_bounds__(256) void k_hidden_update(int R, int K, int d, const float* __restrict__ s_old,
                                                       const float* __restrict__ P_t, const int32_t* __restrict__ tok,
                                                       const int32_t* __restrict__ par, float* __restrict__ s_new,
                                                       DT* __restrict__ h_out) {
    const int b0 = blockIdx.x * 4 + (int)(threadIdx.x / kWave);
    if (b0 >= R) return;  // uniform over the wavefront
    const int b[1] = {b0}, t[1] = {tok[b0]}, p[1] = {par[b0]};
    hidden_update_wave<DT, REG, kRegMaxD / (kWave * 4), 1>(b, t, p, K, d, s_old, P_t, s_new, h_out);
}

// Persistent decode of the steps t0..L-1 (all sparse, LDS selection) with the
// stand-in model between them: one workgroup per query runs every step and
// every hidden update of its beams, so the steps need no launches in between
// (queries share nothing, so no workgroup waits for another).  Buffers [0]
// hold step t0's inputs; outputs of step t go to hist_tok/hist_par [t] and to
// the other buffer of the pair, which becomes the next step's input.
template <typename DT, int NT, int CH, bool REG>
__global__ __launch_bounds__(NT) void k_decode_tail(const StepDev* __restrict__ steps, int t0, int L, int K, int d,
                                                    int V, int R, const DT* __restrict__ W,
                                                    const float* __restrict__ P, float* s0, float* s1, DT* h,
                                                    int32_t* rows0, int32_t* rows1, float* acc0, float* acc1,
                                                    int32_t* __restrict__ hist_tok, int32_t* __restrict__ hist_par,
                                                    uint64_t* __restrict__ clk) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ uint64_t best[kWave];
    __shared__ int32_t rows_l[2][kWave];  // the query's beam rows, current and next step
    __shared__ float acc_l[2][kWave];
    const int q = blockIdx.x;
    const int wv = threadIdx.x / kWave;
    constexpr int NW = NT / kWave;
    // values per lane per slot in the register-resident update: d <= 512 * CH
    constexpr int NV = 2 * CH;
    constexpr int NB = NV <= 4 ? 2 : 1;
    float* sb[2] = {s0, s1};
    int32_t* rb[2] = {rows0, rows1};
    float* ab[2] = {acc0, acc1};
    for (int k = threadIdx.x; k < K; k += NT) {
        rows_l[0][k] = rows0[(int64_t)q * K + k];
        acc_l[0][k] = acc0[(int64_t)q * K + k];
    }
    __syncthreads();
    int cur = 0;
    for (int t = t0; t < L; ++t) {
        // phase clock (when asked): device wall clock at the step's start and
        // once its outputs are written
        if (clk && threadIdx.x == 0) clk[((int64_t)q * L + t) * 2] = wall_clock64();
        const StepDev st = steps[t];
        const int Kc = min(K, max(st.S, 1));
        int32_t* ot = hist_tok + (int64_t)t * R;
        int32_t* op = hist_par + (int64_t)t * R;
        step_query_block<DT, NT, CH>(st, q, K, Kc, d, h, W + (int64_t)t * V * d, rows_l[cur], acc_l[cur], nullptr,
                                     nullptr, 0, 0, ot, op, rb[cur ^ 1], ab[cur ^ 1], smem, best, rows_l[cur ^ 1],
                                     acc_l[cur ^ 1]);
        __syncthreads();
        if (clk && threadIdx.x == 0) clk[((int64_t)q * L + t) * 2 + 1] = wall_clock64();
        if (t + 1 < L) {
            // winners from LDS: the same (token, parent) the step wrote out
            const float* Pt = P + (int64_t)t * V * d;
            for (int k0 = wv; k0 < K; k0 += NW * NB) {
                int bb[NB], tt[NB], pp[NB];
#pragma unroll
                for (int u = 0; u < NB; ++u) {
                    const int k = k0 + u * NW;
                    const uint64_t key = k < K ? best[k] : 0ull;
                    bb[u] = k < K ? q * K + k : -1;
                    tt[u] = key ? 65535 - (int)(key & 0xFFFFu) : -1;
                    pp[u] = key ? 1023 - (int)((key >> 16) & 1023u) : -1;
                }
                hidden_update_wave<DT, REG, NV, NB>(bb, tt, pp, K, d, sb[cur], Pt, sb[cur ^ 1], h);
            }
            __syncthreads();
        }
        cur ^= 1;
    }
}

// Does nothing: the fixed cost of a dispatch (launch, wave start and drain)
// for the overhead floor.
__global__ void k_empty(int) {}

__global__ void k_backtrace(int R, int K, int L, const int32_t* __restrict__ hist_tok,
                            const int32_t* __restrict__ hist_par, int32_t* __restrict__ seqs) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= R) return;
    const int base = (b / K) * K;
    int cur = b;
    bool dead = false;
    for (int t = L - 1; t >= 0; --t) {
        const int tk = dead ? -1 : hist_tok[(int64_t)t * R + cur];
        if (tk < 0) dead = true;
        seqs[(int64_t)b * L + t] = dead ? -1 : tk;
        if (!dead) cur = base + hist_par[(int64_t)t * R + cur];
    }
    if (dead)
        for (int t = 0; t < L; ++t) seqs[(int64_t)b * L + t] = -1;
}

// Wire-format results, one workgroup per query (FlashTrie App. D.3, "Output
// serialization"): the live beams (finite log-prob) of the query's best-first
// slots written in ascending order of score, the beam of live rank r into wire
// slot n_o - 1 - r; the end offset of each sequence is the running sum of the
// lengths in wire order, from a block scan over the slots (every live sequence
// has L tokens); log-probs in float64 times the length normalisation `norm`
// (FlashTrie App. E, eq. 2).  Layout at out + q * stride: uint64 n_o, float64
// logp_norm[n_o], uint64 sent_offset[n_o], uint32 tokens[n_o * L].  Each
// thread owns `run` consecutive slots (K <= 1024, run <= 4 at 256 threads).
template <int NT>
__global__ __launch_bounds__(NT) void k_wire(int K, int L, const int32_t* __restrict__ seqs,
                                             const float* __restrict__ logp, double norm,
                                             unsigned char* __restrict__ out, int64_t stride,
                                             int64_t* __restrict__ nbytes) {
    __shared__ int red_i[NT / kWave];
    const int q = blockIdx.x, tid = threadIdx.x;
    const int run = (K + NT - 1) / NT;
    const int b0 = tid * run;
    const float* lq = logp + (int64_t)q * K;
    uint32_t on = 0;
    int c = 0;
    for (int j = 0; j < run; ++j) {
        const int i = b0 + j;
        const bool live = i < K && lq[i] > -INFINITY;
        on |= (uint32_t)live << j;
        c += live;
    }
    int n_o;
    int r = block_exclusive_scan<NT>(c, red_i, &n_o);
    unsigned char* o = out + (int64_t)q * stride;
    double* lp = reinterpret_cast<double*>(o + 8);
    uint64_t* off = reinterpret_cast<uint64_t*>(o + 8 + 8 * (int64_t)n_o);
    uint32_t* tok = reinterpret_cast<uint32_t*>(o + 8 + 16 * (int64_t)n_o);
    const int64_t total = (int64_t)n_o * L;
    for (int j = 0; j < run; ++j) {
        if (!(on >> j & 1u)) continue;
        const int i = b0 + j;
        const int w = n_o - 1 - r;
        // wire slots 0..w hold the live ranks r..n_o-1
        const int64_t end = total - (int64_t)r * L;
        lp[w] = (double)lq[i] * norm;
        off[w] = (uint64_t)end;
        const int32_t* sq = seqs + ((int64_t)q * K + i) * L;
        for (int t = 0; t < L; ++t) tok[end - L + t] = (uint32_t)sq[t];
        ++r;
    }
    if (tid == 0) {
        *reinterpret_cast<uint64_t*>(o) = (uint64_t)n_o;
        if (nbytes) nbytes[q] = 8 + 16 * (int64_t)n_o + 4 * total;
    }
}

}  // namespace

// ---- launchers -----------------------------------------------------------------

int expand_threads(const StepDev&) { return kExpandThreads; }

int query_threads(int K) { return K >= 16 ? 1024 : 512; }

int64_t query_scores_floats(int K, int S) { return (int64_t)K * kWave + S; }

bool query_threads_ok(int nt) { return nt == 256 || nt == 512 || nt == 1024; }

// The persistent decode runs every step and every hidden update of a query in
// one workgroup; with 512 threads its per-wave register budget doubles (the
// 1024-thread build spills the update's registers).  The per-query step gives
// the same bits at either size (every sum is per wave or over fixed slots).
int tail_threads(int) { return 512; }

size_t expand_lds_bytes(int S, int d, bool dense) { return (size_t)expand_lds(S, d, dense, kExpandThreads).total; }

int expand_bitmap_max_v() { return 64 * kWave; }

size_t query_lds_bytes(int S, int K, int Kc, int d, int nt) {
    return (size_t)query_lds(S, K, Kc, d, query_threads_ok(nt) ? nt : query_threads(K)).total;
}

size_t tail_lds_bytes(int S, int K, int Kc, int d) { return (size_t)query_lds(S, K, Kc, d, tail_threads(K)).total; }

hipError_t launch_step_query(const StepDev& st, cb_dtype dt, int Q, int K, int Kc, int d, int nt, const void* hidden,
                             const void* W, const int32_t* beam_rows, const float* acc, const uint64_t* pre,
                             const int32_t* pre_off, int64_t pre_cap, int pre_min, int32_t* tok, int32_t* par,
                             int32_t* rows, float* logp, int G, float* gz, int* gcnt, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int NT = nt == 256 || nt == 512 || nt == 1024 ? nt : query_threads(K);
    const QueryLds lay = query_lds(st.S, K, Kc, d, NT);
    const int CH = (d + kWave * 8 - 1) / (kWave * 8);
    if (G < 1 || !gz || !gcnt) G = 1;
    const int64_t gz_stride = query_scores_floats(K, st.S);
#define CB_QUERY(DT, NTV, CHV)                                                                           \
    CB_LAUNCH((k_step_query<DT, NTV, CHV>), dim3(Q * G), dim3(NTV), lay.total, s, st, K, Kc, d,     \
                       (const DT*)hidden, (const DT*)W, beam_rows, acc, pre, pre_off, pre_cap, pre_min, tok, par, rows, \
                       logp, G, gz, gz_stride, gcnt)
#define CB_QUERY_NT(DT, CHV)                              \
    do {                                                  \
        if (NT == 1024) CB_QUERY(DT, 1024, CHV);          \
        else if (NT == 512) CB_QUERY(DT, 512, CHV);       \
        else CB_QUERY(DT, 256, CHV);                      \
    } while (0)
    if (dt == CB_BF16) {
        if (CH <= 1) CB_QUERY_NT(uint16_t, 1);
        else if (CH == 2) CB_QUERY_NT(uint16_t, 2);
        else CB_QUERY_NT(uint16_t, 4);
    } else {
        if (CH <= 1) CB_QUERY_NT(float, 1);
        else if (CH == 2) CB_QUERY_NT(float, 2);
        else CB_QUERY_NT(float, 4);
    }
#undef CB_QUERY_NT
#undef CB_QUERY
    return hipGetLastError();
}

hipError_t launch_beam_expand(const StepDev& st, bool dense, cb_dtype dt, int R, int K, int Kc, int d,
                              const void* hidden, const void* W, const float* Z, const float* Zp, int64_t ldz,
                              const int32_t* n_live, const int32_t* ci_of, const int32_t* beam_rows,
                              const float* acc, uint64_t* keys, uint64_t* side, bool* sided, int mode,
                              hipStream_t s, int32_t* tok, int32_t* par, int32_t* orows, float* logp,
                              bool* solo_done) {
    *sided = false;
    if (solo_done) *solo_done = false;
    if (R <= 0) return hipSuccess;
    const int split_ok = dt == CB_BF16 ? 1 : 0;
    if (dense && split_ok && (st.store == CB_STORE_BITMAP || mode == CB_MODE_UNCONSTRAINED) &&
        ldz <= 64 * kWave && ldz % 4 == 0) {
        const int M = (int)((ldz + kWave - 1) / kWave);
        const dim3 grid((R + 3) / 4);
        // a query's one live beam writes the query's outputs itself
        const bool direct = tok && mode != CB_MODE_UNCONSTRAINED;
        const MergeOut mo{direct ? tok : nullptr, par, orows, logp};
        if (solo_done) *solo_done = direct;
#define CB_EXPAND_BM_MODE(MV, MD)                                                                            \
    CB_LAUNCH((k_expand_bitmap<MV, MD>), grid, dim3(256), 0, s, st, R, K, Kc, (int)ldz, d, Z, Zp, n_live, \
                       ci_of, beam_rows, acc, keys, mo)
#define CB_EXPAND_BM(MV)                                                                          \
    do {                                                                                          \
        if (mode == CB_MODE_FILTER_FIRST) CB_EXPAND_BM_MODE(MV, CB_MODE_FILTER_FIRST);            \
        else if (mode == CB_MODE_SCORE_FIRST) CB_EXPAND_BM_MODE(MV, CB_MODE_SCORE_FIRST);         \
        else CB_EXPAND_BM_MODE(MV, CB_MODE_UNCONSTRAINED);                                        \
    } while (0)
        if (M <= 4) CB_EXPAND_BM(4);
        else if (M <= 8) CB_EXPAND_BM(8);
        else if (M <= 16) CB_EXPAND_BM(16);
        else if (M <= 32) CB_EXPAND_BM(32);
        else CB_EXPAND_BM(64);
#undef CB_EXPAND_BM
#undef CB_EXPAND_BM_MODE
        return hipGetLastError();
    }
    if (dense && st.store == CB_STORE_CSR && mode == CB_MODE_FILTER_FIRST) {
        *sided = true;
        CB_LAUNCH((k_expand_csr_wave<8>), dim3((R + 3) / 4), dim3(256), 0, s, st, R, K, Kc, d, ldz, Z, Zp, n_live,
                  ci_of, split_ok, beam_rows, acc, keys, side);
        return hipGetLastError();
    }
    const ExpandLds lay = expand_lds(st.S, d, dense, kExpandThreads);
    *sided = true;
#define CB_EXPAND(DT, DENSE, CHV)                                                                            \
    CB_LAUNCH((k_beam_expand<DT, DENSE, kExpandThreads, CHV>), dim3(R), dim3(kExpandThreads), lay.total, s, \
              st, K, Kc, d, (const DT*)hidden, (const DT*)W, Z, Zp, ldz, n_live, ci_of, split_ok, beam_rows, acc, \
              keys, side, mode)
#define CB_EXPAND_SPARSE(DT)                                   \
    do {                                                       \
        if (d <= 512) CB_EXPAND(DT, false, 1);                 \
        else if (d <= 1024) CB_EXPAND(DT, false, 2);           \
        else if (d <= 2048) CB_EXPAND(DT, false, 4);           \
        else CB_EXPAND(DT, false, 0);                          \
    } while (0)
    if (dt == CB_BF16) {
        if (dense) CB_EXPAND(uint16_t, true, 0); else CB_EXPAND_SPARSE(uint16_t);
    } else {
        if (dense) CB_EXPAND(float, true, 0); else CB_EXPAND_SPARSE(float);
    }
#undef CB_EXPAND_SPARSE
#undef CB_EXPAND
    return hipGetLastError();
}

hipError_t launch_query_merge(const StepDev& st, int Q, int K, int Kc, const uint64_t* keys, const uint64_t* side,
                              const int32_t* beam_rows, int32_t* tok, int32_t* par, int32_t* rows, float* logp,
                              int mode, hipStream_t s, bool solo_done) {
    if (Q <= 0) return hipSuccess;
    const int M = (K * Kc + kWave - 1) / kWave;
    const dim3 grid((Q + 3) / 4);
    const MergeOut mo{tok, par, rows, logp};
    const int sd = solo_done ? 1 : 0;
#define CB_MERGE(MV)                                                                                          \
    CB_LAUNCH((k_query_merge_w<MV>), grid, dim3(256), 0, s, st, Q, K, Kc, keys, side, beam_rows, mo, mode, sd)
    if (M <= 1) CB_MERGE(1);
    else if (M <= 4) CB_MERGE(4);
    else if (M <= 16) CB_MERGE(16);
    else CB_MERGE(64);
#undef CB_MERGE
    return hipGetLastError();
}

hipError_t launch_live_rows(const StepDev& st, int R, const int32_t* beam_rows, const float* acc, int32_t* live,
                            int32_t* n_live, int32_t* ci_of, hipStream_t s) {
    CB_LAUNCH((k_live_rows<1024>), dim3(1), dim3(1024), 0, s, st, R, beam_rows, acc, live, n_live, ci_of);
    return hipGetLastError();
}

bool gemm_finds_live(cb_dtype dt, int R) { return dt == CB_BF16 && R <= kFoldSlots; }

bool gemm_full_ok(cb_dtype dt) { return dt == CB_BF16; }

hipError_t launch_gemm_scores(cb_dtype dt, int R, int V, int d, const int32_t* live, int32_t* n_live,
                              const void* H, const void* W, float* Z, float* Zp, const StepDev& st,
                              const int32_t* beam_rows, const float* acc, int32_t* ci_of, bool full,
                              hipStream_t s) {
    if (R <= 0) return hipSuccess;
    if (dt == CB_BF16) {
        static const hipError_t lds_ok = hipFuncSetAttribute(
            (const void*)k_gemm_bf16, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
        if (lds_ok != hipSuccess) return lds_ok;
        const int fold = full || gemm_finds_live(dt, R) ? R : 0;
        const int grid = full ? ((R + kBM - 1) / kBM) * ((V + kBN - 1) / kBN) : gemm_grid(R, V);
        CB_LAUNCH(k_gemm_bf16, dim3(grid), dim3(kGemmThreads), kGemmLds, s, V, d, live, n_live,
                  (const uint16_t*)H, (const uint16_t*)W, Z, Zp, (int64_t)V, st, fold, beam_rows, acc, ci_of,
                  full ? 1 : 0);
    } else {
        dim3 grid((V + 15) / 16, (R + 15) / 16);
        CB_LAUNCH(k_gemm_f32, grid, dim3(256), 0, s, V, d, live, n_live, (const float*)H, (const float*)W,
                           Z, (int64_t)V);
    }
    return hipGetLastError();
}

int gemm_blocks(cb_dtype dt, int R, int V, bool full) {
    if (dt == CB_BF16 && full) return ((R + kBM - 1) / kBM) * ((V + kBN - 1) / kBN);
    return dt == CB_BF16 ? gemm_grid(R, V) : ((V + 15) / 16) * ((R + 15) / 16);
}

size_t split_scores_floats(int V) { return (size_t)kSplitMax * kSplitRows * (size_t)V; }

hipError_t launch_decode_init(int Q, int K, int d, cb_dtype dt, const float* q, float* s_out, void* h_out,
                              int32_t* rows, float* acc, hipStream_t st) {
    const int R = Q * K;
    if (R <= 0) return hipSuccess;
    if (dt == CB_BF16)
        CB_LAUNCH((k_decode_init<uint16_t, 256>), dim3(R), dim3(256), 0, st, K, d, q, s_out,
                           (uint16_t*)h_out, rows, acc);
    else
        CB_LAUNCH((k_decode_init<float, 256>), dim3(R), dim3(256), 0, st, K, d, q, s_out, (float*)h_out,
                           rows, acc);
    return hipGetLastError();
}

// Whether the register-resident hidden update applies: d a multiple of 256,
// at most kRegMaxD, and P (hence every row of every P_t) 16-byte aligned.
static bool hidden_vec_ok(int d, const float* P) {
    return d % (kWave * 4) == 0 && d <= kRegMaxD && (reinterpret_cast<uintptr_t>(P) & 15) == 0;
}

hipError_t launch_hidden_update(int R, int K, int d, cb_dtype dt, const float* s_old, const float* P_t,
                                const int32_t* tok, const int32_t* par, float* s_new, void* h_out,
                                hipStream_t st) {
    if (R <= 0) return hipSuccess;
    const dim3 grid((R + 3) / 4);
    const bool vec = hidden_vec_ok(d, P_t);
#define CB_HU(DT, V) \
    CB_LAUNCH((k_hidden_update<DT, V>), grid, dim3(256), 0, st, R, K, d, s_old, P_t, tok, par, s_new, (DT*)h_out)
    if (dt == CB_BF16) {
        if (vec) CB_HU(uint16_t, true); else CB_HU(uint16_t, false);
    } else {
        if (vec) CB_HU(float, true); else CB_HU(float, false);
    }
#undef CB_HU
    return hipGetLastError();
}

hipError_t launch_decode_tail(const StepDev* d_steps, size_t lds, int t0, int L, int Q, int K, int d, int V,
                              cb_dtype dt, const void* W, const float* P, float* s0, float* s1, void* h,
                              int32_t* rows0, int32_t* rows1, float* acc0, float* acc1, int32_t* hist_tok,
                              int32_t* hist_par, uint64_t* clk, hipStream_t s) {
    if (Q <= 0 || t0 >= L) return hipSuccess;
    // built for 512-thread workgroups only (tail_threads)
    const int CH = (d + kWave * 8 - 1) / (kWave * 8);
    const int R = Q * K;
    const bool vec = hidden_vec_ok(d, P);
#define CB_TAIL(DT, NTV, CHV, VV)                                                                                  \
    CB_LAUNCH((k_decode_tail<DT, NTV, CHV, VV>), dim3(Q), dim3(NTV), lds, s, d_steps, t0, L, K, d, V, R, \
                       (const DT*)W, P, s0, s1, (DT*)h, rows0, rows1, acc0, acc1, hist_tok, hist_par, clk)
#define CB_TAIL_V(DT, NTV, CHV) \
    do { if (vec) CB_TAIL(DT, NTV, CHV, true); else CB_TAIL(DT, NTV, CHV, false); } while (0)
#define CB_TAIL_NT(DT, CHV) CB_TAIL_V(DT, 512, CHV)
    if (dt == CB_BF16) {
        if (CH <= 1) CB_TAIL_NT(uint16_t, 1);
        else if (CH == 2) CB_TAIL_NT(uint16_t, 2);
        else CB_TAIL_NT(uint16_t, 4);
    } else {
        if (CH <= 1) CB_TAIL_NT(float, 1);
        else if (CH == 2) CB_TAIL_NT(float, 2);
        else CB_TAIL_NT(float, 4);
    }
#undef CB_TAIL_NT
#undef CB_TAIL_V
#undef CB_TAIL
    return hipGetLastError();
}

hipError_t launch_empty(int blocks, int threads, hipStream_t s) {
    CB_LAUNCH(k_empty, dim3(blocks), dim3(threads), 0, s, 0);
    return hipGetLastError();
}

hipError_t launch_backtrace(int R, int K, int L, const int32_t* hist_tok, const int32_t* hist_par, int32_t* seqs,
                            hipStream_t s) {
    if (R <= 0) return hipSuccess;
    CB_LAUNCH(k_backtrace, dim3((R + 255) / 256), dim3(256), 0, s, R, K, L, hist_tok, hist_par, seqs);
    return hipGetLastError();
}

hipError_t launch_wire(int Q, int K, int L, const int32_t* seqs, const float* logp, double norm, void* out,
                       int64_t stride, int64_t* nbytes, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    CB_LAUNCH((k_wire<256>), dim3(Q), dim3(256), 0, s, K, L, seqs, logp, norm, (unsigned char*)out, stride, nbytes);
    return hipGetLastError();
}


}  // namespace cb
