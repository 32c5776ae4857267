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
__device__ void emit(const StepDev& st, int q, int K, int i, uint64_t key, const int32_t* __restrict__ beam_rows,
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
    int qkeys, stage, list, z, h, tok, total;
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
    l.total = l.tok + ((S * 2 + 15) & ~15);
    return l;
}

// ---- sparse step: one workgroup per query ----------------------------------

template <typename DT, int NT, int CH>
__global__ __launch_bounds__(NT) void k_step_query(StepDev st, int K, int Kc, int d,
                                                   const DT* __restrict__ hidden, const DT* __restrict__ W,
                                                   const int32_t* __restrict__ beam_rows,
                                                   const float* __restrict__ acc, const uint64_t* __restrict__ pre,
                                                   const int32_t* __restrict__ pre_off, int64_t pre_cap,
                                                   int32_t* __restrict__ out_tok,
                                                   int32_t* __restrict__ out_par, int32_t* __restrict__ out_rows,
                                                   float* __restrict__ out_logp) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red_f[NT / kWave];
    __shared__ int red_i[NT / kWave];
    __shared__ uint64_t bcast;
    __shared__ uint64_t best[kWave];
    __shared__ int nbig;
    __shared__ int big[kWave];
    const QueryLds lay = query_lds(st.S, K, Kc, d, NT);
    uint64_t* qkeys = reinterpret_cast<uint64_t*>(smem + lay.qkeys);
    uint64_t* stage = reinterpret_cast<uint64_t*>(smem + lay.stage);
    int* list = reinterpret_cast<int*>(smem + lay.list);
    float* z_s = reinterpret_cast<float*>(smem + lay.z);
    float* h_s = reinterpret_cast<float*>(smem + lay.h);
    uint16_t* tok_s = reinterpret_cast<uint16_t*>(smem + lay.tok);

    const int q = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    constexpr int NW = NT / kWave;
    if (tid == 0) nbig = 0;
    __syncthreads();

    // phase 1: one wave per beam with a narrow CSR row; each wave takes two
    // beams at a time so that their chains of dependent loads overlap
    for (int k0 = wv; k0 < K; k0 += 2 * NW) {
        int kk[2], tk[2], n[2];
        int64_t b[2];
        float a[2];
        bool small[2];
        uint32_t e0[2];
        int32_t r[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            kk[u] = k0 + u * NW;
            b[u] = (int64_t)q * K + kk[u];
            r[u] = kk[u] < K ? beam_rows[b[u]] : -1;
            a[u] = kk[u] < K ? acc[b[u]] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bool live = kk[u] < K && beam_live(st, r[u], a[u]);
            e0[u] = live ? st.row_ptr[r[u]] : 0u;
            n[u] = live ? (int)(st.row_ptr[r[u] + 1] - e0[u]) : 0;
            small[u] = live && n[u] <= kSmallRow && st.store == CB_STORE_CSR;
            if (kk[u] < K) {
                if (!live) {
                    if (lane < Kc) qkeys[kk[u] * Kc + lane] = 0ull;
                } else if (!small[u]) {
                    if (lane == 0) big[atomicAdd(&nbig, 1)] = kk[u];
                }
            }
            tk[u] = small[u] && lane < n[u] ? (int)st.tok[e0[u] + lane] : 0;
        }
        if (!small[0] && !small[1]) continue;
        // rows whose scores were computed apart are read, the others scored here
        bool dots[2];
        float z[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bool ready = pre && small[u] && n[u] > kPreMin;
            dots[u] = small[u] && !ready;
            if (ready && lane < n[u])
                z[u] = __uint_as_float((uint32_t)(pre[(int64_t)q * pre_cap + pre_off[(int64_t)q * (K + 1) + kk[u]] +
                                                      lane] >> 32));
        }
        float hr[2][CH][8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int i = c * kWave * 8 + lane * 8;
                if (dots[u] && i < d) load8(hidden + b[u] * d + i, hr[u][c]);
                else
#pragma unroll
                    for (int e = 0; e < 8; ++e) hr[u][c][e] = 0.f;
            }
        const int nmax = max(dots[0] ? n[0] : 0, dots[1] ? n[1] : 0);
        // kTok tokens of each of the two beams at a time: all their W_t row
        // loads are issued before any is reduced, so the latencies overlap
        // (as many as the register budget of a 1024-thread workgroup allows)
        constexpr int kTok = CH >= 4 ? 1 : 4 / CH;
        for (int j0 = 0; j0 < nmax; j0 += kTok) {
            Raw8<DT> wr8[2][kTok][CH];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int jj = 0; jj < kTok; ++jj) {
                    const int j = j0 + jj;
                    const int tj = lane_bcast(tk[u], j < kWave ? j : 0);
                    const bool on = dots[u] && j < n[u];
                    const DT* wr = W + (int64_t)tj * d;
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        const int i = c * kWave * 8 + lane * 8;
                        if (on && i < d) wr8[u][jj][c].load(wr + i);
                        else wr8[u][jj][c].zero();
                    }
                }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int jj = 0; jj < kTok; ++jj) {
                    float sv = 0.f;
#pragma unroll
                    for (int c = 0; c < CH; ++c) sv = wr8[u][jj][c].dot(hr[u][c], sv);
                    const float t = wave_sum(sv);
                    if (dots[u] && lane == j0 + jj) z[u] = t;
                }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (!small[u]) continue;
            const bool on = lane < n[u];
            const float m = wave_max(on ? z[u] : -INFINITY);
            const float se = wave_sum(on ? expf(z[u] - m) : 0.f);
            const float lse = m + logf(se);
            uint64_t key = on ? make_key(a[u] + (z[u] - lse), kk[u], tk[u]) : 0ull;
            if (n[u] > Kc) key = wave_sort_desc(key);
            if (lane < Kc) qkeys[kk[u] * Kc + lane] = key;
        }
    }
    __syncthreads();

    // phase 2: wide rows and bitmap rows, the whole block per beam
    const int nb = nbig;
    for (int i = 0; i < nb; ++i) {
        const int k = big[i];
        const int64_t b = (int64_t)q * K + k;
        const int32_t r = beam_rows[b];
        const float a = acc[b];
        const uint32_t e0 = st.row_ptr[r];
        const int n = (int)(st.row_ptr[r + 1] - e0);
        block_fill_tokens<NT>(st, r, e0, n, tok_s, red_i);
        if (pre) {  // scored apart, across many workgroups
            const uint64_t* zp = pre + (int64_t)q * pre_cap + pre_off[(int64_t)q * (K + 1) + k];
            for (int j = tid; j < n; j += NT) z_s[j] = __uint_as_float((uint32_t)(zp[j] >> 32));
            __syncthreads();
        } else {
            for (int x = tid; x < d; x += NT) h_s[x] = to_f32(hidden[b * d + x]);
            __syncthreads();
            block_scores<DT, NT>(h_s, W, d, tok_s, n, z_s);
            __syncthreads();
        }
        const float lse = block_lse<NT>(z_s, n, red_f);
        auto keyf = [&](int j) { return make_key(a + (z_s[j] - lse), k, (int)tok_s[j]); };
        uint64_t* slot = qkeys + k * Kc;
        if (n <= Kc) {
            for (int j = tid; j < Kc; j += NT) slot[j] = j < n ? keyf(j) : 0ull;
        } else {
            block_select_top<NT>(n, Kc, keyf, slot, stage, list, red_i, &bcast);
        }
        __syncthreads();
    }

    // phase 3: the query's K best
    block_select_top<NT>(K * Kc, K, [&](int j) { return qkeys[j]; }, best, stage, list, red_i, &bcast);
    __syncthreads();
    for (int i = tid; i < K; i += NT) emit(st, q, K, i, best[i], beam_rows, out_tok, out_par, out_rows, out_logp);
}

// ---- dense step: per-beam expansion and per-query merge --------------------

template <typename DT, bool DENSE, int NT>
__global__ __launch_bounds__(NT) void k_beam_expand(StepDev st, int K, int Kc, int d,
                                                    const DT* __restrict__ hidden, const DT* __restrict__ W,
                                                    const float* __restrict__ Z, const float* __restrict__ Zp,
                                                    int64_t ldz, const int32_t* __restrict__ n_live,
                                                    const int32_t* __restrict__ ci_of, int split_ok,
                                                    const int32_t* __restrict__ beam_rows,
                                                    const float* __restrict__ acc, uint64_t* __restrict__ keys_out) {
    auto split_of = [&](const int32_t* nl) { return split_ok ? gemm_split(*nl, (int)ldz, d) : 1; };
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red_f[NT / kWave];
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
    if (!DENSE)
        for (int i = tid; i < d; i += NT) h_s[i] = to_f32(hidden[(int64_t)b * d + i]);
    __syncthreads();
    if (DENSE) {
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
    } else {
        block_scores<DT, NT>(h_s, W, d, tok_s, n, z_s);
    }
    __syncthreads();
    const float lse = block_lse<NT>(z_s, n, red_f);
    const int parent = b % K;
    auto keyf = [&](int j) { return make_key(a + (z_s[j] - lse), parent, (int)tok_s[j]); };
    if (n <= Kc) {
        for (int j = tid; j < Kc; j += NT) out[j] = j < n ? keyf(j) : 0ull;
        return;
    }
    block_select_top<NT>(n, Kc, keyf, out, stage, list, red_i, &bcast);
}

// Dense path on a bitmap step: one wavefront per beam, four beams per
// workgroup.  Lane l owns the M consecutive columns l*M .. l*M+M-1: their
// scores (16-byte loads, summed over the k-slices, if any) and validity bits
// stay in registers; softmax and the beam's best min(K, n) keys use wave
// reductions only.  Requires V <= 64*M and V % 4 == 0.
template <int M>
__global__ __launch_bounds__(256) void k_expand_bitmap(StepDev st, int R, int K, int Kc, int V, int d,
                                                       const float* __restrict__ Z, const float* __restrict__ Zp,
                                                       const int32_t* __restrict__ n_live,
                                                       const int32_t* __restrict__ ci_of,
                                                       const int32_t* __restrict__ beam_rows,
                                                       const float* __restrict__ acc, uint64_t* __restrict__ keys_out) {
    static_assert(M % 4 == 0, "columns are read 4 at a time");
    __shared__ uint64_t wl_all[4][kWaveListCap];
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
    const int c0 = lane * M;
    const uint32_t* rb = st.bits + (int64_t)r * st.words;
    const int split = gemm_split(*n_live, V, d);
    const float* zb = (split == 1 ? Z + (int64_t)b * V : Zp + (int64_t)ci_of[b] * V) + c0;
    float z[M];
#pragma unroll
    for (int i = 0; i < M; ++i) z[i] = 0.f;
#pragma unroll
    for (int x = 0; x < kSplitMax; ++x) {
        if (x < split) {
#pragma unroll
            for (int i = 0; i < M; i += 4) {
                if (c0 + i < V) {
                    const float4 v4 = *reinterpret_cast<const float4*>(zb + (int64_t)x * kSplitRows * V + i);
                    z[i] += v4.x;
                    z[i + 1] += v4.y;
                    z[i + 2] += v4.z;
                    z[i + 3] += v4.w;
                }
            }
        }
    }
    uint32_t on = 0;  // validity of this lane's columns, bit i for column c0 + i (M <= 32 per word)
    uint32_t on_hi = 0;
#pragma unroll
    for (int i = 0; i < M; i += 32) {
        // columns c0+i .. c0+i+31 lie in at most two bitmap words
        const int c = c0 + i;
        const int w = c >> 5, sh = c & 31;
        uint32_t lo = c < V ? rb[w] : 0u;
        uint32_t hi = (sh && c + 32 - sh < V) ? rb[w + 1] : 0u;
        uint32_t bits = sh ? ((lo >> sh) | (hi << (32 - sh))) : lo;
        if (M - i < 32) bits &= (1u << (M - i)) - 1u;
        if (i == 0) on = bits; else on_hi = bits;
    }
    auto valid = [&](int i) { return ((i < 32 ? on >> i : on_hi >> (i - 32)) & 1u) != 0; };
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < M; ++i)
        if (valid(i)) m = fmaxf(m, z[i]);
    m = wave_max(m);
    float se = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i)
        if (valid(i)) se += expf(z[i] - m);
    const float lse = m + logf(wave_sum(se));
    const int parent = b % K;
    uint32_t sc[M];
#pragma unroll
    for (int i = 0; i < M; ++i) sc[i] = valid(i) ? score_order_bits(a + (z[i] - lse)) : 0u;
    const uint64_t best = wave_top<M>(
        Kc, [&](int i) { return sc[i]; },
        [&](int i) { return ((uint64_t)sc[i] << 32) | ((uint64_t)(1023 - parent) << 16) | (uint64_t)(65535 - (c0 + i)); },
        wl_all[wv]);
    if (lane < Kc) out[lane] = best;
}

// Dense path, per query: one wavefront per query, four queries per workgroup;
// lane l owns keys l + 64 i (i < M) of the query's K*Kc.
template <int M>
__global__ __launch_bounds__(256) void k_query_merge_w(StepDev st, int Q, int K, int Kc,
                                                       const uint64_t* __restrict__ keys,
                                                       const int32_t* __restrict__ beam_rows,
                                                       int32_t* __restrict__ out_tok, int32_t* __restrict__ out_par,
                                                       int32_t* __restrict__ out_rows, float* __restrict__ out_logp) {
    __shared__ uint64_t wl_all[4][kWaveListCap];
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int q = blockIdx.x * 4 + wv;
    if (q >= Q) return;
    const int n = K * Kc;
    const uint64_t* src = keys + (int64_t)q * n;
    uint64_t kv[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int c = lane + kWave * i;
        kv[i] = c < n ? src[c] : 0ull;
    }
    const uint64_t best = wave_top<M>(K, [&](int i) { return (uint32_t)(kv[i] >> 32); }, [&](int i) { return kv[i]; },
                                      wl_all[wv]);
    if (lane < K) emit(st, q, K, lane, best, beam_rows, out_tok, out_par, out_rows, out_logp);
}

// ---- full-codebook scores of the live beams (dense path) ------------------

// Compact list of the live beam slots (ascending), their count, and the
// compact index of every slot (-1 when dead).
template <int NT>
__global__ __launch_bounds__(NT) void k_live_rows(StepDev st, int R, const int32_t* __restrict__ beam_rows,
                                                  const float* __restrict__ acc, int32_t* __restrict__ live,
                                                  int32_t* __restrict__ n_live, int32_t* __restrict__ ci_of) {
    __shared__ int red_i[NT / kWave];
    int base = 0;
    for (int b0 = 0; b0 < R; b0 += NT) {
        const int b = b0 + threadIdx.x;
        const int on = b < R && beam_live(st, beam_rows[b], acc[b]);
        int tot;
        const int pos = base + block_exclusive_scan<NT>(on, red_i, &tot);
        if (on) live[pos] = b;
        if (b < R) ci_of[b] = on ? pos : -1;
        base += tot;
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

__global__ __launch_bounds__(kGemmThreads) void k_gemm_bf16(int V, int d, const int32_t* __restrict__ live,
                                                            const int32_t* __restrict__ n_live,
                                                            const uint16_t* __restrict__ H,
                                                            const uint16_t* __restrict__ W, float* __restrict__ Z,
                                                            float* __restrict__ Zp, int64_t ldz) {
    extern __shared__ __align__(16) uint16_t gsm[];
    uint16_t* As = gsm;                     // [2][kBM * kLDP]
    uint16_t* Bs = gsm + 2 * kBM * kLDP;    // [2][kBN * kLDP]
    __shared__ int rows_s[kBM];
    constexpr int NT = kGemmThreads;
    constexpr int CA = kBM * kBK / 8 / NT, CB = kBN * kBK / 8 / NT;  // 16-byte chunks per thread
    constexpr int TJ = kWN / 32;
    const int nl = *n_live;
    const int split = gemm_split(nl, V, d);
    const int mt = (nl + kBM - 1) / kBM, nt = (V + kBN - 1) / kBN;
    const int N = mt * nt * split;
    const int L = blockIdx.x;
    if (L >= N) return;
    const int full = (N / 8) * 8;
    const int lin = L < full ? (L % 8) * (full / 8) + L / 8 : L;
    const int zs = lin % split, tile = lin / split;
    const int m0 = (tile % mt) * kBM, n0 = (tile / mt) * kBN;
    const int klen = d / split, kbeg = zs * klen;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid < kBM) rows_s[tid] = m0 + tid < nl ? live[m0 + tid] : -1;
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

template <typename DT, int NT>
__global__ __launch_bounds__(NT) void k_hidden_update(int K, int d, const float* __restrict__ s_old,
                                                      const float* __restrict__ P_t, const int32_t* __restrict__ tok,
                                                      const int32_t* __restrict__ par, float* __restrict__ s_new,
                                                      DT* __restrict__ h_out) {
    __shared__ double red[NT / kWave];
    const int b = blockIdx.x;
    const int tk = tok[b];
    DT* hb = h_out + (int64_t)b * d;
    if (tk < 0) {
        for (int i = threadIdx.x; i < d; i += NT) store_h(hb + i, 0.f);
        return;
    }
    const int p = (b / K) * K + par[b];
    const float* sp = s_old + (int64_t)p * d;
    const float* pv = P_t + (int64_t)tk * d;
    float* sn = s_new + (int64_t)b * d;
    for (int i = threadIdx.x; i < d; i += NT) sn[i] = sp[i] + pv[i];
    __syncthreads();
    normalise_into<DT, NT>(sn, d, hb, red);
}

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

}  // namespace

// ---- launchers -----------------------------------------------------------------

int expand_threads(const StepDev&) { return kExpandThreads; }

int query_threads(int K) { return K >= 16 ? 1024 : 512; }

size_t expand_lds_bytes(int S, int d, bool dense) { return (size_t)expand_lds(S, d, dense, kExpandThreads).total; }

int expand_bitmap_max_v() { return 64 * kWave; }

size_t query_lds_bytes(int S, int K, int Kc, int d) {
    return (size_t)query_lds(S, K, Kc, d, query_threads(K)).total;
}

hipError_t launch_step_query(const StepDev& st, cb_dtype dt, int Q, int K, int Kc, int d, const void* hidden,
                             const void* W, const int32_t* beam_rows, const float* acc, const uint64_t* pre,
                             const int32_t* pre_off, int64_t pre_cap, int32_t* tok, int32_t* par, int32_t* rows,
                             float* logp, hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int NT = query_threads(K);
    const QueryLds lay = query_lds(st.S, K, Kc, d, NT);
    const int CH = (d + kWave * 8 - 1) / (kWave * 8);
#define CB_QUERY(DT, NTV, CHV)                                                                           \
    hipLaunchKernelGGL((k_step_query<DT, NTV, CHV>), dim3(Q), dim3(NTV), lay.total, s, st, K, Kc, d,     \
                       (const DT*)hidden, (const DT*)W, beam_rows, acc, pre, pre_off, pre_cap, tok, par, rows, logp)
#define CB_QUERY_NT(DT, CHV) \
    do { if (NT == 1024) CB_QUERY(DT, 1024, CHV); else CB_QUERY(DT, 512, CHV); } while (0)
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
                              const float* acc, uint64_t* keys, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const int split_ok = dt == CB_BF16 ? 1 : 0;
    if (dense && split_ok && st.store == CB_STORE_BITMAP && ldz <= 64 * kWave && ldz % 4 == 0) {
        const int M = (int)((ldz + kWave - 1) / kWave);
        const dim3 grid((R + 3) / 4);
#define CB_EXPAND_BM(MV)                                                                                        \
    hipLaunchKernelGGL((k_expand_bitmap<MV>), grid, dim3(256), 0, s, st, R, K, Kc, (int)ldz, d, Z, Zp, n_live, \
                       ci_of, beam_rows, acc, keys)
        if (M <= 4) CB_EXPAND_BM(4);
        else if (M <= 8) CB_EXPAND_BM(8);
        else if (M <= 16) CB_EXPAND_BM(16);
        else if (M <= 32) CB_EXPAND_BM(32);
        else CB_EXPAND_BM(64);
#undef CB_EXPAND_BM
        return hipGetLastError();
    }
    const ExpandLds lay = expand_lds(st.S, d, dense, kExpandThreads);
#define CB_EXPAND(DT, DENSE)                                                                                     \
    hipLaunchKernelGGL((k_beam_expand<DT, DENSE, kExpandThreads>), dim3(R), dim3(kExpandThreads), lay.total, s, \
                       st, K, Kc, d, (const DT*)hidden, (const DT*)W, Z, Zp, ldz, n_live, ci_of, split_ok,        \
                       beam_rows, acc, keys)
    if (dt == CB_BF16) {
        if (dense) CB_EXPAND(uint16_t, true); else CB_EXPAND(uint16_t, false);
    } else {
        if (dense) CB_EXPAND(float, true); else CB_EXPAND(float, false);
    }
#undef CB_EXPAND
    return hipGetLastError();
}

hipError_t launch_query_merge(const StepDev& st, int Q, int K, int Kc, const uint64_t* keys,
                              const int32_t* beam_rows, int32_t* tok, int32_t* par, int32_t* rows, float* logp,
                              hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int M = (K * Kc + kWave - 1) / kWave;
    const dim3 grid((Q + 3) / 4);
#define CB_MERGE(MV)                                                                                      \
    hipLaunchKernelGGL((k_query_merge_w<MV>), grid, dim3(256), 0, s, st, Q, K, Kc, keys, beam_rows, tok, par, \
                       rows, logp)
    if (M <= 1) CB_MERGE(1);
    else if (M <= 4) CB_MERGE(4);
    else if (M <= 16) CB_MERGE(16);
    else CB_MERGE(64);
#undef CB_MERGE
    return hipGetLastError();
}

hipError_t launch_live_rows(const StepDev& st, int R, const int32_t* beam_rows, const float* acc, int32_t* live,
                            int32_t* n_live, int32_t* ci_of, hipStream_t s) {
    hipLaunchKernelGGL((k_live_rows<1024>), dim3(1), dim3(1024), 0, s, st, R, beam_rows, acc, live, n_live, ci_of);
    return hipGetLastError();
}

hipError_t launch_gemm_scores(cb_dtype dt, int R, int V, int d, const int32_t* live, const int32_t* n_live,
                              const void* H, const void* W, float* Z, float* Zp, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    if (dt == CB_BF16) {
        static const hipError_t lds_ok = hipFuncSetAttribute(
            (const void*)k_gemm_bf16, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
        if (lds_ok != hipSuccess) return lds_ok;
        hipLaunchKernelGGL(k_gemm_bf16, dim3(gemm_grid(R, V)), dim3(kGemmThreads), kGemmLds, s, V, d, live, n_live,
                           (const uint16_t*)H, (const uint16_t*)W, Z, Zp, (int64_t)V);
    } else {
        dim3 grid((V + 15) / 16, (R + 15) / 16);
        hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, s, V, d, live, n_live, (const float*)H, (const float*)W,
                           Z, (int64_t)V);
    }
    return hipGetLastError();
}

int gemm_blocks(cb_dtype dt, int R, int V) {
    return dt == CB_BF16 ? gemm_grid(R, V) : ((V + 15) / 16) * ((R + 15) / 16);
}

size_t split_scores_floats(int V) { return (size_t)kSplitMax * kSplitRows * (size_t)V; }

hipError_t launch_decode_init(int Q, int K, int d, cb_dtype dt, const float* q, float* s_out, void* h_out,
                              int32_t* rows, float* acc, hipStream_t st) {
    const int R = Q * K;
    if (R <= 0) return hipSuccess;
    if (dt == CB_BF16)
        hipLaunchKernelGGL((k_decode_init<uint16_t, 256>), dim3(R), dim3(256), 0, st, K, d, q, s_out,
                           (uint16_t*)h_out, rows, acc);
    else
        hipLaunchKernelGGL((k_decode_init<float, 256>), dim3(R), dim3(256), 0, st, K, d, q, s_out, (float*)h_out,
                           rows, acc);
    return hipGetLastError();
}

hipError_t launch_hidden_update(int R, int K, int d, cb_dtype dt, const float* s_old, const float* P_t,
                                const int32_t* tok, const int32_t* par, float* s_new, void* h_out,
                                hipStream_t st) {
    if (R <= 0) return hipSuccess;
    if (dt == CB_BF16)
        hipLaunchKernelGGL((k_hidden_update<uint16_t, 256>), dim3(R), dim3(256), 0, st, K, d, s_old, P_t, tok, par,
                           s_new, (uint16_t*)h_out);
    else
        hipLaunchKernelGGL((k_hidden_update<float, 256>), dim3(R), dim3(256), 0, st, K, d, s_old, P_t, tok, par,
                           s_new, (float*)h_out);
    return hipGetLastError();
}

hipError_t launch_backtrace(int R, int K, int L, const int32_t* hist_tok, const int32_t* hist_par, int32_t* seqs,
                            hipStream_t s) {
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_backtrace, dim3((R + 255) / 256), dim3(256), 0, s, R, K, L, hist_tok, hist_par, seqs);
    return hipGetLastError();
}


}  // namespace cb
