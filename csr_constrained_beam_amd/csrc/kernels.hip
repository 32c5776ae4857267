// Device kernels of one constrained beam-search step on gfx950 (wave64).
//
// Step layout (one decoding step t over R = Q*K beam slots):
//   [dense path only] k_gemm_bf16 / k_gemm_f32: Z = H * W_t^T over the whole
//       codebook (ZeroGR: "full scoring" = one regular matrix product).
//   k_beam_expand: one workgroup per beam slot.
//       a1 slot fill: the beam's row gives its valid tokens, written in order
//          into LDS slots 0..n-1 (CSR rows are copied, bitmap rows are
//          enumerated with a block-wide popcount scan).  Slots depend only on
//          the beam and the position (ZeroGR: fixed candidate slots, valid
//          tokens filling from the front).
//       a2 scores: sparse path = one wavefront per token, W_t row read in
//          place (coalesced 16-byte lanes), hidden vector staged in LDS,
//          fixed-order wave reduction; dense path = gather of the valid
//          columns of Z.
//       a3 log-softmax over the n valid slots only, added to the beam's
//          accumulated log-prob (ZeroGR "The pipeline", stage 4).
//       a4 (first half) the beam's best min(K, n) candidates as 64-bit keys
//          (a beam cannot place more than K candidates among the K best).
//   k_query_merge: one workgroup per query; bitonic sort of its K*min(K,S)
//       keys in LDS, the best K become the next beams; each survivor's next
//       row is the edge position of its token in the parent's row.
//
// Candidate key: [63:32] order-preserving bits of the float32 score,
// [25:16] 1023 - parent slot, [15:0] 65535 - token.  Sorting keys descending
// orders by (score desc, parent asc, token asc); key 0 marks an empty slot.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "cb_internal.h"

namespace cb {
namespace {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// float32 -> bf16, round to nearest, ties to even (inputs finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t score_order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float score_from_order_bits(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t make_key(float score, int parent, int token) {
    return ((uint64_t)score_order_bits(score) << 32) | ((uint64_t)(1023 - parent) << 16) |
           (uint64_t)(65535 - token);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Block reductions in a fixed order (deterministic); every thread gets the result.
template <int NT>
__device__ float block_max(float v, float* red) {
    v = wave_max(v);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

template <int NT, typename T>
__device__ T block_sum(T v, T* red) {
    v = wave_sum(v);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    T r = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) r += red[i];
    __syncthreads();
    return r;
}

// Exclusive prefix sum of c over the block; *total receives the block sum.
template <int NT>
__device__ int block_exclusive_scan(int c, int* red, int* total) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int x = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) red[w] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
        int v = red[i];
        off += (i < w) ? v : 0;
        tot += v;
    }
    __syncthreads();
    *total = tot;
    return off + x - c;
}

// Bitonic sort of n (power of two) keys in LDS, descending.  Caller syncs before.
template <int NT>
__device__ void bitonic_sort_desc(uint64_t* a, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += NT) {
                int ixj = i ^ j;
                if (ixj > i) {
                    uint64_t x = a[i], y = a[ixj];
                    bool desc = (i & k) == 0;
                    if (desc ? (x < y) : (x > y)) {
                        a[i] = y;
                        a[ixj] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
}

__host__ __device__ inline int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// LDS layout of k_beam_expand (bytes), shared by host launcher and kernel.
struct ExpandLds {
    int keys, z, h, tok, total;
};
__host__ __device__ inline ExpandLds expand_lds(int S, int Kc, int d, bool dense) {
    ExpandLds l;
    int nk = S > Kc ? next_pow2(S) : 0;
    l.keys = 0;
    l.z = l.keys + nk * 8;
    l.h = l.z + ((S * 4 + 15) & ~15);
    l.tok = l.h + (dense ? 0 : d * 4);
    l.total = l.tok + ((S * 2 + 15) & ~15);
    return l;
}

// 8 consecutive elements of a W_t row (16-byte aligned) as float.
__device__ __forceinline__ void load8(const uint16_t* p, float* o) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xFFFF0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xFFFF0000u);
    o[4] = __uint_as_float(v.z << 16);
    o[5] = __uint_as_float(v.z & 0xFFFF0000u);
    o[6] = __uint_as_float(v.w << 16);
    o[7] = __uint_as_float(v.w & 0xFFFF0000u);
}
__device__ __forceinline__ void load8(const float* p, float* o) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename DT, bool DENSE, int NT>
__global__ __launch_bounds__(NT) void k_beam_expand(StepDev st, int K, int Kc, int d,
                                                    const DT* __restrict__ hidden, const DT* __restrict__ W,
                                                    const float* __restrict__ Z, int64_t ldz,
                                                    const int32_t* __restrict__ beam_rows,
                                                    const float* __restrict__ acc, uint64_t* __restrict__ keys_out) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red_f[NT / kWave];
    __shared__ int red_i[NT / kWave];
    const ExpandLds lay = expand_lds(st.S, Kc, d, DENSE);
    uint64_t* keys_s = reinterpret_cast<uint64_t*>(smem + lay.keys);
    float* z_s = reinterpret_cast<float*>(smem + lay.z);
    float* h_s = reinterpret_cast<float*>(smem + lay.h);
    uint16_t* tok_s = reinterpret_cast<uint16_t*>(smem + lay.tok);

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    uint64_t* out = keys_out + (int64_t)b * Kc;
    const int32_t r = beam_rows[b];
    const float a = acc[b];
    if (r < 0 || (int64_t)r >= st.n_rows || !(a > -INFINITY)) {
        for (int j = tid; j < Kc; j += NT) out[j] = 0;
        return;
    }
    const uint32_t e0 = st.row_ptr[r];
    const int n = (int)(st.row_ptr[r + 1] - e0);

    // a1: slot fill
    if (st.store == CB_STORE_CSR) {
        for (int j = tid; j < n; j += NT) tok_s[j] = st.tok[e0 + j];
    } else {
        const uint32_t* rb = st.bits + (int64_t)r * st.words;
        int base = 0;
        for (int w0 = 0; w0 < st.words; w0 += NT) {
            const int w = w0 + tid;
            uint32_t word = w < st.words ? rb[w] : 0u;
            int tot;
            int pos = base + block_exclusive_scan<NT>(__popc(word), red_i, &tot);
            while (word) {
                const int bit = __ffs(word) - 1;
                tok_s[pos++] = (uint16_t)(w * 32 + bit);
                word &= word - 1;
            }
            base += tot;
        }
    }
    if (!DENSE) {
        const DT* hb = hidden + (int64_t)b * d;
        for (int i = tid; i < d; i += NT) h_s[i] = to_f32(hb[i]);
    }
    __syncthreads();

    // a2: scores of the valid slots
    if (DENSE) {
        const float* zb = Z + (int64_t)b * ldz;
        for (int j = tid; j < n; j += NT) z_s[j] = zb[tok_s[j]];
    } else {
        const int lane = tid & (kWave - 1);
        for (int j = tid / kWave; j < n; j += NT / kWave) {
            const DT* wr = W + (int64_t)tok_s[j] * d;
            float s = 0.f;
            for (int i = lane * 8; i < d; i += kWave * 8) {
                float w8[8];
                load8(wr + i, w8);
                const float4 h0 = *reinterpret_cast<const float4*>(h_s + i);
                const float4 h1 = *reinterpret_cast<const float4*>(h_s + i + 4);
                s = fmaf(h0.x, w8[0], s);
                s = fmaf(h0.y, w8[1], s);
                s = fmaf(h0.z, w8[2], s);
                s = fmaf(h0.w, w8[3], s);
                s = fmaf(h1.x, w8[4], s);
                s = fmaf(h1.y, w8[5], s);
                s = fmaf(h1.z, w8[6], s);
                s = fmaf(h1.w, w8[7], s);
            }
            s = wave_sum(s);
            if (lane == 0) z_s[j] = s;
        }
    }
    __syncthreads();

    // a3: log-softmax over the valid slots, plus the accumulated log-prob
    float m = -INFINITY;
    for (int j = tid; j < n; j += NT) m = fmaxf(m, z_s[j]);
    m = block_max<NT>(m, red_f);
    float se = 0.f;
    for (int j = tid; j < n; j += NT) se += expf(z_s[j] - m);
    se = block_sum<NT>(se, red_f);
    const float lse = m + logf(se);
    const int parent = b % K;

    // a4 (per beam): best min(K, n) candidates
    if (n <= Kc) {
        for (int j = tid; j < Kc; j += NT)
            out[j] = j < n ? make_key(a + (z_s[j] - lse), parent, tok_s[j]) : 0ull;
        return;
    }
    const int n2 = next_pow2(n);
    for (int j = tid; j < n2; j += NT) keys_s[j] = j < n ? make_key(a + (z_s[j] - lse), parent, tok_s[j]) : 0ull;
    __syncthreads();
    bitonic_sort_desc<NT>(keys_s, n2);
    for (int j = tid; j < Kc; j += NT) out[j] = keys_s[j];
}

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
    const uint32_t* rb = st.bits + (int64_t)r * st.words;
    const int w = token >> 5;
    uint32_t c = 0;
    for (int i = 0; i < w; ++i) c += __popc(rb[i]);
    c += __popc(rb[w] & ((1u << (token & 31)) - 1u));
    return (int32_t)(e0 + c);
}

template <int NT>
__global__ __launch_bounds__(NT) void k_query_merge(StepDev st, int K, int Kc, int P2,
                                                    const uint64_t* __restrict__ keys,
                                                    const int32_t* __restrict__ beam_rows,
                                                    int32_t* __restrict__ out_tok, int32_t* __restrict__ out_par,
                                                    int32_t* __restrict__ out_rows, float* __restrict__ out_logp) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t* sk = reinterpret_cast<uint64_t*>(smem);
    const int q = blockIdx.x;
    const int M = K * Kc;
    const uint64_t* src = keys + (int64_t)q * M;
    for (int i = threadIdx.x; i < P2; i += NT) sk[i] = i < M ? src[i] : 0ull;
    __syncthreads();
    bitonic_sort_desc<NT>(sk, P2);
    for (int i = threadIdx.x; i < K; i += NT) {
        const int64_t o = (int64_t)q * K + i;
        const uint64_t key = sk[i];
        if (key == 0ull) {
            out_tok[o] = -1;
            out_par[o] = -1;
            out_rows[o] = -1;
            out_logp[o] = -INFINITY;
            continue;
        }
        const int parent = 1023 - (int)((key >> 16) & 1023u);
        const int token = 65535 - (int)(key & 0xFFFFu);
        const int32_t r = beam_rows[(int64_t)q * K + parent];
        out_tok[o] = token;
        out_par[o] = parent;
        out_rows[o] = edge_of(st, r, token);
        out_logp[o] = score_from_order_bits((uint32_t)(key >> 32));
    }
}

// ---- full-codebook scores (dense path) ------------------------------------

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64, kLDP = kBK + 8;

// Z[R][V] (row pitch ldz) = H[R][d] * W[V][d]^T, bf16 in, float32 accumulate on
// MFMA 32x32x16.  256 threads = 4 waves, each a 64x64 quarter of the tile.
__global__ __launch_bounds__(256) void k_gemm_bf16(int R, int V, int d, const uint16_t* __restrict__ H,
                                                   const uint16_t* __restrict__ W, float* __restrict__ Z,
                                                   int64_t ldz) {
    __shared__ __align__(16) uint16_t As[kBM * kLDP];
    __shared__ __align__(16) uint16_t Bs[kBN * kLDP];
    const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = (wv >> 1) * 64, wn = (wv & 1) * 64;
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    for (int k0 = 0; k0 < d; k0 += kBK) {
        for (int c = tid; c < kBM * kBK / 8; c += 256) {
            const int rr = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
            uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
            if (m0 + rr < R) va = *reinterpret_cast<const uint4*>(H + (int64_t)(m0 + rr) * d + k0 + kc);
            if (n0 + rr < V) vb = *reinterpret_cast<const uint4*>(W + (int64_t)(n0 + rr) * d + k0 + kc);
            *reinterpret_cast<uint4*>(As + rr * kLDP + kc) = va;
            *reinterpret_cast<uint4*>(Bs + rr * kLDP + kc) = vb;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            bf16x8_t av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                uint4 u = *reinterpret_cast<const uint4*>(As + (wm + i * 32 + (lane & 31)) * kLDP + kk + (lane >> 5) * 8);
                av[i] = __builtin_bit_cast(bf16x8_t, u);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint4 u = *reinterpret_cast<const uint4*>(Bs + (wn + j * 32 + (lane & 31)) * kLDP + kk + (lane >> 5) * 8);
                bv[j] = __builtin_bit_cast(bf16x8_t, u);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
                const int col = n0 + wn + j * 32 + (lane & 31);
                if (row < R && col < V) Z[(int64_t)row * ldz + col] = acc[i][j][e];
            }
}

// float32 full-codebook scores: 16x16 output tile per workgroup, one output
// per thread, the k loop in ascending order.
__global__ __launch_bounds__(256) void k_gemm_f32(int R, int V, int d, const float* __restrict__ H,
                                                  const float* __restrict__ W, float* __restrict__ Z, int64_t ldz) {
    __shared__ float As[16][17], Bs[16][17];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int row = blockIdx.y * 16 + ty, col = blockIdx.x * 16 + tx;
    float s = 0.f;
    for (int k0 = 0; k0 < d; k0 += 16) {
        const int ar = blockIdx.y * 16 + ty, bc = blockIdx.x * 16 + ty;
        As[ty][tx] = (ar < R && k0 + tx < d) ? H[(int64_t)ar * d + k0 + tx] : 0.f;
        Bs[ty][tx] = (bc < V && k0 + tx < d) ? W[(int64_t)bc * d + k0 + tx] : 0.f;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) s = fmaf(As[ty][k], Bs[tx][k], s);
        __syncthreads();
    }
    if (row < R && col < V) Z[(int64_t)row * ldz + col] = s;
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

int expand_threads(const StepDev& st) { return (st.S <= 8 && st.store == CB_STORE_CSR) ? 64 : 256; }

hipError_t launch_beam_expand(const StepDev& st, bool dense, cb_dtype dt, int R, int K, int Kc, int d,
                              const void* hidden, const void* W, const float* Z, int64_t ldz,
                              const int32_t* beam_rows, const float* acc, uint64_t* keys, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const ExpandLds lay = expand_lds(st.S, Kc, d, dense);
    const bool narrow = expand_threads(st) == 64;
    const dim3 grid(R);
#define CB_EXPAND(DT, DENSE, NT)                                                                      \
    hipLaunchKernelGGL((k_beam_expand<DT, DENSE, NT>), grid, dim3(NT), lay.total, s, st, K, Kc, d,   \
                       (const DT*)hidden, (const DT*)W, Z, ldz, beam_rows, acc, keys)
    if (dt == CB_BF16) {
        if (dense) { if (narrow) CB_EXPAND(uint16_t, true, 64); else CB_EXPAND(uint16_t, true, 256); }
        else { if (narrow) CB_EXPAND(uint16_t, false, 64); else CB_EXPAND(uint16_t, false, 256); }
    } else {
        if (dense) { if (narrow) CB_EXPAND(float, true, 64); else CB_EXPAND(float, true, 256); }
        else { if (narrow) CB_EXPAND(float, false, 64); else CB_EXPAND(float, false, 256); }
    }
#undef CB_EXPAND
    return hipGetLastError();
}

hipError_t launch_query_merge(const StepDev& st, int Q, int K, int Kc, const uint64_t* keys,
                              const int32_t* beam_rows, int32_t* tok, int32_t* par, int32_t* rows, float* logp,
                              hipStream_t s) {
    if (Q <= 0) return hipSuccess;
    const int P2 = next_pow2(K * Kc);
    hipLaunchKernelGGL((k_query_merge<kMergeThreads>), dim3(Q), dim3(kMergeThreads), (size_t)P2 * 8, s, st, K, Kc, P2, keys, beam_rows,
                       tok, par, rows, logp);
    return hipGetLastError();
}

hipError_t launch_gemm_scores(cb_dtype dt, int R, int V, int d, const void* H, const void* W, float* Z,
                              hipStream_t s) {
    if (R <= 0) return hipSuccess;
    if (dt == CB_BF16) {
        dim3 grid((V + kBN - 1) / kBN, (R + kBM - 1) / kBM);
        hipLaunchKernelGGL(k_gemm_bf16, grid, dim3(256), 0, s, R, V, d, (const uint16_t*)H, (const uint16_t*)W, Z,
                           (int64_t)V);
    } else {
        dim3 grid((V + 15) / 16, (R + 15) / 16);
        hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, s, R, V, d, (const float*)H, (const float*)W, Z,
                           (int64_t)V);
    }
    return hipGetLastError();
}

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

size_t expand_lds_bytes(int S, int Kc, int d, bool dense) { return (size_t)expand_lds(S, Kc, d, dense).total; }

}  // namespace cb
