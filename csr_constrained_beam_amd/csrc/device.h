// Device primitives shared by the step kernels (wave64, gfx950): number
// formats and candidate keys, wave and workgroup reductions, sorting
// networks, scoring of valid tokens, next rows, output slots, and the tiling
// constants of the full-codebook product.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "cb_internal.h"

// Every launch of the library goes through this: an ordinary launch, or,
// while the thread's timing events are set (eager kernel timing only), the
// launch with those events attached to its dispatch.
#define CB_LAUNCH(kernel, grid, block, lds, stream, ...)                                                   \
    do {                                                                                                   \
        const ::cb::LaunchEvents cb_ev_ = ::cb::launch_events();                                          \
        if (cb_ev_.start || cb_ev_.stop)                                                                   \
            hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, cb_ev_.start, cb_ev_.stop, 0, __VA_ARGS__); \
        else                                                                                               \
            hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                             \
    } while (0)

namespace cb {
namespace {

constexpr int kWave = 64;
constexpr int kSmallRow = 64;  // rows up to this many tokens take the one-wave path

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// float32 -> bf16, round to nearest, ties to even (inputs finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// e^x for the terms of the softmax sums (x <= 0, or -inf): the hardware
// base-2 exponential of x * log2(e).  Relative error ~1e-7 (the rounding of
// the product), exact at x = 0, 0 at -inf; one multiply and one transcendental
// instead of the library's range reduction.
__device__ __forceinline__ float exp_sm(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

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

// ---- wave and block primitives ----------------------------------------------
//
// Cross-lane exchanges avoid the LDS crossbar (ds_bpermute, ~100 cycles each,
// serialised by the dependent chains of sorting networks): partner lane^1 and
// lane^2 by DPP quad permutes, lane^4 and lane^8 by DPP row shifts (one per
// direction, selected by the lane's bit), lane^16 and lane^32 by the gfx950
// permlane16/permlane32 swaps.  Broadcasts from a uniform lane use readlane.

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16 || J == 32, "lane_xor: J is a power of two < 64");
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (J == 4 || J == 8) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 | J, 0xF, 0xF, false);  // lane+J
        const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 | J, 0xF, 0xF, false);  // lane-J
        return (lane_id() & J) ? dn : up;
    } else if constexpr (J == 16) {
        const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane_id() & 16) ? q[0] : q[1];
    } else {
        const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane_id() & 32) ? q[0] : q[1];
    }
}

// When j is a compile-time constant after unrolling the switch folds away;
// otherwise (loops over runtime sizes) one ds_bpermute beats a runtime switch.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int j) {
    if (!__builtin_constant_p(j)) return (uint32_t)__shfl_xor((int)v, j);
    switch (j) {
        case 1: return lane_xor<1>(v);
        case 2: return lane_xor<2>(v);
        case 4: return lane_xor<4>(v);
        case 8: return lane_xor<8>(v);
        case 16: return lane_xor<16>(v);
        default: return lane_xor<32>(v);
    }
}
__device__ __forceinline__ int lane_xor(int v, int j) { return (int)lane_xor((uint32_t)v, j); }
__device__ __forceinline__ float lane_xor(float v, int j) { return __uint_as_float(lane_xor(__float_as_uint(v), j)); }
__device__ __forceinline__ double lane_xor(double v, int j) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint64_t r = ((uint64_t)lane_xor((uint32_t)(u >> 32), j) << 32) | lane_xor((uint32_t)u, j);
    return __longlong_as_double((long long)r);
}

// Value of lane 63 - lane: mirror within each row of 16, then swap rows.
__device__ __forceinline__ uint32_t lane_reverse(uint32_t v) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row_mirror
    return lane_xor<32>(lane_xor<16>(m));
}

// Broadcast from a lane index that is the same for the whole wave.
__device__ __forceinline__ int lane_bcast(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += lane_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, lane_xor(v, o));
    return v;
}

// Max / sum over the aligned groups of w lanes (w a power of two <= 64,
// uniform over the wave): only the butterfly steps below w.  When the lanes
// from n <= w on hold the neutral value, lanes 0..w-1 get the result of all 64
// lanes, in the same order (the skipped steps would only add the neutral
// value), so a row of n tokens needs log2(w) steps instead of six.
__device__ __forceinline__ float wave_max_w(float v, int w) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        if (o < w) v = fmaxf(v, lane_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum_w(float v, int w) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        if (o < w) v += lane_xor(v, o);
    return v;
}
__device__ __forceinline__ int pow2_at_least(int n) { return n <= 1 ? 1 : 1 << (32 - __clz(n - 1)); }

// Inclusive prefix sum over the wave (butterfly: after the step with distance
// o every lane knows the total of its aligned block of 2o lanes).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    int pre = x, sum = x;
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = lane_xor(sum, o);
        if (lane & o) pre += t;
        sum += t;
    }
    return pre;
}

__device__ __forceinline__ uint64_t lane_reverse64(uint64_t v) {
    return ((uint64_t)lane_reverse((uint32_t)(v >> 32)) << 32) | lane_reverse((uint32_t)v);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
    return ((uint64_t)lane_xor((uint32_t)(v >> 32), m) << 32) | lane_xor((uint32_t)v, m);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Bitonic sort of the wave's 64 keys (one per lane), descending across lanes.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t o = shfl_xor64(v, j);
            const bool take_max = ((lane & j) == 0) == ((lane & k) == 0);
            v = take_max ? umax64(v, o) : umin64(v, o);
        }
    return v;
}

// a, b sorted descending across lanes: the 64 largest of a and b, descending.
// (max(a[l], b[63-l]) is a bitonic sequence holding them; a half-cleaner
// cascade sorts it.)
__device__ __forceinline__ uint64_t wave_merge_top(uint64_t a, uint64_t b) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t c = umax64(a, lane_reverse64(b));
#pragma unroll
    for (int j = kWave / 2; j > 0; j >>= 1) {
        const uint64_t o = shfl_xor64(c, j);
        c = ((lane & j) == 0) ? umax64(c, o) : umin64(c, o);
    }
    return c;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bitonic sort of the wave's 64 values (one per lane), descending across lanes.
__device__ __forceinline__ uint32_t wave_sort_desc32(uint32_t v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint32_t o = lane_xor(v, j);
            const bool take_max = ((lane & j) == 0) == ((lane & k) == 0);
            v = take_max ? (v > o ? v : o) : (v < o ? v : o);
        }
    return v;
}

constexpr int kWaveListCap = 256;  // keys per window of wave_top (its list holds 64 more)

// The Kc (<= 64) largest keys of the wave, descending in lanes 0..Kc-1 (0 when
// fewer).  Lane l owns M candidates; score(i) is the high half of candidate i's
// key (the order bits of its score, 0 = empty) and key(i) the full key.  tau =
// the Kc-th largest lane maximum of the scores bounds the answer from below
// (every key of the answer has a score >= tau); the candidates with score >=
// tau get their full keys compacted (ballot order) into the wave's LDS list wl
// [CAP], a window at a time, and are sorted with wave64 bitonic networks (a
// single window of at most 64 keys is ranked instead).  No block barriers.
// With TRASH, wl holds CAP + 64 entries and the list is filled without
// branches: a key outside the current window goes to its lane's slot past
// the window (the per-column loop is otherwise one divergent branch per
// column).
template <int M, int CAP = kWaveListCap, bool TRASH = (CAP == kWaveListCap), class ScoreF, class KeyF>
__device__ uint64_t wave_top(int Kc, ScoreF score, KeyF key, uint64_t* wl) {
    static_assert(CAP >= kWave && CAP % kWave == 0, "windows hold whole waves of keys");
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) mx = max(mx, score(i));
    uint32_t tau = (uint32_t)lane_bcast((int)wave_sort_desc32(mx), Kc - 1);
    if (tau == 0) tau = 1;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) cnt += score(i) >= tau;
    const int incl = wave_inclusive_scan(cnt);
    const int total = lane_bcast(incl, kWave - 1);
    uint64_t best = 0;
    bool first = true;
    for (int s0 = 0; s0 < total; s0 += CAP) {
        int pos = incl - cnt;
        if constexpr (TRASH) {
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const bool take = score(i) >= tau;
                const unsigned p = (unsigned)(pos - s0);
                wl[take && p < (unsigned)CAP ? (int)p : CAP + lane] = key(i);
                pos += take;
            }
        } else {
#pragma unroll
            for (int i = 0; i < M; ++i) {
                if (score(i) >= tau) {
                    if (pos >= s0 && pos < s0 + CAP) wl[pos - s0] = key(i);
                    ++pos;
                }
            }
        }
        wave_lds_sync();
        const int w = min(CAP, total - s0);
        if (total <= kWave) {
            // a single window: each key's rank (number of larger keys; keys
            // are unique) is its output lane, placed through the LDS list
            const uint64_t v = lane < w ? wl[lane] : 0ull;
            int rank = 0;
            for (int j = 0; j < w; ++j) rank += wl[j] > v;  // broadcast reads
            wave_lds_sync();
            if (lane < w) wl[rank] = v;
            wave_lds_sync();
            best = lane < w ? wl[lane] : 0ull;
            wave_lds_sync();
            break;
        }
        for (int c0 = 0; c0 < w; c0 += kWave) {
            const uint64_t v = wave_sort_desc(c0 + lane < w ? wl[c0 + lane] : 0ull);
            best = first ? v : wave_merge_top(best, v);
            first = false;
        }
        wave_lds_sync();
    }
    return best;
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
    const int x = wave_inclusive_scan(c);
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

// The 64 largest of one key per thread, descending, in the lanes of wave 0.
// The waves' sorted lists are merged pairwise as a tree.  stage: LDS [NT/2].
// All threads call.
template <int NT>
__device__ uint64_t block_top64(uint64_t v, uint64_t* stage) {
    v = wave_sort_desc(v);
    const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int half = NT / kWave / 2; half >= 1; half >>= 1) {
        if (w >= half && w < 2 * half) stage[(w - half) * kWave + lane] = v;
        __syncthreads();
        if (w < half) v = wave_merge_top(v, stage[w * kWave + lane]);
        __syncthreads();
    }
    return v;
}

// The Kc (<= 64) largest of the n keys key(0..n-1) (0 = empty), descending,
// written by wave 0 to out[0..Kc) (0-padded).  stage: LDS [NT]; list: LDS
// int [n].  All threads call; out is complete after the next barrier.
template <int NT, class KeyF>
__device__ void block_select_top(int n, int Kc, KeyF key, uint64_t* out, uint64_t* stage, int* list, int* red_i,
                                 uint64_t* bcast) {
    const int tid = threadIdx.x;
    if (n <= NT) {
        const uint64_t top = block_top64<NT>(tid < n ? key(tid) : 0ull, stage);
        if (tid < Kc) out[tid] = top;
        return;
    }
    uint64_t mx = 0;
    for (int j = tid; j < n; j += NT) mx = umax64(mx, key(j));
    const uint64_t t = block_top64<NT>(mx, stage);
    if (tid == Kc - 1) *bcast = t;
    __syncthreads();
    const uint64_t tau = umax64(*bcast, 1ull);
    int c = 0;
    for (int j = tid; j < n; j += NT) c += key(j) >= tau;
    int total;
    int pos = block_exclusive_scan<NT>(c, red_i, &total);
    for (int j = tid; j < n; j += NT)
        if (key(j) >= tau) list[pos++] = j;
    __syncthreads();
    uint64_t best = 0;
    for (int base = 0; base < total; base += NT) {
        const uint64_t top = block_top64<NT>(base + tid < total ? key(list[base + tid]) : 0ull, stage);
        if (tid < kWave) best = base == 0 ? top : wave_merge_top(best, top);
    }
    if (tid < Kc) out[tid] = best;
}

// Append the keys of the lanes where p holds to the LDS list keys[*count ..]
// (wave-aggregated: one LDS atomic per wave).  Their order in the list is
// immaterial (keys are unique).
__device__ __forceinline__ void wave_append(bool p, uint64_t v, uint64_t* keys, int* count) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t mask = __ballot(p);
    if (mask == 0ull) return;
    int base = 0;
    if (lane == 0) base = atomicAdd(count, __popcll(mask));
    base = __shfl(base, 0);
    if (p) keys[base + __popcll(mask & ((1ull << lane) - 1ull))] = v;
}

// The Kc (<= 64) largest of the m keys in the LDS list keys[0..m), descending,
// written by wave 0 to out[0..Kc) (0-padded); out is complete after the next
// barrier.  Keys are unique and nonzero.  Up to 64 keys: one wave ranks them.  Up to NT: only the
// ceil(m / 64) waves that hold keys sort and merge them as a tree.  More: the
// threshold selection.  stage: LDS [NT]; list: LDS int [m].  All threads call.
template <int NT>
__device__ __forceinline__ void block_select_list(int m, int Kc, const uint64_t* keys, uint64_t* out, uint64_t* stage, int* list,
                                  int* red_i, uint64_t* bcast) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    if (m > NT) {
        block_select_top<NT>(m, Kc, [&](int j) { return keys[j]; }, out, stage, list, red_i, bcast);
        return;
    }
    if (m <= kWave) {
        // one key per lane of wave 0; a key's rank is the number of larger keys
        // (keys are unique and nonzero), so it lands directly in its output
        // slot: m independent compares instead of a sorting network
        if (w == 0) {
            const uint64_t v = lane < m ? keys[lane] : 0ull;
            int rank = 0;
            for (int j = 0; j < m; ++j) rank += keys[j] > v;  // broadcast reads
            if (lane < m && rank < Kc) out[rank] = v;
            if (lane >= m && lane < Kc) out[lane] = 0ull;
        }
        return;
    }
    const int nw = (m + kWave - 1) / kWave;
    uint64_t v = 0ull;
    if (w < nw) v = wave_sort_desc(tid < m ? keys[tid] : 0ull);
    for (int s = 1; s < nw; s <<= 1) {  // uniform: m is the same for every thread
        if (w < nw && (w & (2 * s - 1)) == s) stage[(w >> 1) * kWave + lane] = v;
        __syncthreads();
        if (w + s < nw && (w & (2 * s - 1)) == 0) v = wave_merge_top(v, stage[((w + s) >> 1) * kWave + lane]);
        __syncthreads();
    }
    if (w == 0 && lane < Kc) out[lane] = v;
}

// 8 consecutive elements (16-byte aligned) as float.
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
// 8 consecutive elements kept raw in registers (loaded now, converted later),
// so that several rows' loads can be in flight before any is used.
typedef unsigned int cb_u32x4 __attribute__((ext_vector_type(4)));
typedef float cb_f32x8 __attribute__((ext_vector_type(8)));
template <typename DT>
struct Raw8;
template <>
struct Raw8<uint16_t> {
    cb_u32x4 v;
    __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const cb_u32x4*>(p); }
    __device__ __forceinline__ void zero() { v = cb_u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float dot(const float* h, float s) const {
        s = fmaf(h[0], __uint_as_float(v.x << 16), s);
        s = fmaf(h[1], __uint_as_float(v.x & 0xFFFF0000u), s);
        s = fmaf(h[2], __uint_as_float(v.y << 16), s);
        s = fmaf(h[3], __uint_as_float(v.y & 0xFFFF0000u), s);
        s = fmaf(h[4], __uint_as_float(v.z << 16), s);
        s = fmaf(h[5], __uint_as_float(v.z & 0xFFFF0000u), s);
        s = fmaf(h[6], __uint_as_float(v.w << 16), s);
        s = fmaf(h[7], __uint_as_float(v.w & 0xFFFF0000u), s);
        return s;
    }
    // the same sum with the hidden values also kept raw (converted here, so
    // that their loads need not complete before the next loads are issued)
    __device__ __forceinline__ float dot_raw(const Raw8& h, float s) const {
        float hf[8];
        hf[0] = __uint_as_float(h.v.x << 16);
        hf[1] = __uint_as_float(h.v.x & 0xFFFF0000u);
        hf[2] = __uint_as_float(h.v.y << 16);
        hf[3] = __uint_as_float(h.v.y & 0xFFFF0000u);
        hf[4] = __uint_as_float(h.v.z << 16);
        hf[5] = __uint_as_float(h.v.z & 0xFFFF0000u);
        hf[6] = __uint_as_float(h.v.w << 16);
        hf[7] = __uint_as_float(h.v.w & 0xFFFF0000u);
        return dot(hf, s);
    }
};
template <>
struct Raw8<float> {
    cb_f32x8 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const cb_f32x8*>(p); }
    __device__ __forceinline__ void zero() { v = cb_f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ float dot(const float* h, float s) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(h[i], v[i], s);
        return s;
    }
    __device__ __forceinline__ float dot_raw(const Raw8& h, float s) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(h.v[i], v[i], s);
        return s;
    }
};

__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

__device__ __forceinline__ float dot8(const float* h, const float* w, float s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf(h[i], w[i], s);
    return s;
}

__device__ __forceinline__ bool beam_live(const StepDev& st, int32_t r, float a) {
    return r >= 0 && (int64_t)r < st.n_rows && a > -INFINITY;
}

// a1 for one beam, whole block: the row's valid tokens in ascending order into
// tok_s[0..n).
template <int NT>
__device__ void block_fill_tokens(const StepDev& st, int32_t r, uint32_t e0, int n, uint16_t* tok_s, int* red_i) {
    if (st.store == CB_STORE_CSR) {
        for (int j = threadIdx.x; j < n; j += NT) tok_s[j] = st.tok[e0 + j];
        return;
    }
    const uint32_t* rb = st.bits + (int64_t)r * st.words;
    int base = 0;
    for (int w0 = 0; w0 < st.words; w0 += NT) {
        const int w = w0 + threadIdx.x;
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

// a2 (sparse) for one beam, whole block: z_s[j] = <h, W_t[tok_s[j]]>, one wave
// per token, up to four tokens in flight per wave.
template <typename DT, int NT>
__device__ void block_scores(const float* h_s, const DT* __restrict__ W, int d, const uint16_t* tok_s, int n,
                             float* z_s) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int NW = NT / kWave;
    constexpr int U = 4;
    for (int j0 = threadIdx.x / kWave; j0 < n; j0 += U * NW) {
        const DT* wr[U];
        float s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * NW;
            wr[u] = W + (int64_t)tok_s[j < n ? j : j0] * d;
            s[u] = 0.f;
        }
        for (int i = lane * 8; i < d; i += kWave * 8) {
            float h[8];
            load8(h_s + i, h);
            // raw loads of the U rows first (no use inside the guards), so
            // that they are in flight together
            Raw8<DT> w8[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (j0 + u * NW < n) w8[u].load(wr[u] + i);
                else w8[u].zero();
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (j0 + u * NW < n) s[u] = w8[u].dot(h, s[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float t = wave_sum(s[u]);
            if (lane == 0 && j0 + u * NW < n) z_s[j0 + u * NW] = t;
        }
    }
}

// block_scores for d <= CH * 512: every wave takes U tokens at a time with all
// their W_t row chunks in flight at once (the plain version waits one round
// trip per chunk), h held in registers; U = BUDGET / (VGPRs of one token's
// raw row chunks).  Products summed in the same order as block_scores (chunk
// by chunk, then the wave butterfly), so z is identical.
template <typename DT, int NT, int CH, int BUDGET = 48>
__device__ void block_scores_ch(const float* h_s, const DT* __restrict__ W, int d, const uint16_t* tok_s, int n,
                                float* z_s) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int NW = NT / kWave;
    constexpr int kRegs = CH * (sizeof(DT) == 2 ? 4 : 8);  // VGPRs per token in flight
    constexpr int U = BUDGET / kRegs > 0 ? BUDGET / kRegs : 1;
    float h[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int i = c * kWave * 8 + lane * 8;
        if (i < d) load8(h_s + i, h[c]);
        else
#pragma unroll
            for (int e = 0; e < 8; ++e) h[c][e] = 0.f;
    }
    for (int j0 = threadIdx.x / kWave; j0 < n; j0 += U * NW) {
        Raw8<DT> w8[U][CH];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * NW;
            const DT* wr = W + (int64_t)tok_s[j < n ? j : j0] * d;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int i = c * kWave * 8 + lane * 8;
                if (j < n && i < d) w8[u][c].load(wr + i);
                else w8[u][c].zero();
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float sv = 0.f;
#pragma unroll
            for (int c = 0; c < CH; ++c) sv = w8[u][c].dot(h[c], sv);
            const float t = wave_sum(sv);
            if (lane == 0 && j0 + u * NW < n) z_s[j0 + u * NW] = t;
        }
    }
}

// a3 for one beam, whole block: log-sum-exp of z_s[0..n).  The sum runs over
// kLseSlots fixed slots (slot s takes the terms s, s + kLseSlots, ...); the
// slots form groups of 64, each summed by one wave's butterfly, and the group
// sums are added in group order.  Every workgroup size gives the same bits
// (a wave takes the groups w, w + NW, ...), so the per-query step at any size,
// the persistent decode and the per-beam expansion agree exactly; the maximum
// is exact in any order.  red_f: LDS [max(NT / 64, kLseSlots / 64)].
constexpr int kLseSlots = 512;
constexpr int kLseGroups = kLseSlots / 64;
template <int NT>
__device__ float block_lse(const float* z_s, int n, float* red_f) {
    constexpr int NW = NT / kWave;
    float m = -INFINITY;
    for (int j = threadIdx.x; j < n; j += NT) m = fmaxf(m, z_s[j]);
    m = block_max<NT>(m, red_f);
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
    for (int g0 = 0; g0 < kLseGroups; g0 += NW) {
        const int g = g0 + w;
        if (g < kLseGroups) {  // uniform over the wave
            float se = 0.f;
            for (int j = g * kWave + lane; j < n; j += kLseSlots) se += exp_sm(z_s[j] - m);
            se = wave_sum(se);
            if (lane == 0) red_f[g] = se;
        }
    }
    __syncthreads();
    float r = red_f[0];
#pragma unroll
    for (int i = 1; i < kLseGroups; ++i) r += red_f[i];
    __syncthreads();
    return m + logf(r);
}

// Entries of the reduction scratch a block needs (block_max / block_sum /
// block_lse).
template <int NT>
constexpr int red_slots() {
    return NT / kWave > kLseGroups ? NT / kWave : kLseGroups;
}


// ---- full-codebook product tiling (shared with its consumers) ---------------

constexpr int kBM = 128, kBN = 128, kBK = 64, kLDP = kBK + 8;
constexpr int kWM = 32, kWN = 64;  // per-wave tile: 1 x 2 MFMA 32x32 blocks
constexpr int kGemmThreads = (kBM / kWM) * (kBN / kWN) * 64;
constexpr int kGemmLds = 2 * (kBM + kBN) * kLDP * 2;  // double-buffered A and B tiles (bytes)
constexpr int kSplitMax = 2;   // k-slices for steps with few live beams (more cost the consumer more than they save)
constexpr int kSplitRows = 2 * kBM;
constexpr int kCUs = 256;

// Number of k-slices the full-codebook product uses for n_live live beams:
// more than one only when the tiles alone would leave most compute units idle.
// The slices' partial sums are added in slice order by the consumer.
// A negative count marks a product over every beam slot (no compaction):
// one slice, scores indexed by slot.
__host__ __device__ inline int gemm_split(int n_live, int V, int d) {
    const int tiles = ((n_live + kBM - 1) / kBM) * ((V + kBN - 1) / kBN);
    int s = 1;
    if (n_live < 0 || n_live > kSplitRows) return 1;
    while (s < kSplitMax && tiles * s * 2 <= kCUs && (d / kBK) % (s * 2) == 0) s *= 2;
    return s;
}

__host__ __device__ inline int gemm_grid(int R, int V) {
    const int nt = (V + kBN - 1) / kBN;
    const int full = ((R + kBM - 1) / kBM) * nt;
    const int split = kSplitMax * ((kSplitRows + kBM - 1) / kBM) * nt;
    return full > split ? full : split;
}

}  // namespace
}  // namespace cb
