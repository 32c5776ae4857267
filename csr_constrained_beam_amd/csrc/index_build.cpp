// Host construction of the step-sliced prefix index.
//
// The catalog is sorted and made duplicate free (it is a set: STATIC sec. 4.1).
// In sorted order the distinct length-t prefixes are contiguous runs, so one
// pass per step yields the step table (ZeroGR summary, "Why slice the index by
// decoding step?"): row r of step t is the r-th distinct length-t prefix; its
// edges are the distinct length-(t+1) prefixes that extend it, ascending by
// token, and the position of an edge is the row it leads to in step t+1 (no
// next-row array is stored).  Wide steps keep a bitmap per row instead of the
// token list, so that a row's columns line up with a full-codebook score row
// (ZeroGR: dense tables for steps where many tokens are valid).
#include <algorithm>
#include <cstring>
#include <thread>

#include "cb_internal.h"

namespace cb {
namespace {

int bits_for(int V) {
    int b = 1;
    while ((1 << b) < V) ++b;
    return b;
}

int n_threads() {
    unsigned h = std::thread::hardware_concurrency();
    return (int)std::max(1u, std::min(h ? h : 1u, 16u));
}

template <class F>
void parallel_for(int64_t n, F&& f) {
    int T = n_threads();
    if (n < 65536 || T == 1) {
        f(int64_t(0), n);
        return;
    }
    std::vector<std::thread> th;
    for (int i = 0; i < T; ++i) {
        int64_t lo = n * i / T, hi = n * (i + 1) / T;
        th.emplace_back([&f, lo, hi] { f(lo, hi); });
    }
    for (auto& x : th) x.join();
}

// A catalog row packed most-significant token first, so that comparing the
// words in order compares the rows lexicographically.
template <int NW>
struct Packed {
    uint64_t w[NW];
    bool operator<(const Packed& o) const {
        for (int i = 0; i < NW; ++i)
            if (w[i] != o.w[i]) return w[i] < o.w[i];
        return false;
    }
    bool operator==(const Packed& o) const {
        for (int i = 0; i < NW; ++i)
            if (w[i] != o.w[i]) return false;
        return true;
    }
};

template <class T>
void parallel_sort(std::vector<T>& v) {
    int T_ = n_threads();
    int64_t n = (int64_t)v.size();
    if (n < (1 << 20) || T_ == 1) {
        std::sort(v.begin(), v.end());
        return;
    }
    std::vector<int64_t> cut(T_ + 1);
    for (int i = 0; i <= T_; ++i) cut[i] = n * i / T_;
    {
        std::vector<std::thread> th;
        for (int i = 0; i < T_; ++i)
            th.emplace_back([&, i] { std::sort(v.begin() + cut[i], v.begin() + cut[i + 1]); });
        for (auto& x : th) x.join();
    }
    for (int width = 1; width < T_; width *= 2) {
        std::vector<std::thread> th;
        for (int i = 0; i + width < T_; i += 2 * width) {
            int64_t lo = cut[i], mid = cut[i + width], hi = cut[std::min(i + 2 * width, T_)];
            th.emplace_back([&, lo, mid, hi] { std::inplace_merge(v.begin() + lo, v.begin() + mid, v.begin() + hi); });
        }
        for (auto& x : th) x.join();
    }
}

template <int NW>
cb_status build_impl(const int32_t* sids, int64_t n, int32_t L, int32_t V, int32_t store, cb_index* idx,
                     StepUploader* up) {
    const int b = bits_for(V);
    const int per = 64 / b;
    const uint64_t mask = (uint64_t(1) << b) - 1;
    auto token_of = [&](const Packed<NW>& p, int t) -> int32_t {
        int sh = (per - 1 - t % per) * b;
        return (int32_t)((p.w[t / per] >> sh) & mask);
    };

    std::vector<Packed<NW>> keys;
    try {
        keys.resize((size_t)n);
    } catch (...) {
        set_error("cb_build_index: host allocation failed");
        return CB_ENOMEM;
    }
    parallel_for(n, [&](int64_t lo, int64_t hi) {
        for (int64_t i = lo; i < hi; ++i) {
            Packed<NW> p;
            for (int k = 0; k < NW; ++k) p.w[k] = 0;
            for (int t = 0; t < L; ++t) p.w[t / per] |= (uint64_t)sids[i * L + t] << ((per - 1 - t % per) * b);
            keys[(size_t)i] = p;
        }
    });
    parallel_sort(keys);
    keys.erase(std::unique(keys.begin(), keys.end()), keys.end());
    const int64_t N = (int64_t)keys.size();
    idx->n_items = N;

    // fd[i] = first position where item i differs from item i-1 (-1 for i = 0).
    std::vector<int8_t> fd((size_t)N);
    parallel_for(N, [&](int64_t lo, int64_t hi) {
        for (int64_t i = lo; i < hi; ++i) {
            if (i == 0) {
                fd[0] = -1;
                continue;
            }
            int t = 0;
            while (t < L && token_of(keys[(size_t)i], t) == token_of(keys[(size_t)i - 1], t)) ++t;
            fd[(size_t)i] = (int8_t)t;  // t < L: rows are distinct
        }
    });

    idx->steps.assign((size_t)L, StepTable());
    idx->words = (V + 31) / 32;
    const int words = idx->words;
    // chunks of consecutive sorted items; each chunk's first row and first
    // edge are known in advance (prefix sums of the chunks' counts), so every
    // chunk fills its own part of the tables independently
    const int64_t C = std::max<int64_t>(1, std::min<int64_t>(256, N / 4096));
    std::vector<int64_t> cut((size_t)C + 1);
    for (int64_t c = 0; c <= C; ++c) cut[(size_t)c] = N * c / C;
    auto over_chunks = [&](auto&& f) {
        const int T_ = std::min<int>(n_threads(), (int)C);
        if (T_ <= 1) {
            for (int64_t c = 0; c < C; ++c) f(c);
            return;
        }
        std::vector<std::thread> th;
        for (int w = 0; w < T_; ++w)
            th.emplace_back([&, w] {
                for (int64_t c = w; c < C; c += T_) f(c);
            });
        for (auto& x : th) x.join();
    };
    std::vector<int64_t> r0((size_t)C + 1), e0((size_t)C + 1);
    for (int t = 0; t < L; ++t) {
        StepTable& T = idx->steps[(size_t)t];
        // pass 1: rows (items where a new length-t prefix starts) and edges
        // (items where a new length-(t+1) prefix starts) of every chunk
        over_chunks([&](int64_t c) {
            int64_t nr = 0, ne = 0;
            for (int64_t i = cut[(size_t)c]; i < cut[(size_t)c + 1]; ++i) {
                nr += fd[(size_t)i] < t;
                ne += fd[(size_t)i] <= t;
            }
            r0[(size_t)c + 1] = nr;
            e0[(size_t)c + 1] = ne;
        });
        r0[0] = e0[0] = 0;
        for (int64_t c = 0; c < C; ++c) {
            r0[(size_t)c + 1] += r0[(size_t)c];
            e0[(size_t)c + 1] += e0[(size_t)c];
        }
        const int64_t nr = r0[(size_t)C], ne = e0[(size_t)C];
        T.n_rows = nr;
        T.n_edges = ne;
        const int64_t bitmap_bytes = nr * (int64_t)words * 6;  // bits + rank directory
        const int64_t csr_bytes = ne * 2;
        const bool bitmap = store == CB_STORE_BITMAP || (store == CB_STORE_AUTO && bitmap_bytes < csr_bytes);
        try {
            T.row_ptr.resize((size_t)nr + 1);
            if (bitmap) {
                T.bits.assign((size_t)(nr * words), 0u);
                T.rank.assign((size_t)(nr * words), 0);
            } else {
                T.tok.resize((size_t)ne);
                // first token of every row, read together with row_ptr so that a
                // one-token row needs no second dependent read
                T.tok0.resize((size_t)nr);
            }
        } catch (...) {
            // the caller frees the index once the upload thread has stopped
            set_error("cb_build_index: host allocation failed");
            return CB_ENOMEM;
        }
        // pass 2: every chunk fills its rows and edges at its precomputed
        // positions (a row whose edges straddle chunks gets its bitmap bits
        // from both, hence the atomic OR)
        over_chunks([&](int64_t c) {
            int64_t r = r0[(size_t)c], e = e0[(size_t)c];
            for (int64_t i = cut[(size_t)c]; i < cut[(size_t)c + 1]; ++i) {
                const int f = fd[(size_t)i];
                if (f > t) continue;
                const uint32_t v = (uint32_t)token_of(keys[(size_t)i], t);
                if (f < t) {
                    T.row_ptr[(size_t)r] = (uint32_t)e;
                    if (!bitmap) T.tok0[(size_t)r] = (uint16_t)v;
                    ++r;
                }
                if (bitmap)
                    __atomic_fetch_or(&T.bits[(size_t)((r - 1) * words + (v >> 5))], 1u << (v & 31), __ATOMIC_RELAXED);
                else
                    T.tok[(size_t)e] = (uint16_t)v;
                ++e;
            }
        });
        T.row_ptr[(size_t)nr] = (uint32_t)ne;
        // pass 3, over the rows of every chunk: the widest row and (bitmap)
        // the rank directory
        std::vector<int32_t> Sc((size_t)C, 0);
        over_chunks([&](int64_t c) {
            int32_t S = 0;
            for (int64_t k = nr * c / C; k < nr * (c + 1) / C; ++k) {
                S = std::max<int32_t>(S, (int32_t)(T.row_ptr[(size_t)k + 1] - T.row_ptr[(size_t)k]));
                if (bitmap) {
                    uint32_t cnt = 0;
                    for (int w = 0; w < words; ++w) {
                        T.rank[(size_t)(k * words + w)] = (uint16_t)cnt;
                        cnt += (uint32_t)__builtin_popcount(T.bits[(size_t)(k * words + w)]);
                    }
                }
            }
            Sc[(size_t)c] = S;
        });
        T.S = *std::max_element(Sc.begin(), Sc.end());
        T.store = bitmap ? CB_STORE_BITMAP : CB_STORE_CSR;
        T.bytes = bitmap ? (nr + 1) * 4 + bitmap_bytes : (nr + 1) * 4 + csr_bytes + nr * 2;
        // the finished step is streamed to the device while the next is built
        if (up) up->push(t);
    }
    return CB_OK;
}

}  // namespace

cb_status build_host_tables(const int32_t* sids, int64_t n_items, int32_t L, int32_t V, int32_t store,
                            cb_index* idx, StepUploader* up) {
    const int b = bits_for(V);
    const int per = 64 / b;
    const int nw = (L + per - 1) / per;
    idx->L = L;
    idx->V = V;
    switch (nw) {
        case 1: return build_impl<1>(sids, n_items, L, V, store, idx, up);
        case 2: return build_impl<2>(sids, n_items, L, V, store, idx, up);
        case 3: return build_impl<3>(sids, n_items, L, V, store, idx, up);
        case 4: return build_impl<4>(sids, n_items, L, V, store, idx, up);
        default:
            set_error("cb_build_index: L * ceil(log2 V) exceeds 256 bits");
            return CB_EUNSUPPORTED;
    }
}

}  // namespace cb
