// Save and load of a built step-sliced index (the index rebuild pipeline:
// build once on the host, keep the tables, bring them back to HBM without
// re-sorting the catalog; ZeroGR summary, the index built on the CPU and
// streamed to the GPU).
//
// File layout (little-endian): the 8-byte tag "CBINDEX1"; int32 L, V; int64
// n_items; then per step int64 n_rows, n_edges; int32 S, storage; and the
// step's arrays: row_ptr [n_rows + 1] u32; CSR: tok [n_edges] u16, tok0
// [n_rows] u16; bitmap: bits [n_rows * words] u32, rank [n_rows * words] u16
// (words = ceil(V / 32)); last an FNV-1a 64-bit hash of every byte before it.
// Loading checks every structural invariant of the tables, so a damaged file
// is rejected on the host instead of reaching a kernel.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <memory>

#include "cb_internal.h"

namespace cb {
namespace {

constexpr char kTag[8] = {'C', 'B', 'I', 'N', 'D', 'E', 'X', '1'};

struct Writer {
    FILE* f;
    uint64_t h = 1469598103934665603ull;
    bool ok = true;
    void put(const void* p, size_t n) {
        const unsigned char* c = static_cast<const unsigned char*>(p);
        for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 1099511628211ull;
        ok = ok && std::fwrite(p, 1, n, f) == n;
    }
    template <typename T>
    void val(T v) { put(&v, sizeof v); }
};

struct Reader {
    FILE* f;
    uint64_t h = 1469598103934665603ull;
    bool ok = true;
    void get(void* p, size_t n) {
        if (!ok || std::fread(p, 1, n, f) != n) {
            ok = false;
            return;
        }
        const unsigned char* c = static_cast<const unsigned char*>(p);
        for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 1099511628211ull;
    }
    template <typename T>
    T val() {
        T v{};
        get(&v, sizeof v);
        return v;
    }
};

// The host arrays of step t (device tables are copied back).
template <typename T>
bool fetch(const std::vector<T>& host, const T* dev, size_t n, std::vector<T>& out) {
    if (!host.empty() || n == 0) {
        out = host;
        return out.size() == n;
    }
    out.resize(n);
    return hipMemcpy(out.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

bool fail(const std::string& m) {
    set_error("cb_index_load: " + m);
    return false;
}

// Structural checks of one loaded step (prev_edges: edges of step t-1).
bool check_step(const StepTable& T, int t, int64_t prev_edges, int32_t V, int32_t words) {
    const std::string at = " (step " + std::to_string(t) + ")";
    if (T.n_rows != (t == 0 ? 1 : prev_edges)) return fail("row count does not follow the previous step" + at);
    if (T.row_ptr.size() != (size_t)T.n_rows + 1 || T.row_ptr[0] != 0 || T.row_ptr.back() != (uint64_t)T.n_edges)
        return fail("row pointers do not span the edges" + at);
    int32_t S = 0;
    for (int64_t r = 0; r < T.n_rows; ++r) {
        if (T.row_ptr[(size_t)r + 1] <= T.row_ptr[(size_t)r]) return fail("a row without edges" + at);
        S = std::max<int32_t>(S, (int32_t)(T.row_ptr[(size_t)r + 1] - T.row_ptr[(size_t)r]));
    }
    if (S != T.S) return fail("widest row differs from its record" + at);
    if (T.store == CB_STORE_CSR) {
        if (T.tok0.size() != (size_t)T.n_rows) return fail("first-token array size" + at);
        for (int64_t r = 0; r < T.n_rows; ++r) {
            const uint32_t a = T.row_ptr[(size_t)r], b = T.row_ptr[(size_t)r + 1];
            if (T.tok0[(size_t)r] != T.tok[a]) return fail("first token differs from the row's" + at);
            for (uint32_t e = a; e < b; ++e)
                if (T.tok[e] >= V || (e > a && T.tok[e] <= T.tok[e - 1]))
                    return fail("tokens out of range or not ascending within a row" + at);
        }
    } else if (T.store == CB_STORE_BITMAP) {
        for (int64_t r = 0; r < T.n_rows; ++r) {
            uint32_t c = 0;
            for (int w = 0; w < words; ++w) {
                const size_t x = (size_t)r * words + w;
                if (T.rank[x] != c) return fail("rank directory inconsistent" + at);
                uint32_t bits = T.bits[x];
                if (w == words - 1 && (V & 31)) bits &= ~((1u << (V & 31)) - 1u);
                else bits = 0u;
                if (bits) return fail("bit set for a token >= V" + at);
                c += (uint32_t)__builtin_popcount(T.bits[x]);
            }
            if (c != T.row_ptr[(size_t)r + 1] - T.row_ptr[(size_t)r]) return fail("bitmap row size" + at);
        }
    } else {
        return fail("unknown storage" + at);
    }
    return true;
}

}  // namespace
}  // namespace cb

using namespace cb;

extern "C" {

cb_status cb_index_save(const cb_index* idx, const char* path) {
    clear_error();
    if (!idx || !path) {
        set_error("cb_index_save: index or path is NULL");
        return CB_EINVAL;
    }
    std::unique_ptr<FILE, int (*)(FILE*)> f(std::fopen(path, "wb"), std::fclose);
    if (!f) {
        set_error(std::string("cb_index_save: cannot open ") + path);
        return CB_EINVAL;
    }
    Writer w{f.get()};
    w.put(kTag, sizeof kTag);
    w.val<int32_t>(idx->L);
    w.val<int32_t>(idx->V);
    w.val<int64_t>(idx->n_items);
    DeviceGuard guard(idx->device);  // restores the caller's device on return
    if (!guard.ok) {
        set_error("cb_index_save: cannot select the index's device");
        return CB_EHIP;
    }
    for (const auto& T : idx->steps) {
        w.val<int64_t>(T.n_rows);
        w.val<int64_t>(T.n_edges);
        w.val<int32_t>(T.S);
        w.val<int32_t>(T.store);
        std::vector<uint32_t> rp, bits;
        std::vector<uint16_t> tok, tok0, rank;
        const size_t cells = (size_t)T.n_rows * idx->words;
        bool ok = fetch(T.row_ptr, T.d_row_ptr, (size_t)T.n_rows + 1, rp);
        if (T.store == CB_STORE_CSR)
            ok = ok && fetch(T.tok, T.d_tok, (size_t)T.n_edges, tok) && fetch(T.tok0, T.d_tok0, (size_t)T.n_rows, tok0);
        else
            ok = ok && fetch(T.bits, T.d_bits, cells, bits) && fetch(T.rank, T.d_rank, cells, rank);
        if (!ok) {
            set_error("cb_index_save: reading the tables back failed");
            return CB_EHIP;
        }
        w.put(rp.data(), rp.size() * 4);
        if (T.store == CB_STORE_CSR) {
            w.put(tok.data(), tok.size() * 2);
            w.put(tok0.data(), tok0.size() * 2);
        } else {
            w.put(bits.data(), bits.size() * 4);
            w.put(rank.data(), rank.size() * 2);
        }
    }
    const uint64_t h = w.h;
    w.put(&h, sizeof h);
    if (!w.ok) {
        set_error(std::string("cb_index_save: write failed: ") + path);
        return CB_EINVAL;
    }
    return CB_OK;
}

cb_status cb_index_load(const char* path, int32_t device, cb_index** out) {
    clear_error();
    if (!path || !out) {
        set_error("cb_index_load: path or out is NULL");
        return CB_EINVAL;
    }
    *out = nullptr;
    std::unique_ptr<FILE, int (*)(FILE*)> f(std::fopen(path, "rb"), std::fclose);
    if (!f) {
        set_error(std::string("cb_index_load: cannot open ") + path);
        return CB_EINVAL;
    }
    Reader r{f.get()};
    char tag[8];
    r.get(tag, sizeof tag);
    if (!r.ok || std::memcmp(tag, kTag, sizeof tag) != 0) {
        set_error("cb_index_load: not an index file (tag)");
        return CB_EINVAL;
    }
    std::unique_ptr<cb_index> idx(new (std::nothrow) cb_index());
    if (!idx) {
        set_error("cb_index_load: host allocation failed");
        return CB_ENOMEM;
    }
    idx->L = r.val<int32_t>();
    idx->V = r.val<int32_t>();
    idx->n_items = r.val<int64_t>();
    if (!r.ok || idx->L < 1 || idx->L > 64 || idx->V < 2 || idx->V > 65535 || idx->n_items < 1 ||
        idx->n_items >= (int64_t(1) << 31)) {
        set_error("cb_index_load: bad header");
        return CB_EINVAL;
    }
    idx->words = (idx->V + 31) / 32;
    idx->steps.resize((size_t)idx->L);
    int64_t prev_edges = 0;
    for (int t = 0; t < idx->L; ++t) {
        StepTable& T = idx->steps[(size_t)t];
        T.n_rows = r.val<int64_t>();
        T.n_edges = r.val<int64_t>();
        T.S = r.val<int32_t>();
        T.store = r.val<int32_t>();
        if (!r.ok || T.n_rows < 1 || T.n_edges < T.n_rows || T.n_edges > idx->n_items ||
            T.n_rows > idx->n_items || (T.store != CB_STORE_CSR && T.store != CB_STORE_BITMAP)) {
            set_error("cb_index_load: bad step record (step " + std::to_string(t) + ")");
            return CB_EINVAL;
        }
        const size_t cells = (size_t)T.n_rows * idx->words;
        try {
            T.row_ptr.resize((size_t)T.n_rows + 1);
            if (T.store == CB_STORE_CSR) {
                T.tok.resize((size_t)T.n_edges);
                T.tok0.resize((size_t)T.n_rows);
            } else {
                T.bits.resize(cells);
                T.rank.resize(cells);
            }
        } catch (...) {
            set_error("cb_index_load: host allocation failed");
            return CB_ENOMEM;
        }
        r.get(T.row_ptr.data(), T.row_ptr.size() * 4);
        if (T.store == CB_STORE_CSR) {
            r.get(T.tok.data(), T.tok.size() * 2);
            r.get(T.tok0.data(), T.tok0.size() * 2);
            T.bytes = (T.n_rows + 1) * 4 + T.n_edges * 2 + T.n_rows * 2;
        } else {
            r.get(T.bits.data(), T.bits.size() * 4);
            r.get(T.rank.data(), T.rank.size() * 2);
            T.bytes = (T.n_rows + 1) * 4 + T.n_rows * (int64_t)idx->words * 6;
        }
        if (!r.ok) {
            set_error("cb_index_load: file ends early (step " + std::to_string(t) + ")");
            return CB_EINVAL;
        }
        if (!check_step(T, t, prev_edges, idx->V, idx->words)) return CB_EINVAL;
        prev_edges = T.n_edges;
    }
    if (prev_edges != idx->n_items) {
        set_error("cb_index_load: the last step's edges differ from the item count");
        return CB_EINVAL;
    }
    const uint64_t h = r.h;
    const uint64_t stored = r.val<uint64_t>();
    if (!r.ok || stored != h) {
        set_error("cb_index_load: hash mismatch (damaged file)");
        return CB_EINVAL;
    }
    idx->device = device;
    cb_index* raw = idx.release();
    if (device >= 0) {
        const cb_status st = upload_index(raw);  // frees raw on failure
        if (st != CB_OK) return st;
    }
    *out = raw;
    return CB_OK;
}

}  // extern "C"
