/* Seeded catalog drawing for the large Zipf-family workloads.
 *
 * Generation only: this file draws token sequences and rejects repeated ones.
 * It contains none of the decoding arithmetic.
 *
 * Randomness is counter-based: every uniform is splitmix64 of a word built
 * from (seed, draw number, level, purpose), so draw k is the same whatever
 * the thread count.  Item k of the output is the k-th distinct sequence in
 * draw order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline double uniform01(uint64_t seed, uint64_t draw, uint64_t level, uint64_t purpose) {
    uint64_t x = mix64(seed ^ mix64(draw * 0x1000193ull + level * 0x10001ull + purpose * 0x3C6EF372FE94F82Bull));
    return (double)(x >> 11) * (1.0 / 9007199254740992.0);
}

static inline int64_t upper_bound(const double* cdf, int64_t n, double u) {
    int64_t lo = 0, hi = n;  /* first index with cdf[i] > u */
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (cdf[mid] > u) hi = mid; else lo = mid + 1;
    }
    return lo < n ? lo : n - 1;
}

static int64_t gcd64(int64_t a, int64_t b) { while (b) { int64_t t = a % b; a = b; b = t; } return a; }

typedef struct {
    uint64_t seed;
    int L, codebook, eos, min_len, max_len;
    const double* cdf;
    const int64_t* units;
    int64_t n_units;
} params_t;

/* Draw sequence number `k` into row[0..L). */
static void draw_one(const params_t* p, uint64_t k, int32_t* row) {
    uint64_t h = mix64(p->seed ^ 0xA5A5A5A5A5A5A5A5ull);
    int len = p->L;
    if (p->eos >= 0) {
        double u = uniform01(p->seed, k, 0, 7);
        len = p->min_len + (int)(u * (double)(p->max_len - p->min_len + 1));
        if (len > p->max_len) len = p->max_len;
    }
    for (int t = 0; t < p->L; ++t) {
        if (t >= len) { row[t] = p->eos; continue; }
        double u = uniform01(p->seed, k, (uint64_t)t, 1);
        int64_t r = upper_bound(p->cdf, p->codebook, u);
        uint64_t hm = mix64(h);
        int64_t a = p->units[hm % (uint64_t)p->n_units];
        int64_t b = (int64_t)((hm >> 32) % (uint64_t)p->codebook);
        int64_t tok = (a * r + b) % p->codebook;
        row[t] = (int32_t)tok;
        h = mix64(h ^ ((uint64_t)(tok + 1) * (0x100000001B3ull + (uint64_t)t)));
    }
}

static uint64_t row_hash(const int32_t* row, int L) {
    uint64_t h = 0x12345678ull;
    for (int t = 0; t < L; ++t) h = mix64(h ^ ((uint64_t)(uint32_t)row[t] + ((uint64_t)t << 40)));
    return h;
}

/* Draw distinct sequences until n_items exist.  out: int32 [n_items][L].
 * eos < 0: fixed length L.  Otherwise length ~ U{min_len..max_len} and the
 * tail holds eos.  Returns the number of draws used, or -1 on allocation
 * failure. */
int64_t synth_zipf_items(uint64_t seed, int64_t n_items, int L, int codebook, int eos,
                         double zipf_s, int min_len, int max_len, int32_t* out) {
    double* cdf = (double*)malloc(sizeof(double) * (size_t)codebook);
    int64_t* units = (int64_t*)malloc(sizeof(int64_t) * (size_t)codebook);
    if (!cdf || !units) { free(cdf); free(units); return -1; }
    double acc = 0.0;
    for (int i = 0; i < codebook; ++i) { acc += pow((double)(i + 1), -zipf_s); cdf[i] = acc; }
    for (int i = 0; i < codebook; ++i) cdf[i] /= acc;
    int64_t nu = 0;
    for (int64_t a = 1; a < codebook; ++a) if (gcd64(a, codebook) == 1) units[nu++] = a;
    params_t p = {seed, L, codebook, eos, min_len, max_len, cdf, units, nu};

    /* open-addressing set of (hash, item index) */
    uint64_t cap = 1;
    while (cap < (uint64_t)n_items * 2) cap <<= 1;
    uint64_t* hs = (uint64_t*)calloc(cap, sizeof(uint64_t));
    int64_t* ix = (int64_t*)malloc(cap * sizeof(int64_t));
    const int64_t B = 1 << 20;
    int32_t* buf = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * (size_t)L);
    if (!hs || !ix || !buf) { free(cdf); free(units); free(hs); free(ix); free(buf); return -1; }

    int64_t have = 0;
    uint64_t next = 0;
    while (have < n_items) {
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < B; ++i) draw_one(&p, next + (uint64_t)i, buf + i * L);
        for (int64_t i = 0; i < B && have < n_items; ++i) {
            const int32_t* row = buf + i * L;
            uint64_t h = row_hash(row, L) | 1ull;  /* 0 marks an empty slot */
            uint64_t s = h & (cap - 1);
            int dup = 0;
            while (hs[s]) {
                if (hs[s] == h && memcmp(out + ix[s] * L, row, sizeof(int32_t) * (size_t)L) == 0) { dup = 1; break; }
                s = (s + 1) & (cap - 1);
            }
            if (dup) continue;
            hs[s] = h;
            ix[s] = have;
            memcpy(out + have * L, row, sizeof(int32_t) * (size_t)L);
            ++have;
        }
        next += (uint64_t)B;
    }
    free(cdf); free(units); free(hs); free(ix); free(buf);
    return (int64_t)next;
}
