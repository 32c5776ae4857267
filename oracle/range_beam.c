/* Second CPU oracle: beam search over the sorted catalog (no trie).
 *
 * TEST INFRASTRUCTURE ONLY (see trie_beam.c).  Same definition as the trie
 * oracle, computed another way, so that the two check each other and so that
 * catalogs too large for a pointer trie (100M items of 12 tokens) can still be
 * decoded on the host:
 *
 *  - The catalog is sorted lexicographically and repeats are dropped.  The
 *    items that start with a prefix p of length t form one contiguous range
 *    [lo, hi) of the sorted catalog; the valid next tokens of p are the
 *    distinct tokens at position t inside that range (the constraint of
 *    ZeroGR "What problem is it solving?" and STATIC sec. 4.1), found by binary
 *    search since they are sorted.
 *  - The row of p (its rank among the distinct length-t prefixes) is
 *    rank_t[lo], where rank_t[i] counts the distinct length-t prefixes among
 *    sorted items 0..i, minus one.  A row r is mapped back to its range by
 *    binary search of r in the non-decreasing array rank_t.
 *  - Scoring, softmax over the valid tokens, the float32 rounding points and
 *    the selection order are those of the trie oracle (filter first; ZeroGR
 *    "The pipeline").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct or_range {
    int L, V;
    int64_t n;           /* distinct items */
    int32_t* items;      /* sorted distinct items [n][L] */
    int32_t** rank;      /* rank[t][i], t = 1..L (rank[0] unused) */
    int64_t* count;      /* distinct prefixes per depth [L+1] */
} or_range;

void orr_free(or_range* R) {
    if (!R) return;
    free(R->items);
    if (R->rank)
        for (int t = 0; t <= R->L; ++t) free(R->rank[t]);
    free(R->rank);
    free(R->count);
    free(R);
}

or_range* orr_build(const int32_t* sids, int64_t n, int L, int V) {
    if (L < 1 || V < 1 || n < 0) return NULL;
    for (int64_t i = 0; i < n * L; ++i)
        if (sids[i] < 0 || sids[i] >= V) return NULL;
    or_range* R = (or_range*)calloc(1, sizeof(or_range));
    int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n ? n : 1));
    int64_t* tmp = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n ? n : 1));
    int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * ((size_t)V + 1));
    if (!R || !order || !tmp || !cnt) {
        free(order); free(tmp); free(cnt); orr_free(R);
        return NULL;
    }
    R->L = L;
    R->V = V;
    for (int64_t i = 0; i < n; ++i) order[i] = i;
    for (int t = L - 1; t >= 0; --t) {  /* stable counting sort, last position first */
        memset(cnt, 0, sizeof(int64_t) * ((size_t)V + 1));
        for (int64_t k = 0; k < n; ++k) cnt[sids[order[k] * L + t] + 1]++;
        for (int v = 0; v < V; ++v) cnt[v + 1] += cnt[v];
        for (int64_t k = 0; k < n; ++k) tmp[cnt[sids[order[k] * L + t]]++] = order[k];
        int64_t* sw = order; order = tmp; tmp = sw;
    }
    free(tmp);
    free(cnt);
    R->items = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n ? n : 1) * (size_t)L);
    if (!R->items) { free(order); orr_free(R); return NULL; }
    int64_t m = 0;
    for (int64_t k = 0; k < n; ++k) {
        const int32_t* row = sids + order[k] * L;
        if (m > 0 && memcmp(R->items + (m - 1) * L, row, sizeof(int32_t) * (size_t)L) == 0) continue;
        memcpy(R->items + m * L, row, sizeof(int32_t) * (size_t)L);
        ++m;
    }
    free(order);
    R->n = m;
    R->rank = (int32_t**)calloc((size_t)L + 1, sizeof(int32_t*));
    R->count = (int64_t*)calloc((size_t)L + 1, sizeof(int64_t));
    if (!R->rank || !R->count) { orr_free(R); return NULL; }
    R->count[0] = 1;
    /* first position where item i differs from item i-1 (0 for i = 0): item i
     * starts a new length-t prefix iff that position is < t */
    unsigned char* fd = (unsigned char*)malloc((size_t)(m ? m : 1));
    if (!fd) { orr_free(R); return NULL; }
    for (int64_t i = 0; i < m; ++i) {
        int u = 0;
        if (i > 0)
            while (u < L && R->items[i * L + u] == R->items[(i - 1) * L + u]) ++u;
        fd[i] = (unsigned char)u;
    }
    for (int t = 1; t <= L; ++t) {
        R->rank[t] = (int32_t*)malloc(sizeof(int32_t) * (size_t)(m ? m : 1));
        if (!R->rank[t]) { free(fd); orr_free(R); return NULL; }
        int64_t c = -1;
        for (int64_t i = 0; i < m; ++i) {
            if (fd[i] < t) ++c;
            R->rank[t][i] = (int32_t)c;
        }
        R->count[t] = c + 1;
    }
    free(fd);
    return R;
}

int64_t orr_n_items(const or_range* R) { return R->n; }

int64_t orr_level_count(const or_range* R, int depth) {
    if (depth < 0 || depth > R->L) return -1;
    return R->count[depth];
}

/* first index in [lo, hi) whose token at position t is > v (tokens there ascend) */
static int64_t upper_tok(const or_range* R, int64_t lo, int64_t hi, int t, int32_t v) {
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (R->items[mid * R->L + t] <= v) lo = mid + 1; else hi = mid;
    }
    return lo;
}

/* range [lo, hi) of the prefix with row `row` at depth t */
static int range_of_row(const or_range* R, int t, int64_t row, int64_t* lo, int64_t* hi) {
    if (t < 0 || t > R->L || row < 0 || row >= R->count[t]) return -1;
    if (t == 0) { *lo = 0; *hi = R->n; return 0; }
    const int32_t* rk = R->rank[t];
    int64_t a = 0, b = R->n;
    while (a < b) { int64_t mid = a + (b - a) / 2; if (rk[mid] < row) a = mid + 1; else b = mid; }
    int64_t c = a, e = R->n;
    while (c < e) { int64_t mid = c + (e - c) / 2; if (rk[mid] <= row) c = mid + 1; else e = mid; }
    *lo = a;
    *hi = c;
    return 0;
}

/* children of row `row` at depth t: tokens ascending, their rows at depth t+1 */
int orr_children_of_row(const or_range* R, int t, int64_t row, int32_t* tokens, int64_t* rows, int64_t cap) {
    if (t < 0 || t >= R->L) return -1;
    int64_t lo, hi;
    if (range_of_row(R, t, row, &lo, &hi) != 0) return -1;
    int k = 0;
    for (int64_t j = lo; j < hi;) {
        const int32_t v = R->items[j * R->L + t];
        if (k < cap) {
            if (tokens) tokens[k] = v;
            if (rows) rows[k] = R->rank[t + 1][j];
        }
        ++k;
        j = upper_tok(R, j, hi, t, v);
    }
    return k;
}

typedef struct {
    float score;
    int32_t parent;
    int32_t token;
    int64_t row;
} rcand_t;

static int rcand_cmp(const void* a, const void* b) {
    const rcand_t* x = (const rcand_t*)a;
    const rcand_t* y = (const rcand_t*)b;
    if (x->score != y->score) return x->score > y->score ? -1 : 1;
    if (x->parent != y->parent) return x->parent < y->parent ? -1 : 1;
    if (x->token != y->token) return x->token < y->token ? -1 : 1;
    return 0;
}

/* All candidates of one query (K slots), sorted best first; *out malloc'ed.
 * rows[k] < 0 = dead.  Beams are scored in parallel (OpenMP) when threads > 1. */
static int64_t query_cands(const or_range* R, int t, int K, int d, const float* h, const float* Wt,
                           const int64_t* rows, const float* acc, rcand_t** out, int threads) {
    int64_t* off = (int64_t*)calloc((size_t)K + 1, sizeof(int64_t));
    if (!off) return -1;
    for (int k = 0; k < K; ++k) {
        int64_t c = 0;
        if (rows[k] >= 0) c = orr_children_of_row(R, t, rows[k], NULL, NULL, 0);
        off[k + 1] = off[k] + (c > 0 ? c : 0);
    }
    const int64_t total = off[K];
    rcand_t* c = (rcand_t*)malloc(sizeof(rcand_t) * (size_t)(total ? total : 1));
    if (!c) { free(off); return -1; }
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 0 ? threads : 1)
    for (int k = 0; k < K; ++k) {
        const int64_t nk = off[k + 1] - off[k];
        if (nk == 0) continue;
        int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)nk);
        int64_t* rw = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
        double* z = (double*)malloc(sizeof(double) * (size_t)nk);
        if (!tok || !rw || !z) {
            #pragma omp atomic write
            err = 1;
            free(tok); free(rw); free(z);
            continue;
        }
        orr_children_of_row(R, t, rows[k], tok, rw, nk);
        const float* hb = h + (int64_t)k * d;
        double zmax = -INFINITY;
        for (int64_t j = 0; j < nk; ++j) {
            const float* w = Wt + (int64_t)tok[j] * d;
            double s = 0.0;
            for (int i = 0; i < d; ++i) s += (double)hb[i] * (double)w[i];
            z[j] = s;
            if (s > zmax) zmax = s;
        }
        double se = 0.0;
        for (int64_t j = 0; j < nk; ++j) se += exp(z[j] - zmax);
        const double lse = zmax + log(se);
        for (int64_t j = 0; j < nk; ++j) {
            rcand_t* o = &c[off[k] + j];
            const float logp = (float)(z[j] - lse);
            o->score = (float)((double)acc[k] + (double)logp);
            o->parent = k;
            o->token = tok[j];
            o->row = rw[j];
        }
        free(tok); free(rw); free(z);
    }
    free(off);
    if (err) { free(c); return -1; }
    qsort(c, (size_t)total, sizeof(rcand_t), rcand_cmp);
    *out = c;
    return total;
}

/* Teacher-forced step; arguments and outputs as or_step of the trie oracle. */
int orr_step(const or_range* R, int t, int Q, int K, int d, const float* h, const float* Wt, const int64_t* rows,
             const float* acc, int32_t* out_tok, int32_t* out_par, int64_t* out_row, float* out_logp,
             int64_t cand_cap, int64_t* cand_count, int32_t* c_tok, int32_t* c_par, int64_t* c_row, float* c_score,
             int threads) {
    if (t < 0 || t >= R->L || Q < 0 || K < 1 || d < 1) return -1;
    for (int64_t b = 0; b < (int64_t)Q * K; ++b)
        if (rows[b] >= R->count[t]) return -1;
    for (int q = 0; q < Q; ++q) {
        rcand_t* c = NULL;
        const int64_t m = query_cands(R, t, K, d, h + (int64_t)q * K * d, Wt, rows + (int64_t)q * K,
                                      acc + (int64_t)q * K, &c, threads);
        if (m < 0) return -2;
        for (int k = 0; k < K; ++k) {
            const int64_t o = (int64_t)q * K + k;
            out_tok[o] = k < m ? c[k].token : -1;
            out_par[o] = k < m ? c[k].parent : -1;
            out_row[o] = k < m ? c[k].row : -1;
            out_logp[o] = k < m ? c[k].score : -INFINITY;
        }
        if (cand_count) cand_count[q] = m;
        for (int64_t j = 0; j < m && j < cand_cap; ++j) {
            const int64_t o = (int64_t)q * cand_cap + j;
            if (c_tok) c_tok[o] = c[j].token;
            if (c_par) c_par[o] = c[j].parent;
            if (c_row) c_row[o] = c[j].row;
            if (c_score) c_score[o] = c[j].score;
        }
        free(c);
    }
    return 0;
}

static float round_bf16_r(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    u = u + 0x7FFFu + ((u >> 16) & 1u);
    u &= 0xFFFF0000u;
    memcpy(&v, &u, 4);
    return v;
}

static void hidden_r(const float* s, int d, int bf16, float* h) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += (double)s[i] * (double)s[i];
    const double nrm = sqrt(ss);
    for (int i = 0; i < d; ++i) {
        const float v = (float)((double)s[i] / nrm);
        h[i] = bf16 ? round_bf16_r(v) : v;
    }
}

/* Free-running decode; arguments and outputs as or_decode of the trie oracle. */
int orr_decode(const or_range* R, int Q, int K, int d, int bf16, const float* q, const float* P, const float* W,
               int32_t* seqs, float* logp, int64_t* rows_out, float* tr_h, int64_t* tr_rows_in, float* tr_acc_in,
               int32_t* tr_tok, int32_t* tr_par, int64_t* tr_rows_out, float* tr_logp_out, int threads) {
    const int L = R->L, V = R->V;
    if (Q < 0 || K < 1 || d < 1) return -1;
    const int64_t RB = (int64_t)Q * K;
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)K);
    int64_t* rows2 = (int64_t*)malloc(sizeof(int64_t) * (size_t)K);
    float* acc = (float*)malloc(sizeof(float) * (size_t)K);
    float* acc2 = (float*)malloc(sizeof(float) * (size_t)K);
    float* s = (float*)calloc((size_t)K * d, sizeof(float));
    float* s2 = (float*)calloc((size_t)K * d, sizeof(float));
    float* h = (float*)calloc((size_t)K * d, sizeof(float));
    int32_t* seq = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * L);
    int32_t* seq2 = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * L);
    int err = 0;
    if (!rows || !rows2 || !acc || !acc2 || !s || !s2 || !h || !seq || !seq2) err = -2;
    for (int qi = 0; qi < Q && !err; ++qi) {
        for (int k = 0; k < K; ++k) { rows[k] = -1; acc[k] = -INFINITY; }
        for (int64_t i = 0; i < (int64_t)K * L; ++i) seq[i] = -1;
        rows[0] = 0;
        acc[0] = 0.0f;
        memcpy(s, q + (int64_t)qi * d, sizeof(float) * (size_t)d);
        for (int t = 0; t < L && !err; ++t) {
            for (int k = 0; k < K; ++k) {
                if (rows[k] >= 0) hidden_r(s + (int64_t)k * d, d, bf16, h + (int64_t)k * d);
                else memset(h + (int64_t)k * d, 0, sizeof(float) * (size_t)d);
            }
            if (tr_h) memcpy(tr_h + ((int64_t)t * RB + (int64_t)qi * K) * d, h, sizeof(float) * (size_t)K * d);
            for (int k = 0; k < K; ++k) {
                const int64_t o = (int64_t)t * RB + (int64_t)qi * K + k;
                if (tr_rows_in) tr_rows_in[o] = rows[k];
                if (tr_acc_in) tr_acc_in[o] = acc[k];
            }
            rcand_t* c = NULL;
            const int64_t m = query_cands(R, t, K, d, h, W + (int64_t)t * V * d, rows, acc, &c, threads);
            if (m < 0) { err = -2; break; }
            for (int k = 0; k < K; ++k) {
                const int64_t o = (int64_t)t * RB + (int64_t)qi * K + k;
                if (k < m) {
                    const rcand_t* ck = &c[k];
                    rows2[k] = ck->row;
                    acc2[k] = ck->score;
                    memcpy(seq2 + (int64_t)k * L, seq + (int64_t)ck->parent * L, sizeof(int32_t) * (size_t)L);
                    seq2[(int64_t)k * L + t] = ck->token;
                    if (t + 1 < L) {
                        const float* sp = s + (int64_t)ck->parent * d;
                        const float* pv = P + ((int64_t)t * V + ck->token) * d;
                        for (int i = 0; i < d; ++i) s2[(int64_t)k * d + i] = (float)((double)sp[i] + (double)pv[i]);
                    }
                } else {
                    rows2[k] = -1;
                    acc2[k] = -INFINITY;
                    for (int i = 0; i < L; ++i) seq2[(int64_t)k * L + i] = -1;
                }
                if (tr_tok) tr_tok[o] = k < m ? c[k].token : -1;
                if (tr_par) tr_par[o] = k < m ? c[k].parent : -1;
                if (tr_rows_out) tr_rows_out[o] = k < m ? c[k].row : -1;
                if (tr_logp_out) tr_logp_out[o] = k < m ? c[k].score : -INFINITY;
            }
            free(c);
            { int64_t* x = rows; rows = rows2; rows2 = x; }
            { float* x = acc; acc = acc2; acc2 = x; }
            { float* x = s; s = s2; s2 = x; }
            { int32_t* x = seq; seq = seq2; seq2 = x; }
        }
        for (int k = 0; k < K && !err; ++k) {
            const int64_t o = (int64_t)qi * K + k;
            memcpy(seqs + o * L, seq + (int64_t)k * L, sizeof(int32_t) * (size_t)L);
            logp[o] = acc[k];
            rows_out[o] = rows[k];
        }
    }
    free(rows); free(rows2); free(acc); free(acc2); free(s); free(s2); free(h); free(seq); free(seq2);
    return err;
}
