/* CPU oracle for catalog-constrained beam search over Semantic IDs.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this code.  It shares nothing with the
 * HIP library: it never reads the library's step tables, kernels or headers.
 *
 * What it computes (the plain definition, written out):
 *
 *  - Catalog and constraint.  A catalog is a set of token sequences of length
 *    L over a codebook of V tokens.  After a prefix p of length t, token v is
 *    valid iff some catalog item starts with p followed by v (ZeroGR summary,
 *    "What problem is it solving?", the 3-5 -> {1, 4} example; STATIC, sec. 4.1
 *    constraint functions).  The oracle holds the catalog as a pointer trie:
 *    a node per distinct prefix, children sorted by token.  Repeated items
 *    collapse (the catalog is a set, STATIC sec. 4.1).
 *
 *  - Row numbers.  The nodes of depth t are numbered 0.. in breadth-first
 *    order with children visited in ascending token order; this is the rank
 *    of the prefix among the distinct length-t prefixes in lexicographic
 *    order.  A beam's "row" at step t is the number of its depth-t node (ZeroGR
 *    "Why slice the index by decoding step?": a row per prefix, carried
 *    forward by the beam).
 *
 *  - One step, filter first (ZeroGR "The pipeline", stages 2-4).  For every
 *    live beam b (node n_b, accumulated log-prob acc_b, hidden vector h_b) and
 *    every child v of n_b:  z_v = sum_i h_b[i] * W_t[v][i]  (in double);
 *    lse = max z + log(sum_v exp(z_v - max z))  over the children only (the
 *    softmax denominator covers valid tokens only, ZeroGR "Does filtering
 *    first change the recommendations?");  logp_v = float(z_v - lse);
 *    cand = float(acc_b + logp_v).  The K best candidates of a query by
 *    (cand descending, parent slot ascending, token ascending) become the new
 *    beams (ZeroGR "The pipeline", stage 4: selection by the new total).  A
 *    query with fewer than K candidates pads with sentinels
 *    (token = parent = row = -1, logp = -inf): slots without a valid token
 *    score minus infinity and are never selected (ZeroGR, fixed candidate
 *    slots).
 *
 *  - Decode.  Step 0 starts from one live beam per query at the root with
 *    acc = 0; the other K-1 slots are dead.  The hidden vector of the
 *    stand-in model is h = s / ||s||_2 with s = q + sum_{j<t} P_j[token_j]
 *    (s kept in float32, one float32 add per step; the norm and division in
 *    double, then rounded to float32, then to bf16 when the workload stores
 *    bf16).  Output rows at the last step number the catalog items in
 *    lexicographic order.
 *
 * Variants (the same step with another softmax support or no constraint):
 *  - Score first: the softmax denominator covers the whole codebook (lse over
 *    all V tokens of z_v, in double), and only the valid tokens become
 *    candidates (ZeroGR "Does filtering first change the recommendations?":
 *    the two orders differ exactly in the denominator).
 *  - Unconstrained: every token of the codebook is a candidate and the
 *    denominator covers all of them; no catalog (ZeroGR summary: decoding
 *    without constraints as the speed reference).  Beams stay "live" at a
 *    placeholder node, so every output row is 0.
 *
 * Floating point: double inside, with float32 rounding at exactly the points
 * listed above (logp, cand, s, h), so that the final selection is made on
 * float32 values, as on the device.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct node {
    int32_t token;       /* label of the edge from the parent (-1 at the root) */
    int32_t n;           /* number of children */
    int64_t rank;        /* breadth-first number among nodes of the same depth */
    struct node* first;  /* first child (smallest token) */
    struct node* next;   /* next sibling (next larger token) */
} node;

typedef struct or_trie {
    int L, V;
    int64_t n_items;
    node* root;
    node** pools;       /* node storage, in blocks */
    int64_t n_pools, pool_fill, pool_cap;
    int64_t* count;     /* nodes per depth, [L+1] */
    node*** level;      /* level[t][rank] for t < L */
} or_trie;

#define POOL_BLOCK (1 << 20)

static node* new_node(or_trie* T, int32_t token) {
    if (T->n_pools == 0 || T->pool_fill == POOL_BLOCK) {
        if (T->n_pools == T->pool_cap) {
            int64_t nc = T->pool_cap ? T->pool_cap * 2 : 64;
            node** np = (node**)realloc(T->pools, sizeof(node*) * (size_t)nc);
            if (!np) return NULL;
            T->pools = np;
            T->pool_cap = nc;
        }
        node* blk = (node*)malloc(sizeof(node) * POOL_BLOCK);
        if (!blk) return NULL;
        T->pools[T->n_pools++] = blk;
        T->pool_fill = 0;
    }
    node* x = &T->pools[T->n_pools - 1][T->pool_fill++];
    x->token = token;
    x->n = 0;
    x->rank = -1;
    x->first = NULL;
    x->next = NULL;
    return x;
}

/* Child of x labelled tok, or NULL. */
static const node* find_child(const node* x, int32_t tok) {
    for (const node* c = x->first; c; c = c->next)
        if (c->token == tok) return c;
    return NULL;
}

void or_free(or_trie* T) {
    if (!T) return;
    for (int64_t p = 0; p < T->n_pools; ++p) free(T->pools[p]);
    free(T->pools);
    if (T->level)
        for (int t = 0; t <= T->L; ++t) free(T->level[t]);
    free(T->level);
    free(T->count);
    free(T);
}

/* Build the trie of the catalog sids[n][L] (tokens in [0, V)).  Returns NULL
 * on a token out of range, L < 1, V < 1 or allocation failure.
 *
 * Items are inserted in lexicographic order (a stable counting sort per token
 * position, last position first).  In that order an item shares with the
 * previous one the path down to the first position where they differ; below
 * it every node is new, and the new child at the divergence point has a larger
 * token than every existing sibling, so it is appended as the last child.  An
 * item equal to the previous one is a repeat and adds nothing. */
or_trie* or_build(const int32_t* sids, int64_t n, int L, int V) {
    if (L < 1 || V < 1 || n < 0) return NULL;
    for (int64_t i = 0; i < n * L; ++i)
        if (sids[i] < 0 || sids[i] >= V) return NULL;
    or_trie* T = (or_trie*)calloc(1, sizeof(or_trie));
    if (!T) return NULL;
    T->L = L;
    T->V = V;
    T->root = new_node(T, -1);
    if (!T->root) { or_free(T); return NULL; }
    int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n ? n : 1));
    int64_t* tmp = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n ? n : 1));
    int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * ((size_t)V + 1));
    node** path = (node**)malloc(sizeof(node*) * ((size_t)L + 1));
    if (!order || !tmp || !cnt || !path) {
        free(order); free(tmp); free(cnt); free(path); or_free(T);
        return NULL;
    }
    for (int64_t i = 0; i < n; ++i) order[i] = i;
    for (int t = L - 1; t >= 0; --t) {
        memset(cnt, 0, sizeof(int64_t) * ((size_t)V + 1));
        for (int64_t k = 0; k < n; ++k) cnt[sids[order[k] * L + t] + 1]++;
        for (int v = 0; v < V; ++v) cnt[v + 1] += cnt[v];
        for (int64_t k = 0; k < n; ++k) tmp[cnt[sids[order[k] * L + t]]++] = order[k];
        int64_t* sw = order; order = tmp; tmp = sw;
    }
    free(tmp);
    free(cnt);
    path[0] = T->root;
    int64_t prev = -1;
    for (int64_t k = 0; k < n; ++k) {
        const int64_t i = order[k];
        int t0 = 0;
        if (prev >= 0)
            while (t0 < L && sids[i * L + t0] == sids[prev * L + t0]) ++t0;
        if (t0 == L) continue;  /* repeated item */
        for (int t = t0; t < L; ++t) {
            node* c = new_node(T, sids[i * L + t]);
            if (!c) { free(order); free(path); or_free(T); return NULL; }
            node* parent = path[t];
            if (parent->n == 0) parent->first = c;
            else path[t + 1]->next = c;  /* path[t+1] is parent's last child */
            parent->n++;
            path[t + 1] = c;
        }
        T->n_items++;
        prev = i;
    }
    free(order);
    free(path);
    /* breadth-first numbering, children in ascending token order */
    T->count = (int64_t*)calloc((size_t)L + 1, sizeof(int64_t));
    T->level = (node***)calloc((size_t)L + 1, sizeof(node**));
    if (!T->count || !T->level) { or_free(T); return NULL; }
    T->count[0] = 1;
    T->level[0] = (node**)malloc(sizeof(node*));
    if (!T->level[0]) { or_free(T); return NULL; }
    T->level[0][0] = T->root;
    T->root->rank = 0;
    for (int t = 0; t < L; ++t) {
        int64_t m = 0;
        for (int64_t r = 0; r < T->count[t]; ++r) m += T->level[t][r]->n;
        const int keep = t + 1 < L;  /* leaves need no rank -> node table */
        if (keep) {
            T->level[t + 1] = (node**)malloc(sizeof(node*) * (size_t)(m ? m : 1));
            if (!T->level[t + 1]) { or_free(T); return NULL; }
        }
        int64_t k = 0;
        for (int64_t r = 0; r < T->count[t]; ++r)
            for (node* c = T->level[t][r]->first; c; c = c->next) {
                c->rank = k;
                if (keep) T->level[t + 1][k] = c;
                ++k;
            }
        T->count[t + 1] = m;
    }
    return T;
}

int64_t or_n_items(const or_trie* T) { return T->n_items; }

/* Number of distinct length-`depth` prefixes. */
int64_t or_level_count(const or_trie* T, int depth) {
    if (depth < 0 || depth > T->L) return -1;
    return T->count[depth];
}

static int fill_children(const node* x, int32_t* tokens, int64_t* ranks, int64_t cap) {
    int64_t j = 0;
    for (const node* c = x->first; c; c = c->next, ++j)
        if (j < cap) {
            if (tokens) tokens[j] = c->token;
            if (ranks) ranks[j] = c->rank;
        }
    return x->n;
}

/* Children of the prefix prefix[0..len): tokens ascending and their row
 * numbers at depth len+1.  Returns the child count, -1 if the prefix is not
 * in the catalog. */
int or_children(const or_trie* T, const int32_t* prefix, int len, int32_t* tokens, int64_t* ranks, int64_t cap) {
    if (len < 0 || len >= T->L) return -1;
    const node* x = T->root;
    for (int t = 0; t < len && x; ++t) x = find_child(x, prefix[t]);
    if (!x) return -1;
    return fill_children(x, tokens, ranks, cap);
}

/* Children of the node with number `row` at depth `depth` (< L). */
int or_children_of_row(const or_trie* T, int depth, int64_t row, int32_t* tokens, int64_t* ranks, int64_t cap) {
    if (depth < 0 || depth >= T->L || row < 0 || row >= T->count[depth]) return -1;
    return fill_children(T->level[depth][row], tokens, ranks, cap);
}

/* The prefix (tokens from the root) of node `row` at depth `depth` (< L).
 * Plain and slow: each parent is found by scanning the level above. */
int or_prefix_of_row(const or_trie* T, int depth, int64_t row, int32_t* out) {
    if (depth < 0 || depth >= T->L || row < 0 || row >= T->count[depth]) return -1;
    const node* target = T->level[depth][row];
    for (int t = depth; t > 0; --t) {
        out[t - 1] = target->token;
        const node* parent = NULL;
        for (int64_t r = 0; r < T->count[t - 1] && !parent; ++r)
            for (const node* c = T->level[t - 1][r]->first; c; c = c->next)
                if (c == target) { parent = T->level[t - 1][r]; break; }
        if (!parent) return -1;
        target = parent;
    }
    return depth;
}

/* ---- one step ------------------------------------------------------------ */

typedef struct {
    float score;
    int32_t parent;
    int32_t token;
    const node* child;
} cand_t;

static int cand_cmp(const void* a, const void* b) {
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->score != y->score) return x->score > y->score ? -1 : 1;
    if (x->parent != y->parent) return x->parent < y->parent ? -1 : 1;
    if (x->token != y->token) return x->token < y->token ? -1 : 1;
    return 0;
}

/* All candidates of one query, sorted best first.  h: [K][d], nodes: [K]
 * (NULL = dead), acc: [K].  Returns the count, or -1 on allocation failure;
 * *out is malloc'ed. */
/* Softmax support and candidate set of one step. */
enum { OR_FILTER_FIRST = 0, OR_SCORE_FIRST = 1, OR_UNCONSTRAINED = 2 };

/* log sum_v exp(z_v) over the whole codebook, z_v = <h, W_t[v]> in double. */
static double lse_all_tokens(const float* hb, const float* Wt, int V, int d, double* zall) {
    double zmax = -INFINITY;
    for (int v = 0; v < V; ++v) {
        const float* w = Wt + (int64_t)v * d;
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += (double)hb[i] * (double)w[i];
        zall[v] = s;
        if (s > zmax) zmax = s;
    }
    double se = 0.0;
    for (int v = 0; v < V; ++v) se += exp(zall[v] - zmax);
    return zmax + log(se);
}

static int64_t query_candidates(const or_trie* T, int t, int K, int d, const float* h, const float* Wt,
                                const node* const* nodes, const float* acc, int mode, cand_t** out) {
    int64_t total = 0;
    for (int k = 0; k < K; ++k)
        if (nodes[k]) total += mode == OR_UNCONSTRAINED ? T->V : nodes[k]->n;
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(total ? total : 1));
    double* z = NULL;
    int32_t zcap = 0;
    if (!c) return -1;
    int64_t m = 0;
    if (mode != OR_FILTER_FIRST) {
        double* zall = (double*)malloc(sizeof(double) * (size_t)T->V);
        if (!zall) { free(c); return -1; }
        for (int k = 0; k < K; ++k) {
            const node* x = nodes[k];
            if (!x) continue;
            const double lse = lse_all_tokens(h + (int64_t)k * d, Wt, T->V, d, zall);
            if (mode == OR_UNCONSTRAINED) {
                for (int v = 0; v < T->V; ++v) {
                    float logp = (float)(zall[v] - lse);
                    c[m].score = (float)((double)acc[k] + (double)logp);
                    c[m].parent = k;
                    c[m].token = v;
                    c[m].child = T->root;  /* placeholder: the beam stays live, row 0 */
                    ++m;
                }
            } else {
                for (const node* ch = x->first; ch; ch = ch->next) {
                    float logp = (float)(zall[ch->token] - lse);
                    c[m].score = (float)((double)acc[k] + (double)logp);
                    c[m].parent = k;
                    c[m].token = ch->token;
                    c[m].child = ch;
                    ++m;
                }
            }
        }
        free(zall);
        qsort(c, (size_t)m, sizeof(cand_t), cand_cmp);
        *out = c;
        return m;
    }
    for (int k = 0; k < K; ++k) {
        const node* x = nodes[k];
        if (!x || x->n == 0) continue;
        if (x->n > zcap) {
            double* nz = (double*)realloc(z, sizeof(double) * (size_t)x->n);
            if (!nz) { free(z); free(c); return -1; }
            z = nz;
            zcap = x->n;
        }
        const float* hb = h + (int64_t)k * d;
        double zmax = -INFINITY;
        int32_t j = 0;
        for (const node* ch = x->first; ch; ch = ch->next, ++j) {
            const float* w = Wt + (int64_t)ch->token * d;
            double s = 0.0;
            for (int i = 0; i < d; ++i) s += (double)hb[i] * (double)w[i];
            z[j] = s;
            if (s > zmax) zmax = s;
        }
        double se = 0.0;
        for (j = 0; j < x->n; ++j) se += exp(z[j] - zmax);
        double lse = zmax + log(se);
        j = 0;
        for (const node* ch = x->first; ch; ch = ch->next, ++j) {
            float logp = (float)(z[j] - lse);
            c[m].score = (float)((double)acc[k] + (double)logp);
            c[m].parent = k;
            c[m].token = ch->token;
            c[m].child = ch;
            ++m;
        }
    }
    free(z);
    (void)t;
    (void)T;
    qsort(c, (size_t)m, sizeof(cand_t), cand_cmp);
    *out = c;
    return m;
}

/* Teacher-forced single step for Q queries of K beam slots.
 *   h     [Q*K][d]  hidden vectors (float32 values; bf16-representable for
 *                   bf16 workloads)
 *   Wt    [V][d]    output layer of step t
 *   rows  [Q*K]     depth-t row per slot, -1 = dead
 *   acc   [Q*K]     accumulated log-prob per slot
 * Outputs [Q*K]: tokens, parents (slot within the query), rows (depth t+1),
 * logp (new accumulated log-prob), best first, sentinel-padded.
 * Optional full candidate lists (any of c_* may be NULL): cand_count[Q] and
 * [Q][cand_cap] arrays, sorted best first.
 * Returns 0, -1 on bad arguments, -2 on allocation failure. */
int or_step_mode(const or_trie* T, int t, int Q, int K, int d, const float* h, const float* Wt,
                 const int64_t* rows, const float* acc,
                 int32_t* out_tok, int32_t* out_par, int64_t* out_row, float* out_logp,
                 int64_t cand_cap, int64_t* cand_count, int32_t* c_tok, int32_t* c_par, int64_t* c_row,
                 float* c_score, int nthreads, int mode) {
    if (t < 0 || t >= T->L || Q < 0 || K < 1 || d < 1 || mode < 0 || mode > 2) return -1;
    for (int64_t b = 0; b < (int64_t)Q * K; ++b)
        if (rows[b] >= T->count[t]) return -1;
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int q = 0; q < Q; ++q) {
        const node* nodes[1024];
        const node** np = K <= 1024 ? nodes : (const node**)malloc(sizeof(node*) * (size_t)K);
        if (!np) {
            #pragma omp atomic write
            err = -2;
            continue;
        }
        for (int k = 0; k < K; ++k) {
            int64_t r = rows[(int64_t)q * K + k];
            np[k] = r < 0 ? NULL : (mode == OR_UNCONSTRAINED ? T->root : T->level[t][r]);
        }
        cand_t* c = NULL;
        int64_t m = query_candidates(T, t, K, d, h + (int64_t)q * K * d, Wt, np, acc + (int64_t)q * K, mode, &c);
        if (np != nodes) free(np);
        if (m < 0) {
            #pragma omp atomic write
            err = -2;
            continue;
        }
        for (int k = 0; k < K; ++k) {
            int64_t o = (int64_t)q * K + k;
            if (k < m) {
                out_tok[o] = c[k].token;
                out_par[o] = c[k].parent;
                out_row[o] = c[k].child->rank;
                out_logp[o] = c[k].score;
            } else {
                out_tok[o] = -1;
                out_par[o] = -1;
                out_row[o] = -1;
                out_logp[o] = -INFINITY;
            }
        }
        if (cand_count) cand_count[q] = m;
        for (int64_t j = 0; j < m && j < cand_cap; ++j) {
            int64_t o = (int64_t)q * cand_cap + j;
            if (c_tok) c_tok[o] = c[j].token;
            if (c_par) c_par[o] = c[j].parent;
            if (c_row) c_row[o] = c[j].child->rank;
            if (c_score) c_score[o] = c[j].score;
        }
        free(c);
    }
    return err;
}

int or_step(const or_trie* T, int t, int Q, int K, int d, const float* h, const float* Wt,
            const int64_t* rows, const float* acc,
            int32_t* out_tok, int32_t* out_par, int64_t* out_row, float* out_logp,
            int64_t cand_cap, int64_t* cand_count, int32_t* c_tok, int32_t* c_par, int64_t* c_row, float* c_score,
            int nthreads) {
    return or_step_mode(T, t, Q, K, d, h, Wt, rows, acc, out_tok, out_par, out_row, out_logp, cand_cap, cand_count,
                        c_tok, c_par, c_row, c_score, nthreads, OR_FILTER_FIRST);
}

/* ---- the stand-in model's hidden vector and the full decode --------------- */

static float round_bf16(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    u = u + 0x7FFFu + ((u >> 16) & 1u);  /* round to nearest, ties to even */
    u &= 0xFFFF0000u;
    memcpy(&v, &u, 4);
    return v;
}

static void hidden_of_state(const float* s, int d, int bf16, float* h) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += (double)s[i] * (double)s[i];
    double nrm = sqrt(ss);
    for (int i = 0; i < d; ++i) {
        float v = (float)((double)s[i] / nrm);
        h[i] = bf16 ? round_bf16(v) : v;
    }
}

/* Free-running decode of Q queries, K beams, all L steps.
 *   q [Q][d], P [L-1][V][d], W [L][V][d] (float32 values).
 * Outputs: seqs [Q*K][L] (-1 for dead slots), logp [Q*K], rows [Q*K]
 * (item number among the sorted distinct catalog items, -1 dead).
 * Optional per-step trace (NULL to skip), all indexed [t][Q*K]...:
 *   tr_h [L][Q*K][d] hidden vectors fed to step t (zeros for dead slots),
 *   tr_rows_in / tr_acc_in: beam state fed to step t,
 *   tr_tok / tr_par / tr_rows_out / tr_logp_out: step t's outputs.
 * Returns 0, -1 on bad arguments, -2 on allocation failure. */
int or_decode_mode(const or_trie* T, int Q, int K, int d, int bf16,
                   const float* q, const float* P, const float* W,
                   int32_t* seqs, float* logp, int64_t* rows,
                   float* tr_h, int64_t* tr_rows_in, float* tr_acc_in,
                   int32_t* tr_tok, int32_t* tr_par, int64_t* tr_rows_out, float* tr_logp_out,
                   int nthreads, int mode) {
    const int L = T->L, V = T->V;
    if (Q < 0 || K < 1 || d < 1 || mode < 0 || mode > 2) return -1;
    const int64_t R = (int64_t)Q * K;
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int qi = 0; qi < Q; ++qi) {
        const node** nodes = (const node**)calloc((size_t)K, sizeof(node*));
        const node** nn = (const node**)calloc((size_t)K, sizeof(node*));
        float* acc = (float*)malloc(sizeof(float) * (size_t)K);
        float* acc2 = (float*)malloc(sizeof(float) * (size_t)K);
        float* s = (float*)calloc((size_t)K * d, sizeof(float));
        float* s2 = (float*)calloc((size_t)K * d, sizeof(float));
        float* h = (float*)calloc((size_t)K * d, sizeof(float));
        int32_t* seq = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * L);
        int32_t* seq2 = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * L);
        if (!nodes || !nn || !acc || !acc2 || !s || !s2 || !h || !seq || !seq2) {
            #pragma omp atomic write
            err = -2;
            goto done;
        }
        for (int k = 0; k < K; ++k) acc[k] = -INFINITY;
        for (int64_t i = 0; i < (int64_t)K * L; ++i) seq[i] = -1;
        nodes[0] = T->root;
        acc[0] = 0.0f;
        memcpy(s, q + (int64_t)qi * d, sizeof(float) * (size_t)d);
        for (int t = 0; t < L; ++t) {
            for (int k = 0; k < K; ++k) {
                if (nodes[k]) hidden_of_state(s + (int64_t)k * d, d, bf16, h + (int64_t)k * d);
                else memset(h + (int64_t)k * d, 0, sizeof(float) * (size_t)d);
            }
            if (tr_h) memcpy(tr_h + ((int64_t)t * R + (int64_t)qi * K) * d, h, sizeof(float) * (size_t)K * d);
            for (int k = 0; k < K; ++k) {
                int64_t o = (int64_t)t * R + (int64_t)qi * K + k;
                if (tr_rows_in) tr_rows_in[o] = nodes[k] ? nodes[k]->rank : -1;
                if (tr_acc_in) tr_acc_in[o] = acc[k];
            }
            cand_t* c = NULL;
            int64_t m = query_candidates(T, t, K, d, h, W + (int64_t)t * V * d, nodes, acc, mode, &c);
            if (m < 0) {
                #pragma omp atomic write
                err = -2;
                goto done;
            }
            for (int k = 0; k < K; ++k) {
                int64_t o = (int64_t)t * R + (int64_t)qi * K + k;
                if (k < m) {
                    const cand_t* ck = &c[k];
                    nn[k] = ck->child;
                    acc2[k] = ck->score;
                    memcpy(seq2 + (int64_t)k * L, seq + (int64_t)ck->parent * L, sizeof(int32_t) * (size_t)L);
                    seq2[(int64_t)k * L + t] = ck->token;
                    if (t + 1 < L) {
                        const float* sp = s + (int64_t)ck->parent * d;
                        const float* pv = P + ((int64_t)t * V + ck->token) * d;
                        for (int i = 0; i < d; ++i) s2[(int64_t)k * d + i] = (float)((double)sp[i] + (double)pv[i]);
                    }
                    if (tr_tok) tr_tok[o] = ck->token;
                    if (tr_par) tr_par[o] = ck->parent;
                    if (tr_rows_out) tr_rows_out[o] = ck->child->rank;
                    if (tr_logp_out) tr_logp_out[o] = ck->score;
                } else {
                    nn[k] = NULL;
                    acc2[k] = -INFINITY;
                    for (int i = 0; i < L; ++i) seq2[(int64_t)k * L + i] = -1;
                    if (tr_tok) tr_tok[o] = -1;
                    if (tr_par) tr_par[o] = -1;
                    if (tr_rows_out) tr_rows_out[o] = -1;
                    if (tr_logp_out) tr_logp_out[o] = -INFINITY;
                }
            }
            free(c);
            { const node** tn = nodes; nodes = nn; nn = tn; }
            { float* ta = acc; acc = acc2; acc2 = ta; }
            { float* ts = s; s = s2; s2 = ts; }
            { int32_t* tq = seq; seq = seq2; seq2 = tq; }
        }
        for (int k = 0; k < K; ++k) {
            int64_t o = (int64_t)qi * K + k;
            memcpy(seqs + o * L, seq + (int64_t)k * L, sizeof(int32_t) * (size_t)L);
            logp[o] = acc[k];
            rows[o] = nodes[k] ? nodes[k]->rank : -1;
        }
    done:
        free(nodes); free(nn); free(acc); free(acc2); free(s); free(s2); free(h); free(seq); free(seq2);
    }
    return err;
}

int or_decode(const or_trie* T, int Q, int K, int d, int bf16,
              const float* q, const float* P, const float* W,
              int32_t* seqs, float* logp, int64_t* rows,
              float* tr_h, int64_t* tr_rows_in, float* tr_acc_in,
              int32_t* tr_tok, int32_t* tr_par, int64_t* tr_rows_out, float* tr_logp_out,
              int nthreads) {
    return or_decode_mode(T, Q, K, d, bf16, q, P, W, seqs, logp, rows, tr_h, tr_rows_in, tr_acc_in, tr_tok, tr_par,
                          tr_rows_out, tr_logp_out, nthreads, OR_FILTER_FIRST);
}

/* Hidden vector of a float32 state vector, as the decode computes it
 * (exposed so that teacher-forced tests feed both sides the same h). */
void or_hidden(const float* s, int64_t n, int d, int bf16, float* h) {
    for (int64_t b = 0; b < n; ++b) hidden_of_state(s + b * d, d, bf16, h + b * d);
}
