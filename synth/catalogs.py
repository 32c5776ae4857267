"""Seeded catalogs of Semantic-ID token sequences.

A catalog is an int32 array of shape (n_items, L): one row per item, every
token in [0, V).  Rows are distinct.  The generators below only draw token
sequences; they do not index, score or rank anything.

Generators (one per workload shape):

* ``clustered``: level-1 token ~ Zipf(s) over a seeded permutation of the
  codebook; a prefix seen for the first time receives c ~ Poisson(mean)
  (conditioned on c >= 1) children, a uniformly random c-subset of the
  codebook; an item walks top-down choosing uniformly among the children;
  repeated items are rejected until n_items distinct ones exist.
* ``clustered_collision``: the same walk for the first L-1 levels, with
  repeats allowed; the last token is the occurrence index of that (L-1)-token
  code among the items drawn so far (0, 1, ...), and a draw that would create
  occurrence number ``max_collisions`` is rejected.
* ``hybrid``: tree first.  Level 1 holds every codebook token; each level-1
  prefix receives Geometric(mean level2_mean) children; every deeper prefix
  receives Geometric(mean later_mean) children; children are uniform random
  subsets.  Exactly n_items leaves are then sampled without replacement.
* ``zipf_prefix``: every level's token is rank ~ Zipf(s) mapped through a
  bijection of the codebook, rank -> (a_p * rank + b_p) mod V, whose (a_p,
  b_p) are hashed from the prefix drawn so far (a_p a unit mod V); repeated
  items are rejected until n_items distinct ones exist.
* ``zipf_varlen``: like ``zipf_prefix`` over a codebook of ``codebook``
  tokens, with item length ~ Uniform{min_len..max_len}; positions past the
  length hold the end token EOS = ``codebook``, so rows have a fixed width
  and V = codebook + 1.
"""

import numpy as np

def _zipf_cdf(V, s):
    w = np.arange(1, V + 1, dtype=np.float64) ** (-float(s))
    c = np.cumsum(w)
    return c / c[-1]


def _zipf_ranks(rng, cdf, n):
    """0-based ranks with P(rank = k) proportional to (k + 1) ** -s."""
    u = rng.random(n)
    r = np.searchsorted(cdf, u, side="right")
    return np.minimum(r, len(cdf) - 1).astype(np.int64)


def _poisson_at_least_one(rng, lam):
    while True:
        c = int(rng.poisson(lam))
        if c >= 1:
            return c


def _clustered_walk(rng, perm, cdf, children, depth, V, fanout_mean):
    prefix = (int(perm[_zipf_ranks(rng, cdf, 1)[0]]),)
    for _ in range(1, depth):
        kids = children.get(prefix)
        if kids is None:
            c = min(_poisson_at_least_one(rng, fanout_mean), V)
            kids = rng.choice(V, size=c, replace=False)
            children[prefix] = kids
        prefix = prefix + (int(kids[rng.integers(len(kids))]),)
    return prefix


def clustered(n_items, L, V, seed, zipf_s=1.1, fanout_mean=4.0):
    rng = np.random.default_rng([seed, 1])
    perm = rng.permutation(V)
    cdf = _zipf_cdf(V, zipf_s)
    children = {}
    seen = set()
    items = []
    draws = 0
    while len(items) < n_items:
        draws += 1
        if draws > 1000 * n_items + 10_000:
            raise RuntimeError("clustered catalog: too many repeated draws")
        code = _clustered_walk(rng, perm, cdf, children, L, V, fanout_mean)
        if code not in seen:
            seen.add(code)
            items.append(code)
    return np.asarray(items, dtype=np.int32).reshape(n_items, L)


def clustered_collision(n_items, L, V, seed, zipf_s=1.1, fanout_mean=4.0, max_collisions=8):
    rng = np.random.default_rng([seed, 1])
    perm = rng.permutation(V)
    cdf = _zipf_cdf(V, zipf_s)
    children = {}
    counts = {}
    items = []
    draws = 0
    while len(items) < n_items:
        draws += 1
        if draws > 1000 * n_items + 10_000:
            raise RuntimeError("collision catalog: too many rejected draws")
        code = _clustered_walk(rng, perm, cdf, children, L - 1, V, fanout_mean)
        c = counts.get(code, 0)
        if c >= max_collisions:
            continue
        counts[code] = c + 1
        items.append(code + (c,))
    return np.asarray(items, dtype=np.int32).reshape(n_items, L)


def _random_subsets(rng, counts, V):
    """For group i, a uniformly random subset of range(V) of size counts[i].

    Returns the members flattened group by group, ascending within a group.
    Large groups are drawn without replacement one by one; small groups are
    drawn with replacement and their repeated members redrawn until distinct
    (the procedure is symmetric in the codebook, so each subset is uniform).
    """
    counts = np.minimum(np.asarray(counts, dtype=np.int64), V)
    n = len(counts)
    offs = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=offs[1:])
    out = np.empty(offs[-1], dtype=np.int64)
    big = counts > 64
    for i in np.nonzero(big)[0]:
        out[offs[i]:offs[i + 1]] = np.sort(rng.choice(V, size=int(counts[i]), replace=False))
    small = np.nonzero(~big)[0]
    if len(small):
        sc = counts[small]
        grp = np.repeat(np.arange(len(small), dtype=np.int64), sc)
        vals = rng.integers(0, V, size=len(grp))
        while True:
            key = grp * V + vals
            order = np.argsort(key, kind="stable")
            ks = key[order]
            dup = np.zeros(len(ks), dtype=bool)
            dup[1:] = ks[1:] == ks[:-1]
            if not dup.any():
                break
            redo = order[dup]
            vals[redo] = rng.integers(0, V, size=len(redo))
        vals = vals[np.argsort(grp * V + vals, kind="stable")]
        so = np.zeros(len(small) + 1, dtype=np.int64)
        np.cumsum(sc, out=so[1:])
        dst = np.repeat(offs[small] - so[:-1], sc) + np.arange(so[-1])
        out[dst] = vals
    return out


def hybrid(n_items, L, V, seed, level2_mean=300.0, later_mean=3.0):
    rng = np.random.default_rng([seed, 1])
    prefixes = np.arange(V, dtype=np.int32)[:, None]
    for level in range(1, L):
        mean = level2_mean if level == 1 else later_mean
        c = np.minimum(rng.geometric(1.0 / mean, size=len(prefixes)), V)
        kids = _random_subsets(rng, c, V).astype(np.int32)
        prefixes = np.concatenate([np.repeat(prefixes, c, axis=0), kids[:, None]], axis=1)
    if len(prefixes) < n_items:
        raise RuntimeError(f"hybrid tree has {len(prefixes)} leaves < {n_items}")
    pick = np.sort(rng.choice(len(prefixes), size=n_items, replace=False))
    items = prefixes[pick]
    return np.ascontiguousarray(items[rng.permutation(n_items)])


def branch(n_items, L, V, seed, B=64):
    """Exact branch factor B: the root has n1 = round(n_items / B^(L-1))
    children (at least 1, at most V), every node below has exactly B children,
    all uniform random token subsets; the catalog is every leaf, n1 * B^(L-1)
    items (within a few percent of n_items).  ``n_items`` only sets n1."""
    rng = np.random.default_rng([seed, 1, B])
    n1 = int(min(V, max(1, round(n_items / float(B) ** (L - 1)))))
    prefixes = np.sort(rng.choice(V, size=n1, replace=False)).astype(np.int32)[:, None]
    for _ in range(1, L):
        c = np.full(len(prefixes), min(B, V), dtype=np.int64)
        kids = _random_subsets(rng, c, V).astype(np.int32)
        prefixes = np.concatenate([np.repeat(prefixes, c, axis=0), kids[:, None]], axis=1)
    return np.ascontiguousarray(prefixes[rng.permutation(len(prefixes))])


def zipf_prefix(n_items, L, V, seed, zipf_s=1.0):
    from ._native import zipf_items
    return zipf_items(seed, n_items, L, V, -1, zipf_s, L, L)


def zipf_varlen(n_items, L, V, seed, zipf_s=1.2, min_len=4, max_len=12, codebook=32_000):
    from ._native import zipf_items
    assert V == codebook + 1 and L == max_len
    return zipf_items(seed, n_items, L, codebook, codebook, zipf_s, min_len, max_len)


_GENERATORS = {
    "clustered": clustered,
    "clustered_collision": clustered_collision,
    "hybrid": hybrid,
    "branch": branch,
    "zipf_prefix": zipf_prefix,
    "zipf_varlen": zipf_varlen,
}


def make_catalog(cfg, n_items=None):
    """Draw the catalog of a ``synth.Config`` (optionally with another item
    count).  Returns int32 (n_items, L)."""
    n = cfg.n_items if n_items is None else int(n_items)
    gen = _GENERATORS[cfg.generator]
    return gen(n, cfg.L, cfg.V, cfg.seed, **cfg.params)
