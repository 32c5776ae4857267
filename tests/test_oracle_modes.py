"""Pins of the oracle's score-first and unconstrained variants (CPU).

Score first: the softmax denominator covers the whole codebook and only the
valid tokens become candidates (ZeroGR, "Does filtering first change the
recommendations?").  Unconstrained: every token is a candidate (ZeroGR
summary: decoding without constraints as the speed reference).  Pinned by an
independent brute-force enumerator, by the full-product catalog on which the
three variants must coincide, and by the per-beam constant shift between the
two softmax supports.
"""

import itertools

import numpy as np
import pytest

import oracle
from oracle import brute


def inputs(rng, Q, L, V, d):
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((max(L - 1, 1), V, d)) / np.sqrt(d)).astype(np.float32)
    W = (rng.standard_normal((L, V, d)) / np.sqrt(d)).astype(np.float32)
    return q, P, W


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_score_first_wide_beam_returns_every_item_with_its_full_softmax_score(seed):
    rng = np.random.default_rng(seed)
    V, L, d = 5, 3, 8
    items = np.unique(rng.integers(0, V, size=(25, L)), axis=0).astype(np.int32)
    q, P, W = inputs(rng, 1, L, V, d)
    T = oracle.Trie(items, V)
    K = len(items)
    out = T.decode(K, q, P, W, bf16=False, mode="score_first")
    got = {tuple(s): lp for s, lp in zip(out["seqs"].tolist(), out["logp"].tolist())}
    assert set(got) == {tuple(x) for x in items.tolist()}
    want = brute.item_scores(items.tolist(), q[0], P, W, bf16=False, support="all")
    for it, w in zip(items.tolist(), want):
        assert np.float32(got[tuple(it)]) == np.float32(w), (it, got[tuple(it)], w)
    # best first, ties by (parent, token) cannot occur with random scores
    assert np.all(np.diff(out["logp"]) <= 0)


@pytest.mark.parametrize("bf16", [False, True])
def test_unconstrained_wide_beam_enumerates_the_codebook_product(bf16):
    rng = np.random.default_rng(5)
    V, L, d = 3, 3, 8
    items = np.array([[0, 1, 2], [2, 2, 2]], np.int32)  # the catalog plays no part
    q, P, W = inputs(rng, 1, L, V, d)
    if bf16:
        W = brute_bf16(W)
    T = oracle.Trie(items, V)
    K = V ** L
    out = T.decode(K, q, P, W, bf16=bf16, mode="unconstrained")
    allseq = [tuple(x) for x in itertools.product(range(V), repeat=L)]
    got = {tuple(s): lp for s, lp in zip(out["seqs"].tolist(), out["logp"].tolist())}
    assert set(got) == set(allseq)
    assert np.all(out["rows"] == 0)
    want = brute.item_scores(allseq, q[0], P, W, bf16=bf16, support="all")
    for it, w in zip(allseq, want):
        assert np.float32(got[it]) == np.float32(w), (it, got[it], w)


def brute_bf16(W):
    b = W.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return b.view(np.float32)


def test_variants_coincide_on_the_full_product_catalog():
    rng = np.random.default_rng(9)
    V, L, d, K, Q = 4, 3, 16, 6, 3
    items = np.array(list(itertools.product(range(V), repeat=L)), np.int32)
    q, P, W = inputs(rng, Q, L, V, d)
    T = oracle.Trie(items, V)
    ff = T.decode(K, q, P, W, bf16=False)
    sf = T.decode(K, q, P, W, bf16=False, mode="score_first")
    un = T.decode(K, q, P, W, bf16=False, mode="unconstrained")
    for o in (sf, un):
        assert np.array_equal(o["seqs"], ff["seqs"])
        assert np.array_equal(o["logp"], ff["logp"])
    assert np.array_equal(sf["rows"], ff["rows"])
    assert np.all(un["rows"] == 0)


@pytest.mark.parametrize("seed", [0, 3])
def test_score_first_shifts_each_beam_by_a_constant_below_zero(seed):
    """Teacher forced from the same beams: per beam, score-first log-probs are
    the filter-first ones shifted by lse(valid) - lse(all) <= 0."""
    rng = np.random.default_rng(seed)
    V, L, d, K = 16, 3, 12, 4
    items = np.unique(rng.integers(0, V, size=(200, L)), axis=0).astype(np.int32)
    T = oracle.Trie(items, V)
    t = 1
    rows = np.array([0, 1, 2, -1], np.int64)  # three live beams and a dead slot
    h = rng.standard_normal((K, d)).astype(np.float32)
    Wt = (rng.standard_normal((V, d)) / np.sqrt(d)).astype(np.float32)
    acc = np.zeros(K, np.float32)
    ff = T.step(t, K, h, Wt, rows, acc, candidates=True)
    sf = T.step(t, K, h, Wt, rows, acc, candidates=True, mode="score_first")
    assert ff["cand_count"][0] == sf["cand_count"][0]
    n = int(ff["cand_count"][0])
    key = lambda o, j: (int(o["cand_parents"][0][j]), int(o["cand_tokens"][0][j]))
    fmap = {key(ff, j): float(ff["cand_scores"][0][j]) for j in range(n)}
    smap = {key(sf, j): float(sf["cand_scores"][0][j]) for j in range(n)}
    assert fmap.keys() == smap.keys()
    for k in range(3):
        diffs = [smap[c] - fmap[c] for c in fmap if c[0] == k]
        z = h[k].astype(np.float64) @ Wt.astype(np.float64).T
        valid = [c[1] for c in fmap if c[0] == k]
        lv = np.log(np.sum(np.exp(z[valid] - z[valid].max()))) + z[valid].max()
        la = np.log(np.sum(np.exp(z - z.max()))) + z.max()
        assert la >= lv
        for x in diffs:
            assert x <= 1e-6
            assert abs(x - (lv - la)) <= 1e-5 * (1 + abs(la))
