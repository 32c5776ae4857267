"""Pins of the second CPU oracle (sorted ranges, no trie).

The sorted-range oracle exists so that catalogs too large for a pointer trie
can still be decoded on the host.  It is pinned against brute-force
enumeration over the catalog, the W = 0 closed form, and the pinned trie
oracle (a different construction of the same valid sets and row numbers).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from synth import get_config, make_catalog, make_dense
from tests.test_oracle_pins import random_catalog


def both(items, V):
    return oracle.Trie(items, V), oracle.SortedRange(items, V)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_children_equal_catalog_scan(seed):
    """Valid next tokens of every prefix = distinct tokens that follow it in
    the catalog; rows = lexicographic rank of the extended prefix."""
    rng = np.random.default_rng(seed)
    V, L = 7, 4
    items = random_catalog(rng, 60, L, V)
    S = oracle.SortedRange(np.concatenate([items, items[:9]])[rng.permutation(69)], V)
    assert S.n_items == len(items)
    lst = [tuple(r) for r in items.tolist()]
    for t in range(L):
        prefixes = sorted({r[:t] for r in lst})
        nxt = sorted({r[:t + 1] for r in lst})
        assert S.level_count(t) == len(prefixes)
        for row, p in enumerate(prefixes):
            tok, rows = S.children_of_row(t, row)
            exp = sorted(brute.valid_tokens(lst, p))
            assert tok.tolist() == exp
            assert rows.tolist() == [nxt.index(p + (v,)) for v in exp]
        assert S.children_of_row(t, len(prefixes)) is None
    assert S.level_count(L) == len(lst)


def test_bad_tokens_rejected():
    with pytest.raises(ValueError):
        oracle.SortedRange(np.array([[0, 5]], np.int32), 5)
    with pytest.raises(ValueError):
        oracle.SortedRange(np.array([[0, -1]], np.int32), 5)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_tables_equal_trie(name):
    cfg = get_config(name)
    items = make_catalog(cfg)
    T, S = both(items, cfg.V)
    assert T.n_items == S.n_items
    for t in range(cfg.L):
        n = T.level_count(t)
        assert S.level_count(t) == n
        for r in range(n):
            a, b = T.children_of_row(t, r), S.children_of_row(t, r)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("seed,bf16", [(0, False), (1, True)])
def test_wide_beam_returns_every_item_with_its_path_score(seed, bf16):
    rng = np.random.default_rng(seed)
    V, L, d = 6, 3, 5
    items = random_catalog(rng, 9, L, V)
    S = oracle.SortedRange(items[rng.permutation(len(items))], V)
    K = 12
    q = rng.standard_normal((1, d)).astype(np.float32)
    P = rng.standard_normal((L - 1, V, d)).astype(np.float32)
    W = rng.standard_normal((L, V, d)).astype(np.float32)
    if bf16:
        W = torch.tensor(W).bfloat16().float().numpy()
    out = S.decode(K, q, P, W, bf16=bf16)
    live = out["rows"] >= 0
    lst = [tuple(r) for r in items.tolist()]
    got = {tuple(s): lp for s, lp in zip(out["seqs"][live].tolist(), out["logp"][live].tolist())}
    exp = dict(zip(lst, brute.item_scores(lst, q[0], P, W, bf16)))
    assert set(got) == set(exp)
    for k in exp:
        assert abs(got[k] - exp[k]) <= 2 * np.spacing(np.float32(abs(exp[k]) + 1.0))
    assert (out["seqs"][~live] == -1).all() and np.isneginf(out["logp"][~live]).all()


def test_w_zero_uniform_and_tiebreak():
    """W = 0: every valid token scores log(1/n) and the order is the
    tie-break alone (parent ascending, then token ascending)."""
    items = np.array([[0, 1], [0, 3], [2, 0], [2, 1], [2, 2]], np.int32)
    S = oracle.SortedRange(items, 4)
    K, d = 2, 3
    h = np.ones((K, d), np.float32)
    Wt = np.zeros((4, d), np.float32)
    o = S.step(1, K, h, Wt, np.array([0, 1]), np.zeros(K, np.float32), candidates=True)
    n = int(o["cand_count"][0])
    assert n == 5
    assert o["cand_parents"][0, :n].tolist() == [0, 0, 1, 1, 1]
    assert o["cand_tokens"][0, :n].tolist() == [1, 3, 0, 1, 2]
    exp = [math.log(1 / 2)] * 2 + [math.log(1 / 3)] * 3
    assert np.allclose(o["cand_scores"][0, :n], exp, rtol=0, atol=1e-7)
    assert o["rows"].tolist() == [0, 1]


@pytest.mark.parametrize("name,bf16", [("tiny", False), ("small", True)])
def test_decode_trace_equals_trie(name, bf16):
    cfg = get_config(name)
    items = make_catalog(cfg)
    dense = make_dense(cfg, Q=min(cfg.Q, 32))
    T, S = both(items, cfg.V)
    a = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=bf16, trace=True, threads=4)
    b = S.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=bf16, trace=True, threads=4)
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_step_candidates_equal_trie():
    cfg = get_config("small")
    items = make_catalog(cfg)
    dense = make_dense(cfg, Q=8)
    T, S = both(items, cfg.V)
    ref = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=True, trace=True)
    for t in range(cfg.L):
        args = (t, cfg.K, ref["trace_h"][t], dense["W"][t], ref["trace_rows_in"][t], ref["trace_acc_in"][t])
        a = T.step(*args, candidates=True)
        b = S.step(*args, candidates=True, threads=3)
        for k in a:
            assert np.array_equal(a[k], b[k]), (t, k)


def test_hybrid_subset_decode_equals_trie():
    """The hybrid generator (full-product first level, wide second level) at
    one tenth of its catalog size, 16 queries."""
    cfg = get_config("hybrid", n_items=1_000_000)
    items = make_catalog(cfg)
    dense = make_dense(cfg, Q=16)
    T, S = both(items, cfg.V)
    for t in range(cfg.L + 1):
        assert T.level_count(t) == S.level_count(t)
    a = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=True, trace=True, threads=8)
    b = S.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=True, trace=True, threads=8)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
