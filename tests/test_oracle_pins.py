"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the fact it checks.  None of them compares the oracle with
itself: expected values come from the pages' worked examples (golden files),
closed forms, a library routine (torch) on a special case that reduces to
textbook beam search, or brute-force enumeration.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from synth import get_config, make_catalog, make_dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    spec = {"item": []}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            vals = [int(v) for v in vals]
            if key == "item":
                spec["item"].append(vals)
            else:
                spec[key] = vals
    return spec


def random_catalog(rng, n, L, V):
    items = set()
    while len(items) < n:
        items.add(tuple(int(x) for x in rng.integers(0, V, size=L)))
    return np.array(sorted(items), dtype=np.int32)


# ---------------------------------------------------------------- valid sets

def test_worked_example_prefix_3_5():
    """ZeroGR: after 3-5 only tokens 1 and 4 are valid."""
    g = read_golden("worked_example.txt")
    T = oracle.Trie(np.array(g["item"], np.int32), g["V"][0])
    tok, _ = T.children(g["prefix"])
    assert tok.tolist() == g["valid"]


def test_depth_only_list_is_rejected():
    """A token that is valid at this depth under another prefix (a depth-only
    list admits a strict superset, FlashTrie App. I) must not be admitted."""
    g = read_golden("worked_example.txt")
    items = np.array(g["item"], np.int32)
    T = oracle.Trie(items, g["V"][0])
    depth = len(g["prefix"])
    assert sorted(set(items[:, depth].tolist())) == g["depth_only"]
    tok, _ = T.children(g["prefix"])
    extra = set(g["depth_only"]) - set(tok.tolist())
    assert extra == {2, 7, 9}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_children_equal_catalog_scan(seed):
    rng = np.random.default_rng(seed)
    items = random_catalog(rng, 40, 3, 6)
    T = oracle.Trie(items[rng.permutation(len(items))], 6)
    lst = [tuple(r) for r in items.tolist()]
    prefixes = {()} | {it[:t] for it in lst for t in range(1, 3)}
    for p in prefixes:
        tok, _ = T.children(list(p))
        assert tok.tolist() == brute.valid_tokens(lst, p)
    # absent prefixes are reported as absent
    for _ in range(20):
        p = tuple(int(x) for x in rng.integers(0, 6, size=2))
        if p not in prefixes:
            assert T.children(list(p)) is None


def test_rows_are_lexicographic_ranks():
    """Row r of depth t is the r-th smallest distinct length-t prefix; the
    child's row equals the rank of prefix + token at depth t + 1."""
    rng = np.random.default_rng(7)
    items = random_catalog(rng, 60, 4, 5)
    T = oracle.Trie(items[rng.permutation(len(items))], 5)
    for t in range(0, 5):
        distinct = sorted({tuple(r[:t]) for r in items.tolist()})
        assert T.level_count(t) == len(distinct)
        for r, p in enumerate(distinct):
            if t < 4:
                assert tuple(T.prefix_of_row(t, r).tolist()) == p
                tok, rows = T.children_of_row(t, r)
                nxt = sorted({tuple(x[:t + 1]) for x in items.tolist()})
                for v, row in zip(tok.tolist(), rows.tolist()):
                    assert nxt.index(p + (v,)) == row


def test_duplicate_items_collapse():
    items = np.array([[1, 2], [1, 2], [0, 3], [1, 2]], np.int32)
    T = oracle.Trie(items, 4)
    assert T.n_items == 2


def test_bad_tokens_rejected():
    with pytest.raises(ValueError):
        oracle.Trie(np.array([[0, 4]], np.int32), 4)
    with pytest.raises(ValueError):
        oracle.Trie(np.array([[0, -1]], np.int32), 4)


def test_csr_fragment_numbering():
    """STATIC sec. 4.2.1: C[5:7] = [2, 3], V[5:7] = [6, 7] under breadth-first
    state numbering (root = 0): the edge at position e leads to state e + 1."""
    g = read_golden("csr_fragment.txt")
    items = np.array(g["item"], np.int32)
    L = g["L"][0]
    T = oracle.Trie(items, g["V"][0])
    # global state id of a node = nodes in shallower levels + its row
    base = [sum(T.level_count(u) for u in range(t)) for t in range(L + 1)]
    edge_tok, edge_dst = [], []
    for t in range(L):
        for r in range(T.level_count(t)):
            tok, rows = T.children_of_row(t, r)
            edge_tok += tok.tolist()
            edge_dst += [base[t + 1] + x for x in rows.tolist()]
    lo, hi = g["edges"]
    assert edge_tok[lo:hi] == g["tokens"]
    assert edge_dst[lo:hi] == g["targets"]
    assert edge_dst == [e + 1 for e in range(len(edge_dst))]


# ---------------------------------------------------------------- one step

def _step_inputs(T, t, rows, d, rng, h=None, W=None, acc=None):
    R = len(rows)
    if h is None:
        h = rng.standard_normal((R, d)).astype(np.float32)
    if W is None:
        W = (rng.standard_normal((T.V, d)) / math.sqrt(d)).astype(np.float32)
    if acc is None:
        acc = np.where(np.asarray(rows) >= 0, -rng.random(R), -np.inf).astype(np.float32)
    return h, W, acc


def test_w_zero_gives_log_one_over_n_and_tiebreak_order():
    """W = 0: every valid token of a row scores log(1/n) exactly; with equal
    fanouts and equal accumulated scores every candidate ties, so the output
    order is fixed by the tie-break alone (parent ascending, token
    ascending)."""
    V, L = 5, 3
    # every prefix has exactly 3 children: tokens {0, 2, 4}
    items = np.array([[a, b, c] for a in (0, 2, 4) for b in (0, 2, 4) for c in (0, 2, 4)], np.int32)
    T = oracle.Trie(items, V)
    K, d = 4, 8
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, d)).astype(np.float32)
    P = rng.standard_normal((L - 1, V, d)).astype(np.float32)
    W = np.zeros((L, V, d), np.float32)
    out = T.decode(K, q, P, W, bf16=False, trace=True)
    lg = np.float32(-math.log(3.0))
    acc = np.float32(0.0)
    for t in range(L):
        tok = out["trace_tokens"][t].reshape(2, K)
        par = out["trace_parents"][t].reshape(2, K)
        lp = out["trace_logp_out"][t].reshape(2, K)
        acc = np.float32(acc + lg)
        live = min(K, 3 ** t)  # live beams entering step t
        expect = [(p, v) for p in range(live) for v in (0, 2, 4)][:K]
        n = len(expect)
        expect += [(-1, -1)] * (K - n)
        for qi in range(2):
            assert list(zip(par[qi].tolist(), tok[qi].tolist())) == expect
            assert (lp[qi][:n] == acc).all() and np.isneginf(lp[qi][n:]).all()


def test_single_child_scores_zero():
    """A row with one valid token: log-softmax over one token is 0 exactly,
    so the accumulated score is carried unchanged."""
    items = np.array([[1, 3, 0], [1, 3, 2], [2, 0, 1]], np.int32)
    T = oracle.Trie(items, 4)
    rng = np.random.default_rng(0)
    rows = np.array([T.children([])[1][0], T.children([])[1][1]], np.int64)  # prefixes (1,), (2,)
    h, W, acc = _step_inputs(T, 1, rows, 6, rng)
    out = T.step(1, 2, h, W, rows, acc)
    assert sorted(out["logp"].tolist()) == sorted(acc.tolist())


def test_two_token_row_closed_form():
    """Prefix 3-5 of the worked example has the two valid tokens {1, 4}:
    logp(1) = -log(1 + exp(z4 - z1)), logp(4) = -log(1 + exp(z1 - z4)), with
    z_v = W_t[v][0] exactly for the one-hot hidden vector e_0."""
    g = read_golden("worked_example.txt")
    T = oracle.Trie(np.array(g["item"], np.int32), g["V"][0])
    d = 4
    # row of prefix 3-5 at depth 2
    r35 = int(T.children([3])[1][T.children([3])[0].tolist().index(5)])
    h = np.zeros((1, d), np.float32)
    h[0, 0] = 1.0
    W = np.zeros((10, d), np.float32)
    W[1, 0], W[4, 0] = 0.75, -0.5
    out = T.step(2, 1, h, W, np.array([r35], np.int64), np.zeros(1, np.float32), candidates=True)
    sc = dict(zip(out["cand_tokens"][0, :2].tolist(), out["cand_scores"][0, :2].tolist()))
    z1, z4 = 0.75, -0.5
    assert sc[1] == np.float32(-math.log1p(math.exp(z4 - z1)))
    assert sc[4] == np.float32(-math.log1p(math.exp(z1 - z4)))


@pytest.mark.parametrize("seed", [0, 1])
def test_softmax_sums_to_one_over_valid_tokens(seed):
    cfg = get_config("tiny")
    items = make_catalog(cfg)
    T = oracle.Trie(items, cfg.V)
    rng = np.random.default_rng(seed)
    K = 8
    rows = np.full(2 * K, -1, np.int64)
    rows[:K] = rng.choice(T.level_count(1), K, replace=False)
    rows[K:K + 3] = rng.choice(T.level_count(1), 3, replace=False)
    h, W, acc = _step_inputs(T, 1, rows, 16, rng)
    out = T.step(1, K, h, W, rows, acc, candidates=True)
    for qi in range(2):
        n = out["cand_count"][qi]
        par = out["cand_parents"][qi, :n]
        sc = out["cand_scores"][qi, :n].astype(np.float64)
        for k in np.unique(par):
            lp = sc[par == k] - float(acc[qi * K + k])
            assert abs(np.exp(lp).sum() - 1.0) < 1e-5
            assert len(lp) == len(T.children_of_row(1, int(rows[qi * K + k]))[0])


def test_full_product_catalog_equals_textbook_beam_search():
    """When every sequence of V^L is in the catalog every token is valid at
    every step, so filter-first decoding is plain beam search with
    log_softmax over the whole codebook (torch.log_softmax + torch.topk)."""
    V, L, K, d, Q = 8, 3, 5, 16, 3
    items = np.array(np.meshgrid(*[np.arange(V)] * L, indexing="ij")).reshape(L, -1).T.astype(np.int32)
    T = oracle.Trie(items, V)
    rng = np.random.default_rng(11)
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((L - 1, V, d)) / 4).astype(np.float32)
    W = (rng.standard_normal((L, V, d)) / 4).astype(np.float32)
    out = T.decode(K, q, P, W, bf16=False, trace=True)
    for qi in range(Q):
        s = torch.tensor(q[qi:qi + 1], dtype=torch.float32)
        acc = torch.zeros(1, dtype=torch.float32)
        seqs = [[]]
        for t in range(L):
            h = (s.double() / s.double().norm(dim=1, keepdim=True)).float()
            logits = h.double() @ torch.tensor(W[t], dtype=torch.float64).T
            lp = torch.log_softmax(logits, dim=1).float()
            tot = (acc[:, None] + lp).reshape(-1)
            val, idx = torch.topk(tot, K)
            par, tok = (idx // V), (idx % V)
            got_tok = out["trace_tokens"][t][qi * K:(qi + 1) * K]
            got_par = out["trace_parents"][t][qi * K:(qi + 1) * K]
            got_lp = out["trace_logp_out"][t][qi * K:(qi + 1) * K]
            assert got_tok.tolist() == tok.tolist()
            assert got_par.tolist() == par.tolist()
            np.testing.assert_allclose(got_lp, val.numpy(), rtol=0, atol=1e-6)
            acc = val
            seqs = [seqs[p] + [v] for p, v in zip(par.tolist(), tok.tolist())]
            if t + 1 < L:
                s = s[par] + torch.tensor(P[t], dtype=torch.float32)[tok]
        assert out["seqs"][qi * K:(qi + 1) * K].tolist() == seqs


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("seed,bf16", [(0, False), (1, False), (2, True), (3, True)])
def test_wide_beam_returns_every_item_with_its_path_score(seed, bf16):
    """Beam width >= catalog size: nothing is ever pruned, so the final beams
    are exactly the catalog items, scored along their own paths (brute-force
    enumeration over the catalog, no trie)."""
    rng = np.random.default_rng(seed)
    V, L, d = 6, 3, 5
    items = random_catalog(rng, 9, L, V)
    T = oracle.Trie(items[rng.permutation(len(items))], V)
    K = 12
    q = rng.standard_normal((1, d)).astype(np.float32)
    P = rng.standard_normal((L - 1, V, d)).astype(np.float32)
    W = rng.standard_normal((L, V, d)).astype(np.float32)
    if bf16:
        W = torch.tensor(W).bfloat16().float().numpy()
    out = T.decode(K, q, P, W, bf16=bf16)
    live = out["rows"] >= 0
    assert live.sum() == len(items)
    got = {tuple(s): lp for s, lp in zip(out["seqs"][live].tolist(), out["logp"][live].tolist())}
    lst = [tuple(r) for r in items.tolist()]
    exp = dict(zip(lst, brute.item_scores(lst, q[0], P, W, bf16)))
    assert set(got) == set(exp)
    for k in exp:
        assert abs(got[k] - exp[k]) <= 2 * np.spacing(np.float32(abs(exp[k]) + 1.0))
    # dead slots are sentinels
    assert (out["seqs"][~live] == -1).all() and np.isneginf(out["logp"][~live]).all()
    # final rows number the sorted distinct items
    order = sorted(lst)
    for s, r in zip(out["seqs"][live].tolist(), out["rows"][live].tolist()):
        assert order.index(tuple(s)) == r


def test_single_item_catalog():
    items = np.array([[2, 0, 1, 3]], np.int32)
    T = oracle.Trie(items, 4)
    K, d = 3, 4
    rng = np.random.default_rng(1)
    out = T.decode(K, rng.standard_normal((2, d)), rng.standard_normal((3, 4, d)),
                   rng.standard_normal((4, 4, d)), bf16=False)
    for qi in range(2):
        assert out["seqs"][qi * K].tolist() == [2, 0, 1, 3]
        assert out["logp"][qi * K] == 0.0
        assert out["rows"][qi * K] == 0
        assert (out["seqs"][qi * K + 1:(qi + 1) * K] == -1).all()
        assert np.isneginf(out["logp"][qi * K + 1:(qi + 1) * K]).all()


def test_decode_invariants_tiny():
    cfg = get_config("tiny")
    items = make_catalog(cfg)
    T = oracle.Trie(items, cfg.V)
    dense = make_dense(cfg)
    out = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=False, trace=True)
    cat = {tuple(r) for r in items.tolist()}
    live = out["rows"] >= 0
    assert live.all()  # the tiny catalog has enough items for every beam
    for s in out["seqs"].tolist():
        assert tuple(s) in cat
    K = cfg.K
    for t in range(cfg.L):
        tok, par = out["trace_tokens"][t], out["trace_parents"][t]
        lp, rin = out["trace_logp_out"][t], out["trace_rows_in"][t]
        ain = out["trace_acc_in"][t]
        for qi in range(cfg.Q):
            sl = slice(qi * K, (qi + 1) * K)
            keys = list(zip((-lp[sl]).tolist(), par[sl].tolist(), tok[sl].tolist()))
            assert keys == sorted(keys)  # best first under the tie-break
            for k in range(K):
                b = qi * K + k
                if tok[b] < 0:
                    continue
                pb = qi * K + par[b]
                assert rin[pb] >= 0  # parent is live
                assert lp[b] <= ain[pb]  # scores never increase
                ctok, crow = T.children_of_row(t, int(rin[pb]))
                j = ctok.tolist().index(int(tok[b]))
                assert out["trace_rows_out"][t][b] == crow[j]


def test_hidden_rule_unit_norm_and_bf16_rounding():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((6, 32)).astype(np.float32) * 3
    T = oracle.Trie(np.array([[0]], np.int32), 1)
    h = T.hidden(s, bf16=False)
    np.testing.assert_allclose(np.linalg.norm(h.astype(np.float64), axis=1), 1.0, atol=1e-6)
    np.testing.assert_allclose(h, s / np.linalg.norm(s.astype(np.float64), axis=1, keepdims=True), rtol=1e-6)
    hb = T.hidden(s, bf16=True)
    # torch's float32 -> bfloat16 conversion rounds to nearest even
    assert (hb == torch.tensor(h).bfloat16().float().numpy()).all()
