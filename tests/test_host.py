"""CPU tests of the host side of the library: the C ABI surface and the
step-table builder (no kernel is launched; indexes are built host-only)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from synth import get_config, make_catalog

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cb.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cb_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def cb():
    import csr_constrained_beam_amd as m
    m._lib.lib()
    return m


def test_library_exports_every_declared_symbol(cb):
    names = declared_functions()
    assert len(names) >= 14
    L = cb._lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(cb._lib.SIGNATURES), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", cb.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (cb_\w+)", out))
    assert set(names) <= exported


def test_library_is_built_for_gfx950(cb):
    """The in-tree build carries a gfx950 code object (its bundle id string)."""
    blob = open(cb.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def check_against_oracle(cb, items, V, store):
    idx = cb.Index(items, V, device=-1, store=store)
    T = oracle.Trie(items, V)
    L = items.shape[1]
    assert idx.shape["n_items"] == T.n_items
    for t in range(L):
        info = idx.info(t)
        assert info["n_rows"] == T.level_count(t)
        assert info["n_edges"] == T.level_count(t + 1)
        fan = 0
        for r in range(info["n_rows"]):
            tok, nxt = idx.row(t, r)
            otok, orow = T.children_of_row(t, r)
            assert tok.tolist() == otok.tolist()
            assert nxt.tolist() == orow.tolist()
            fan = max(fan, len(tok))
        assert info["max_fanout"] == fan
        if store != "auto":
            assert info["storage"] == store
    return idx


@pytest.mark.parametrize("store", ["auto", "csr", "bitmap"])
def test_step_tables_equal_oracle_trie_tiny(cb, store):
    cfg = get_config("tiny")
    check_against_oracle(cb, make_catalog(cfg), cfg.V, store)


def test_step_tables_equal_oracle_trie_small(cb):
    cfg = get_config("small")
    idx = check_against_oracle(cb, make_catalog(cfg), cfg.V, "auto")
    # the collision level only ever uses tokens 0..7
    for r in range(0, idx.info(3)["n_rows"], 97):
        tok, _ = idx.row(3, r)
        assert tok.max() < 8


@pytest.mark.parametrize("seed", [0, 1])
def test_step_tables_random_unsorted_with_duplicates(cb, seed):
    rng = np.random.default_rng(seed)
    items = rng.integers(0, 7, size=(300, 4)).astype(np.int32)  # many repeats
    for store in ("auto", "csr", "bitmap"):
        check_against_oracle(cb, items, 7, store)


def test_worked_example_row(cb):
    """ZeroGR's 3-5 example through the library's own tables."""
    from tests.test_oracle_pins import read_golden
    g = read_golden("worked_example.txt")
    items = np.array(g["item"], np.int32)
    for store in ("csr", "bitmap"):
        idx = cb.Index(items, g["V"][0], device=-1, store=store)
        # row of prefix (3,) at step 1, then of (3, 5) at step 2
        tok0, nxt0 = idx.row(0, 0)
        r3 = int(nxt0[tok0.tolist().index(3)])
        tok1, nxt1 = idx.row(1, r3)
        r35 = int(nxt1[tok1.tolist().index(5)])
        tok2, _ = idx.row(2, r35)
        assert tok2.tolist() == g["valid"]


def test_last_step_rows_rank_the_sorted_catalog(cb):
    cfg = get_config("tiny")
    items = make_catalog(cfg)
    idx = cb.Index(items, cfg.V, device=-1)
    order = {tuple(r): i for i, r in enumerate(sorted(map(tuple, items.tolist())))}
    for it in items[:200].tolist():
        r = 0
        for t in range(cfg.L):
            tok, nxt = idx.row(t, r)
            r = int(nxt[tok.tolist().index(it[t])])
        assert r == order[tuple(it)]


@pytest.mark.parametrize("args,status", [
    (dict(items=[[0, 5]], V=5), -1),          # token out of range
    (dict(items=[[0, -1]], V=5), -1),
    (dict(items=np.zeros((1, 0)), V=5), -1),  # L = 0
    (dict(items=[[0, 1]], V=1), -1),          # V < 2
    (dict(items=[[0, 1]], V=70000), -4),      # V beyond 16-bit tokens
])
def test_build_errors(cb, args, status):
    with pytest.raises(cb.CbError) as e:
        cb.Index(np.array(args["items"], np.int32).reshape(len(args["items"]), -1), args["V"], device=-1)
    assert e.value.status == status
    assert cb._lib.lib().cb_last_error()


def test_host_only_index_cannot_plan(cb):
    idx = cb.Index(np.array([[0, 1], [1, 0]], np.int32), 2, device=-1)
    with pytest.raises(cb.CbError) as e:
        idx.plan(1, 2, 8, "f32")
    assert e.value.status == -1


def test_null_arguments_rejected(cb):
    L = cb._lib.lib()
    assert L.cb_build_index(None, 1, 1, 2, -1, 0, ctypes.byref(ctypes.c_void_p())) == -1
    assert L.cb_index_info(None, 0, None) == -1
    assert L.cb_step(None, 0, 0, None, None, None, None, None, None, None, None, None) == -1
    assert L.cb_decode(None, 0, None, None, None, None, None, None, None, None, None, None) == -1
    L.cb_free_index(None)
    L.cb_plan_destroy(None)


def test_wire_arguments_checked_on_the_host(cb):
    """The wire-format call checks its sizes before touching the device."""
    L = cb._lib.lib()
    v = ctypes.c_int64()
    assert L.cb_wire_bytes(3, 2, ctypes.byref(v)) == 0 and v.value == 80  # 8 + 16*3 + 4*3*2
    assert L.cb_wire_bytes(1, 7, ctypes.byref(v)) == 0 and v.value == 56  # 52 rounded up to 8
    assert cb.wire_bytes(1024, 8) == 8 + 16 * 1024 + 4 * 1024 * 8
    assert L.cb_wire_bytes(0, 2, ctypes.byref(v)) == -1
    assert L.cb_wire_results(0, 4, 3, None, None, 0.0, None, 8 + 64 + 48, None, None) == 0  # no queries
    assert L.cb_wire_results(1, 1025, 3, None, None, 0.0, None, 1 << 20, None, None) == -1  # K above 1024
    assert L.cb_wire_results(1, 4, 3, None, None, 0.0, None, 64, None, None) == -1  # stride too small
    assert L.cb_wire_results(1, 4, 3, None, None, float("inf"), None, 128, None, None) == -1
    assert L.cb_wire_results(1, 4, 3, None, None, 0.0, None, 128, None, None) == -1  # NULL arrays


@pytest.mark.parametrize("store", ["auto", "csr", "bitmap"])
def test_chunked_build_equals_oracle_at_chunk_boundaries(cb, store):
    """A catalog of 200k items is built in 48 chunks of consecutive sorted
    items, each filling its rows and edges at positions computed in advance.
    Every row that holds a chunk's first or last item (rows straddling two
    chunks included), and a sample of the others, equal the oracle trie's."""
    rng = np.random.default_rng(17)
    V, L, n = 96, 4, 200_000
    items = rng.integers(0, V, size=(n, L)).astype(np.int32)
    items[:, 0] %= 5  # few wide level-1 rows, so that rows straddle chunks
    u = np.unique(items, axis=0)
    N = len(u)
    C = max(1, min(256, N // 4096))
    assert C > 8
    idx = cb.Index(items, V, device=-1, store=store)
    T = oracle.Trie(items, V)
    assert idx.shape["n_items"] == N == T.n_items
    for t in range(L):
        info = idx.info(t)
        assert info["n_rows"] == T.level_count(t) and info["n_edges"] == T.level_count(t + 1)
        if t == 0:
            row_of = np.zeros(N, np.int64)
        else:
            change = np.ones(N, bool)
            change[1:] = (u[1:, :t] != u[:-1, :t]).any(axis=1)
            row_of = np.cumsum(change) - 1
        rows = {int(row_of[b]) for c in range(C + 1) for b in (N * c // C - 1, N * c // C) if 0 <= b < N}
        rows |= set(rng.integers(0, info["n_rows"], size=200).tolist())
        fan = max(len(T.children_of_row(t, r)[0]) for r in range(info["n_rows"]))
        assert info["max_fanout"] == fan
        for r in sorted(rows):
            tok, nxt = idx.row(t, r)
            otok, orow = T.children_of_row(t, r)
            assert tok.tolist() == otok.tolist(), (t, r)
            assert nxt.tolist() == orow.tolist(), (t, r)


def test_static_umax_reproduces_the_capacity_rule():
    """The bench compares index bytes with STATIC's bound (sec. 5.3) at
    K1 = 12, K2 = 4 bytes (App. B.3): the page's own numbers are 17.3 MB for
    the dense levels at |V| = 2048, d = 2, 72 MB per million items for the
    six later levels of L = 8, about 90 MB per million in all."""
    import bench
    dense = bench.static_umax(2048, 0, 2, 2)
    assert abs(dense - 17_301_504) < 1
    assert abs(bench.static_umax(2048, 1_000_000, 8, 2) - dense - 72e6) < 1
    assert 89e6 < bench.static_umax(2048, 1_000_000, 8, 2) < 90e6
