"""GPU parity of the radix-select path (beam widths up to 1024).

The radix path writes every candidate's key to HBM and finds each query's
K-th largest key by radix select (FlashTrie's beam widths of 100 to 1000,
sec. 4.2).  It is checked against the CPU oracles on the same seeded inputs:
forced on the tiny and small workloads at their own beam widths (where the
LDS selection also runs), at beam widths 100 to 1000, on massive exact ties
(which exercise the in-workgroup end of the radix select), and on a reduced
catalog of the large-library generator (V = 32,001, variable lengths).
"""

import math

import numpy as np
import pytest

import oracle
from synth import get_config, make_catalog, make_dense
from tests.parity import compare_step, logp_ok

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402

DEV = torch.device("cuda:0")
_CACHE = {}


def dev_w(W, dtype):
    t = torch.from_numpy(np.ascontiguousarray(W, np.float32)).to(DEV)
    return t.bfloat16() if dtype == "bf16" else t


def dev_h(h, dtype):
    t = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(DEV)
    return t.bfloat16() if dtype == "bf16" else t


def workload(name, oracle_cls=oracle.Trie, **over):
    key = (name, oracle_cls.__name__, tuple(sorted(over.items())))
    if key not in _CACHE:
        _CACHE.clear()
        cfg = get_config(name, **over)
        print("building", name, over, flush=True)
        items = make_catalog(cfg)
        dense = make_dense(cfg)
        T = oracle_cls(items, cfg.V)
        ref = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=cfg.dtype == "bf16", trace=True, threads=16)
        if cfg.dtype == "bf16":
            W = torch.from_numpy(dense["W_bits"].view(np.int16)).to(DEV).view(torch.bfloat16)
        else:
            W = torch.from_numpy(dense["W"]).to(DEV)
        _CACHE[key] = dict(cfg=cfg, items=items, dense=dense, T=T, ref=ref, W=W)
    return _CACHE[key]


def step_all(plan, w, path, select, K=None):
    """Teacher-forced steps on the oracle's beam state; returns the exemptions.
    path "sparse_tm": the sparse path with its scores grouped by token."""
    cfg, T, ref = w["cfg"], w["T"], w["ref"]
    K = K or cfg.K
    ex_total = 0
    for t in range(cfg.L):
        plan.set_path(t, "sparse" if path == "sparse_tm" else path)
        plan.set_option(t, "token_major", 2 if path == "sparse_tm" else 1)
        plan.set_select(t, select)
        print("step", t, plan.get_path(t), plan.get_select(t), flush=True)
        h, rows, acc = ref["trace_h"][t], ref["trace_rows_in"][t], ref["trace_acc_in"][t]
        o = T.step(t, K, h, w["dense"]["W"][t], rows, acc, candidates=True, threads=16)
        out = plan.step(t, dev_h(h, cfg.dtype), w["W"][t], torch.from_numpy(rows.astype(np.int32)).to(DEV),
                        torch.from_numpy(acc).to(DEV))
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in zip(("tokens", "parents", "rows", "logp"), out)}
        ex, gap, fails = compare_step(o, g, K, cfg.dtype)
        assert not fails, "step %d:\n" % t + "\n".join(fails[:10])
        ex_total += ex
    return ex_total


@pytest.mark.parametrize("name", ["tiny", "small"])
@pytest.mark.parametrize("path", ["sparse", "dense", "sparse_tm"])
@pytest.mark.parametrize("store", ["auto", "bitmap"])
def test_radix_step_parity_at_workload_width(name, path, store):
    w = workload(name)
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0, store=store)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    ex = step_all(plan, w, path, "radix")
    if name == "tiny":
        assert ex == 0


@pytest.mark.parametrize("K", [100, 256, 1000])
@pytest.mark.parametrize("path", ["sparse", "dense", "sparse_tm"])
def test_wide_beam_step_parity(K, path):
    w = workload("small", K=K, Q=6)
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, K, cfg.d, cfg.dtype)
    for t in range(cfg.L):
        assert plan.get_select(t) == "radix"
    step_all(plan, w, path, "auto", K=K)


@pytest.mark.parametrize("K", [100, 1000])
def test_wide_beam_decode_parity(K):
    w = workload("small", K=K, Q=6)
    cfg, ref = w["cfg"], w["ref"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, K, cfg.d, cfg.dtype)
    q = torch.from_numpy(w["dense"]["q"]).to(DEV)
    P = torch.from_numpy(w["dense"]["P"]).to(DEV)
    out = plan.decode(q, P, w["W"], trace=True)
    torch.cuda.synchronize()
    check_decode(w, out, K, plan)


def check_decode(w, out, K, plan):
    """Per query: identical to the oracle, or the first differing step is a
    near tie (teacher-forced comparison at that step)."""
    cfg, ref, T = w["cfg"], w["ref"], w["T"]
    seqs, logp, rows = (out[k].cpu().numpy() for k in ("seqs", "logp", "rows"))
    tr = out["trace_rows"].cpu().numpy()
    if len(w["items"]) <= 10_000_000:  # (larger catalogs: outputs equal to the oracle's are in it)
        catalog = {tuple(r) for r in w["items"].tolist()}
        for s_ in seqs[rows >= 0][:3000].tolist():
            assert tuple(s_) in catalog
    diverged = 0
    for qi in range(cfg.Q):
        sl = slice(qi * K, (qi + 1) * K)
        if np.array_equal(seqs[sl], ref["seqs"][sl]):
            assert np.array_equal(rows[sl], ref["rows"][sl])
            ok, err = logp_ok(logp[sl], ref["logp"][sl], cfg.dtype)
            assert ok.all(), (qi, err.max())
            continue
        diverged += 1
        g_rows = [tr[t][sl] for t in range(1, cfg.L)] + [rows[sl]]
        r_rows = [ref["trace_rows_in"][t][sl] for t in range(1, cfg.L)] + [ref["rows"][sl]]
        t0 = next(t for t in range(cfg.L) if not np.array_equal(g_rows[t], r_rows[t]))
        print("query", qi, "first differs at step", t0, flush=True)
        o = T.step(t0, K, ref["trace_h"][t0][sl], w["dense"]["W"][t0], ref["trace_rows_in"][t0][sl],
                   ref["trace_acc_in"][t0][sl], candidates=True, threads=16)
        got = plan.step(t0, dev_h(ref["trace_h"][t0][sl], cfg.dtype), w["W"][t0],
                        torch.from_numpy(ref["trace_rows_in"][t0][sl].astype(np.int32)).to(DEV),
                        torch.from_numpy(ref["trace_acc_in"][t0][sl]).to(DEV))
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in zip(("tokens", "parents", "rows", "logp"), got)}
        ex, gap, fails = compare_step(o, g, K, cfg.dtype)
        assert not fails, "\n".join(fails[:5])
        assert ex > 0
    assert diverged <= max(1, cfg.Q // 4)


def test_massive_exact_ties_follow_the_tie_break():
    """16 x 4096 full product, W = 0: at step 1 all 65,536 candidates of a
    query have the same float32 score, so the order is (parent, token)
    alone and the radix select has to resolve all 64 key bits."""
    V, d, Q, K = 4096, 64, 2, 128
    items = np.array([(a, b) for a in range(16) for b in range(V)], np.int32)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((1, V, d)) / math.sqrt(d)).astype(np.float32)
    W = np.zeros((2, V, d), np.float32)
    T = oracle.Trie(items, V)
    ref = T.decode(K, q, P, W, bf16=False, trace=True)
    idx = cb.Index(items, V, device=0)
    plan = idx.plan(Q, K, d, "f32")
    for path in ("sparse", "dense", "sparse_tm"):
        for t in range(2):
            plan.set_path(t, "sparse" if path == "sparse_tm" else path)
            plan.set_option(t, "token_major", 2 if path == "sparse_tm" else 1)
        out = plan.decode(torch.from_numpy(q).to(DEV), torch.from_numpy(P).to(DEV), torch.from_numpy(W).to(DEV))
        torch.cuda.synchronize()
        seqs = out["seqs"].cpu().numpy()
        assert np.array_equal(seqs, ref["seqs"]), path
        assert np.array_equal(out["rows"].cpu().numpy(), ref["rows"])
        ok, _ = logp_ok(out["logp"].cpu().numpy(), ref["logp"], "f32")
        assert ok.all()
        # the first query's beams: parent 0 (token 0 at step 0), tokens 0..127
        assert seqs[:K, 0].tolist() == [0] * K and seqs[:K, 1].tolist() == list(range(K))


def test_few_score_levels_many_ties():
    """W = 0 at step 0 and two W rows at step 1: a query's 12,288 step-1
    candidates take six distinct scores (two per beam), each shared by about
    2,000 candidates, so the K-th key lies inside a tie group."""
    V, d, Q, K = 4096, 64, 1, 1000
    items = np.array([(a, b) for a in range(3) for b in range(V)], np.int32)
    rng = np.random.default_rng(6)
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((1, V, d)) / math.sqrt(d)).astype(np.float32)
    W = np.zeros((2, V, d), np.float32)
    W[1, : V // 2 - 100, 0] = 1.0  # tokens below 1948 score higher at step 1 when h[0] > 0
    T = oracle.Trie(items, V)
    ref = T.decode(K, q, P, W, bf16=False, trace=True)
    idx = cb.Index(items, V, device=0)
    plan = idx.plan(Q, K, d, "f32")
    out = plan.decode(torch.from_numpy(q).to(DEV), torch.from_numpy(P).to(DEV), torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(out["seqs"].cpu().numpy(), ref["seqs"])
    ok, _ = logp_ok(out["logp"].cpu().numpy(), ref["logp"], "f32")
    assert ok.all()


@pytest.mark.parametrize("K", [100, 1000])
def test_large_generator_reduced_catalog(K):
    """The large-library generator (Zipf tokens, lengths 4-12 padded with
    EOS, V = 32,001, d = 1024 bf16) on 2M items, one query, checked against
    the sorted-range oracle; both scoring paths teacher forced, then the
    tuned free-running decode."""
    w = workload("large", oracle_cls=oracle.SortedRange, n_items=2_000_000, K=K)
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, K, cfg.d, cfg.dtype)
    for path in ("sparse", "dense", "sparse_tm"):
        print("teacher forced", path, flush=True)
        step_all(plan, w, path, "auto", K=K)
    for t in range(cfg.L):
        plan.set_path(t, "auto")
        plan.set_option(t, "token_major", 0)
    q = torch.from_numpy(w["dense"]["q"]).to(DEV)
    P = torch.from_numpy(w["dense"]["P"]).to(DEV)
    plan.tune(q, P, w["W"], reps=2)
    print("paths", [plan.get_path(t) for t in range(cfg.L)], flush=True)
    out = plan.decode(q, P, w["W"], trace=True)
    torch.cuda.synchronize()
    check_decode(w, out, K, plan)


def test_radix_errors():
    w = workload("tiny")
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    with pytest.raises(cb.CbError) as e:
        idx.plan(1, 1025, cfg.d, cfg.dtype)
    assert e.value.status == -5
    plan = idx.plan(1, 100, cfg.d, cfg.dtype)
    with pytest.raises(cb.CbError) as e:
        plan.set_select(0, "lds")
    assert e.value.status == -5
    plan.set_select(0, "radix")
    assert plan.get_select(0) == "radix"
    assert plan.get_option(0, "token_major") == 1
    plan.set_option(0, "token_major", 2)
    assert plan.get_option(0, "token_major") == 2
    with pytest.raises(cb.CbError) as e:
        plan.set_option(0, "token_major", 3)
    assert e.value.status == -1
    wide = idx.plan(1, 100, 2056, cfg.dtype)  # W_t rows wider than the registers hold
    with pytest.raises(cb.CbError) as e:
        wide.set_option(0, "token_major", 2)
    assert e.value.status == -1


@pytest.mark.parametrize("prepass", [1, 2])
def test_token_major_decode_with_and_without_prepass(prepass):
    """Every step scored by token, with and without the one-token pre-pass,
    repeated (the per-token counts are cleared between steps): the decode
    equals the per-chunk scoring's up to near ties and holds to the oracle."""
    w = workload("small", K=100, Q=6)
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    q = torch.from_numpy(w["dense"]["q"]).to(DEV)
    P = torch.from_numpy(w["dense"]["P"]).to(DEV)
    for t in range(cfg.L):
        plan.set_path(t, "sparse")
        plan.set_option(t, "radix_prepass", prepass)
        plan.set_option(t, "token_major", 2)
    first = None
    for rep in range(2):
        out = plan.decode(q, P, w["W"], trace=True)
        torch.cuda.synchronize()
        check_decode(w, out, cfg.K, plan)
        if first is None:
            first = {k: out[k].clone() for k in ("seqs", "logp", "rows")}
        else:
            for k in first:
                assert torch.equal(first[k], out[k]), k
