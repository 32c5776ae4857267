"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Every call goes through the C ABI (via the ctypes binding).  Step tests are
teacher forced: each step gets the oracle's beam state and hidden vectors, so
a difference at one step cannot hide or cause differences later.
"""

import math

import numpy as np
import pytest

import oracle
from synth import get_config, make_catalog, make_dense
from tests.parity import compare_step, force_beam_form, logp_ok

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402  (fails loudly if the library is not built)

DEV = torch.device("cuda:0")
_CACHE = {}


def to_dev_w(dense, cfg):
    if cfg.dtype == "bf16":
        return torch.from_numpy(dense["W_bits"].view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(dense["W"]).to(DEV)


def to_dev_h(h, cfg):
    t = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(DEV)
    return t.to(torch.bfloat16) if cfg.dtype == "bf16" else t


def workload(name, **over):
    key = (name, tuple(sorted(over.items())))
    if key not in _CACHE:
        cfg = get_config(name, **over)
        items = make_catalog(cfg)
        dense = make_dense(cfg)
        T = oracle.Trie(items, cfg.V)
        ref = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=cfg.dtype == "bf16", trace=True, threads=8)
        _CACHE[key] = dict(cfg=cfg, items=items, dense=dense, T=T, ref=ref, W=to_dev_w(dense, cfg))
    return _CACHE[key]


def gpu_step(plan, t, h, Wt, rows, acc):
    out = plan.step(t, h, Wt, rows, acc)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in zip(("tokens", "parents", "rows", "logp"), out)}


@pytest.mark.parametrize("name", ["tiny", "small"])
@pytest.mark.parametrize("path", ["sparse", "dense", "auto", "sparse_split", "sparse_split_all", "sparse_beam",
                                  "sparse_qsplit", "sparse_qsplit8"])
@pytest.mark.parametrize("store", ["auto", "csr", "bitmap"])
def test_step_parity_teacher_forced(name, path, store):
    w = workload(name)
    cfg, T, ref = w["cfg"], w["T"], w["ref"]
    idx = cb.Index(w["items"], cfg.V, device=0, store=store)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    total_exempt = 0
    for t in range(cfg.L):
        print("case", name, path, store, "step", t, flush=True)
        if path == "sparse_split_all":  # every multi-token row scored apart
            plan.set_path(t, "sparse_split")
            plan.set_split_rows(t, 1)
        elif path == "sparse_beam":  # one workgroup per beam, then the per-query merge
            plan.set_path(t, "sparse")
            force_beam_form(plan, t)
        elif path in ("sparse_qsplit", "sparse_qsplit8"):  # four or eight workgroups per query
            plan.set_path(t, "sparse")
            plan.set_option(t, "query_split", 8 if path == "sparse_qsplit8" else 4)
        else:
            plan.set_path(t, path)
        h = ref["trace_h"][t]
        rows = ref["trace_rows_in"][t]
        acc = ref["trace_acc_in"][t]
        o = T.step(t, cfg.K, h, w["dense"]["W"][t], rows, acc, candidates=True, threads=8)
        g = gpu_step(plan, t, to_dev_h(h, cfg), w["W"][t],
                     torch.from_numpy(rows.astype(np.int32)).to(DEV), torch.from_numpy(acc).to(DEV))
        ex, gap, fails = compare_step(o, g, cfg.K, cfg.dtype)
        assert not fails, "\n".join(fails[:10])
        total_exempt += ex
    if name == "tiny":
        assert total_exempt == 0


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_decode_parity_free_running(name):
    w = workload(name)
    cfg, T, ref = w["cfg"], w["T"], w["ref"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    q = torch.from_numpy(w["dense"]["q"]).to(DEV)
    P = torch.from_numpy(w["dense"]["P"]).to(DEV)
    out = plan.decode(q, P, w["W"], trace=True)
    torch.cuda.synchronize()
    seqs, logp, rows = (out[k].cpu().numpy() for k in ("seqs", "logp", "rows"))
    th = out["trace_h"].float().cpu().numpy()
    # hidden vectors of step 0 are computed from q alone: identical on both sides
    assert np.array_equal(th[0], ref["trace_h"][0])
    if np.array_equal(seqs, ref["seqs"]):
        assert np.array_equal(rows, ref["rows"])
        ok, err = logp_ok(logp, ref["logp"], cfg.dtype)
        assert ok.all(), err.max()
        for t in range(cfg.L):
            d = np.abs(th[t] - ref["trace_h"][t])
            assert (d <= 1e-2 * np.abs(ref["trace_h"][t]) + 1e-30).all()
    else:
        # a divergence is allowed only where the step chose between near-tied candidates
        assert name != "tiny", "tiny must decode identically"
        tr = out["trace_rows"].cpu().numpy()
        g_rows = [tr[t] for t in range(1, cfg.L)] + [rows]
        r_rows = [ref["trace_rows_in"][t] for t in range(1, cfg.L)] + [ref["rows"]]
        first = next(t for t in range(cfg.L) if not np.array_equal(g_rows[t], r_rows[t]))
        o = T.step(first, cfg.K, ref["trace_h"][first], w["dense"]["W"][first], ref["trace_rows_in"][first],
                   ref["trace_acc_in"][first], candidates=True)
        g = gpu_step(plan, first, to_dev_h(ref["trace_h"][first], cfg), w["W"][first],
                     torch.from_numpy(ref["trace_rows_in"][first].astype(np.int32)).to(DEV),
                     torch.from_numpy(ref["trace_acc_in"][first]).to(DEV))
        ex, gap, fails = compare_step(o, g, cfg.K, cfg.dtype)
        assert not fails and ex > 0


def test_decode_is_deterministic():
    w = workload("small")
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    q = torch.from_numpy(w["dense"]["q"]).to(DEV)
    P = torch.from_numpy(w["dense"]["P"]).to(DEV)
    a = plan.decode(q, P, w["W"])
    b = plan.decode(q, P, w["W"])
    torch.cuda.synchronize()
    for k in ("seqs", "logp", "rows"):
        assert torch.equal(a[k], b[k])


def small_problem(items, V, K, d, Q, seed, dtype="f32", zero_w=False):
    items = np.asarray(items, np.int32)
    L = items.shape[1]
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((max(L - 1, 1), V, d)) / math.sqrt(d)).astype(np.float32)[: L - 1]
    W = np.zeros((L, V, d), np.float32) if zero_w else (rng.standard_normal((L, V, d)) / math.sqrt(d)).astype(np.float32)
    if dtype == "bf16":
        W = torch.from_numpy(W).bfloat16().float().numpy()
    T = oracle.Trie(items, V)
    ref = T.decode(K, q, P if L > 1 else None, W, bf16=dtype == "bf16", trace=True)
    idx = cb.Index(items, V, device=0)
    plan = idx.plan(Q, K, d, dtype)
    Wd = torch.from_numpy(W).to(DEV)
    if dtype == "bf16":
        Wd = Wd.bfloat16()
    Pd = torch.from_numpy(np.ascontiguousarray(P)).to(DEV) if L > 1 else None
    out = plan.decode(torch.from_numpy(q).to(DEV), Pd, Wd)
    torch.cuda.synchronize()
    return ref, {k: v.cpu().numpy() for k, v in out.items()}, plan


def test_single_item_catalog_gpu():
    ref, got, _ = small_problem([[2, 0, 1, 3]], 4, K=3, d=8, Q=2, seed=1)
    for qi in range(2):
        assert got["seqs"][qi * 3].tolist() == [2, 0, 1, 3]
        assert got["logp"][qi * 3] == 0.0 and got["rows"][qi * 3] == 0
        assert (got["seqs"][qi * 3 + 1:(qi + 1) * 3] == -1).all()
        assert np.isneginf(got["logp"][qi * 3 + 1:(qi + 1) * 3]).all()


def test_zero_w_ties_follow_the_tie_break_gpu():
    items = [[a, b, c] for a in (0, 2, 4) for b in (0, 2, 4) for c in (0, 2, 4)]
    for path in ("sparse", "dense"):
        rng = np.random.default_rng(3)
        K, d, Q, V = 4, 8, 2, 5
        T = oracle.Trie(np.array(items, np.int32), V)
        idx = cb.Index(np.array(items, np.int32), V, device=0)
        plan = idx.plan(Q, K, d, "f32")
        q = torch.from_numpy(rng.standard_normal((Q, d)).astype(np.float32)).to(DEV)
        P = torch.from_numpy(rng.standard_normal((2, V, d)).astype(np.float32)).to(DEV)
        W = torch.zeros((3, V, d), dtype=torch.float32, device=DEV)
        for t in range(3):
            plan.set_path(t, path)
        out = plan.decode(q, P, W, trace=True)
        torch.cuda.synchronize()
        ref = T.decode(K, q.cpu().numpy(), P.cpu().numpy(), W.cpu().numpy(), bf16=False)
        assert np.array_equal(out["seqs"].cpu().numpy(), ref["seqs"])
        lp = out["logp"].cpu().numpy()
        ok, err = logp_ok(lp, ref["logp"], "f32")
        assert ok.all()
        # all four final beams tie: order is parent ascending then token ascending
        assert (lp == lp[0]).all()


def test_fewer_candidates_than_beams_gpu():
    items = [[0, 1], [0, 2], [1, 1]]
    ref, got, _ = small_problem(items, 3, K=8, d=16, Q=3, seed=2)
    assert np.array_equal(got["seqs"], ref["seqs"])
    assert np.array_equal(got["rows"], ref["rows"])
    live = ref["rows"] >= 0
    assert live.reshape(3, 8).sum(axis=1).tolist() == [3, 3, 3]
    assert np.isneginf(got["logp"][~live]).all()


def test_full_product_catalog_gpu_equals_oracle():
    V, L = 8, 3
    items = np.array(np.meshgrid(*[np.arange(V)] * L, indexing="ij")).reshape(L, -1).T
    ref, got, _ = small_problem(items, V, K=5, d=16, Q=3, seed=11)
    assert np.array_equal(got["seqs"], ref["seqs"])
    ok, _ = logp_ok(got["logp"], ref["logp"], "f32")
    assert ok.all()


def test_rows_outside_the_table_are_dead_beams():
    cfg = get_config("tiny")
    w = workload("tiny")
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    n1 = idx.info(1)["n_rows"]
    R = cfg.Q * cfg.K
    rows = torch.full((R,), n1 + 5, dtype=torch.int32, device=DEV)
    acc = torch.zeros(R, dtype=torch.float32, device=DEV)
    h = torch.randn(R, cfg.d, device=DEV)
    g = gpu_step(plan, 1, h, w["W"][1], rows, acc)
    assert (g["tokens"] == -1).all() and np.isneginf(g["logp"]).all()


def test_q_below_q_max_and_q_zero():
    w = workload("tiny")
    cfg, T, ref = w["cfg"], w["T"], w["ref"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q + 3, cfg.K, cfg.d, cfg.dtype)
    t = 1
    Qs = 2
    R = Qs * cfg.K
    h = ref["trace_h"][t][:R]
    rows = ref["trace_rows_in"][t][:R]
    acc = ref["trace_acc_in"][t][:R]
    o = T.step(t, cfg.K, h, w["dense"]["W"][t], rows, acc, candidates=True)
    g = gpu_step(plan, t, to_dev_h(h, cfg), w["W"][t], torch.from_numpy(rows.astype(np.int32)).to(DEV),
                 torch.from_numpy(acc).to(DEV))
    ex, gap, fails = compare_step(o, g, cfg.K, cfg.dtype)
    assert not fails
    e = torch.empty(0, dtype=torch.int32, device=DEV)
    plan.step(t, torch.empty((0, cfg.d), device=DEV), w["W"][t], e, torch.empty(0, device=DEV))


def test_step_argument_errors():
    w = workload("tiny")
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    R = cfg.Q * cfg.K
    h = torch.zeros((R, cfg.d), device=DEV)
    rows = torch.zeros(R, dtype=torch.int32, device=DEV)
    acc = torch.zeros(R, device=DEV)
    with pytest.raises(cb.CbError):
        plan.step(cfg.L, h, w["W"][0], rows, acc)  # t out of range
    big = torch.zeros(((cfg.Q + 1) * cfg.K, cfg.d), device=DEV)
    with pytest.raises(cb.CbError):
        plan.step(0, big, w["W"][0], torch.zeros((cfg.Q + 1) * cfg.K, dtype=torch.int32, device=DEV),
                  torch.zeros((cfg.Q + 1) * cfg.K, device=DEV))  # Q > Q_max
    with pytest.raises(cb.CbError) as e:
        idx.plan(1, 2000, cfg.d, cfg.dtype)
    assert e.value.status == -5


def test_plan_released_after_its_index():
    """Destroying a plan after its index (as a garbage collector may order
    them) touches nothing of the index and leaves no HIP error pending."""
    w = workload("tiny")
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    idx.close()
    plan.close()
