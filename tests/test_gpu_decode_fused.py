"""GPU: the persistent decode (the trailing sparse steps in one launch, one
workgroup per query) against the step-by-step decode and the oracle.

The persistent form runs the same per-query step and the same hidden update
as the step-by-step form, so its outputs must be equal bit for bit; the
step-by-step decode itself is held to the oracle by the parity tests.
"""

import numpy as np
import pytest

import oracle
from tests.parity import logp_ok

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402
from tests.test_gpu_parity import DEV, workload  # noqa: E402


def set_paths(plan, L, mode):
    for t in range(L):
        if mode == "all_sparse":
            plan.set_path(t, "sparse")
        elif mode == "first_dense":
            plan.set_path(t, "dense" if t == 0 else "sparse")
        elif mode == "middle_dense":
            plan.set_path(t, "dense" if t == L // 2 else "sparse")
        elif mode == "middle_per_beam":  # one step in the per-beam form splits the trailing run
            plan.set_path(t, "sparse")
            plan.set_option(t, "sparse_form", 1 if t == L // 2 else 0)
        else:
            plan.set_path(t, "auto")


def decode_both(plan, q, P, W):
    plan.set_decode_fusion(False)
    a = plan.decode(q, P, W)
    plan.set_decode_fusion(True)
    plan.profile_start(capacity=1024)
    b = plan.decode(q, P, W)
    recs = plan.profile_stop()
    torch.cuda.synchronize()
    # phase clock: one entry per persistent step, selection time positive
    tails = [r for r in recs if r["kernel"] == "decode_tail"]
    ph = plan.profile_phases()
    if tails:
        L = plan.L
        assert [x["step"] for x in ph] == list(range(tails[0]["step"], L))
        assert all(x["select_us"] > 0 and x["update_us"] >= 0 for x in ph)
        assert ph[-1]["update_us"] == 0 and all(x["update_us"] > 0 for x in ph[:-1])
        assert sum(x["select_us"] + x["update_us"] for x in ph) <= tails[0]["us"] * 1.05 + 5
    else:
        assert ph == []
    return a, b, recs


def expected_tail(plan, L):
    t = L
    while (t > 0 and plan.get_path(t - 1) == "sparse" and plan.get_select(t - 1) == "lds"
           and plan.get_option(t - 1, "sparse_form") == 0):
        t -= 1
    return t if L - t >= 2 else L


@pytest.mark.parametrize("name", ["tiny", "small"])
@pytest.mark.parametrize("mode", ["auto", "all_sparse", "first_dense", "middle_dense", "middle_per_beam"])
def test_persistent_decode_equals_step_by_step(name, mode):
    w = workload(name)
    cfg, ref = w["cfg"], w["ref"]
    print("case", name, mode, flush=True)
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    set_paths(plan, cfg.L, mode)
    q = torch.from_numpy(w["dense"]["q"]).to(DEV)
    P = torch.from_numpy(w["dense"]["P"]).to(DEV)
    a, b, recs = decode_both(plan, q, P, w["W"])
    for k in ("seqs", "logp", "rows"):
        assert torch.equal(a[k], b[k]), k
    t0 = expected_tail(plan, cfg.L)
    tails = [r for r in recs if r["kernel"] == "decode_tail"]
    if t0 < cfg.L:
        assert len(tails) == 1 and tails[0]["step"] == t0 and tails[0]["blocks"] == cfg.Q
        assert not [r for r in recs if r["step"] >= t0 and r["kernel"] != "decode_tail"]
    else:
        assert not tails
    if name == "tiny":  # identical to the oracle
        seqs, logp, rows = (b[k].cpu().numpy() for k in ("seqs", "logp", "rows"))
        assert np.array_equal(seqs, ref["seqs"]) and np.array_equal(rows, ref["rows"])
        ok, err = logp_ok(logp, ref["logp"], cfg.dtype)
        assert ok.all(), err.max()


def test_persistent_decode_fewer_queries_and_repeat():
    """Q below Q_max, then the full batch, then Q = 0, on one plan."""
    w = workload("small")
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    set_paths(plan, cfg.L, "all_sparse")
    q = torch.from_numpy(w["dense"]["q"]).to(DEV)
    P = torch.from_numpy(w["dense"]["P"]).to(DEV)
    full_a, full_b, _ = decode_both(plan, q, P, w["W"])
    for Q in (3, 1, cfg.Q):
        a, b, _ = decode_both(plan, q[:Q].contiguous(), P, w["W"])
        for k in ("seqs", "logp", "rows"):
            assert torch.equal(a[k], b[k]), (Q, k)
            assert torch.equal(b[k], full_b[k][:Q * cfg.K]), (Q, k)
    z = plan.decode(q[:0], P, w["W"])
    torch.cuda.synchronize()
    assert z["seqs"].numel() == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 256, 200])
def test_persistent_decode_hidden_widths(dtype, d):
    """Hidden widths on and off the 4-wide update (d a multiple of 256), both
    element types, a catalog with dead beams and a single-child chain; the
    whole decode runs in one launch and equals the oracle's."""
    rng = np.random.default_rng(7)
    items = np.unique(rng.integers(0, 12, size=(400, 5)), axis=0)
    items = np.unique(np.concatenate([items, np.array([[11, 11, 11, 11, 3]])]), axis=0).astype(np.int32)
    V, K, Q, L = 12, 8, 5, 5
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((L - 1, V, d)) / np.sqrt(d)).astype(np.float32)
    W = (rng.standard_normal((L, V, d)) / np.sqrt(d)).astype(np.float32)
    Wd = torch.from_numpy(W).to(DEV)
    if dtype == "bf16":
        Wd = Wd.bfloat16()
        W = Wd.float().cpu().numpy()
    ref = oracle.Trie(items, V).decode(K, q, P, W, bf16=dtype == "bf16")
    idx = cb.Index(items, V, device=0)
    plan = idx.plan(Q, K, d, dtype)
    set_paths(plan, L, "all_sparse")
    a, b, recs = decode_both(plan, torch.from_numpy(q).to(DEV), torch.from_numpy(P).to(DEV), Wd)
    for k in ("seqs", "logp", "rows"):
        assert torch.equal(a[k], b[k]), k
    assert [r["kernel"] for r in recs] == ["decode_tail"]
    seqs, logp, rows = (b[k].cpu().numpy() for k in ("seqs", "logp", "rows"))
    assert np.array_equal(seqs, ref["seqs"]) and np.array_equal(rows, ref["rows"])
    ok, err = logp_ok(logp, ref["logp"], dtype)
    assert ok.all(), err.max()


def test_fusion_switch_and_traced_decode_unfused():
    w = workload("tiny")
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    assert plan.get_decode_fusion() is True
    set_paths(plan, cfg.L, "all_sparse")
    q = torch.from_numpy(w["dense"]["q"]).to(DEV)
    P = torch.from_numpy(w["dense"]["P"]).to(DEV)
    plan.profile_start(capacity=1024)
    tr = plan.decode(q, P, w["W"], trace=True)  # traced: one launch per step
    recs = plan.profile_stop()
    assert "decode_tail" not in {r["kernel"] for r in recs}
    b = plan.decode(q, P, w["W"])
    torch.cuda.synchronize()
    for k in ("seqs", "logp", "rows"):
        assert torch.equal(tr[k], b[k]), k


def test_tune_chooses_the_faster_decode_form():
    w = workload("small")
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    q = torch.from_numpy(w["dense"]["q"]).to(DEV)
    P = torch.from_numpy(w["dense"]["P"]).to(DEV)
    assert plan.tune_decode_times() == (-1.0, -1.0)
    plan.tune(q, P, w["W"], reps=3)
    stepwise, persistent = plan.tune_decode_times()
    assert stepwise > 0 and persistent > 0
    assert plan.get_decode_fusion() == (persistent <= stepwise)
    plan.set_decode_fusion(True)
    assert plan.get_decode_fusion() is True
    plan.set_decode_fusion(False)
    assert plan.get_decode_fusion() is False
    plan.set_decode_fusion("auto")
    assert plan.get_decode_fusion() == (persistent <= stepwise)
