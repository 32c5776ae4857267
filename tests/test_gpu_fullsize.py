"""GPU parity at the full workload sizes, in the benchmark's launch
configuration (all queries of the batch, beam width and hidden width of the
workload, the tuned per-step paths), plus both scoring paths forced.

The oracle builds its own pointer trie of the whole catalog; every query's
outputs are compared.  Teacher forcing: every step gets the oracle's beam
state and hidden vectors.
"""

import numpy as np
import pytest

import oracle
from synth import get_config, make_catalog, make_dense
from tests.parity import compare_step, force_beam_form, logp_ok

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402

DEV = torch.device("cuda:0")
_CACHE = {}


def big(name):
    if name in _CACHE:
        return _CACHE[name]
    _CACHE.clear()  # one full-size workload resident at a time
    cfg = get_config(name)
    print("building", name, flush=True)
    items = make_catalog(cfg)
    dense = make_dense(cfg)
    T = oracle.Trie(items, cfg.V)
    bf16 = cfg.dtype == "bf16"
    ref = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=bf16, trace=True, threads=16)
    idx = cb.Index(items, cfg.V, device=0)
    if bf16:
        W = torch.from_numpy(dense["W_bits"].view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        W = torch.from_numpy(dense["W"]).to(DEV)
    q = torch.from_numpy(dense["q"]).to(DEV)
    P = torch.from_numpy(dense["P"]).to(DEV)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    plan.tune(q, P, W, reps=2)
    _CACHE[name] = dict(cfg=cfg, items=items, dense=dense, T=T, ref=ref, idx=idx, plan=plan, W=W, q=q, P=P)
    return _CACHE[name]


@pytest.mark.parametrize("name", ["production", "hybrid"])
def test_fullsize_decode(name):
    w = big(name)
    cfg, ref, plan = w["cfg"], w["ref"], w["plan"]
    print("paths", [plan.get_path(t) for t in range(cfg.L)], flush=True)
    out = plan.decode(w["q"], w["P"], w["W"], trace=True)
    torch.cuda.synchronize()
    seqs, logp, rows = (out[k].cpu().numpy() for k in ("seqs", "logp", "rows"))
    catalog = {tuple(r) for r in w["items"].tolist()}
    for s_ in seqs[rows >= 0][:2000].tolist():
        assert tuple(s_) in catalog
    K = cfg.K
    tr = out["trace_rows"].cpu().numpy()
    diverged = 0
    for qi in range(cfg.Q):
        sl = slice(qi * K, (qi + 1) * K)
        if np.array_equal(seqs[sl], ref["seqs"][sl]):
            assert np.array_equal(rows[sl], ref["rows"][sl])
            ok, err = logp_ok(logp[sl], ref["logp"][sl], cfg.dtype)
            assert ok.all(), (qi, err.max())
            continue
        diverged += 1
        # the first step where this query's beams differ must be a near tie
        g_rows = [tr[t][sl] for t in range(1, cfg.L)] + [rows[sl]]
        r_rows = [ref["trace_rows_in"][t][sl] for t in range(1, cfg.L)] + [ref["rows"][sl]]
        t0 = next(t for t in range(cfg.L) if not np.array_equal(g_rows[t], r_rows[t]))
        o = w["T"].step(t0, K, ref["trace_h"][t0][sl], w["dense"]["W"][t0], ref["trace_rows_in"][t0][sl],
                        ref["trace_acc_in"][t0][sl], candidates=True)
        hd = torch.from_numpy(np.ascontiguousarray(ref["trace_h"][t0][sl])).to(DEV)
        if cfg.dtype == "bf16":
            hd = hd.bfloat16()
        gt = plan.step(t0, hd, w["W"][t0], torch.from_numpy(ref["trace_rows_in"][t0][sl].astype(np.int32)).to(DEV),
                       torch.from_numpy(ref["trace_acc_in"][t0][sl]).to(DEV))
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in zip(("tokens", "parents", "rows", "logp"), gt)}
        ex, gap, fails = compare_step(o, g, K, cfg.dtype)
        assert not fails, "\n".join(fails[:5])
        assert ex > 0
    print("queries diverging at a near tie:", diverged, "of", cfg.Q)
    # observed on the current kernels: no query diverges on either workload
    assert diverged == 0


@pytest.mark.parametrize("name", ["production", "hybrid"])
@pytest.mark.parametrize("paths", ["tuned", "sparse"])
def test_fullsize_persistent_decode(name, paths):
    """The untraced decode (trailing sparse steps in one persistent launch)
    equals the step-by-step decode bit for bit, on the tuned paths and with
    every step forced sparse."""
    w = big(name)
    cfg = w["cfg"]
    plan = w["plan"] if paths == "tuned" else w["idx"].plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    if paths == "sparse":
        for t in range(cfg.L):
            plan.set_path(t, "sparse")
    plan.set_decode_fusion(False)
    a = plan.decode(w["q"], w["P"], w["W"])
    plan.set_decode_fusion(True)
    plan.profile_start(capacity=1024)
    b = plan.decode(w["q"], w["P"], w["W"])
    recs = plan.profile_stop()
    torch.cuda.synchronize()
    tail = [r["step"] for r in recs if r["kernel"] == "decode_tail"]
    print("paths", [plan.get_path(t) + "/" + plan.get_select(t) for t in range(cfg.L)], "tail from", tail,
          flush=True)
    if paths == "sparse":
        assert len(tail) == 1
    for k in ("seqs", "logp", "rows"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("name", ["production", "hybrid"])
@pytest.mark.parametrize("path", ["tuned", "dense", "sparse", "sparse_split", "sparse_beam", "sparse_qsplit"])
def test_fullsize_teacher_forced(name, path):
    w = big(name)
    cfg, ref, plan, T = w["cfg"], w["ref"], w["plan"], w["T"]
    K = cfg.K
    S = cfg.Q * K
    forms = [plan.get_option(t, "sparse_form") for t in range(cfg.L)]
    splits = [plan.get_option(t, "query_split") for t in range(cfg.L)]
    try:
        for t in range(cfg.L):
            if path == "sparse_beam":
                plan.set_path(t, "sparse")
                print("per-beam form:", force_beam_form(plan, t), flush=True)
            elif path == "sparse_qsplit":
                plan.set_path(t, "sparse")
                plan.set_option(t, "sparse_form", 0)
                plan.set_option(t, "query_split", 4)
            elif path != "tuned":
                plan.set_path(t, path)
                plan.set_option(t, "sparse_form", 0)
                plan.set_option(t, "query_split", 1)
            print(name, path, "step", t, plan.get_path(t), flush=True)
            h = ref["trace_h"][t]
            hd = torch.from_numpy(h).to(DEV)
            if cfg.dtype == "bf16":
                hd = hd.bfloat16()
            rows = ref["trace_rows_in"][t]
            acc = ref["trace_acc_in"][t]
            gt = plan.step(t, hd, w["W"][t], torch.from_numpy(rows.astype(np.int32)).to(DEV),
                           torch.from_numpy(acc).to(DEV))
            torch.cuda.synchronize()
            g = {k: v[:S].cpu().numpy() for k, v in zip(("tokens", "parents", "rows", "logp"), gt)}
            o = T.step(t, K, h[:S], w["dense"]["W"][t], rows[:S], acc[:S], candidates=True, threads=16)
            ex, gap, fails = compare_step(o, g, K, cfg.dtype)
            assert not fails, "\n".join(fails[:5])
    finally:
        for t in range(cfg.L):
            plan.set_path(t, "auto")
            plan.set_option(t, "sparse_form", forms[t])
            plan.set_option(t, "query_split", splits[t])
