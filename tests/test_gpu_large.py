"""GPU parity on the full large-library workload: 100M variable-length items
(lengths 4 to 12, EOS padded to 12 steps), V = 32,001, d = 1024 bf16, one
query, beam widths 1000 (the workload's) and 100 / 250 / 500 (its sweep).

The sorted-range oracle decodes the same query on the host (a pointer trie of
this catalog does not fit the host's memory).  The beam width is the whole
output, so every output is compared: the free-running decode with the tuned
per-step paths, and every step teacher forced on the oracle's beam state.
Building the inputs takes minutes of host time; progress is printed.
"""

import time

import numpy as np
import pytest

import oracle
from synth import get_config, make_catalog, make_dense
from tests.parity import compare_step

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402
from tests.test_gpu_radix import DEV, check_decode, dev_h  # noqa: E402

_W = {}


def large():
    if _W:
        return _W
    cfg = get_config("large")
    t0 = time.time()
    print("drawing 100M items", flush=True)
    items = make_catalog(cfg)
    print("catalog %.0f s; drawing W, P" % (time.time() - t0), flush=True)
    dense = make_dense(cfg)
    print("building the device index", flush=True)
    idx = cb.Index(items, cfg.V, device=0)
    print("index %.0f s; building the sorted-range oracle" % (time.time() - t0), flush=True)
    S = oracle.SortedRange(items, cfg.V)
    print("oracle %.0f s" % (time.time() - t0), flush=True)
    W = torch.from_numpy(dense["W_bits"].view(np.int16)).to(DEV).view(torch.bfloat16)
    q = torch.from_numpy(dense["q"]).to(DEV)
    P = torch.from_numpy(dense["P"]).to(DEV)
    _W.update(cfg=cfg, items=items, dense=dense, idx=idx, T=S, W=W, q=q, P=P, refs={})
    return _W


def ref_for(w, K):
    if K not in w["refs"]:
        d = w["dense"]
        t0 = time.time()
        w["refs"][K] = w["T"].decode(K, d["q"], d["P"], d["W"], bf16=True, trace=True, threads=16)
        print("oracle decode K=%d: %.1f s" % (K, time.time() - t0), flush=True)
    return w["refs"][K]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("K", [1000, 100, 250, 500])
def test_large_decode_full_size(K):
    w = large()
    cfg = w["cfg"]
    ref = ref_for(w, K)
    plan = w["idx"].plan(cfg.Q, K, cfg.d, cfg.dtype)
    plan.tune(w["q"], w["P"], w["W"], reps=2)
    print("K", K, "paths", [plan.get_path(t) for t in range(cfg.L)], flush=True)
    out = plan.decode(w["q"], w["P"], w["W"], trace=True)
    torch.cuda.synchronize()
    view = dict(cfg=get_config("large", K=K), items=w["items"], dense=w["dense"], T=w["T"], ref=ref, W=w["W"])
    check_decode(view, out, K, plan)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("path", ["sparse", "dense", "sparse_tm"])
def test_large_teacher_forced_full_size(path):
    """Every step at full size on the oracle's beam state; sparse_tm: the
    sparse scores grouped by token."""
    w = large()
    cfg = w["cfg"]
    K = cfg.K
    ref = ref_for(w, K)
    plan = w["idx"].plan(cfg.Q, K, cfg.d, cfg.dtype)
    for t in range(cfg.L):
        plan.set_path(t, "sparse" if path == "sparse_tm" else path)
        if path == "sparse_tm":
            plan.set_option(t, "token_major", 2)
        h, rows, acc = ref["trace_h"][t], ref["trace_rows_in"][t], ref["trace_acc_in"][t]
        o = w["T"].step(t, K, h, w["dense"]["W"][t], rows, acc, candidates=True, threads=16)
        got = plan.step(t, dev_h(h, cfg.dtype), w["W"][t], torch.from_numpy(rows.astype(np.int32)).to(DEV),
                        torch.from_numpy(acc).to(DEV))
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in zip(("tokens", "parents", "rows", "logp"), got)}
        ex, gap, fails = compare_step(o, g, K, cfg.dtype)
        print("step", t, path, "candidates", int(o["cand_count"][0]), "near-tie exemptions", ex, flush=True)
        assert not fails, "step %d:\n" % t + "\n".join(fails[:10])
