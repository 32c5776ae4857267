"""GPU parity at the shapes of the scaling sweeps that take other kernel
branches than the five workloads: a 32,768-token codebook (the root and
wide steps go to the radix selection, the dense expansion to the per-beam
gather), 256 queries (8,192 beam slots: the live-beam list of the dense
path is built apart), and the branch-factor catalogs at B = 8 and B = 512
(rows of 512 tokens on the block-per-row phase).  Item counts are reduced so
that the oracle finishes in seconds.

Per shape: the tuned plan's free-running decode against the oracle's
(identical, or diverging only at near ties), and every step teacher forced
on the tuned, dense and sparse paths against the oracle's candidates, all
queries compared.
"""

import numpy as np
import pytest

import oracle
from synth import get_config, make_catalog, make_dense
from tests.parity import compare_step, decode_vs_oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402

DEV = torch.device("cuda:0")

SHAPES = {
    "codebook_32768": ("production", dict(n_items=300_000, V=32_768, Q=32)),
    "batch_256": ("production", dict(n_items=1_000_000, Q=256)),
    "branch_8": ("branch", dict(params={"B": 8}, Q=16)),
    "branch_512": ("branch", dict(params={"B": 512}, Q=16)),
}
_CACHE = {}


def shape(key):
    if key in _CACHE:
        return _CACHE[key]
    _CACHE.clear()
    name, over = SHAPES[key]
    cfg = get_config(name, **over)
    print("building", key, flush=True)
    items = make_catalog(cfg)
    dense = make_dense(cfg)
    T = oracle.Trie(items, cfg.V)
    ref = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=True, trace=True, threads=16)
    idx = cb.Index(items, cfg.V, device=0)
    W = torch.from_numpy(dense["W_bits"].view(np.int16)).to(DEV).view(torch.bfloat16)
    q = torch.from_numpy(dense["q"]).to(DEV)
    P = torch.from_numpy(dense["P"]).to(DEV)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    plan.tune(q, P, W, reps=2)
    _CACHE[key] = dict(cfg=cfg, items=items, dense=dense, T=T, ref=ref, idx=idx, plan=plan, W=W, q=q, P=P)
    return _CACHE[key]


@pytest.mark.parametrize("key", sorted(SHAPES))
def test_sweep_shape_decode(key):
    w = shape(key)
    cfg, plan = w["cfg"], w["plan"]
    print(key, "paths", [plan.get_path(t) + "/" + plan.get_select(t) for t in range(cfg.L)], flush=True)
    out = plan.decode(w["q"], w["P"], w["W"], trace=True)
    torch.cuda.synchronize()
    rec = {k: out[k].cpu().numpy() for k in ("trace_rows", "rows", "seqs")}
    vs = decode_vs_oracle(w["T"], w["ref"], rec, w["dense"]["W"], cfg.L, cfg.K, cfg.Q)
    print(key, "decode vs oracle:", vs, flush=True)
    assert not vs["unexplained"], vs


@pytest.mark.parametrize("key", sorted(SHAPES))
@pytest.mark.parametrize("path", ["tuned", "dense", "sparse"])
def test_sweep_shape_teacher_forced(key, path):
    w = shape(key)
    cfg, ref, plan, T = w["cfg"], w["ref"], w["plan"], w["T"]
    K = cfg.K
    try:
        for t in range(cfg.L):
            if path != "tuned":
                plan.set_path(t, path)
            print(key, path, "step", t, plan.get_path(t), plan.get_select(t), flush=True)
            h, rows, acc = ref["trace_h"][t], ref["trace_rows_in"][t], ref["trace_acc_in"][t]
            gt = plan.step(t, torch.from_numpy(h).to(DEV).bfloat16(), w["W"][t],
                           torch.from_numpy(rows.astype(np.int32)).to(DEV), torch.from_numpy(acc).to(DEV))
            torch.cuda.synchronize()
            g = {k: v.cpu().numpy() for k, v in zip(("tokens", "parents", "rows", "logp"), gt)}
            o = T.step(t, K, h, w["dense"]["W"][t], rows, acc, candidates=True, threads=16)
            ex, gap, fails = compare_step(o, g, K, cfg.dtype)
            assert not fails, "\n".join(fails[:5])
    finally:
        if path != "tuned":
            for t in range(cfg.L):
                plan.set_path(t, "auto")
