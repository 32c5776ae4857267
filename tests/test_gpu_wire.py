"""GPU: wire-format records of a decode's results (cb_wire_results;
FlashTrie App. D.3, "Output serialization"), byte for byte against the
oracle's writer: on the oracle's own decode where the GPU decode equals it,
on the GPU decode's outputs otherwise, at beam widths up to 1024 and with
dead slots anywhere."""

import numpy as np
import pytest

import oracle
from synth import get_config, make_catalog, make_dense
from tests.parity import tolerance

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402

DEV = torch.device("cuda:0")


def records_of(out, nbytes):
    out, nbytes = out.cpu().numpy(), nbytes.cpu().numpy()
    return [out[q, :nbytes[q]].tobytes() for q in range(out.shape[0])]


def gpu_decode(cfg, K=None):
    K = K or cfg.K
    items, dense = make_catalog(cfg), make_dense(cfg)
    idx = cb.Index(items, cfg.V, device=0)
    plan = idx.plan(cfg.Q, K, cfg.d, cfg.dtype)
    W = torch.from_numpy(dense["W_bits"].view(np.int16)).to(DEV).view(torch.bfloat16) if cfg.dtype == "bf16" \
        else torch.from_numpy(dense["W"]).to(DEV)
    out = plan.decode(torch.from_numpy(dense["q"]).to(DEV), torch.from_numpy(dense["P"]).to(DEV), W)
    torch.cuda.synchronize()
    return items, dense, out


@pytest.mark.parametrize("alpha", [0.0, 0.6, 1.0])
def test_wire_tiny_equals_oracle_decode(alpha):
    cfg = get_config("tiny")
    items, dense, out = gpu_decode(cfg)
    print("case tiny alpha", alpha, flush=True)
    T = oracle.Trie(items, cfg.V)
    ref = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=cfg.dtype == "bf16")
    assert np.array_equal(out["seqs"].cpu().numpy(), ref["seqs"])  # the tiny decode is exact
    w, nb = cb.wire_results(out["seqs"], out["logp"], cfg.K, alpha)
    got = records_of(w, nb)
    # byte for byte against the oracle's writer on the same results
    assert got == oracle.wire_records(out["seqs"].cpu().numpy(), out["logp"].cpu().numpy(), cfg.K, alpha)
    # and against the oracle's own decode: the same sequences and offsets, the
    # log-probs within the step tolerance (float32 sums of the two decodes)
    want = oracle.wire_records(ref["seqs"], ref["logp"].astype(np.float32), cfg.K, alpha)
    for g, r in zip(got, want):
        assert len(g) == len(r)
        lg, sg = oracle.wire_parse(g)
        lr, sr = oracle.wire_parse(r)
        assert sg == sr
        # a sum of L step log-probs, each within the step tolerance
        rel, _ = tolerance(cfg.dtype)
        for a, b in zip(lg, lr):
            assert abs(a - b) <= cfg.L * rel * max(1.0, abs(b)), (a, b)


@pytest.mark.parametrize("K", [8, 100, 1000])
def test_wire_small_decode(K):
    """The GPU decode's own outputs (radix selection above K = 64; the small
    catalog leaves dead slots at K = 1000)."""
    # at K = 1000 a catalog of 600 items leaves dead slots in every query
    cfg = get_config("small", Q=4, **({"n_items": 600} if K == 1000 else {}))
    items, dense, out = gpu_decode(cfg, K)
    print("case small K", K, flush=True)
    w, nb = cb.wire_results(out["seqs"], out["logp"], K, 0.6)
    got = records_of(w, nb)
    seqs, logp = out["seqs"].cpu().numpy(), out["logp"].cpu().numpy()
    assert got == oracle.wire_records(seqs, logp, K, 0.6)
    n_live = [int(np.isfinite(logp[q * K:(q + 1) * K]).sum()) for q in range(cfg.Q)]
    assert [oracle.wire_parse(g)[1].__len__() for g in got] == n_live
    if K == 1000:
        assert min(n_live) < K


@pytest.mark.parametrize("K", [1, 33, 1024])
def test_wire_dead_slots_anywhere(K):
    """Synthetic results with dead slots between live ones and a query with
    none live; the record stride above the minimum."""
    rng = np.random.default_rng(K)
    Q, L = 5, 6
    seqs = rng.integers(0, 1 << 20, size=(Q * K, L)).astype(np.int32)
    logp = (-rng.random(Q * K) * 10).astype(np.float32)
    logp[rng.random(Q * K) < 0.3] = -np.inf
    logp[2 * K:3 * K] = -np.inf
    seqs[~np.isfinite(logp)] = -1
    stride = cb.wire_bytes(K, L) + 24
    w, nb = cb.wire_results(torch.from_numpy(seqs).to(DEV), torch.from_numpy(logp).to(DEV), K, 1.0, stride=stride)
    got = records_of(w, nb)
    assert got == oracle.wire_records(seqs, logp, K, 1.0)
    assert len(got[2]) == 8


def test_wire_argument_errors():
    seqs = torch.zeros((8, 3), dtype=torch.int32, device=DEV)
    logp = torch.zeros(8, dtype=torch.float32, device=DEV)
    with pytest.raises(cb.CbError):
        cb.wire_results(seqs, logp, 4, stride=cb.wire_bytes(4, 3) - 8)
    with pytest.raises(cb.CbError):
        cb.wire_results(seqs, logp, 4, alpha=float("nan"))
