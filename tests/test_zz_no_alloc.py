"""GPU: the allocation-free step (cb_step_noalloc, workspace in a static
device array) against cb_step on a plan (its own workspace), through the C ABI.

Both run the same kernels on the same inputs, so the outputs must be equal
bit for bit.  Every case makes two calls in a row on the static array, the
second with fewer queries, so that what the first call left in the array
cannot leak into the second.  A step whose workspace exceeds the array is
refused before any launch.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402
from csr_constrained_beam_amd import _lib as C  # noqa: E402
from tests.test_gpu_parity import DEV, to_dev_h, workload  # noqa: E402

NAMES = ("tokens", "parents", "rows", "logp")


def _inputs(w, t, R):
    ref, cfg = w["ref"], w["cfg"]
    h = to_dev_h(ref["trace_h"][t][:R], cfg)
    rows = torch.from_numpy(ref["trace_rows_in"][t][:R].astype(np.int32)).to(DEV)
    acc = torch.from_numpy(np.ascontiguousarray(ref["trace_acc_in"][t][:R])).to(DEV)
    return h, rows, acc


def _same(a, b, what):
    for n, x, y in zip(NAMES, a, b):
        assert torch.equal(x, y), "%s: %s differs between cb_step_noalloc and cb_step" % (what, n)


@pytest.mark.parametrize("name", ["tiny", "small"])
@pytest.mark.parametrize("path", ["dense", "sparse", "auto"])
def test_noalloc_matches_plan_step(name, path):
    w = workload(name)
    cfg = w["cfg"]
    idx = cb.Index(w["items"], cfg.V, device=0)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    for t in range(cfg.L):
        plan.set_path(t, path)
        plan.set_select(t, "lds")
    for t in range(cfg.L):
        # two calls in a row: all queries, then the first half of them
        for Qc in (cfg.Q, max(1, cfg.Q // 2)):
            print("case", name, path, "step", t, "Q", Qc, flush=True)
            R = Qc * cfg.K
            h, rows, acc = _inputs(w, t, R)
            a = idx.step_noalloc(t, cfg.K, h, w["W"][t], rows, acc, path=path)
            b = plan.step(t, h, w["W"][t], rows, acc)
            torch.cuda.synchronize()
            _same(a, b, "%s step %d Q %d" % (name, t, Qc))


def test_noalloc_wide_hidden_sparse_route():
    """d = 4096: the sparse step is a per-beam expansion + merge whose
    candidate keys lie in the static array."""
    rng = np.random.default_rng(3)
    V, d, K, Q, L = 300, 4096, 16, 5, 3
    items = np.unique(rng.integers(0, 40, size=(3000, L)).astype(np.int32) * 7 % V, axis=0)
    idx = cb.Index(items, V, device=0)
    plan = idx.plan(Q, K, d, "bf16")
    W = (torch.randn((L, V, d), generator=torch.Generator().manual_seed(1)) / d ** 0.5).to(DEV).bfloat16()
    q = torch.randn((Q, d), generator=torch.Generator().manual_seed(2)).to(DEV)
    P = (torch.randn((L - 1, V, d), generator=torch.Generator().manual_seed(4)) / d ** 0.5).to(DEV)
    for t in range(L):
        plan.set_path(t, "sparse")
    rec = plan.decode(q, P, W, trace=True)
    torch.cuda.synchronize()
    for t in range(L):
        for Qc in (Q, 2):
            print("case wide step", t, "Q", Qc, flush=True)
            R = Qc * K
            h, rows, acc = rec["trace_h"][t][:R], rec["trace_rows"][t][:R], rec["trace_acc"][t][:R]
            a = idx.step_noalloc(t, K, h, W[t], rows, acc, path="sparse")
            b = plan.step(t, h, W[t], rows, acc)
            torch.cuda.synchronize()
            _same(a, b, "wide step %d Q %d" % (t, Qc))


def test_noalloc_refuses_workspace_beyond_the_array():
    # 4096 beams x 4096 tokens of float32 scores (64 MiB) > the 32 MiB array
    rng = np.random.default_rng(7)
    V, d, K, Q = 4096, 64, 64, 64
    items = rng.integers(0, V, size=(20000, 2)).astype(np.int32)
    idx = cb.Index(items, V, device=0, store="bitmap")
    R = Q * K
    h = torch.zeros((R, d), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((V, d), dtype=torch.bfloat16, device=DEV)
    rows = torch.full((R,), -1, dtype=torch.int32, device=DEV)
    acc = torch.full((R,), float("-inf"), dtype=torch.float32, device=DEV)
    with pytest.raises(C.CbError) as e:
        idx.step_noalloc(0, K, h, W, rows, acc, path="dense")
    assert e.value.status == C.CB_ECAPACITY
    assert "workspace" in str(e.value)
