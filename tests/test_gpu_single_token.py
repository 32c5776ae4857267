"""GPU parity of the per-query sparse step's two branches and its workgroup
sizes, against the oracle, through the C ABI.

Identity branch: every live row of a query has one valid token, the live
slots come first and their accumulated log-probs do not increase; slot i of
the output is then beam i (log-softmax over one token is exactly 0, and the
(score desc, parent asc) order of the candidates is the slot order).  The
general branch takes the same rows with the slots permuted (log-probs out of
order, a dead slot between live ones) or with one multi-token row in the
query.  Both must equal the oracle's step on the same inputs, at every
workgroup size (256, 512, 1024 threads), bit for bit across sizes.
"""

import numpy as np
import pytest

import oracle
from tests.parity import compare_step

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402
from tests.test_gpu_parity import DEV, gpu_step  # noqa: E402


def catalog(multi):
    """L = 4, V = 64: 8 level-1 tokens, 3 children each at level 2, then one
    child per prefix at levels 3 and 4 (single-token rows at steps 2 and 3);
    with ``multi`` one level-3 prefix gets a second child."""
    rng = np.random.default_rng(4)
    items = []
    for a in range(8):
        for b in rng.choice(64, size=3, replace=False):
            c = int(rng.integers(64))
            items.append((a, int(b), c, int(rng.integers(64))))
    if multi:
        a, b, c, _ = items[5]
        items.append((a, b, c, (items[5][3] + 7) % 64))
    return np.unique(np.array(items, np.int32), axis=0)


def _device_inputs(h, rows, acc, dtype):
    hd = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(DEV)
    if dtype == "bf16":
        hd = hd.to(torch.bfloat16)
    return hd, torch.from_numpy(rows.astype(np.int32)).to(DEV), torch.from_numpy(np.ascontiguousarray(acc)).to(DEV)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("order", ["sorted", "permuted", "dead_between"])
def test_single_token_steps(dtype, multi, order):
    items = catalog(multi)
    V, L, d, K, Q = 64, 4, 256, 8, 4
    rng = np.random.default_rng(9)
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((L - 1, V, d)) / np.sqrt(d)).astype(np.float32)
    W = (rng.standard_normal((L, V, d)) / np.sqrt(d)).astype(np.float32)
    Wd = torch.from_numpy(W).to(DEV)
    if dtype == "bf16":
        Wd = Wd.bfloat16()
        W = Wd.float().cpu().numpy()
    T = oracle.Trie(items, V)
    ref = T.decode(K, q, P, W, bf16=dtype == "bf16", trace=True)
    idx = cb.Index(items, V, device=0)
    plan = idx.plan(Q, K, d, dtype)
    for t in (2, 3):
        h = ref["trace_h"][t].copy()
        rows = ref["trace_rows_in"][t].copy()
        acc = ref["trace_acc_in"][t].copy()
        if order != "sorted":
            # permute the slots within each query (all arrays alike); the
            # dead_between case also kills one live slot in the middle
            for qq in range(Q):
                sl = slice(qq * K, (qq + 1) * K)
                perm = rng.permutation(K) if order == "permuted" else np.arange(K)
                h[sl], rows[sl], acc[sl] = h[sl][perm], rows[sl][perm], acc[sl][perm]
                if order == "dead_between":
                    rows[qq * K + 1], acc[qq * K + 1] = -1, -np.inf
        o = T.step(t, K, h, W[t], rows, acc, candidates=True)
        outs = []
        for nt in (256, 512, 1024):
            print("case", dtype, "multi", multi, order, "step", t, "threads", nt, flush=True)
            plan.set_path(t, "sparse")
            plan.set_select(t, "lds")
            plan.set_step_threads(t, nt)
            hd, rd, ad = _device_inputs(h, rows, acc, dtype)
            g = gpu_step(plan, t, hd, Wd[t], rd, ad)
            ex, gap, fails = compare_step(o, g, K, dtype)
            assert not fails, "\n".join(fails[:10])
            outs.append(g)
        for g in outs[1:]:
            for k in ("tokens", "parents", "rows", "logp"):
                assert np.array_equal(g[k], outs[0][k]), "workgroup sizes disagree on " + k


@pytest.mark.parametrize("K", [8, 32])
def test_workgroup_sizes_agree_on_every_phase(K):
    """Rows of every scoring phase (1, 2-4, 5-64, > 64 tokens): the three
    workgroup sizes, and two and four workgroups per query, give identical
    bits, and the oracle's results."""
    from tests.test_gpu_widths import catalog as wide_catalog
    items, V = wide_catalog(11)
    L, Q, d = 3, 6, 1024
    rng = np.random.default_rng(2)
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((L - 1, V, d)) / np.sqrt(d)).astype(np.float32)
    Wd = (torch.from_numpy(rng.standard_normal((L, V, d)).astype(np.float32)) / d ** 0.5).to(DEV).bfloat16()
    W = Wd.float().cpu().numpy()
    T = oracle.Trie(items, V)
    ref = T.decode(K, q, P, W, bf16=True, trace=True, threads=8)
    idx = cb.Index(items, V, device=0)
    plan = idx.plan(Q, K, d, "bf16")
    for t in range(L):
        h, rows, acc = ref["trace_h"][t], ref["trace_rows_in"][t], ref["trace_acc_in"][t]
        o = T.step(t, K, h, W[t], rows, acc, candidates=True, threads=8)
        outs = []
        for nt, qs in ((256, 1), (512, 1), (1024, 1), (1024, 2), (256, 4), (1024, 4)):
            print("case K", K, "step", t, "threads", nt, "workgroups per query", qs, flush=True)
            plan.set_path(t, "sparse")
            plan.set_select(t, "lds")
            plan.set_step_threads(t, nt)
            plan.set_option(t, "query_split", qs)
            hd, rd, ad = _device_inputs(h, rows, acc, "bf16")
            for rep in range(2):  # the arrival counts are left at zero for the next launch
                g = gpu_step(plan, t, hd, Wd[t], rd, ad)
                ex, gap, fails = compare_step(o, g, K, "bf16")
                assert not fails, "\n".join(fails[:10])
            outs.append(g)
        for g in outs[1:]:
            for k in ("tokens", "parents", "rows", "logp"):
                assert np.array_equal(g[k], outs[0][k]), "workgroup sizes disagree on " + k


def wide_catalog(multi):
    """64 level-1 tokens with 4 children each (256 rows at step 2), then one
    child per prefix at levels 3 and 4; with ``multi`` one level-3 prefix gets
    a second child."""
    rng = np.random.default_rng(6)
    items = []
    for a in range(64):
        for b in rng.choice(64, size=4, replace=False):
            items.append((a, int(b), int(rng.integers(64)), int(rng.integers(64))))
    if multi:
        a, b, c, x = items[11]
        items.append((a, b, c, (x + 5) % 64))
    return np.unique(np.array(items, np.int32), axis=0)


@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("order", ["sorted", "permuted", "dead_between"])
def test_single_token_steps_wide_beam(multi, order):
    """Beam width 100 (radix selection): the one-token pre-pass finishes the
    query in place (sorted), by a sort of its keys (permuted, dead slot
    between live ones), or leaves it to the radix kernels (a two-token row)."""
    items = wide_catalog(multi)
    V, L, d, K, Q = 64, 4, 256, 100, 2
    rng = np.random.default_rng(12)
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((L - 1, V, d)) / np.sqrt(d)).astype(np.float32)
    Wd = (torch.from_numpy((rng.standard_normal((L, V, d)) / np.sqrt(d)).astype(np.float32))).to(DEV).bfloat16()
    W = Wd.float().cpu().numpy()
    T = oracle.Trie(items, V)
    ref = T.decode(K, q, P, W, bf16=True, trace=True)
    idx = cb.Index(items, V, device=0)
    plan = idx.plan(Q, K, d, "bf16")
    for t in (2, 3):
        h = ref["trace_h"][t].copy()
        rows = ref["trace_rows_in"][t].copy()
        acc = ref["trace_acc_in"][t].copy()
        if order != "sorted":
            for qq in range(Q):
                sl = slice(qq * K, (qq + 1) * K)
                perm = rng.permutation(K) if order == "permuted" else np.arange(K)
                h[sl], rows[sl], acc[sl] = h[sl][perm], rows[sl][perm], acc[sl][perm]
                if order == "dead_between":
                    rows[qq * K + 3], acc[qq * K + 3] = -1, -np.inf
        print("case wide beam multi", multi, order, "step", t, plan.get_select(t), flush=True)
        assert plan.get_select(t) == "radix"
        o = T.step(t, K, h, W[t], rows, acc, candidates=True)
        plan.set_path(t, "sparse")
        hd, rd, ad = _device_inputs(h, rows, acc, "bf16")
        g = gpu_step(plan, t, hd, Wd[t], rd, ad)
        ex, gap, fails = compare_step(o, g, K, "bf16")
        assert not fails, "\n".join(fails[:10])
