"""GPU parity of a decoding step at hidden widths of two to four 512-element
chunks, float32 and bf16, on the sparse path with both workgroup sizes of the
per-query kernel (512 threads for K < 16, 1024 otherwise) and on the dense
path (the full-codebook product, then the expansion and merge).  Widths above
2048 (beyond what the fused per-query kernel keeps in registers) take the
sparse steps as a per-beam expansion + per-query merge: d = 4096 is checked
on that route, on the dense path and on the radix selection; the same form,
forced at every width, is checked as "sparse_beam".

The catalog is built so that the rows of its steps cover every scoring phase
of the per-query kernel: rows of one token (not scored: log-softmax 0), of
2-4 tokens (one wavefront), of 5-64 tokens (the block-wide task list) and of
more than 64 tokens (the block per row).  Each step is teacher forced from the
oracle's trace and compared with the oracle's candidates; the persistent
decode must equal the step-by-step decode bit for bit.
"""

import numpy as np
import pytest

import oracle
from tests.parity import compare_step, force_beam_form

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402
from tests.test_gpu_parity import DEV, gpu_step  # noqa: E402

# children of the level-1 prefixes: one of each scoring phase and the edges
# between them (4 | 5 and 64 | 65 are the phase boundaries)
FANOUTS = [1, 2, 3, 4, 5, 6, 12, 30, 64, 65, 100, 250]


def catalog(seed):
    rng = np.random.default_rng(seed)
    V = 300
    items = []
    for a, f in enumerate(FANOUTS * 3):
        for b in rng.choice(V, size=f, replace=False):
            for c in rng.choice(V, size=int(rng.integers(1, 6)), replace=False):
                items.append((a, int(b), int(c)))
    return np.unique(np.array(items, np.int32), axis=0), V


def test_catalog_covers_every_phase():
    items, V = catalog(11)
    T = oracle.Trie(items, V)
    fan1 = sorted({len(T.children_of_row(1, r)[0]) for r in range(len(np.unique(items[:, 0])))})
    assert fan1 == sorted(set(FANOUTS))
    assert len(T.children_of_row(0, 0)[0]) == 3 * len(FANOUTS)  # the root row: 36 tokens


@pytest.mark.parametrize("dtype,d", [("f32", 1024), ("f32", 2048), ("bf16", 1536), ("bf16", 2048),
                                     ("f32", 4096), ("bf16", 4096)])
@pytest.mark.parametrize("K", [8, 32])
@pytest.mark.parametrize("path", ["sparse", "dense", "sparse_beam", "sparse_qsplit"])
def test_step_hidden_widths(dtype, d, K, path):
    _run_widths(dtype, d, K, path, "lds")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_wide_hidden_radix(dtype):
    _run_widths(dtype, 4096, 32, "sparse", "radix")


@pytest.mark.parametrize("dtype,d", [("f32", 1024), ("bf16", 2048)])
@pytest.mark.parametrize("K", [8, 32])
@pytest.mark.parametrize("split_rows", [1, 16])
def test_step_split_scoring(dtype, d, K, split_rows):
    """Rows above split_rows tokens scored apart across many workgroups, the
    rest by the per-query kernel, on rows of every scoring phase."""
    _run_widths(dtype, d, K, "sparse_split", "lds", split_rows=split_rows)


@pytest.mark.parametrize("dtype,d", [("f32", 200), ("f32", 1024), ("bf16", 520), ("bf16", 1536), ("bf16", 2048)])
def test_step_token_major_widths(dtype, d):
    """The radix selection's sparse scores grouped by token at hidden widths
    of one to four 512-element chunks, partial chunks included, on rows of
    every scoring phase."""
    _run_widths(dtype, d, 32, "sparse", "radix", token_major=True)


def _run_widths(dtype, d, K, path, select, split_rows=0, token_major=False):
    items, V = catalog(11)
    L, Q = 3, 6
    rng = np.random.default_rng(5)
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((L - 1, V, d)) / np.sqrt(d)).astype(np.float32)
    W = (rng.standard_normal((L, V, d)) / np.sqrt(d)).astype(np.float32)
    Wd = torch.from_numpy(W).to(DEV)
    if dtype == "bf16":
        Wd = Wd.bfloat16()
        W = Wd.float().cpu().numpy()
    bf16 = dtype == "bf16"
    T = oracle.Trie(items, V)
    ref = T.decode(K, q, P, W, bf16=bf16, trace=True, threads=8)
    idx = cb.Index(items, V, device=0)
    plan = idx.plan(Q, K, d, dtype)
    for t in range(L):
        plan.set_path(t, "sparse" if path in ("sparse_beam", "sparse_qsplit") else path)
        plan.set_select(t, select)
        if path == "sparse_beam":  # one workgroup per beam, then the per-query merge
            force_beam_form(plan, t)
        if path == "sparse_qsplit":  # four workgroups per query
            plan.set_option(t, "query_split", 4)
        if split_rows:
            plan.set_split_rows(t, split_rows)
        if token_major:
            plan.set_option(t, "token_major", 2)
    for t in range(L):
        print("case", dtype, d, "K", K, path, "step", t, flush=True)
        h = ref["trace_h"][t]
        rows = ref["trace_rows_in"][t]
        acc = ref["trace_acc_in"][t]
        o = T.step(t, K, h, W[t], rows, acc, candidates=True, threads=8)
        hd = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(DEV)
        if bf16:
            hd = hd.to(torch.bfloat16)
        g = gpu_step(plan, t, hd, Wd[t], torch.from_numpy(rows.astype(np.int32)).to(DEV),
                     torch.from_numpy(acc).to(DEV))
        ex, gap, fails = compare_step(o, g, K, dtype)
        assert not fails, "\n".join(fails[:10])
    # the persistent decode (one launch for every step) against the step-by-step one
    print("case", dtype, d, "K", K, path, select, "decode", flush=True)
    qd, Pd = torch.from_numpy(q).to(DEV), torch.from_numpy(P).to(DEV)
    plan.set_decode_fusion(False)
    a = plan.decode(qd, Pd, Wd)
    plan.set_decode_fusion(True)
    b = plan.decode(qd, Pd, Wd)
    torch.cuda.synchronize()
    for k in ("seqs", "logp", "rows"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_csr_expansion_rows_across_windows(dtype):
    """The dense path on a CSR step expands each beam by one wavefront, 512
    tokens per window: rows of 1 to 1,500 tokens (window boundaries at 512
    and 1,024 on both sides) against the oracle, teacher forced."""
    rng = np.random.default_rng(3)
    V, d, Q, K, L = 2048, 64, 4, 16, 2
    fan = [1, 2, 63, 64, 65, 511, 512, 513, 1024, 1025, 1500]
    items = np.array([(a, int(b)) for a, f in enumerate(fan) for b in rng.choice(V, size=f, replace=False)], np.int32)
    q = rng.standard_normal((Q, d)).astype(np.float32)
    P = (rng.standard_normal((L - 1, V, d)) / np.sqrt(d)).astype(np.float32)
    W = (rng.standard_normal((L, V, d)) / np.sqrt(d)).astype(np.float32)
    Wd = torch.from_numpy(W).to(DEV)
    if dtype == "bf16":
        Wd = Wd.bfloat16()
        W = Wd.float().cpu().numpy()
    T = oracle.Trie(items, V)
    ref = T.decode(K, q, P, W, bf16=dtype == "bf16", trace=True, threads=8)
    idx = cb.Index(items, V, device=0, store="csr")
    plan = idx.plan(Q, K, d, dtype)
    for t in range(L):
        plan.set_path(t, "dense")
        h, rows, acc = ref["trace_h"][t], ref["trace_rows_in"][t], ref["trace_acc_in"][t]
        o = T.step(t, K, h, W[t], rows, acc, candidates=True, threads=8)
        hd = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(DEV)
        if dtype == "bf16":
            hd = hd.to(torch.bfloat16)
        g = gpu_step(plan, t, hd, Wd[t], torch.from_numpy(rows.astype(np.int32)).to(DEV),
                     torch.from_numpy(acc).to(DEV))
        ex, gap, fails = compare_step(o, g, K, dtype)
        assert not fails, "step %d:\n" % t + "\n".join(fails[:10])
    assert sorted(len(T.children_of_row(1, r)[0]) for r in range(len(fan))) == sorted(fan)
