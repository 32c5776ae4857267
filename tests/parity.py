"""Comparison of device step outputs with the oracle (test helper).

Tolerances (written here, used by every parity test):

* log-probs, float32 workloads: |gpu - ref| <= 1e-5 * max(1, |ref|).
* log-probs, bf16 workloads: |gpu - ref| <= 2e-2 (the stated bar) and, as a
  tighter check derived from the arithmetic, <= 1e-4 * max(1, |ref|): bf16 x
  bf16 products are exact in float32, so the device's scores differ from the
  double-precision oracle only by float32 summation order (about d * 2^-24 *
  sum |h_i w_i|, < 1e-4 for d <= 1024 and unit-norm h).
* tokens, parents and next rows: identical, except at near ties: where the
  device picked a different candidate than the oracle at some output
  position, the two candidates' oracle scores must lie within
  eps_tie = 1e-5 * max(1, |score|) (float32 reassociation moves a score by a
  few ulps, so candidates that close may legitimately swap).  Every device
  output must still be a valid candidate with the oracle's next row and
  score, and the outputs must be sorted by the tie-break.
"""

import numpy as np


def tolerance(dtype):
    return (1e-5, 0.0) if dtype == "f32" else (1e-4, 2e-2)


def logp_ok(got, ref, dtype):
    rel, absb = tolerance(dtype)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    lim = rel * np.maximum(1.0, np.abs(ref))
    ok = err <= lim
    if absb:
        ok &= err <= absb
    return ok, err


def compare_step(ref, got, K, dtype, eps_rel=1e-5):
    """ref: oracle.Trie.step(..., candidates=True) output; got: dict of numpy
    arrays tokens/parents/rows/logp from the device.  Returns (exemptions,
    max_gap, failures[list of str])."""
    fails = []
    exempt = 0
    max_gap = 0.0
    R = len(ref["tokens"])
    Q = R // K
    for q in range(Q):
        sl = slice(q * K, (q + 1) * K)
        n = int(ref["cand_count"][q])
        cands = {}
        for j in range(n):
            cands[(int(ref["cand_parents"][q, j]), int(ref["cand_tokens"][q, j]))] = (
                float(ref["cand_scores"][q, j]), int(ref["cand_rows"][q, j]))
        nv = min(K, n)
        gt, gp, gr, gl = (got[k][sl] for k in ("tokens", "parents", "rows", "logp"))
        rt, rp = ref["tokens"][sl], ref["parents"][sl]
        # sentinels past the valid count
        if not ((gt[nv:] == -1).all() and (gp[nv:] == -1).all() and (gr[nv:] == -1).all()
                and np.isneginf(gl[nv:]).all()):
            fails.append("query %d: expected %d valid outputs then sentinels" % (q, nv))
            continue
        # every output is a real candidate with the right row and score
        keys = []
        for i in range(nv):
            c = (int(gp[i]), int(gt[i]))
            if c not in cands:
                fails.append("query %d pos %d: (parent %d, token %d) is not a valid candidate" % (q, i, *c))
                continue
            sc, row = cands[c]
            if int(gr[i]) != row:
                fails.append("query %d pos %d: next row %d, oracle %d" % (q, i, int(gr[i]), row))
            ok, err = logp_ok([gl[i]], [sc], dtype)
            if not ok[0]:
                fails.append("query %d pos %d: logp %.9g vs oracle %.9g (err %.3g)" % (q, i, gl[i], sc, err[0]))
            keys.append((-float(gl[i]), c[0], c[1]))
        if keys != sorted(keys) or len(set(keys)) != len(keys):
            fails.append("query %d: outputs not sorted by (score desc, parent asc, token asc)" % q)
        # positions where the pick differs: only near ties are allowed
        for i in range(nv):
            a = (int(gp[i]), int(gt[i]))
            b = (int(rp[i]), int(rt[i]))
            if a == b or a not in cands:
                continue
            sa, sb = cands[a][0], cands[b][0]
            gap = abs(sa - sb)
            max_gap = max(max_gap, gap)
            if gap > eps_rel * max(1.0, abs(sb)):
                fails.append("query %d pos %d: picked %s (oracle score %.9g) where the oracle has %s (%.9g)"
                             % (q, i, a, sa, b, sb))
            else:
                exempt += 1
        # the selected sets may differ only at the boundary, within the tie window
        gs = {(int(p), int(t)) for p, t in zip(gp[:nv], gt[:nv])}
        rs = {(int(p), int(t)) for p, t in zip(rp[:nv], rt[:nv])}
        if gs != rs and nv:
            kth = float(ref["cand_scores"][q, nv - 1])
            for c in gs ^ rs:
                if c in cands and abs(cands[c][0] - kth) > eps_rel * max(1.0, abs(kth)):
                    fails.append("query %d: candidate %s (%.9g) differs from the oracle's selection away from "
                                 "the boundary %.9g" % (q, c, cands[c][0], kth))
    return exempt, max_gap, fails


def decode_vs_oracle(T, r0, rec, W, L, K, Q, mode=None):
    """A free-running device decode against the oracle's.  Per query:
    identical item rows and sequences, or the first step where the device's
    outputs differ is checked on the oracle's candidates of that step (same
    inputs on both sides up to it): every position where the picks differ
    must be between candidates whose oracle scores lie within
    1e-5 * max(1, |score|).  T: the oracle; r0: its decode with trace=True;
    rec: the device decode's trace_rows [L][Q*K], rows and seqs (numpy);
    W: [L][V][d] float32; mode: the oracle's decoding variant (None: filter
    first)."""
    g_rows = [np.asarray(rec["trace_rows"][t]) for t in range(1, L)] + [np.asarray(rec["rows"])]
    r_rows = [r0["trace_rows_in"][t] for t in range(1, L)] + [r0["rows"]]
    g_seqs = np.asarray(rec["seqs"])
    identical, tie, bad, max_gap = 0, 0, [], 0.0
    cand = {}
    for q in range(Q):
        sl = slice(q * K, (q + 1) * K)
        first = next((t for t in range(L) if not np.array_equal(g_rows[t][sl], r_rows[t][sl])), None)
        if first is None and np.array_equal(g_seqs[sl], r0["seqs"][sl]):
            identical += 1
            continue
        if first is None:
            bad.append(q)
            continue
        if first not in cand:
            mkw = {"mode": mode} if mode else {}
            cand[first] = T.step(first, K, r0["trace_h"][first], W[first], r0["trace_rows_in"][first],
                                 r0["trace_acc_in"][first], candidates=True, threads=8, **mkw)
        o = cand[first]
        score = {int(o["cand_rows"][q, j]): float(o["cand_scores"][q, j]) for j in range(int(o["cand_count"][q]))}
        ok = True
        for i in range(K):
            a, b = int(g_rows[first][q * K + i]), int(r_rows[first][q * K + i])
            if a == b:
                continue
            if a not in score or b not in score:
                ok = False
                break
            gap = abs(score[a] - score[b])
            max_gap = max(max_gap, gap)
            if gap > 1e-5 * max(1.0, abs(score[b])):
                ok = False
                break
        if ok:
            tie += 1
        else:
            bad.append(q)
    return {"queries": Q, "identical": identical, "near_tie_divergences": tie, "unexplained": bad,
            "max_tie_gap": max_gap}


def force_beam_form(plan, t):
    """Put the sparse path of step t in its per-beam form (one workgroup per
    beam, then the per-query merge); False when the step's widest row does
    not fit that form's LDS (the step then keeps the per-query kernel)."""
    import csr_constrained_beam_amd as cb
    try:
        plan.set_option(t, "sparse_form", 1)
        return True
    except cb.CbError as e:
        if e.status != -5:  # CB_ECAPACITY
            raise
        return False
