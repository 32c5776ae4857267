"""Brute-force enumeration for tiny catalogs (TEST INFRASTRUCTURE ONLY).

Independent of the trie: valid next tokens come from scanning the whole
catalog, and the score of an item is built along its own path.  When the beam
is at least as wide as the catalog, beam search never prunes, so after L steps
its beams must be exactly the catalog items, each with the score computed here
(ZeroGR summary, "The pipeline": log-softmax over the valid tokens only, added
to the accumulated log-probability).

Pure Python loops, float64 (Python floats) inside; float32 rounding at the same
points the decode defines (logp, accumulated score, state vector, hidden
vector), done with numpy scalars.
"""

import math

import numpy as np


def valid_tokens(items, prefix):
    """Tokens v such that some item starts with prefix + (v,), ascending."""
    t = len(prefix)
    return sorted({it[t] for it in items if tuple(it[:t]) == tuple(prefix)})


def _f32(x):
    return float(np.float32(x))


def _bf16(x):
    b = np.array([x], dtype=np.float32).view(np.uint32)[0]
    b = (int(b) + 0x7FFF + ((int(b) >> 16) & 1)) & 0xFFFF0000
    return float(np.array([b], dtype=np.uint32).view(np.float32)[0])


def _hidden(s, bf16):
    nrm = math.sqrt(sum(float(v) * float(v) for v in s))
    h = [_f32(float(v) / nrm) for v in s]
    return [_bf16(v) for v in h] if bf16 else h


def item_scores(items, q, P, W, bf16, support="valid"):
    """Accumulated score of every item of the catalog along its own path.

    items: list of tuples (distinct); q [d]; P [L-1][V][d]; W [L][V][d].
    support: the tokens the softmax denominator covers, "valid" (the tokens
    that continue the prefix in the catalog) or "all" (the whole codebook:
    score first, or no constraint).
    Returns a list of float32-valued floats, one per item."""
    items = [tuple(int(x) for x in it) for it in items]
    L = len(items[0])
    V = len(W[0])
    out = []
    for it in items:
        s = [float(v) for v in q]
        acc = 0.0
        for t in range(L):
            h = _hidden(s, bf16)
            valid = valid_tokens(items, it[:t]) if support == "valid" else list(range(V))
            z = {v: sum(h[i] * float(W[t][v][i]) for i in range(len(h))) for v in valid}
            m = max(z.values())
            lse = m + math.log(sum(math.exp(z[v] - m) for v in valid))
            logp = _f32(z[it[t]] - lse)
            acc = _f32(acc + logp)
            if t + 1 < L:
                s = [_f32(s[i] + float(P[t][it[t]][i])) for i in range(len(s))]
        out.append(acc)
    return out
