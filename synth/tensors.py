"""Seeded dense tensors of a workload.

* q   [Q][d]        ~ N(0, 1): one query vector per query.
* P   [L-1][V][d]   ~ N(0, 1/d): per-step token embeddings of the stand-in
                     model (the hidden vector after step t adds P_t[token]).
* W   [L][V][d]     ~ N(0, 1/d): per-step output layers.

For bf16 workloads W is rounded to bf16 (round to nearest, ties to even)
here, once, as part of drawing the input; both consumers then read the same
bf16 values (``W_bits`` as raw bf16 bit patterns, ``W`` as the exactly equal
float32 values).
"""

import numpy as np


def bf16_round_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even.
    (Inputs here are finite.)"""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u.astype(np.uint64) + np.uint64(0x7FFF) + lsb.astype(np.uint64)) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(seed_words, shape, scale):
    rng = np.random.default_rng(seed_words)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def make_dense(cfg, Q=None, steps=None):
    """Draw q, P and W for ``cfg``.

    Returns a dict with ``q`` (float32 [Q][d]), ``P`` (float32 [L-1][V][d]),
    ``W`` (float32 [L][V][d], bf16-representable values for bf16 workloads)
    and, for bf16 workloads, ``W_bits`` (uint16 [L][V][d]).  ``steps``
    restricts W and P to the first ``steps`` decoding steps.
    """
    Q = cfg.Q if Q is None else int(Q)
    L = cfg.L if steps is None else int(steps)
    d, V, s = cfg.d, cfg.V, cfg.seed
    sc = 1.0 / np.sqrt(d)
    q = _normal([s, 10], (Q, d), 1.0)
    P = np.empty((max(L - 1, 0), V, d), dtype=np.float32)
    for t in range(L - 1):
        P[t] = _normal([s, 20, t], (V, d), sc)
    W = np.empty((L, V, d), dtype=np.float32)
    for t in range(L):
        W[t] = _normal([s, 30, t], (V, d), sc)
    out = {"q": q, "P": P}
    if cfg.dtype == "bf16":
        bits = bf16_round_bits(W)
        out["W_bits"] = bits
        out["W"] = bf16_bits_to_f32(bits)
    else:
        out["W"] = W
    return out
