"""Wire-format results, written on the CPU (TEST INFRASTRUCTURE ONLY: only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it).

FlashTrie (arXiv 2607.10044), App. D.3 "Output serialization": the selected
beams, kept best-first during the search, go on the wire in ascending order of
score; per-beam sequences come from the parent pointers; their lengths are
turned into end offsets by a prefix sum.  The record of n_o beams holding
n_tok tokens is an 8-byte num_beams header followed by n_o float64
``logp_norm``, n_o uint64 ``sent_offset`` and n_tok uint32 ``tokens``;
sequence i is ``tokens[sent_offset[i-1]:sent_offset[i]]`` (with 0 before the
first).  ``logp_norm`` is the length-normalised log-probability of FlashTrie
App. E, eq. 2 (after Wu et al.): the sum of the step log-probs times
(6 / (5 + d))**alpha for a sequence of d tokens.

Readings (the page leaves them open): the records are little-endian; a beam
is on the wire when its log-prob is finite (dead slots, -inf, are left out);
the log-prob of a beam is the decode's float32 accumulated value, widened to
float64 before the normalisation factor is applied.

Parity: pinned by hand-written byte records of small examples
(``tests/golden/wire_records.txt``) and by parse-back invariants
(``tests/test_oracle_wire.py``).
"""

import math
import struct

import numpy as np


def length_norm(d, alpha):
    """(6 / (5 + d)) ** alpha: the length normalisation of a d-token beam."""
    return (6.0 / (5.0 + d)) ** alpha


def record(seqs, logp, alpha=0.0):
    """One query's record.  seqs: int [K][L] best-first, logp: float32 [K]
    (-inf for dead slots).  Returns bytes."""
    seqs = np.asarray(seqs)
    logp = np.asarray(logp, np.float32)
    # the selected beams, best first (dead slots are not selected)
    selected = [i for i in range(len(logp)) if math.isfinite(float(logp[i]))]
    ascending = selected[::-1]
    lengths = [int(seqs.shape[1]) for _ in ascending]
    ends = np.cumsum(lengths, dtype=np.int64) if lengths else np.zeros(0, np.int64)
    out = [struct.pack("<Q", len(ascending))]
    for i, n in zip(ascending, lengths):
        out.append(struct.pack("<d", float(logp[i]) * length_norm(n, alpha)))
    for e in ends:
        out.append(struct.pack("<Q", int(e)))
    for i in ascending:
        out.append(struct.pack("<%dI" % seqs.shape[1], *[int(x) for x in seqs[i]]))
    return b"".join(out)


def records(seqs, logp, K, alpha=0.0):
    """Records of every query of a decode: seqs int [Q*K][L], logp float32
    [Q*K] (the decode's outputs, best-first per query).  Returns a list of
    bytes, one per query."""
    seqs = np.asarray(seqs)
    logp = np.asarray(logp, np.float32)
    Q = len(logp) // K
    return [record(seqs[q * K:(q + 1) * K], logp[q * K:(q + 1) * K], alpha) for q in range(Q)]


def parse(buf):
    """Inverse of ``record``: (logp_norm list, list of token tuples) in wire
    order."""
    n = struct.unpack_from("<Q", buf, 0)[0]
    lp = list(struct.unpack_from("<%dd" % n, buf, 8))
    ends = list(struct.unpack_from("<%dQ" % n, buf, 8 + 8 * n))
    n_tok = ends[-1] if n else 0
    toks = struct.unpack_from("<%dI" % n_tok, buf, 8 + 16 * n)
    seqs, s = [], 0
    for e in ends:
        seqs.append(tuple(toks[s:e]))
        s = e
    return lp, seqs
