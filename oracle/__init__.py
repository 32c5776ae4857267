"""CPU oracle for catalog-constrained beam search (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
``csr_constrained_beam_amd``: the trie, the step and the decode live in
``trie_beam.c``, a second trie-free construction in ``range_beam.c`` (both
compiled here with gcc); ``brute.py`` is an independent pure-Python
enumerator for tiny catalogs.

Parity status of each function (what pins it; see ``tests/test_oracle_pins.py``):

* ``Trie`` valid sets and row numbers: the ZeroGR worked example (prefix 3-5
  admits exactly tokens 1 and 4), a depth-only-list negative case, a scan of
  the catalog for every prefix, the lexicographic rank of every prefix, and
  the STATIC CSR fragment's "next state = edge position + 1" numbering.
* ``Trie.step``: closed forms (W = 0 gives log(1/n) and an order fixed by the
  tie-break alone; a single child gives 0 exactly; a two-token row gives
  -log(1 + exp(z_other - z))), softmax normalisation over valid tokens, and
  textbook beam search on a full-product catalog.
* ``Trie.decode``: brute-force enumeration of every item's path score when the
  beam is at least as wide as the catalog, the single-item catalog, and the
  decode invariants.
* ``Trie.hidden``: the stand-in model's rule is defined by the workload, not by
  the pages; it is pinned by a closed form (unit norm, direction of s) only.
* ``Trie.step`` / ``Trie.decode`` with ``mode="score_first"`` (softmax over
  the whole codebook, valid tokens as candidates) and ``mode="unconstrained"``
  (every token a candidate, row 0): the brute-force enumerator with the
  whole codebook as softmax support (every catalog item, resp. every
  sequence of the codebook product, with its path score when the beam is
  that wide), equality of the three variants on the full-product catalog,
  and the per-beam constant shift lse(valid) - lse(all) <= 0 between the two
  supports (``tests/test_oracle_modes.py``).
* ``SortedRange`` (``range_beam.c``): the same definition computed over the
  sorted catalog without a trie, light enough for 100M-item catalogs.  Pinned
  by a catalog scan of every prefix, brute-force path scores, the W = 0 closed
  form, and equality with the trie oracle (tables, step candidates, decode
  traces) on the tiny, small and hybrid generators
  (``tests/test_oracle_range.py``).
* ``wire_records`` / ``wire_parse`` (``wire.py``): the on-wire record of a
  decode's results (FlashTrie App. D.3, "Output serialization").  Pinned by
  byte records written out by hand from the page's layout
  (``tests/golden/wire_records.txt``) and parse-back invariants
  (``tests/test_oracle_wire.py``).
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "trie_beam.c"), os.path.join(_HERE, "range_beam.c")]
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32p = ctypes.c_void_p


def build(force=False):
    """Compile trie_beam.c and range_beam.c -> liboracle.so (gcc, OpenMP)."""
    stale = not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(x) for x in _SRCS)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_MODES = {"filter_first": 0, "score_first": 1, "unconstrained": 2}


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        lib.or_build.restype = P
        lib.or_build.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
        lib.or_free.restype = None
        lib.or_free.argtypes = [P]
        lib.or_n_items.restype = ctypes.c_int64
        lib.or_n_items.argtypes = [P]
        lib.or_level_count.restype = ctypes.c_int64
        lib.or_level_count.argtypes = [P, ctypes.c_int]
        lib.or_children.restype = ctypes.c_int
        lib.or_children.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int64]
        lib.or_children_of_row.restype = ctypes.c_int
        lib.or_children_of_row.argtypes = [P, ctypes.c_int, ctypes.c_int64, P, P, ctypes.c_int64]
        lib.or_prefix_of_row.restype = ctypes.c_int
        lib.or_prefix_of_row.argtypes = [P, ctypes.c_int, ctypes.c_int64, P]
        lib.or_step.restype = ctypes.c_int
        lib.or_step.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P,
                                P, P, P, P, ctypes.c_int64, P, P, P, P, P, ctypes.c_int]
        lib.or_decode.restype = ctypes.c_int
        lib.or_decode.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P,
                                  P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.or_step_mode.restype = ctypes.c_int
        lib.or_step_mode.argtypes = lib.or_step.argtypes + [ctypes.c_int]
        lib.or_decode_mode.restype = ctypes.c_int
        lib.or_decode_mode.argtypes = lib.or_decode.argtypes + [ctypes.c_int]
        lib.or_hidden.restype = None
        lib.or_hidden.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P]
        lib.orr_build.restype = P
        lib.orr_build.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
        lib.orr_free.restype = None
        lib.orr_free.argtypes = [P]
        lib.orr_n_items.restype = ctypes.c_int64
        lib.orr_n_items.argtypes = [P]
        lib.orr_level_count.restype = ctypes.c_int64
        lib.orr_level_count.argtypes = [P, ctypes.c_int]
        lib.orr_children_of_row.restype = ctypes.c_int
        lib.orr_children_of_row.argtypes = [P, ctypes.c_int, ctypes.c_int64, P, P, ctypes.c_int64]
        lib.orr_step.restype = ctypes.c_int
        lib.orr_step.argtypes = lib.or_step.argtypes
        lib.orr_decode.restype = ctypes.c_int
        lib.orr_decode.argtypes = lib.or_decode.argtypes
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


class Trie:
    """Pointer trie of a catalog (int array [n][L], tokens in [0, V))."""

    _p = "or_"

    def __init__(self, sids, V):
        sids = np.ascontiguousarray(sids, dtype=np.int32)
        if sids.ndim != 2:
            raise ValueError("sids must be [n_items][L]")
        self.L = int(sids.shape[1])
        self.V = int(V)
        self._lib = _load()
        self._h = self._fn("build")(_ptr(sids), sids.shape[0], self.L, self.V)
        if not self._h:
            raise ValueError("oracle build failed (token out of range, bad shape or out of memory)")

    def _fn(self, name):
        return getattr(self._lib, self._p + name)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._fn("free")(h)
            self._h = None

    @property
    def n_items(self):
        return int(self._fn("n_items")(self._h))

    def level_count(self, depth):
        return int(self._fn("level_count")(self._h, depth))

    def children(self, prefix):
        """(tokens, rows) of the children of ``prefix`` (None if absent)."""
        p = np.ascontiguousarray(prefix, dtype=np.int32)
        n = self._lib.or_children(self._h, _ptr(p), len(p), None, None, 0)
        if n < 0:
            return None
        tok = np.empty(n, dtype=np.int32)
        rows = np.empty(n, dtype=np.int64)
        self._lib.or_children(self._h, _ptr(p), len(p), _ptr(tok), _ptr(rows), n)
        return tok, rows

    def children_of_row(self, depth, row):
        f = self._fn("children_of_row")
        n = f(self._h, depth, row, None, None, 0)
        if n < 0:
            return None
        tok = np.empty(n, dtype=np.int32)
        rows = np.empty(n, dtype=np.int64)
        f(self._h, depth, row, _ptr(tok), _ptr(rows), n)
        return tok, rows

    def prefix_of_row(self, depth, row):
        out = np.empty(max(depth, 1), dtype=np.int32)
        r = self._lib.or_prefix_of_row(self._h, depth, row, _ptr(out))
        if r < 0:
            return None
        return out[:depth]

    def step(self, t, K, h, Wt, rows, acc, candidates=False, threads=1, mode="filter_first"):
        """Teacher-forced step.  h [Q*K][d] f32, Wt [V][d] f32, rows [Q*K]
        (-1 dead), acc [Q*K] f32.  Returns dict of tokens, parents, rows,
        logp (each [Q*K]) and, with ``candidates``, every candidate of every
        query sorted best first (``cand_*`` [Q][cap], ``cand_count`` [Q]).
        mode: "filter_first", "score_first" (softmax over the whole codebook,
        valid tokens as candidates) or "unconstrained" (every token, row 0)."""
        m = _MODES[mode]
        if m and type(self) is not Trie:
            raise NotImplementedError("modes other than filter_first: pointer-trie oracle only")
        h = np.ascontiguousarray(h, dtype=np.float32)
        Wt = np.ascontiguousarray(Wt, dtype=np.float32)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        acc = np.ascontiguousarray(acc, dtype=np.float32)
        R = rows.shape[0]
        assert R % K == 0
        Q = R // K
        d = h.shape[1]
        assert h.shape == (R, d) and Wt.shape[1] == d and acc.shape == (R,)
        out = {
            "tokens": np.empty(R, np.int32),
            "parents": np.empty(R, np.int32),
            "rows": np.empty(R, np.int64),
            "logp": np.empty(R, np.float32),
        }
        cap = 0
        cc = ct = cp = cr = cs = None
        if candidates:
            # capacity: the widest query's candidate count
            fan = np.zeros(R, dtype=np.int64)
            for b in np.nonzero(rows >= 0)[0]:
                fan[b] = self.V if m == 2 else self._fn("children_of_row")(self._h, t, int(rows[b]), None, None, 0)
            cap = int(max(1, fan.reshape(Q, K).sum(axis=1).max() if Q else 1))
            cc = np.zeros(Q, np.int64)
            ct = np.full((Q, cap), -1, np.int32)
            cp = np.full((Q, cap), -1, np.int32)
            cr = np.full((Q, cap), -1, np.int64)
            cs = np.full((Q, cap), -np.inf, np.float32)
        args = (self._h, t, Q, K, d, _ptr(h), _ptr(Wt), _ptr(rows), _ptr(acc),
                _ptr(out["tokens"]), _ptr(out["parents"]), _ptr(out["rows"]), _ptr(out["logp"]),
                cap, _ptr(cc), _ptr(ct), _ptr(cp), _ptr(cr), _ptr(cs), threads)
        r = self._lib.or_step_mode(*args, m) if m else self._fn("step")(*args)
        if r != 0:
            raise RuntimeError("or_step failed (%d)" % r)
        if candidates:
            out.update(cand_count=cc, cand_tokens=ct, cand_parents=cp, cand_rows=cr, cand_scores=cs)
        return out

    def decode(self, K, q, P, W, bf16, trace=False, threads=1, mode="filter_first"):
        """Free-running decode.  q [Q][d], P [L-1][V][d], W [L][V][d] (f32).
        mode as for ``step``."""
        m = _MODES[mode]
        if m and type(self) is not Trie:
            raise NotImplementedError("modes other than filter_first: pointer-trie oracle only")
        q = np.ascontiguousarray(q, dtype=np.float32)
        W = np.ascontiguousarray(W, dtype=np.float32)
        Q, d = q.shape
        L = self.L
        if P is None or L == 1:
            P = np.zeros((max(L - 1, 1), self.V, d), np.float32)
        P = np.ascontiguousarray(P, dtype=np.float32)
        assert W.shape == (L, self.V, d) and P.shape[1:] == (self.V, d)
        R = Q * K
        out = {"seqs": np.empty((R, L), np.int32), "logp": np.empty(R, np.float32), "rows": np.empty(R, np.int64)}
        tr = [None] * 7
        if trace:
            tr = [np.zeros((L, R, d), np.float32), np.empty((L, R), np.int64), np.empty((L, R), np.float32),
                  np.empty((L, R), np.int32), np.empty((L, R), np.int32), np.empty((L, R), np.int64),
                  np.empty((L, R), np.float32)]
        args = (self._h, Q, K, d, 1 if bf16 else 0, _ptr(q), _ptr(P), _ptr(W),
                _ptr(out["seqs"]), _ptr(out["logp"]), _ptr(out["rows"]), *[_ptr(a) for a in tr], threads)
        r = self._lib.or_decode_mode(*args, m) if m else self._fn("decode")(*args)
        if r != 0:
            raise RuntimeError("or_decode failed (%d)" % r)
        if trace:
            for k, a in zip(["h", "rows_in", "acc_in", "tokens", "parents", "rows_out", "logp_out"], tr):
                out["trace_" + k] = a
        return out

    def hidden(self, s, bf16):
        s = np.ascontiguousarray(s, dtype=np.float32)
        h = np.empty_like(s)
        self._lib.or_hidden(_ptr(s), s.shape[0], s.shape[1], 1 if bf16 else 0, _ptr(h))
        return h


class SortedRange(Trie):
    """Second oracle over the sorted catalog: a prefix is a range of sorted
    items, its children the distinct tokens found by binary search.  Same
    interface as Trie (children(prefix), prefix_of_row and hidden excepted)."""

    _p = "orr_"

    def children(self, prefix):
        raise NotImplementedError

    def prefix_of_row(self, depth, row):
        raise NotImplementedError


from .wire import length_norm, parse as wire_parse, record as wire_record, records as wire_records  # noqa: E402
