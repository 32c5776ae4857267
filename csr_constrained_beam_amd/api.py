"""Python binding of the C ABI: argument marshalling only.

Every step of the decoding path runs in the HIP library; this module checks
shapes and dtypes, passes raw device pointers and the current HIP stream, and
allocates output tensors with PyTorch.
"""

import ctypes

import numpy as np

from . import _lib as C

_PATHS = {"auto": C.CB_PATH_AUTO, "dense": C.CB_PATH_DENSE, "sparse": C.CB_PATH_SPARSE,
          "sparse_split": C.CB_PATH_SPARSE_SPLIT}
_PATH_NAMES = {v: k for k, v in _PATHS.items()}
_SELECTS = {"auto": C.CB_SELECT_AUTO, "lds": C.CB_SELECT_LDS, "radix": C.CB_SELECT_RADIX}
_SELECT_NAMES = {v: k for k, v in _SELECTS.items()}
_STORES = {"auto": C.CB_STORE_AUTO, "csr": C.CB_STORE_CSR, "bitmap": C.CB_STORE_BITMAP}
_STORE_NAMES = {v: k for k, v in _STORES.items()}
_MODES = {"filter_first": 0, "score_first": 1, "unconstrained": 2}
_MODE_NAMES = {v: k for k, v in _MODES.items()}


def _torch():
    import torch
    return torch


class Index:
    """Step-sliced prefix index of a catalog, resident on ``device``.

    sids: int array [n_items][L] with tokens in [0, V).  ``device=-1`` builds
    host tables only (inspection, no stepping)."""

    def __init__(self, sids, V, device=0, store="auto"):
        sids = np.ascontiguousarray(sids, dtype=np.int32)
        if sids.ndim != 2:
            raise ValueError("sids must be a 2-D [n_items][L] array")
        self._lib = C.lib()
        h = ctypes.c_void_p()
        C.check("cb_build_index", self._lib.cb_build_index(sids.ctypes.data, sids.shape[0], sids.shape[1], int(V),
                                                            int(device), _STORES[store], ctypes.byref(h)))
        self._h = h

    @classmethod
    def load(cls, path, device=0):
        """An index saved by ``save``, uploaded to ``device`` (-1: host only)."""
        self = cls.__new__(cls)
        self._lib = C.lib()
        h = ctypes.c_void_p()
        C.check("cb_index_load", self._lib.cb_index_load(str(path).encode(), int(device), ctypes.byref(h)))
        self._h = h
        return self

    def save(self, path):
        C.check("cb_index_save", self._lib.cb_index_save(self._h, str(path).encode()))

    def size_report(self):
        """Bytes per step and in total, with bytes per catalog item."""
        shape = self.shape
        steps = [dict(t=t, **self.info(t)) for t in range(shape["L"])]
        total = sum(s["bytes"] for s in steps)
        return {"n_items": shape["n_items"], "L": shape["L"], "V": shape["V"], "steps": steps, "bytes": total,
                "bytes_per_item": total / max(1, shape["n_items"])}

    def close(self):
        if getattr(self, "_h", None):
            self._lib.cb_free_index(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def shape(self):
        L, V, dev = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        n = ctypes.c_int64()
        C.check("cb_index_shape", self._lib.cb_index_shape(self._h, ctypes.byref(L), ctypes.byref(V), ctypes.byref(n),
                                                            ctypes.byref(dev)))
        return {"L": L.value, "V": V.value, "n_items": n.value, "device": dev.value}

    @property
    def L(self):
        return self.shape["L"]

    def info(self, t):
        si = C.StepInfo()
        C.check("cb_index_info", self._lib.cb_index_info(self._h, int(t), ctypes.byref(si)))
        return {"n_rows": si.n_rows, "n_edges": si.n_edges, "max_fanout": si.max_fanout,
                "storage": _STORE_NAMES[si.storage], "bytes": si.bytes}

    def row(self, t, r):
        """(tokens, next_rows) of row r of step t, read back to the host."""
        n = ctypes.c_int32()
        C.check("cb_index_row", self._lib.cb_index_row(self._h, int(t), int(r), None, None, 0, ctypes.byref(n)))
        tok = np.empty(n.value, np.int32)
        nxt = np.empty(n.value, np.int64)
        C.check("cb_index_row", self._lib.cb_index_row(self._h, int(t), int(r), tok.ctypes.data, nxt.ctypes.data,
                                                        n.value, ctypes.byref(n)))
        return tok, nxt

    def plan(self, Q_max, K, d, dtype):
        return Plan(self, Q_max, K, d, dtype)

    def step_noalloc(self, t, K, hidden, W_t, rows, acc, path="auto", out=None):
        """One decoding step without a plan (cb_step_noalloc): the library
        allocates nothing; its workspace is a static device array.  hidden
        [Q*K][d] (f32 or bf16), W_t [V][d] of the same type, rows int32 [Q*K],
        acc f32 [Q*K].  Returns (tokens, parents, rows, logp)."""
        torch = _torch()
        K = int(K)
        R = rows.shape[0]
        if R % K:
            raise ValueError("rows length must be a multiple of K")
        code, tdt = _dtype_code(hidden.dtype)
        d = hidden.shape[1]
        dev = self.shape["device"]
        ph = _check_tensor(dev, "hidden", hidden, tdt, (R, d))
        pw = _check_tensor(dev, "W_t", W_t, tdt, (self.shape["V"], d))
        pr = _check_tensor(dev, "rows", rows, torch.int32, (R,))
        pa = _check_tensor(dev, "acc", acc, torch.float32, (R,))
        if out is None:
            out = (torch.empty(R, dtype=torch.int32, device=rows.device),
                   torch.empty(R, dtype=torch.int32, device=rows.device),
                   torch.empty(R, dtype=torch.int32, device=rows.device),
                   torch.empty(R, dtype=torch.float32, device=rows.device))
        ot, op, orow, ol = out
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        C.check("cb_step_noalloc", self._lib.cb_step_noalloc(
            self._h, int(t), R // K, K, int(d), code, _PATHS[path], ph, pw, pr, pa, ctypes.c_void_p(ot.data_ptr()),
            ctypes.c_void_p(op.data_ptr()), ctypes.c_void_p(orow.data_ptr()), ctypes.c_void_p(ol.data_ptr()),
            stream))
        return out


def _check_tensor(device, name, x, dtype, shape):
    """Raw pointer of a contiguous tensor on cuda:device of the given dtype and shape."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.device.index != device:
        raise ValueError("%s must be a tensor on cuda:%d" % (name, device))
    if x.dtype != dtype or tuple(x.shape) != tuple(shape) or not x.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s (got %s %s)"
                         % (name, dtype, tuple(shape), x.dtype, tuple(x.shape)))
    return ctypes.c_void_p(x.data_ptr())


def _dtype_code(dtype):
    torch = _torch()
    if dtype in ("bf16", torch.bfloat16):
        return C.CB_BF16, torch.bfloat16
    if dtype in ("f32", torch.float32):
        return C.CB_F32, torch.float32
    raise ValueError("dtype must be 'f32' or 'bf16'")


class Plan:
    """Workspace and per-step path choice for up to Q_max queries of beam K."""

    def __init__(self, index, Q_max, K, d, dtype):
        self.index = index  # keeps the index alive
        self._lib = index._lib
        self.code, self.tdtype = _dtype_code(dtype)
        self.Q_max, self.K, self.d = int(Q_max), int(K), int(d)
        self.L = index.L
        self.V = index.shape["V"]
        self.device = index.shape["device"]
        h = ctypes.c_void_p()
        C.check("cb_plan_create", self._lib.cb_plan_create(index._h, self.Q_max, self.K, self.d, self.code,
                                                            ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._lib.cb_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def set_path(self, t, path):
        C.check("cb_set_path", self._lib.cb_set_path(self._h, int(t), _PATHS[path]))

    def get_path(self, t):
        v = ctypes.c_int()
        C.check("cb_get_path", self._lib.cb_get_path(self._h, int(t), ctypes.byref(v)))
        return _PATH_NAMES[v.value]

    def set_option(self, t, option, value):
        """Force a form of step t's kernels (cb_set_step_option): option is
        one of "step_threads", "split_rows", "sparse_form", "dense_rows",
        "radix_prepass", "query_split", "token_major"; 0 restores the
        default."""
        C.check("cb_set_step_option", self._lib.cb_set_step_option(self._h, int(t), C.STEP_OPTIONS[option],
                                                                    int(value)))

    def get_option(self, t, option):
        v = ctypes.c_int32()
        C.check("cb_get_step_option", self._lib.cb_get_step_option(self._h, int(t), C.STEP_OPTIONS[option],
                                                                    ctypes.byref(v)))
        return v.value

    def set_step_threads(self, t, threads):
        """Workgroup size of the per-query sparse step at step t (256, 512,
        1024, or 0 for the default)."""
        self.set_option(t, "step_threads", threads)

    def get_step_threads(self, t):
        return self.get_option(t, "step_threads")

    def set_split_rows(self, t, min_tokens):
        """Rows of more than min_tokens tokens that the split sparse path
        scores apart at step t (0: the default, 16)."""
        self.set_option(t, "split_rows", min_tokens)

    def set_select(self, t, select):
        """Top-K selection of step t: "auto", "lds" (K <= 64) or "radix"."""
        C.check("cb_set_select", self._lib.cb_set_select(self._h, int(t), _SELECTS[select]))

    def get_select(self, t):
        v = ctypes.c_int()
        C.check("cb_get_select", self._lib.cb_get_select(self._h, int(t), ctypes.byref(v)))
        return _SELECT_NAMES[v.value]

    def set_mode(self, mode):
        """Decoding variant: "filter_first" (default), "score_first" or
        "unconstrained" (the last two on the dense path only)."""
        C.check("cb_set_mode", self._lib.cb_set_mode(self._h, _MODES[mode]))

    def get_mode(self):
        v = ctypes.c_int()
        C.check("cb_get_mode", self._lib.cb_get_mode(self._h, ctypes.byref(v)))
        return _MODE_NAMES[v.value]

    def set_decode_fusion(self, enable):
        """Persistent decode of the trailing sparse steps: True, False or
        "auto" (the default: chosen by tune, on until measured)."""
        v = -1 if enable == "auto" else (1 if enable else 0)
        C.check("cb_set_decode_fusion", self._lib.cb_set_decode_fusion(self._h, v))

    def tune_decode_times(self):
        """(step-by-step, persistent) decode microseconds from the last tune."""
        a, b = ctypes.c_float(), ctypes.c_float()
        C.check("cb_tune_decode_times", self._lib.cb_tune_decode_times(self._h, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def get_decode_fusion(self):
        v = ctypes.c_int()
        C.check("cb_get_decode_fusion", self._lib.cb_get_decode_fusion(self._h, ctypes.byref(v)))
        return bool(v.value)

    def _stream(self):
        torch = _torch()
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def _check_tensor(self, name, x, dtype, shape):
        return _check_tensor(self.device, name, x, dtype, shape)

    def step(self, t, hidden, W_t, rows, acc, out=None):
        """One decoding step (cb_step).  Returns (tokens, parents, rows, logp)."""
        torch = _torch()
        R = rows.shape[0]
        if R % self.K:
            raise ValueError("rows length must be a multiple of K")
        Q = R // self.K
        ph = self._check_tensor("hidden", hidden, self.tdtype, (R, self.d))
        pw = self._check_tensor("W_t", W_t, self.tdtype, (self.V, self.d))
        pr = self._check_tensor("rows", rows, torch.int32, (R,))
        pa = self._check_tensor("acc", acc, torch.float32, (R,))
        if out is None:
            dev = rows.device
            out = (torch.empty(R, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.int32, device=dev),
                   torch.empty(R, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.float32, device=dev))
        ot, op, orow, ol = out
        C.check("cb_step", self._lib.cb_step(self._h, int(t), Q, ph, pw, pr, pa, ctypes.c_void_p(ot.data_ptr()),
                                             ctypes.c_void_p(op.data_ptr()), ctypes.c_void_p(orow.data_ptr()),
                                             ctypes.c_void_p(ol.data_ptr()), self._stream()))
        return out

    def decode(self, q, P, W, trace=False):
        """Full decode (cb_decode).  q [Q][d] f32, P [L-1][V][d] f32, W [L][V][d]."""
        torch = _torch()
        Q = q.shape[0]
        R = Q * self.K
        dev = q.device
        pq = self._check_tensor("q", q, torch.float32, (Q, self.d))
        pp = self._check_tensor("P", P, torch.float32, (self.L - 1, self.V, self.d)) if self.L > 1 else None
        pw = self._check_tensor("W", W, self.tdtype, (self.L, self.V, self.d))
        out = {"seqs": torch.empty((R, self.L), dtype=torch.int32, device=dev),
               "logp": torch.empty(R, dtype=torch.float32, device=dev),
               "rows": torch.empty(R, dtype=torch.int32, device=dev)}
        tr = [None, None, None]
        if trace:
            out["trace_h"] = torch.empty((self.L, R, self.d), dtype=self.tdtype, device=dev)
            out["trace_rows"] = torch.empty((self.L, R), dtype=torch.int32, device=dev)
            out["trace_acc"] = torch.empty((self.L, R), dtype=torch.float32, device=dev)
            tr = [ctypes.c_void_p(out[k].data_ptr()) for k in ("trace_h", "trace_rows", "trace_acc")]
        C.check("cb_decode", self._lib.cb_decode(self._h, Q, pq, pp, pw, ctypes.c_void_p(out["seqs"].data_ptr()),
                                                 ctypes.c_void_p(out["logp"].data_ptr()),
                                                 ctypes.c_void_p(out["rows"].data_ptr()), *tr, self._stream()))
        return out

    def tune(self, q, P, W, reps=5):
        """Pre-measured path switch (cb_tune); returns per-step timings."""
        torch = _torch()
        Q = q.shape[0]
        pq = self._check_tensor("q", q, torch.float32, (Q, self.d))
        pp = self._check_tensor("P", P, torch.float32, (self.L - 1, self.V, self.d)) if self.L > 1 else None
        pw = self._check_tensor("W", W, self.tdtype, (self.L, self.V, self.d))
        C.check("cb_tune", self._lib.cb_tune(self._h, Q, pq, pp, pw, int(reps), self._stream()))
        res = []
        for t in range(self.L):
            dus, sus = ctypes.c_float(), ctypes.c_float()
            C.check("cb_tune_times", self._lib.cb_tune_times(self._h, t, ctypes.byref(dus), ctypes.byref(sus)))
            res.append({"t": t, "dense_us": dus.value, "sparse_us": sus.value, "path": self.get_path(t)})
        return res

    def profile_start(self, capacity=4096):
        """Record HIP events around every kernel launch from now on."""
        C.check("cb_profile_start", self._lib.cb_profile_start(self._h, int(capacity)))
        self._prof_cap = int(capacity)

    def profile_stop(self):
        """Stop recording; returns one dict per recorded launch."""
        cap = getattr(self, "_prof_cap", 0)
        buf = (C.KernelTime * max(cap, 1))()
        n = ctypes.c_int32()
        C.check("cb_profile_stop", self._lib.cb_profile_stop(self._h, buf, cap, ctypes.byref(n)))
        return [{"step": r.step, "kernel": C.KERNEL_NAMES[r.kernel], "threads": r.threads, "blocks": r.blocks,
                 "us": r.us} for r in buf[:min(n.value, cap)]]

    def profile_phases(self):
        """Per-step phase times (mean over queries, device wall clock) of the
        last persistent decode run while profiling was on, as of the last
        profile_stop: [{"step", "select_us", "update_us"}]."""
        buf = (C.PhaseTime * max(self.L, 1))()
        n = ctypes.c_int32()
        C.check("cb_profile_phases", self._lib.cb_profile_phases(self._h, buf, self.L, ctypes.byref(n)))
        return [{"step": r.step, "select_us": r.select_us, "update_us": r.update_us} for r in buf[:n.value]]


def floor_probe(blocks, threads, n, timed=True):
    """Overhead floor (cb_floor_probe): n launches of an empty kernel of
    ``blocks`` x ``threads`` on the current stream.  timed: returns (mean
    dispatch duration, mean time per launch back to back) in microseconds;
    otherwise only enqueues them (capturable) and returns None."""
    torch = _torch()
    lib = C.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if not timed:
        C.check("cb_floor_probe", lib.cb_floor_probe(int(blocks), int(threads), int(n), None, stream))
        return None
    us = (ctypes.c_float * 2)()
    C.check("cb_floor_probe", lib.cb_floor_probe(int(blocks), int(threads), int(n), us, stream))
    return float(us[0]), float(us[1])


def wire_bytes(K, L):
    """Smallest record stride of the wire format (cb_wire_bytes)."""
    v = ctypes.c_int64()
    C.check("cb_wire_bytes", C.lib().cb_wire_bytes(int(K), int(L), ctypes.byref(v)))
    return v.value


def wire_results(seqs, logp, K, alpha=0.0, out=None, stride=None):
    """Wire-format records of a decode's results (cb_wire_results).

    seqs: device int32 [Q*K][L] and logp: device float32 [Q*K] from
    Plan.decode.  Returns (out, nbytes): out uint8 [Q][stride] on the same
    device, query q's record in out[q, :nbytes[q]] (uint64 n_o, float64
    logp_norm[n_o], uint64 sent_offset[n_o], uint32 tokens[n_o*L]; live beams
    in ascending order of score)."""
    torch = _torch()
    if seqs.dim() != 2 or seqs.dtype != torch.int32 or not seqs.is_contiguous():
        raise ValueError("seqs must be a contiguous int32 [Q*K][L] tensor")
    R, L = seqs.shape
    if R % K:
        raise ValueError("seqs rows must be a multiple of K")
    Q = R // K
    if logp.dtype != torch.float32 or logp.numel() != R or not logp.is_contiguous() or logp.device != seqs.device:
        raise ValueError("logp must be a contiguous float32 [Q*K] tensor on the device of seqs")
    if stride is None:
        stride = wire_bytes(K, L)
    if out is None:
        out = torch.empty((Q, stride), dtype=torch.uint8, device=seqs.device)
    if out.dtype != torch.uint8 or out.numel() < Q * stride or not out.is_contiguous() or out.device != seqs.device:
        raise ValueError("out must be a contiguous uint8 tensor of Q*stride bytes on the device of seqs")
    nbytes = torch.empty(Q, dtype=torch.int64, device=seqs.device)
    with torch.cuda.device(seqs.device):
        stream = ctypes.c_void_p(torch.cuda.current_stream(seqs.device).cuda_stream)
        C.check("cb_wire_results", C.lib().cb_wire_results(
            Q, int(K), int(L), ctypes.c_void_p(seqs.data_ptr()), ctypes.c_void_p(logp.data_ptr()), float(alpha),
            ctypes.c_void_p(out.data_ptr()), int(stride), ctypes.c_void_p(nbytes.data_ptr()), stream))
    return out, nbytes
