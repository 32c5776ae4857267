"""Loader for the C catalog drawer (``_gen.c``), compiled with gcc on first use."""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "_gen.c")
_LIB = os.path.join(_HERE, "_gen.so")
_lib = None


def build(force=False):
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        f = _lib.synth_zipf_items
        f.restype = ctypes.c_int64
        f.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return _lib


def zipf_items(seed, n_items, L, codebook, eos, zipf_s, min_len, max_len):
    out = np.empty((n_items, L), dtype=np.int32)
    r = lib().synth_zipf_items(seed, n_items, L, codebook, eos, zipf_s, min_len, max_len,
                               out.ctypes.data)
    if r < 0:
        raise MemoryError("synth_zipf_items: allocation failed")
    return out
