"""ctypes declarations of the C ABI in include/cb.h.

The shared library is built in-tree (``python -m csr_constrained_beam_amd.build``).
There is no fallback: if it is missing, importing the package's API raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsrbeam.so")

CB_OK, CB_EINVAL, CB_ENOMEM, CB_EHIP, CB_EUNSUPPORTED, CB_ECAPACITY = 0, -1, -2, -3, -4, -5
CB_F32, CB_BF16 = 0, 1
CB_PATH_AUTO, CB_PATH_DENSE, CB_PATH_SPARSE, CB_PATH_SPARSE_SPLIT = 0, 1, 2, 3
CB_STORE_AUTO, CB_STORE_CSR, CB_STORE_BITMAP = 0, 1, 2
CB_SELECT_AUTO, CB_SELECT_LDS, CB_SELECT_RADIX = 0, 1, 2
STEP_OPTIONS = {"step_threads": 0, "split_rows": 1, "sparse_form": 2, "dense_rows": 3, "radix_prepass": 4,
                "query_split": 5, "token_major": 6}

STATUS_NAMES = {0: "CB_OK", -1: "CB_EINVAL", -2: "CB_ENOMEM", -3: "CB_EHIP", -4: "CB_EUNSUPPORTED",
                -5: "CB_ECAPACITY"}

# every symbol the header declares, with (restype, argtypes)
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PP = ctypes.POINTER(ctypes.c_void_p)


class StepInfo(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("n_edges", ctypes.c_int64), ("max_fanout", ctypes.c_int32),
                ("storage", ctypes.c_int32), ("bytes", ctypes.c_int64)]


class KernelTime(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("kernel", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("blocks", ctypes.c_int32), ("us", ctypes.c_float)]


class PhaseTime(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("select_us", ctypes.c_float), ("update_us", ctypes.c_float)]


KERNEL_NAMES = {0: "gemm_bf16", 1: "gemm_f32", 2: "expand_sparse", 3: "expand_dense", 4: "merge",
                5: "step_query", 6: "live_rows", 7: "radix_score_sparse", 8: "radix_score_dense",
                9: "radix_keys", 10: "radix_refine", 11: "radix_collect", 12: "radix_sort",
                13: "decode_tail", 14: "radix_small", 15: "row_lse", 16: "token_lists", 17: "token_score"}

SIGNATURES = {
    "cb_build_index": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _I32, _PP]),
    "cb_index_shape": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "cb_index_info": (ctypes.c_int, [_P, _I32, ctypes.POINTER(StepInfo)]),
    "cb_index_row": (ctypes.c_int, [_P, _I32, _I64, _P, _P, _I32, _P]),
    "cb_free_index": (None, [_P]),
    "cb_plan_create": (ctypes.c_int, [_P, _I32, _I32, _I32, ctypes.c_int, _PP]),
    "cb_set_path": (ctypes.c_int, [_P, _I32, ctypes.c_int]),
    "cb_get_path": (ctypes.c_int, [_P, _I32, _P]),
    "cb_set_step_option": (ctypes.c_int, [_P, _I32, ctypes.c_int, _I32]),
    "cb_get_step_option": (ctypes.c_int, [_P, _I32, ctypes.c_int, _P]),
    "cb_set_select": (ctypes.c_int, [_P, _I32, ctypes.c_int]),
    "cb_get_select": (ctypes.c_int, [_P, _I32, _P]),
    "cb_set_decode_fusion": (ctypes.c_int, [_P, _I32]),
    "cb_get_decode_fusion": (ctypes.c_int, [_P, _P]),
    "cb_tune_decode_times": (ctypes.c_int, [_P, _P, _P]),
    "cb_set_mode": (ctypes.c_int, [_P, ctypes.c_int]),
    "cb_get_mode": (ctypes.c_int, [_P, _P]),
    "cb_step": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "cb_step_noalloc": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, ctypes.c_int, ctypes.c_int, _P, _P, _P, _P, _P,
                                       _P, _P, _P, _P]),
    "cb_decode": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "cb_tune": (ctypes.c_int, [_P, _I32, _P, _P, _P, _I32, _P]),
    "cb_tune_times": (ctypes.c_int, [_P, _I32, _P, _P]),
    "cb_profile_start": (ctypes.c_int, [_P, _I32]),
    "cb_profile_stop": (ctypes.c_int, [_P, _P, _I32, _P]),
    "cb_profile_phases": (ctypes.c_int, [_P, _P, _I32, _P]),
    "cb_index_save": (ctypes.c_int, [_P, ctypes.c_char_p]),
    "cb_index_load": (ctypes.c_int, [ctypes.c_char_p, _I32, _P]),
    "cb_floor_probe": (ctypes.c_int, [_I32, _I32, _I32, _P, _P]),
    "cb_wire_bytes": (ctypes.c_int, [_I32, _I32, _P]),
    "cb_wire_results": (ctypes.c_int, [_I32, _I32, _I32, _P, _P, ctypes.c_double, _P, ctypes.c_int64, _P, _P]),
    "cb_plan_destroy": (None, [_P]),
    "cb_last_error": (ctypes.c_char_p, []),
}

_lib = None


class CbError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s: %s" % (fn, STATUS_NAMES.get(status, status), msg))
        self.status = status


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libcsrbeam.so is not built; run `python -m csr_constrained_beam_amd.build` "
                              "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(fn, status):
    if status != CB_OK:
        raise CbError(fn, status, lib().cb_last_error().decode(errors="replace"))
