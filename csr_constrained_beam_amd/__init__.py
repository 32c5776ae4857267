"""MI355X-native catalog-constrained beam search over Semantic-ID catalogs.

The decoding step (index lookup, scoring, masked log-softmax, per-query top-K)
runs in hand-written HIP kernels for gfx950 behind the C ABI of
``include/cb.h`` (``libcsrbeam.so``); this package is its thin Python binding.
"""

from ._lib import CbError, LIB_PATH
from .api import Index, Plan, floor_probe, wire_bytes, wire_results

__all__ = ["Index", "Plan", "floor_probe", "wire_bytes", "wire_results", "CbError", "LIB_PATH"]
