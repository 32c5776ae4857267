"""Seeded synthetic inputs for the constrained beam-search step.

This package is the only code shared by the CPU oracle (``oracle/``) and the
HIP library (``csr_constrained_beam_amd``): it draws catalogs of Semantic-ID
token sequences and the dense tensors (queries, per-step output layers and the
per-step token embeddings of the stand-in model) from fixed seeds.  It holds
none of the decoding arithmetic: no index, no scoring, no softmax, no
selection.
"""

from .configs import CONFIGS, Config, get_config
from .catalogs import make_catalog
from .tensors import make_dense, bf16_round_bits, bf16_bits_to_f32

__all__ = [
    "CONFIGS",
    "Config",
    "get_config",
    "make_catalog",
    "make_dense",
    "bf16_round_bits",
    "bf16_bits_to_f32",
]
