"""The five synthetic workloads: catalog shape, model width, batch and beam.

Each entry fixes the seed so that every consumer (tests, benchmark, oracle
timing) draws the identical catalog and tensors.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    name: str
    n_items: int          # distinct catalog items after duplicate rejection
    L: int                # Semantic-ID length = number of decoding steps
    V: int                # rows of every per-step output layer W_t (codebook size; +1 for EOS)
    d: int                # hidden width
    dtype: str            # "f32" or "bf16": storage of W_t and of the hidden vectors
    Q: int                # queries per batch
    K: int                # beam width
    seed: int
    generator: str        # catalog generator name in synth.catalogs
    params: dict = field(default_factory=dict, hash=False, compare=False)


CONFIGS = {
    # 1,000 items, L=3, V=256, clustered hierarchy, fp32, 4 queries x beam 8.
    "tiny": Config("tiny", 1_000, 3, 256, 64, "f32", 4, 8, 101, "clustered",
                   {"zipf_s": 1.1, "fanout_mean": 4.0}),
    # 3,700 items, three V=256 levels plus a collision token (< 8), bf16 W.
    "small": Config("small", 3_700, 4, 256, 256, "bf16", 256, 20, 102, "clustered_collision",
                    {"zipf_s": 1.1, "fanout_mean": 4.0, "max_collisions": 8}),
    # 10M items, V=4096, level 1 fully populated, wide level 2, narrow levels 3-4.
    "hybrid": Config("hybrid", 10_000_000, 4, 4096, 512, "bf16", 512, 16, 103, "hybrid",
                     {"level2_mean": 300.0, "later_mean": 3.0}),
    # 20M items, L=8, V=2048, Zipf(1.0) tokens over per-prefix permutations.
    "production": Config("production", 20_000_000, 8, 2048, 1024, "bf16", 64, 32, 104, "zipf_prefix",
                         {"zipf_s": 1.0}),
    # ~1M items in a tree whose rows below the root all hold exactly B tokens
    # (the branch-factor sweep at |C| = 10^6); V = 16,384 so that the root of
    # the smallest B fits.
    "branch": Config("branch", 1_000_000, 3, 16_384, 1024, "bf16", 64, 32, 106, "branch", {"B": 64}),
    # 100M variable-length items (4..12 tokens) over V=32,000, EOS-padded to 12.
    "large": Config("large", 100_000_000, 12, 32_001, 1024, "bf16", 1, 1000, 105, "zipf_varlen",
                    {"zipf_s": 1.2, "min_len": 4, "max_len": 12, "codebook": 32_000}),
}


def get_config(name: str, **overrides) -> Config:
    """Return the named workload, optionally with fields replaced (smaller
    item counts or batches for quick checks)."""
    cfg = CONFIGS[name]
    if not overrides:
        return cfg
    fields = dict(cfg.__dict__)
    fields.update(overrides)
    return Config(**fields)
