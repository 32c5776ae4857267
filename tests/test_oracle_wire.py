"""Pins of the oracle's wire-format writer (FlashTrie App. D.3, "Output
serialization"): byte records written out by hand from the page's layout,
and parse-back invariants on decodes of the oracle itself."""

import math
import os

import numpy as np
import pytest

import oracle
from synth import get_config, make_catalog, make_dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "wire_records.txt")


def golden_cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "case":
            cur = {"name": rest[0], "slots": []}
        elif key in ("K", "L"):
            cur[key] = int(rest[0])
        elif key == "alpha":
            cur["alpha"] = float(rest[0])
        elif key == "slot":
            cur["slots"].append((float(rest[0]), [int(x) for x in rest[1:]]))
        elif key == "bytes":
            cur["bytes"] = bytes.fromhex("".join(rest))
        elif key == "end":
            cases.append(cur)
    return cases


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_wire_record_golden(case):
    assert len(case["slots"]) == case["K"]
    seqs = np.array([s for _, s in case["slots"]], np.int64).reshape(case["K"], case["L"])
    logp = np.array([lp for lp, _ in case["slots"]], np.float32)
    assert oracle.wire_record(seqs, logp, case["alpha"]) == case["bytes"]


def test_wire_parse_inverts_record_on_oracle_decodes():
    """Every live beam appears once, worst first, with its own tokens and its
    log-prob times the length factor; end offsets step by L; the record's
    size is 8 + 16 n_o + 4 n_o L."""
    cfg = get_config("tiny")
    items, dense = make_catalog(cfg), make_dense(cfg)
    T = oracle.Trie(items, cfg.V)
    ref = T.decode(cfg.K, dense["q"], dense["P"], dense["W"], bf16=cfg.dtype == "bf16")
    seqs, logp = ref["seqs"], ref["logp"].astype(np.float32)
    for alpha in (0.0, 0.6, 1.0):
        recs = oracle.wire_records(seqs, logp, cfg.K, alpha)
        assert len(recs) == cfg.Q
        f = (6.0 / (5.0 + cfg.L)) ** alpha
        for q, buf in enumerate(recs):
            lp, sq = oracle.wire_parse(buf)
            live = [i for i in range(cfg.K) if math.isfinite(float(logp[q * cfg.K + i]))]
            assert len(buf) == 8 + 16 * len(live) + 4 * len(live) * cfg.L
            assert sq == [tuple(int(x) for x in seqs[q * cfg.K + i]) for i in live[::-1]]
            assert lp == [float(logp[q * cfg.K + i]) * f for i in live[::-1]]
            assert lp == sorted(lp)  # ascending order of score (alpha scales every beam alike)
            assert all(x in set(map(tuple, items.tolist())) for x in sq)


def test_length_norm_closed_form():
    # Wu et al. normalisation at alpha = 1: 6 / (5 + d); alpha = 0: 1
    assert oracle.length_norm(7, 1.0) == 0.5
    assert oracle.length_norm(1, 1.0) == 1.0
    assert oracle.length_norm(3, 0.0) == 1.0
