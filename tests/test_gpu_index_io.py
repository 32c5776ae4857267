"""GPU: an index written by cb_index_save and read back by cb_index_load
decodes exactly like the index it was saved from (device tables read back
for the save; host-built tables saved and uploaded on load)."""

import numpy as np
import pytest

from synth import get_config, make_catalog, make_dense

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import csr_constrained_beam_amd as cb  # noqa: E402

DEV = torch.device("cuda:0")


def decode(idx, cfg, dense, paths):
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    for t, p in enumerate(paths):
        plan.set_path(t, p)
    W = torch.from_numpy(dense["W_bits"].view(np.int16)).to(DEV).view(torch.bfloat16) if cfg.dtype == "bf16" \
        else torch.from_numpy(dense["W"]).to(DEV)
    out = plan.decode(torch.from_numpy(dense["q"]).to(DEV), torch.from_numpy(dense["P"]).to(DEV), W)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


@pytest.mark.parametrize("name", ["tiny", "small", "hybrid"])
@pytest.mark.parametrize("source", ["device", "host"])
def test_loaded_index_decodes_identically(tmp_path, name, source):
    cfg = get_config(name)
    items = make_catalog(cfg)
    dense = make_dense(cfg)
    print("case", name, source, flush=True)
    built = cb.Index(items, cfg.V, device=0)
    saved_from = built if source == "device" else cb.Index(items, cfg.V, device=-1)
    p = tmp_path / ("%s.cbi" % name)
    saved_from.save(p)
    loaded = cb.Index.load(p, device=0)
    for t in range(cfg.L):
        assert loaded.info(t) == built.info(t)
    for paths in (["auto"] * cfg.L, ["sparse"] * cfg.L):
        a = decode(built, cfg, dense, paths)
        b = decode(loaded, cfg, dense, paths)
        for k in ("seqs", "logp", "rows"):
            assert torch.equal(a[k], b[k]), (paths, k)
