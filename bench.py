"""Benchmark of the constrained beam-search step on one MI355X.

A bench "step" is one pass of the whole hot path over one batch: all L
decoding steps (index lookup, scoring, masked log-softmax and per-query
top-K), teacher forced with the beam states and hidden vectors that a free
running decode of the same batch produced, replayed as one HIP graph.  The
stand-in model's hidden update is outside the timed region (it is timed
separately as part of a full decode).

Prints one JSON line.  `value` is beam expansions per second: one expansion is
one (live beam, valid next token) candidate that is scored, normalised and
offered to the top-K.  `us_per_decode_step` is the mean time of one decoding
step; `pass_ms` gives mean / p50 / p95 / p99 / std over the timed replays.
Per-kernel and per-step times come from event pairs attached to each kernel's
dispatch (hipExtLaunchKernel), i.e. the kernel's own start and end as the GPU
records them, the durations a rocprofv3 kernel trace shows; `roofline` covers
the kernel with the largest share of the pass, with its algorithmic bytes (or
flops) per launch over that mean duration.  `floor` is the overhead floor
(empty kernels, graph nodes) and `copy_gbs` a measured device copy rate.
`cpu_baseline` is the CPU oracle on the host cores (one thread and all the
threads it may use), and `decode_vs_oracle` compares the free-running GPU
decode of the benched batch with the oracle's.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


# Scaling sweeps over the production workload family (L = 8, d = 1024, bf16):
# catalog size at V = 2048, codebook size at 10M items and batch 32, batch size.
SWEEPS = {
    "items": [{"items": n} for n in (100_000, 1_000_000, 10_000_000, 20_000_000, 100_000_000)],
    "codebook": [{"items": 10_000_000, "Q": 32, "V": v} for v in (256, 1024, 2048, 4096, 8192, 16384, 32768)],
    "batch": [{"Q": q} for q in (1, 8, 32, 64, 128, 256)],
    # STATIC's max-branch-factor scaling at |C| = 10^6: rows below the root
    # hold exactly B tokens (L = 3, V = 16,384)
    "branch": [{"config": "branch", "B": b} for b in (8, 16, 32, 64, 128, 256, 512, 1024)],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed passes")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="production")
    ap.add_argument("--K", type=int, default=None, help="beam width other than the workload's (sweeps)")
    ap.add_argument("--items", type=int, default=None, help="catalog size other than the workload's (sweeps)")
    ap.add_argument("--V", type=int, default=None, help="codebook size other than the workload's (sweeps)")
    ap.add_argument("--Q", type=int, default=None, help="batch (queries) other than the workload's (sweeps)")
    ap.add_argument("--B", type=int, default=None, help="branch factor of the 'branch' workload (sweeps)")
    ap.add_argument("--sweep", default=None, choices=sorted(SWEEPS),
                    help="run the named scaling sweep, one child process per point, and print a table")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle time budget")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--path", default="tuned", choices=["tuned", "auto", "dense", "sparse"])
    ap.add_argument("--paths", default=None,
                    help="comma-separated path per step (dense/sparse/sparse_split), no tuning: replays a tuned "
                         "choice without the tuning launches (profiler runs)")
    ap.add_argument("--radix-scoring", default="tuned", choices=["tuned", "chunk", "token"],
                    help="sparse scoring of the radix-selection steps: as tuned, per beam chunk, or by token")
    ap.add_argument("--mode", default="filter_first", choices=["filter_first", "score_first", "unconstrained"],
                    help="decoding variant (the last two run the dense path)")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 256 MiB five times (counter calibration)")
    return ap.parse_args()


def kernel_sources(kernel):
    """Source files that define `kernel` (by its bench name)."""
    main = "radix.hip" if kernel.startswith("radix_") else "kernels.hip"
    return [os.path.join(ROOT, "csr_constrained_beam_amd", "csrc", f) for f in ("device.h", main)]


def kernels_sha1(kernel):
    import hashlib
    h = hashlib.sha1()
    for path in kernel_sources(kernel):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE measurement of the current kernel source, else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernels_sha1") != kernels_sha1(kernel):
        return None
    return rec.get("bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def run_sweep(args):
    """One child bench process per sweep point (each builds its own workload);
    a table on stderr and the list of points as one JSON line."""
    import subprocess
    import tempfile
    rows = []
    for point in SWEEPS[args.sweep]:
        with tempfile.NamedTemporaryFile(suffix=".json", delete=False) as f:
            out = f.name
        cmd = [sys.executable, os.path.abspath(__file__), "--no-cpu", "--steps",
               str(args.steps), "--warmup", str(args.warmup), "--json-out", out, "--mode", args.mode]
        if "config" not in point:
            cmd += ["--config", args.config]
        for k, v in point.items():
            cmd += ["--" + k, str(v)]
        log("sweep %s: %s" % (args.sweep, point))
        rc = subprocess.run(cmd, stdout=subprocess.DEVNULL).returncode
        if rc != 0:
            log("sweep point failed (exit %d): %s" % (rc, point))
            rows.append(dict(point, error=rc))
            break
        with open(out) as f:
            r = json.loads(f.read())
        os.unlink(out)
        rows.append(dict(point, workload=r["config"]["workload"], paths=r["config"]["paths"],
                         ms_per_pass=r["ms_per_step"], us_per_decode_step=r["us_per_decode_step"],
                         expansions_per_pass=r["expansions_per_pass"], expansions_per_s=r["value"],
                         decode_ms=r["decode_ms_as_planned"],
                         decode_ms_persistent=r["decode_ms_with_model_standin"],
                         decode_ms_step_by_step=r["decode_ms_step_by_step"],
                         index_bytes=r["index"]["bytes"], index_build_s=r["index"]["build_s"],
                         n_items=r["index"]["n_items"],
                         step_us=[round(x["kernel_us"]["mean"], 2) for x in r["per_step"]],
                         max_fanout=[x["max_fanout"] for x in r["per_step"]],
                         step_paths=[x["path"] for x in r["per_step"]],
                         sparse_forms=[x["sparse_form"] for x in r["per_step"]],
                         dominant=r["roofline"]["kernel"], dominant_frac=r["roofline"]["frac"]))
        x = rows[-1]
        log("  %s: %.4f ms/pass, %.3g expansions/s, decode %.4f ms, index %.1f MB" % (
            point, x["ms_per_pass"], x["expansions_per_s"], x["decode_ms"], x["index_bytes"] / 1e6))
    line = json.dumps({"sweep": args.sweep, "config": args.config, "points": rows})
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(run with --gpus 1)" % args.gpus, flush=True)
        sys.exit(2)
    if args.sweep:
        return run_sweep(args)

    import torch

    if args.copy_calibration:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}))
        return

    import csr_constrained_beam_amd as cb
    from synth import get_config, make_catalog, make_dense

    over = {k: v for k, v in (("K", args.K), ("n_items", args.items), ("V", args.V), ("Q", args.Q)) if v}
    if args.B:
        over["params"] = dict(get_config(args.config).params, B=args.B)
    cfg = get_config(args.config, **over)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    items = make_catalog(cfg)
    dense = make_dense(cfg)
    log("inputs drawn in %.1f s" % (time.time() - t0))
    t0 = time.time()
    idx = cb.Index(items, cfg.V, device=0)
    build_s = time.time() - t0
    info = [idx.info(t) for t in range(cfg.L)]
    log("index built in %.1f s: %.1f MB" % (build_s, sum(i["bytes"] for i in info) / 1e6))

    es = 2 if cfg.dtype == "bf16" else 4
    if cfg.dtype == "bf16":
        W = torch.from_numpy(dense["W_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        W = torch.from_numpy(dense["W"]).to(dev)
    q = torch.from_numpy(dense["q"]).to(dev)
    P = torch.from_numpy(dense["P"]).to(dev)
    plan = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
    if args.mode != "filter_first":
        plan.set_mode(args.mode)

    # pre-measured path switch (warm-up decode trying both paths per step)
    tune = None
    if args.paths:
        fixed = args.paths.split(",")
        assert len(fixed) == cfg.L, "--paths needs one path per step"
        for t, pth in enumerate(fixed):
            plan.set_path(t, pth)
    elif args.path == "tuned":
        tune = plan.tune(q, P, W, reps=5)
    elif args.path in ("dense", "sparse"):
        for t in range(cfg.L):
            plan.set_path(t, args.path)
    if args.radix_scoring != "tuned":
        for t in range(cfg.L):
            plan.set_option(t, "token_major", 2 if args.radix_scoring == "token" else 1)
    paths = [plan.get_path(t) for t in range(cfg.L)]
    forms = [plan.get_option(t, "sparse_form") for t in range(cfg.L)]
    qsplits = [plan.get_option(t, "query_split") for t in range(cfg.L)]
    tmajor = [plan.get_option(t, "token_major") for t in range(cfg.L)]
    nthreads = [plan.get_option(t, "step_threads") for t in range(cfg.L)]
    log("paths per step:", paths, "sparse form per step (1: per beam):", forms, "workgroups per query:", qsplits,
        "threads:", nthreads, "radix scoring (2: by token):", tmajor)

    # free-running decode: records every step's inputs; also times the full decode
    rec = plan.decode(q, P, W, trace=True)
    torch.cuda.synchronize()

    def time_decodes(fused, n=10):
        plan.set_decode_fusion(fused)
        a = plan.decode(q, P, W)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(n):
            plan.decode(q, P, W)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n, a

    decode_ms_steps, dec_a = time_decodes(False)
    decode_ms, dec_b = time_decodes(True)
    for k in ("seqs", "logp", "rows"):
        assert torch.equal(dec_a[k], dec_b[k]), "persistent decode differs from the step-by-step decode"
    plan.profile_start(capacity=4 * cfg.L * 10)
    plan.decode(q, P, W)
    tail_recs = [r for r in plan.profile_stop() if r["kernel"] == "decode_tail"]
    tail = [r["step"] for r in tail_recs]
    phases = plan.profile_phases()
    plan.set_decode_fusion("auto")
    decode_ms_auto, _ = time_decodes("auto")
    log("decode: %.4f ms step by step, %.4f ms with the persistent tail (from step %s), %.4f ms as the plan "
        "decides" % (decode_ms_steps, decode_ms, tail[0] if tail else "-", decode_ms_auto))
    # wire-format records of the decode's results (one launch after the decode)
    wire_out, _ = cb.wire_results(dec_a["seqs"], dec_a["logp"], cfg.K, 0.6)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(20):
        cb.wire_results(dec_a["seqs"], dec_a["logp"], cfg.K, 0.6, out=wire_out)
    ev1.record()
    torch.cuda.synchronize()
    wire_us = ev0.elapsed_time(ev1) * 1000 / 20
    log("wire-format records: %.2f us per call (%d bytes per query)" % (wire_us, wire_out.shape[1]))
    for ph in phases:
        log("  persistent step %d: selection %.2f us, hidden update %.2f us" % (ph["step"], ph["select_us"],
                                                                             ph["update_us"]))

    L, R, K, Q, d, V = cfg.L, cfg.Q * cfg.K, cfg.K, cfg.Q, cfg.d, cfg.V
    trace_h, trace_rows, trace_acc = rec["trace_h"], rec["trace_rows"], rec["trace_acc"]
    rows_np = trace_rows.cpu().numpy()

    # workload accounting from the library's own tables: a host-side copy of the
    # index, or (catalogs too large to build twice) rows read back from the device
    hidx = cb.Index(items, cfg.V, device=-1) if cfg.n_items <= 50_000_000 else idx
    words = (V + 31) // 32
    steps = []
    for t in range(L):
        live = np.nonzero(rows_np[t] >= 0)[0]
        fan = np.zeros(len(live), np.int64)
        toks = set()
        toks_scored = set()  # sparse paths read W_t rows only for rows of two or more tokens
        for i, b in enumerate(live):
            tk, _ = hidx.row(t, int(rows_np[t][b]))
            if args.mode == "unconstrained":  # every token is a candidate
                tk = np.arange(V)
            fan[i] = len(tk)
            toks.update(tk.tolist())
            if len(tk) > 1:
                toks_scored.update(tk.tolist())
        S = info[t]["max_fanout"]
        Kc = min(K, max(S, 1))
        n_exp = int(fan.sum())
        # a row with one valid token has log-softmax 0 whatever its score: the
        # sparse paths read neither its hidden vector nor its W_t row
        n_scored = int(fan[fan > 1].sum())
        live_scored = int((fan > 1).sum())
        chunks = int(((fan + 63) // 64).sum())
        idx_bytes = len(live) * 8 + (n_exp * 2 if info[t]["storage"] == "csr" else len(live) * words * 4)
        state_bytes = R * 8 + R * Kc * 8
        w_bytes = live_scored * d * es + len(toks_scored) * d * es  # hidden vectors and distinct W_t rows
        steps.append({
            "t": t, "path": paths[t], "sparse_form": forms[t], "query_split": qsplits[t], "step_threads": nthreads[t],
            "token_major": tmajor[t],
            "storage": info[t]["storage"], "live_beams": int(len(live)),
            "expansions": n_exp, "max_fanout": S, "mean_fanout": float(fan.mean()) if len(fan) else 0.0,
            "valid_fraction": n_exp / max(1, len(live) * V), "distinct_tokens": len(toks),
            "bytes": {
                "step_query": R * 8 + idx_bytes + w_bytes + R * 16 + min(R, n_exp) * 8,
                # per-beam expansions also write each survivor's next row and token
                "expand_sparse": state_bytes + R * Kc * 8 + idx_bytes + w_bytes,
                # bitmap rows: the expansion reads whole score rows, writes no side information
                "expand_dense": (state_bytes + idx_bytes + len(live) * V * 4 if info[t]["storage"] == "bitmap"
                                 else state_bytes + R * Kc * 8 + idx_bytes + n_exp * 4),
                "merge": Q * K * Kc * 8 + R * 4 + R * 16 + min(R, n_exp) * 16,
                "gemm_" + cfg.dtype: R * d * es + V * d * es + R * V * 4,
                # radix path: candidates written to HBM as 8-byte keys
                "radix_score_sparse": R * 8 + idx_bytes + w_bytes + n_exp * 8 + chunks * 8,
                "radix_score_dense": R * 8 + idx_bytes + n_exp * 4 + n_exp * 8 + chunks * 8,
                # scores by token: counting sort of the candidates (ranks, lists, offsets),
                # then each distinct W_t row and each scored beam's hidden vector once
                "token_lists": R * 8 + idx_bytes + n_exp * 32 + V * 16,
                "token_score": w_bytes + n_scored * 16,
                # score first: every live beam's whole score row, once; otherwise
                # the chunk pairs of the score pass
                "row_lse": (len(live) * V * 4 + R * 12 if args.mode == "score_first" else chunks * 8 + R * 4),
                "radix_keys": n_exp * 16 + chunks * 8 + len(live) * 4,
                "radix_refine": n_exp * 8,
                "radix_collect": n_exp * 8,
                "radix_sort": min(n_exp, K) * 8 + R * 24,
            },
            "flops": {"gemm_" + cfg.dtype: 2 * len(live) * V * d, "expand_sparse": 2 * d * n_scored,
                      "step_query": 2 * d * n_scored, "radix_score_sparse": 2 * d * n_scored},
            "selection": plan.get_select(t),
        })
    expansions = sum(s["expansions"] for s in steps)
    del hidx

    # teacher-forced pass over all L steps, outputs into fixed buffers
    outs = [tuple(torch.empty(R, dtype=dt, device=dev) for dt in (torch.int32, torch.int32, torch.int32,
                                                                   torch.float32)) for _ in range(L)]

    def one_pass():
        for t in range(L):
            plan.step(t, trace_h[t], W[t], trace_rows[t], trace_acc[t], out=outs[t])

    one_pass()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                one_pass()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                one_pass()
            torch.cuda.synchronize()
        except Exception as e:  # capture not possible: time eager launches
            log("graph capture failed (%s); timing eager launches" % e)
            graph = None
    run = graph.replay if graph is not None else one_pass

    # check the timed pass reproduces the recorded decode (same beams)
    run()
    torch.cuda.synchronize()
    for t in range(L - 1):
        assert torch.equal(outs[t][2], trace_rows[t + 1]), "teacher-forced pass diverged at step %d" % t

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    # the timed region: an event between consecutive replays, so that the
    # whole region's time and each replay's time come from the same run
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        run()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms_per_pass = evs[0].elapsed_time(evs[-1]) / args.steps
    pass_ms = stats([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    log("pass: %.4f ms (p50 %.4f, p99 %.4f)" % (ms_per_pass, pass_ms["p50"], pass_ms["p99"]))

    # score first against filter first on the same batch: share of each
    # query's final items that both orders return (ZeroGR's overlap measure)
    overlap = None
    if args.mode == "score_first":
        ff = idx.plan(cfg.Q, cfg.K, cfg.d, cfg.dtype)
        a = ff.decode(q, P, W)
        b = plan.decode(q, P, W)
        torch.cuda.synchronize()
        sa, ra = a["seqs"].cpu().numpy(), a["rows"].cpu().numpy()
        sb, rb_ = b["seqs"].cpu().numpy(), b["rows"].cpu().numpy()
        fr = []
        for qi in range(Q):
            sl = slice(qi * K, (qi + 1) * K)
            A = {int(x) for x in ra[sl] if x >= 0}
            B = {int(x) for x in rb_[sl] if x >= 0}
            fr.append(len(A & B) / max(1, len(A)))
        overlap = {"mean": float(np.mean(fr)), "min": float(np.min(fr))}
        del ff
        log("score-first vs filter-first item overlap: mean %.4f, min %.4f" % (overlap["mean"], overlap["min"]))

    # per-kernel durations: event pairs attached to each dispatch (its start
    # and end on the GPU), over eager passes of the same inputs
    plan.profile_start(capacity=args.steps * L * 10 + 16)
    for _ in range(args.steps):
        one_pass()
    recs = plan.profile_stop()
    kern = {}
    per_pass_step = np.zeros((args.steps, L))
    per_step_k = [dict() for _ in range(L)]
    seen = [0] * L
    for r in recs:
        t = r["step"]
        k = kern.setdefault(r["kernel"], {"launches": 0, "us": 0.0, "bytes": 0, "flops": 0, "durations": []})
        k["launches"] += 1
        k["us"] += r["us"]
        k["durations"].append(r["us"])
        k["bytes"] += steps[t]["bytes"].get(r["kernel"], 0)
        k["flops"] += steps[t]["flops"].get(r["kernel"], 0)
        kk = per_step_k[t]
        kk[r["kernel"]] = kk.get(r["kernel"], 0.0) + r["us"] / args.steps
    # pass index of each record: records come pass by pass, step by step
    launches_per_pass = len(recs) // args.steps
    for i, r in enumerate(recs[:launches_per_pass * args.steps]):
        per_pass_step[i // launches_per_pass, r["step"]] += r["us"]
    for s_ in steps:
        t = s_["t"]
        s_["kernel_us"] = stats(per_pass_step[:, t].tolist())
        s_["kernels_us"] = {k: round(v, 3) for k, v in per_step_k[t].items()}
    for name, k in kern.items():
        k["mean_us"] = k["us"] / k["launches"]
        k["share"] = k["us"] / sum(x["us"] for x in kern.values())
    dom = max(kern, key=lambda n: kern[n]["us"])
    kd = kern[dom]
    if dom.startswith("gemm"):
        ach = kd["flops"] / (kd["us"] * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": MFMA_PEAK_TFLOPS[cfg.dtype],
                "unit": "TFLOP/s", "frac": ach / MFMA_PEAK_TFLOPS[cfg.dtype],
                "per_launch": kd["flops"] / kd["launches"], "mean_us": kd["mean_us"],
                "traffic": committed_traffic(dom, cfg.name)}
    else:
        ach = kd["bytes"] / (kd["us"] * 1e-6) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "per_launch": kd["bytes"] / kd["launches"], "mean_us": kd["mean_us"],
                "traffic": committed_traffic(dom, cfg.name)}
    roof["timing"] = "dispatch events (kernel start to end on the GPU), eager passes of the benched inputs"
    kernels = {n: {"launches_per_pass": k["launches"] // args.steps, "mean_us": round(k["mean_us"], 3),
                   "p50_us": round(float(np.percentile(k["durations"], 50)), 3),
                   "share": round(k["share"], 4),
                   "GB/s": round(k["bytes"] / (k["us"] * 1e-6) / 1e9, 1),
                   "TFLOP/s": round(k["flops"] / (k["us"] * 1e-6) / 1e12, 2) if k["flops"] else None}
               for n, k in kern.items()}
    kernel_sum_us = sum(k["us"] for k in kern.values()) / args.steps
    log("kernels: %.1f us of dispatch time per pass; dominant %s %.2f us/launch, %.4g %s (%.4f of peak)"
        % (kernel_sum_us, dom, kd["mean_us"], roof["achieved"], roof["unit"], roof["frac"]))

    floor = measure_floor(torch, cb)
    copy_gbs = measure_copy(torch)
    log("floor: graph node of an empty kernel %s; copy %.0f GB/s"
        % (", ".join("%s %.2f us" % (k[len("graph_node_"):-3], v) for k, v in floor.items()), copy_gbs))

    # CPU baseline: the oracle on the host cores, same batch, same L steps; and
    # the free-running GPU decode of this batch against the oracle's
    cpu = None
    vs_oracle = None
    if not args.no_cpu:
        cpu, vs_oracle = cpu_leg(args, cfg, items, dense, rec, L, K, Q, V)

    value = expansions / (ms_per_pass * 1e-3)
    line = {
        "metric": "constrained-decode µs/step and beam-expansions/s; % HBM / MFMA roofline",
        "value": value,
        "unit": "beam-expansions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_pass,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": "%s: %d items, L=%d, V=%d, d=%d, %s W, %d queries x beam %d"
                        % (cfg.name, cfg.n_items, cfg.L, cfg.V, cfg.d, cfg.dtype, cfg.Q, cfg.K),
            "seed": cfg.seed,
            "step": "one teacher-forced pass over all %d decoding steps" % cfg.L,
            "mode": args.mode,
            "graph": graph is not None,
            "paths": paths,
        },
        "us_per_decode_step": ms_per_pass * 1000.0 / L,
        "pass_ms": pass_ms,
        "kernel_us_per_pass": kernel_sum_us,
        "expansions_per_pass": expansions,
        "decode_ms_with_model_standin": decode_ms,
        "decode_ms_step_by_step": decode_ms_steps,
        "decode_ms_as_planned": decode_ms_auto,
        "wire_records_us": wire_us,
        "decode_persistent_chosen_by_tune": plan.get_decode_fusion() if tune is not None else None,
        "decode_persistent_from_step": tail[0] if tail else None,
        "decode_persistent_us": tail_recs[0]["us"] if tail_recs else None,
        "decode_persistent_phases": phases,
        "decode_vs_oracle": vs_oracle,
        "overlap_with_filter_first": overlap,
        "index": index_report(idx, info, build_s, cfg),
        "per_step": steps,
        "kernels": kernels,
        "tune": tune,
        "floor": floor,
        "copy_gbs": copy_gbs,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    for s_ in steps:
        del s_["bytes"], s_["flops"]
    out = json.dumps(line)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(out + "\n")
    print(out, flush=True)


def static_umax(V, n_items, L, d, K1=12, K2=4):
    """STATIC (arXiv 2602.22647) sec. 5.3's upper bound on its index bytes:
    (1/8 + K2) V^d for the d dense-mask levels plus K1 bytes per edge of each
    later level, at most min(V^l, |C|) edges (K1 = 12, K2 = 4 as in its App.
    B.3 capacity planning)."""
    return (0.125 + K2) * float(V) ** d + K1 * sum(min(float(V) ** lv, n_items) for lv in range(d + 1, L + 1))


def index_report(idx, info, build_s, cfg):
    """Index bytes and build time, with STATIC's bound for the same catalog
    shape (its dense levels = the leading bitmap steps here)."""
    n = idx.shape["n_items"]
    total = sum(i["bytes"] for i in info)
    d = 0
    while d < len(info) and info[d]["storage"] == "bitmap":
        d += 1
    um = static_umax(cfg.V, n, cfg.L, d)
    return {"build_s": round(build_s, 2), "bytes": total, "n_items": n, "bytes_per_item": total / max(1, n),
            "rows": [i["n_rows"] for i in info], "storage": [i["storage"] for i in info],
            "static_umax_bytes": um, "static_umax_per_item": um / max(1, n), "static_umax_dense_levels": d}


def stats(xs):
    """mean / p50 / p95 / p99 / std / n of a list of times."""
    a = np.asarray(xs, np.float64)
    return {"mean": float(a.mean()), "p50": float(np.percentile(a, 50)), "p95": float(np.percentile(a, 95)),
            "p99": float(np.percentile(a, 99)), "std": float(a.std()), "n": int(a.size)}


def measure_floor(torch, cb):
    """Overhead floor (FlashTrie's fixed per-launch cost): wall time per node
    of a graph of empty kernels, replayed back to back, at grid shapes the step
    kernels use (64 workgroups of 64 or 1024 threads, 256 and 2048 of 256).
    This is the least a kernel of the graph-replayed pass costs."""
    f = {}
    nodes, reps = 50, 20
    for blocks, threads in ((64, 64), (64, 1024), (256, 256), (2048, 256)):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            cb.floor_probe(blocks, threads, nodes, timed=False)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cb.floor_probe(blocks, threads, nodes, timed=False)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        f["graph_node_%dx%d_us" % (blocks, threads)] = e0.elapsed_time(e1) * 1000.0 / (reps * nodes)
        del g
    return f


def measure_copy(torch):
    """Device-to-device copy of 1 GiB: bytes read plus written per second (GB/s)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_leg(args, cfg, items, dense, rec, L, K, Q, V):
    """The oracle on the host: one thread and all the threads this process may
    use (at most 16, the host share of one GPU), timed per pass over the same
    batch; and the GPU's free-running decode of the batch against the oracle's
    (identical, or diverging only where the step chose between candidates whose
    oracle scores are within 1e-5 relative)."""
    import oracle
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(16, avail))
    t0 = time.time()
    # the pointer trie of 100M 12-token items does not fit the host: sorted ranges instead
    kind = "sorted-range" if cfg.n_items > 50_000_000 else "pointer-trie"
    T = oracle.SortedRange(items, cfg.V) if kind == "sorted-range" else oracle.Trie(items, cfg.V)
    trie_s = time.time() - t0
    bf16 = cfg.dtype == "bf16"
    mkw = {} if args.mode == "filter_first" else {"mode": args.mode}
    r0 = T.decode(K, dense["q"], dense["P"], dense["W"], bf16=bf16, trace=True, threads=threads, **mkw)
    cexp = 0
    for t in range(L):
        for r in r0["trace_rows_in"][t]:
            if r >= 0:
                cexp += V if args.mode == "unconstrained" else len(T.children_of_row(t, int(r))[0])
    runs = {}
    for nth in sorted({1, threads}):
        reps, el = 0, 0.0
        budget = args.cpu_seconds if nth == threads else args.cpu_seconds / 2
        while (el < budget and reps < 1000) or reps == 0:
            t0 = time.time()
            T.decode(K, dense["q"], dense["P"], dense["W"], bf16=bf16, threads=nth, **mkw)
            el += time.time() - t0
            reps += 1
        runs[nth] = (reps, el)
        log("cpu oracle, %d thread(s): %.2f ms per pass (%d passes)" % (nth, 1000 * el / reps, reps))
    reps, el = runs[threads]
    r1, e1 = runs[1]
    cpu = {"value": cexp * reps / el, "unit": "beam-expansions/s", "cores": threads, "kind": "oracle",
           "sample": "the full batch (%d queries x %d steps, %d expansions per pass), %d passes, %.1f s on %d "
                     "threads; %s build (%.1f s) excluded" % (Q, L, cexp, reps, el, threads, kind, trie_s),
           "ms_per_pass": 1000 * el / reps,
           "single_thread": {"value": cexp * r1 / e1, "ms_per_pass": 1000 * e1 / r1, "passes": r1},
           "host_cpus": os.cpu_count(), "affinity_cpus": avail, "cpu_model": cpu_model()}
    vs = None
    if args.mode == "filter_first":
        from tests.parity import decode_vs_oracle
        vs = decode_vs_oracle(T, r0, {k: v.cpu().numpy() for k, v in rec.items() if k in ("trace_rows", "rows", "seqs")},
                              dense["W"], L, K, Q)
        log("decode vs oracle: %s" % vs)
        assert not vs["unexplained"], "free-running GPU decode differs from the oracle away from a near tie"
    return cpu, vs


if __name__ == "__main__":
    main()
