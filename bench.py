#!/usr/bin/env python3
"""Benchmark of the DSA decode step (indexer scores -> exact top-k -> sparse attention)
on one MI355X, through the libdsa C ABI.

One "step" is one decode token through the workload's DSA layers: every stage of
the path (dsa_decode_step) over one batch of synthetic inputs already resident in
HBM. Default workload: 300,000 cached positions, k = 2,048, one query row.

Cold cache by construction: the step cycles through --sets independent input sets
(keys, latent cache, queries), so by the time a set comes back the other sets have
streamed far more than the 256 MB Infinity Cache holds. The timed steps are HIP
graph replays (one graph holds one step per set), bracketed by synchronisations.
A second, eager pass over the same steps has the runtime stamp HIP events with the
start and end of each stage's kernel (dsa_decode_step_timed), which times the
indexer pass and the selection + attention pass live, kernel by kernel; its steps
are queued in chunks behind a short sleep kernel, so they run back to back as in
the graph rather than each starting on an idle GPU.

Prints one JSON line (see the design doc for every field).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode step µs & indexer+gather HBM GB/s, top-2048 at 62k/300k ctx"
HBM_PEAK_GBPS = 8000.0
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_step_ctx300k_hbm_counters.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def device_set(torch, c, s, name):
    """Inputs of rotation set s: set 0 from the shared generator, later sets drawn on the
    GPU with the same distributions (torch generator seeded 9000 + s)."""
    from sparse_attention_decode_scores_amd import inputs
    dev = torch.device("cuda")
    if s == 0:
        d = {}
        for key in ("iq", "iw", "ik"):
            d[key] = torch.from_numpy(np.ascontiguousarray(c[key])).to(dev)
        for key in ("q", "kv"):
            a = np.ascontiguousarray(c[key])
            d[key] = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16
                      else torch.from_numpy(a)).to(dev)
        return d
    g = torch.Generator(device=dev)
    g.manual_seed(9000 + 100 * s + c.get("layer", 0))
    qr, kr = c["qk_range"], c["key_range"]
    w0, w1 = c["w_range"]
    d = {
        "iq": torch.randint(-qr, qr + 1, (c["B"], c["Hi"], c["Di"]), dtype=torch.int8, device=dev, generator=g),
        "iw": torch.randint(w0, w1 + 1, (c["B"], c["Hi"]), dtype=torch.int8, device=dev, generator=g),
        "ik": torch.randint(-kr, kr + 1, (c["N"], c["Di"]), dtype=torch.int8, device=dev, generator=g),
    }
    mul = 1.0 if c["dtype"] == "f32" else 0.5
    for key, shape in (("q", (c["B"], c["Hq"], c["Dk"])), ("kv", (c["N"], c["Dk"]))):
        x = torch.randn(shape, dtype=torch.float32, device=dev, generator=g) * mul
        d[key] = x if c["dtype"] == "f32" else x.to(torch.bfloat16)
    return d


def essential_bytes(c):
    """Algorithmic HBM bytes of one layer: every indexer key once, the scores written,
    the k gathered latent rows, queries, weights and the output."""
    B, N, Di, Dk, Dv, Hq, Hi, k = (c[x] for x in ("B", "N", "Di", "Dk", "Dv", "Hq", "Hi", "k"))
    esz = 4 if c["dtype"] == "f32" else 2
    keys = N * Di
    scores = B * N * 4
    gather = sum(min(k, int(n)) for n in c["ctx_len"]) * Dk * esz
    small = B * Hi * Di + B * Hi + B * Hq * Dk * esz + B * Hq * Dv * 4 + B * k * 4
    return keys, scores, gather, small


def score_kernel_bytes(c):
    """Algorithmic bytes of one launch of the indexer pass: keys read once, queries and
    weights, scores written (the per-position figure is Di + 4*B bytes)."""
    return c["N"] * c["Di"] + c["B"] * c["N"] * 4 + c["B"] * c["Hi"] * (c["Di"] + 1)


def gather_pass_bytes(c):
    """Algorithmic bytes of one launch of the selection + attention pass: the k selected
    latent rows of every query row (Dk values each) and the attention queries. Candidate
    keys and split partials are working data of this design, not counted."""
    esz = 4 if c["dtype"] == "f32" else 2
    rows = sum(min(c["k"], int(n)) for n in c["ctx_len"])
    return rows * c["Dk"] * esz + c["B"] * c["Hq"] * c["Dk"] * esz


def secondary_workload(torch, binding, name, steps, sets):
    """Graph-replayed step time of another workload (GPU-generated inputs only; the
    parity tests cover its correctness): one step = every layer of the workload."""
    from sparse_attention_decode_scores_amd import inputs
    base = dict(inputs.CONFIGS[name])
    layers = base["layers"]
    ctx_len = inputs.ctx_lengths(name)
    data = []
    for st in range(sets):
        per = []
        for l in range(layers):
            c = dict(base, layer=l)
            per.append(device_set(torch, c, 1 + st, name))
        data.append(per)
    B, N, k, Hq, Dv = base["B"], base["N"], base["k"], base["Hq"], base["Dv"]
    ws = binding.new_workspace(B, N, k, Hq, Dv)
    scores = torch.zeros((B, N), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, Dv), dtype=torch.float32, device="cuda")

    def step(st):
        for l in range(layers):
            d = data[st][l]
            binding.dsa_decode_step(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], ctx_len, k, Dv,
                                    base["scale"], scores=scores, idx=idx, out=out, workspace=ws)

    for i in range(2 * sets):
        step(i % sets)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for st in range(sets):
                step(st)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // sets)
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / (reps * sets)
    keys, sc_bytes, gather, small = essential_bytes(dict(base, ctx_len=ctx_len))
    step_bytes = layers * (keys + sc_bytes + gather + small)
    del data
    return {
        "workload": "%s: %d cached positions, k=%d, %d query row(s), %d layers/step (distinct caches)"
                    % (name, N, k, B, layers),
        "us_per_step": round(us, 3),
        "us_per_layer": round(us / layers, 3),
        "step_essential_bytes": step_bytes,
        "step_essential_GBps": round(step_bytes / (us * 1e-6) / 1e9, 1),
        "cache": "cold: %d rotating input sets" % sets,
        "launch": "HIP graph replay of %d step(s) per graph, %d step(s) timed" % (sets, reps * sets),
    }


def measured_traffic(config):
    """HBM bytes per launch of each libdsa kernel from the committed counter summary, or
    None for a kernel whose sources changed since the counters were taken."""
    from sparse_attention_decode_scores_amd.profsum import library_source_sha
    if not os.path.exists(PMC_SUMMARY):
        return {}
    with open(PMC_SUMMARY) as f:
        pmc = json.load(f)
    if pmc.get("kernel_source_sha") != library_source_sha() or pmc.get("config") != config:
        return {}
    return {k: v.get("hbm_bytes_per_launch") for k, v in pmc.get("kernels", {}).items()}


def cpu_baseline(name, layers, budget_s):
    import oracle
    from sparse_attention_decode_scores_amd import inputs
    runs, spent, per_layer = 0, 0.0, []
    layer = 0
    while True:
        c = inputs.make(name, layer % layers)
        t = time.perf_counter()
        oracle.decode_step(c["iq"], c["iw"], c["ik"], c["q"], c["kv"], c["ctx_len"], c["k"], c["Dv"],
                           c["scale"])
        dt = time.perf_counter() - t
        per_layer.append(dt)
        spent += dt
        runs += 1
        layer += 1
        if spent >= budget_s or runs >= 50:
            break
    us_step = float(np.mean(per_layer)) * layers * 1e6
    sample = ("%d oracle decode-step call(s) on layer input(s) of %s (%d positions, k=%d), "
              "%.1f s of CPU work; step = %d layer(s) x mean per-layer time"
              % (runs, name, c["N"], c["k"], spent, layers))
    return {"value": us_step, "unit": "us", "cores": 1, "kind": "oracle", "sample": sample}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--config", default="ctx300k", choices=["ctx16k", "ctx62k_11layers", "ctx300k", "verify8_ctx131k"])
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = default per workload)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--secondary", default="ctx62k_11layers",
                    help="also time this workload (reported beside the headline; 'none' to skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy kernel of 256 MiB (scale reference for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the design for "
              "position-sharding over RCCL is described in DESIGN.md). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    from sparse_attention_decode_scores_amd import binding, inputs

    binding.load_library()
    torch.cuda.set_device(0)
    cfg = inputs.CONFIGS[args.config]
    layers = cfg["layers"]
    R = args.sets or (1 if layers > 1 else 12)
    log("workload", args.config, "layers", layers, "sets", R)

    # inputs: [set][layer]
    host = [inputs.make(args.config, l) for l in range(layers)]
    sets = []
    for s in range(R):
        sets.append([device_set(torch, host[l], s, args.config) for l in range(layers)])
    c = host[0]
    B, N, k, Hq, Dv = c["B"], c["N"], c["k"], c["Hq"], c["Dv"]
    ws = binding.new_workspace(B, N, k, Hq, Dv)
    scores = torch.zeros((B, N), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, Dv), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log("inputs resident: %.2f GB" % (torch.cuda.memory_allocated() / 1e9))

    def step(s, kernel_events=None):
        for l in range(layers):
            d = sets[s][l]
            ev = None if kernel_events is None else kernel_events[l]
            binding.dsa_decode_step(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], host[l]["ctx_len"], k,
                                    Dv, c["scale"], scores=scores, idx=idx, out=out, workspace=ws,
                                    kernel_events=ev)

    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()

    K = args.steps
    graphs = []
    if not args.no_graph:
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            full = torch.cuda.CUDAGraph()
            with torch.cuda.graph(full, stream=stream):
                for s in range(R):
                    step(s)
            tail = None
            if K % R:
                tail = torch.cuda.CUDAGraph()
                with torch.cuda.graph(tail, stream=stream):
                    for s in range(K % R):
                        step(s)
        torch.cuda.synchronize()
        full.replay()
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()
        graphs = [full] * (K // R) + ([tail] if tail is not None else [])

    # ---- timed region: K steps
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    if graphs:
        for g in graphs:
            g.replay()
    else:
        for i in range(K):
            step(i % R)
    e1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    us_step = wall_s * 1e6 / K
    log("timed %d steps: wall %.3f ms, events %.3f ms -> %.2f us/step" % (K, wall_s * 1e3, gpu_ms, us_step))

    # ---- kernel timing pass (eager; events carry each stage kernel's own start and end)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(layers)]
           for _ in range(K)]
    for per_step in evs:  # torch creates the HIP event on first record
        for per_layer in per_step:
            for e in per_layer:
                e.record()
    torch.cuda.synchronize()
    # The host takes longer to issue an eager step than the GPU takes to run it, so
    # steps issued one after another would each start on an idle GPU. Each chunk of
    # steps is therefore queued behind a sleep kernel (longer than the host needs to
    # issue the chunk) and then runs back to back. Every step counts, so these means
    # are the eager pass's means in the kernel trace of the same command.
    chunk = 30
    for i0 in range(0, K, chunk):
        torch.cuda._sleep(16_000_000)  # several ms at the shader clock
        for i in range(i0, min(K, i0 + chunk)):
            step(i % R, evs[i])
    torch.cuda.synchronize()
    st = np.array([[[e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3]), e[4].elapsed_time(e[5])]
                    for e in per_step] for per_step in evs]) * 1e3  # us [K][layers][3]
    score_us = float(st[:, :, 0].mean())
    select_us = float(st[:, :, 1].mean())
    combine_us = float(st[:, :, 2].mean())
    log("kernel durations (eager, HIP events): score %.2f us, select+attend %.2f us, combine %.2f us"
        % (score_us, select_us, combine_us))
    stats = binding.dsa_read_stats(ws, B)

    # reference read rate: a vendor streaming reduction over the same key caches, in the
    # same cold rotation (context for the roofline fraction, not part of the metric)
    rd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4 * R)]
    for i, (r0, r1) in enumerate(rd):
        ikf = sets[i % R][0]["ik"].view(torch.float32)  # the same bytes; values are irrelevant
        r0.record()
        acc = torch.sum(ikf)
        r1.record()
    torch.cuda.synchronize()
    read_us = float(np.mean([r0.elapsed_time(r1) for r0, r1 in rd[R:]])) * 1e3
    read_bytes = c["N"] * c["Di"]

    if args.copy_calibration:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy calibration: 5 x torch.neg over 256 MiB")

    kb = score_kernel_bytes(c)
    achieved = kb / (score_us * 1e-6) / 1e9
    traffic = measured_traffic(args.config)
    gb = gather_pass_bytes(c)
    g_achieved = gb / (select_us * 1e-6) / 1e9
    keys, sc_bytes, gather, small = essential_bytes(c)
    step_bytes = layers * (keys + sc_bytes + gather + small)

    secondary = None
    if args.secondary != "none" and args.secondary != args.config:
        log("secondary workload", args.secondary)
        secondary = secondary_workload(torch, binding, args.secondary, max(8, args.steps // 8), 4)
        log("secondary: %.2f us/step" % secondary["us_per_step"])

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle for about %.0f s" % args.cpu_seconds)
        cpu = cpu_baseline(args.config, layers, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(us_step, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 indexer (int32 accumulate) + bf16 attention (fp32 accumulate)",
        "data": "synthetic (seeded; no model weights or caches)",
        "config": {
            "workload": "%s: %d cached positions, k=%d, %d query row(s), %d layer(s)/step; indexer "
                        "%d heads x %d int8, one shared key per position; attention %d heads over a "
                        "%d-value bf16 latent row (%d output values)"
                        % (args.config, N, k, B, layers, c["Hi"], c["Di"], Hq, c["Dk"], Dv),
            "cache": "cold: %d rotating input sets of %.0f MB each" % (R, layers * (keys + N * c["Dk"] * 2) / 1e6)
                     if R > 1 else "cold: %d layers x %.0f MB streamed per step" % (layers, (keys + N * c["Dk"] * 2) / 1e6),
            "launch": "HIP graph replay of %d step(s) per graph" % R if graphs else "eager launches",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "indexer score pass (k_score_row: int8 MFMA, per-chunk top-m candidates)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic.get("k_score"),
            "algorithmic_bytes_per_launch": kb,
            "launch_us": round(score_us, 3),
        },
        "roofline_gather": {
            "bound": "hbm",
            "kernel": "selection + sparse attention pass (k_select: exact top-k, row gather, split-K attention)",
            "achieved": round(g_achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(g_achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic.get("k_select"),
            "algorithmic_bytes_per_launch": gb,
            "launch_us": round(select_us, 3),
        },
        "cpu_baseline": cpu,
        "secondary": secondary,
        "read_reference": {
            "what": "torch.sum over one layer's key cache (its bytes viewed as fp32), same cold rotation, "
                    "eager; HIP events around each launch, so dispatch latency is included (the "
                    "kernel trace gives the kernel's own time); a streaming-read rate for this buffer",
            "bytes": read_bytes,
            "us": round(read_us, 3),
            "GBps": round(read_bytes / (read_us * 1e-6) / 1e9, 1),
        },
        "kernel_us_events": {"score": round(score_us, 3), "select_attend": round(select_us, 3),
                                   "combine": round(combine_us, 3)},
        "step_essential_bytes": step_bytes,
        "step_essential_GBps": round(step_bytes / (us_step * 1e-6) / 1e9, 1),
        "selection_paths": [s["path"] for s in stats],
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
