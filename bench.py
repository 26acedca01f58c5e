#!/usr/bin/env python3
"""Benchmark of the DSA decode step (indexer scores -> exact top-k -> sparse attention)
on one MI355X, through the libdsa C ABI.

One "step" is one decode token through the workload's DSA layers: every stage of
the path (dsa_decode_step) over one batch of synthetic inputs already resident in
HBM. Default workload: 300,000 cached positions, k = 2,048, one query row.

Cold cache by construction: the step cycles through --sets independent input sets
(keys, latent cache, queries), so by the time a set comes back the other sets have
streamed far more than the 256 MB Infinity Cache holds.

Timings, all on the stream the library launches on:
  - value: K steps as HIP graph replays (one graph holds one step per input set),
    bracketed by synchronisations; mean microseconds per step.
  - kernel durations: an eager pass of the same steps in which the runtime stamps
    HIP events with each stage kernel's own dispatch start and end
    (dsa_decode_step_timed), queued in chunks behind a sleep kernel so that the
    kernels run back to back as in the graph. These feed the roofline figures.
    (Events recorded inside a graph are not restamped on replay, so per-kernel
    times come from this pass.)
  - step_stats: the per-step mean of each replay of the R-step graph, HIP events
    between the replays: median, p10, p90 over replays. (eager_step_span: from the
    eager pass, per step the span from its first kernel's start to its last
    kernel's end, eager launch gaps included.)
  - legs: the forced exhaustive path on the headline workload (and the stand-alone
    exhaustive selection over every position, the path of rows without candidates),
    the 62k-context 11-layer step, the 8-row verify block and the headline workload
    over an FP8 E4M3 latent cache (bf16 queries; the gather reads half the bytes),
    each as graph replays plus the eager kernel pass.
  - cpu_baseline: the CPU oracle on the headline workload, single-threaded and with
    its all-core OpenMP build, per stage, median of 5 after one warm-up.

Prints one JSON line.
"""
import argparse
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode step µs & indexer+gather HBM GB/s, top-2048 at 62k/300k ctx"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 matrix-core peak (5.0 POPS)
POOL_PAGES = 4096           # paged leg: a 1,048,576-token pool of 256-position pages
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_step_ctx300k_hbm_counters.json")

# The pages' own figures, with their hardware (context, not targets).
CONTEXT = {
    "ds4 glm53-m3ultra branch post (rising, 2026-09-09), long-context paragraph": [
        "Apple M3 Ultra, 80 GPU cores, Metal, GLM-5.3-Flash at 4 bits: the rewritten DSA selection "
        "(parallel narrowing scans, then a small sort) saves about 1 ms per generated token",
        "same machine, 300k-token context, end to end (all of the branch's changes): 21.6 -> 37.4 "
        "tokens/s",
        "same machine, 62k-token context, end to end (mostly decode fusion): 24 -> 38 tokens/s",
    ],
    "derived here": [
        "1 ms per token over the model's 11 DSA layers is about 90 us of selection per layer per token "
        "on the M3 Ultra, if each layer selects once per token",
    ],
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- inputs and bytes

def device_set(torch, c, s):
    """Inputs of rotation set s: set 0 from the shared generator, later sets drawn on the
    GPU with the same distributions (torch generator seeded 9000 + 100 s + layer)."""
    dev = torch.device("cuda")
    if s == 0:
        d = {}
        for key in ("iq", "iw", "ik"):
            d[key] = torch.from_numpy(np.ascontiguousarray(c[key])).to(dev)
        for key in ("q", "kv"):
            a = np.ascontiguousarray(c[key])
            if a.dtype == np.uint16:  # bf16 bit patterns
                t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
            elif a.dtype == np.uint8:  # FP8 E4M3 codes
                t = torch.from_numpy(a).view(torch.float8_e4m3fn)
            else:
                t = torch.from_numpy(a)
            d[key] = t.to(dev)
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
        if c["dtype"] == "f32":
            d[key] = x
        elif c["dtype"] == "fp8" and key == "kv":
            d[key] = x.to(torch.float8_e4m3fn)
        else:
            d[key] = x.to(torch.bfloat16)
    return d


def esz(c):
    """Bytes per latent-cache value."""
    return {"f32": 4, "bf16": 2, "fp8": 1}[c["dtype"]]


def qsz(c):
    """Bytes per attention-query value."""
    return 4 if c["dtype"] == "f32" else 2


def rows_gathered(c):
    return sum(min(c["k"], int(n)) for n in c["ctx_len"])


def score_kernel_bytes(c):
    """Algorithmic bytes of one indexer pass: every key read once, plus the queries and
    head weights (Di bytes per position, B*Hi*(Di+1) per launch). The int32 scores it
    writes (4*B bytes per position) are as-built working data, reported apart."""
    return c["N"] * c["Di"] + c["B"] * c["Hi"] * (c["Di"] + 1)


def gather_pass_bytes(c):
    """Algorithmic bytes of one selection + attention pass: the k selected latent rows
    of every query row (Dk values each) and the attention queries."""
    return rows_gathered(c) * c["Dk"] * esz(c) + c["B"] * c["Hq"] * c["Dk"] * qsz(c)


def step_essential_bytes(c):
    """Essential HBM bytes of one layer: keys once, the gathered rows, queries, head
    weights and the attention output (scores and indices are working data)."""
    return (c["N"] * c["Di"] + c["B"] * c["Hi"] * (c["Di"] + 1) + rows_gathered(c) * c["Dk"] * esz(c)
            + c["B"] * c["Hq"] * c["Dk"] * qsz(c) + c["B"] * c["Hq"] * c["Dv"] * 4)


def indexer_int_ops(c):
    """Integer operations of the indexer contraction: a multiply and an add per query
    head, dim and scored position."""
    return 2 * c["Hi"] * c["Di"] * sum(int(n) for n in c["ctx_len"])


# ---------------------------------------------------------------- timing helpers

class Runner:
    """One workload's rotating input sets and outputs, and its timing passes."""

    def __init__(self, torch, binding, name, sets, host_set0=True, paged=False):
        from sparse_attention_decode_scores_amd import inputs
        self.torch, self.binding, self.name = torch, binding, name
        self.paged = paged
        base = dict(inputs.CONFIGS[name])
        self.layers = base["layers"]
        self.hosts = []
        if host_set0:
            self.hosts = [inputs.make(name, l) for l in range(self.layers)]
            self.c = self.hosts[0]
        else:
            self.c = dict(base, ctx_len=inputs.ctx_lengths(name), layer=0)
        self.R = sets
        self.data = []
        for s in range(sets):
            per = []
            for l in range(self.layers):
                c = self.hosts[l] if host_set0 else dict(self.c, layer=l)
                per.append(device_set(torch, c, s if host_set0 else s + 1))
            self.data.append(per)
        if paged:
            self.to_pools()
        c = self.c
        self.ws = binding.new_workspace(c["B"], c["N"], c["k"], c["Hq"], c["Dv"])
        self.scores = torch.zeros((c["B"], c["N"]), dtype=torch.int32, device="cuda")
        self.idx = torch.empty((c["B"], c["k"]), dtype=torch.int32, device="cuda")
        self.out = torch.empty((c["B"], c["Hq"], c["Dv"]), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

    def to_pools(self):
        """Moves every (set, layer) cache into a pair of paged pools of its own, each the size
        of the 1,048,576-token pool of 4,096 pages of 256 positions (at least the
        sequence's pages). The rotating sets stand for the layers of one sequence, which
        share its page table: the sequence takes ceil(N / 256) of the pool's pages in a
        seeded random order (scattered over the pool, the rest left to other sequences),
        and every set's caches are laid out by that one table."""
        torch, c = self.torch, self.c
        page = self.binding.PAGE_SIZE
        n_tab = (c["N"] + page - 1) // page
        pool_pages = max(POOL_PAGES, n_tab)
        g = torch.Generator(device="cuda")
        g.manual_seed(7700)
        pos = torch.arange(c["N"], device="cuda", dtype=torch.int64)
        table = torch.randperm(pool_pages, generator=g, device="cuda")[:n_tab].to(torch.int32).contiguous()
        rows = table[pos // page].to(torch.int64) * page + pos % page
        for d in (d for per in self.data for d in per):
            ik, kv = d.pop("ik"), d.pop("kv")
            d["ik_pool"] = torch.zeros((pool_pages * page, c["Di"]), dtype=torch.int8, device="cuda")
            d["kv_pool"] = torch.zeros((pool_pages * page, c["Dk"]), dtype=kv.dtype, device="cuda")
            d["ik_pool"].index_copy_(0, rows, ik)
            d["kv_pool"].index_copy_(0, rows, kv)
            d["page_table"] = table
            del ik, kv
        self.pool_pages = pool_pages
        torch.cuda.synchronize()

    def bytes_per_set(self):
        c = self.c
        return self.layers * (c["N"] * c["Di"] + c["N"] * c["Dk"] * esz(c))

    def step(self, s, flags=0, kernel_events=None):
        c = self.c
        for l in range(self.layers):
            d = self.data[s][l]
            ev = None if kernel_events is None else kernel_events[l]
            if self.paged:
                self.binding.dsa_decode_step_paged(d["iq"], d["iw"], d["ik_pool"], d["q"], d["kv_pool"],
                                                   d["page_table"], c["ctx_len"], c["k"], c["Dv"], c["scale"],
                                                   N=c["N"], scores=self.scores, idx=self.idx, out=self.out,
                                                   workspace=self.ws, flags=flags, kernel_events=ev)
                continue
            self.binding.dsa_decode_step(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], c["ctx_len"], c["k"],
                                         c["Dv"], c["scale"], scores=self.scores, idx=self.idx, out=self.out,
                                         workspace=self.ws, flags=flags, kernel_events=ev)

    def capture(self, sets, flags=0):
        torch = self.torch
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for s in sets:
                    self.step(s, flags)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        return g

    def graph_us(self, steps, flags=0):
        """Mean us per step over `steps` graph-replayed steps (R steps per graph)."""
        torch = self.torch
        full = self.capture(range(self.R), flags)
        reps = max(1, steps // self.R)
        full.replay()  # the first replay uploads the graph: not timed
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            full.replay()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / (reps * self.R)
        del full
        return us, reps * self.R

    def full_row_select_us(self, calls):
        """Mean time of a forced stand-alone selection over the last step's scores (no
        candidate pass: the exhaustive path over every position), `calls` launches queued
        back to back behind a sleep kernel between two HIP events (gaps included)."""
        torch, c = self.torch, self.c
        ws = self.binding.new_workspace(c["B"], c["N"], c["k"], 1, 1)
        idx = torch.empty((c["B"], c["k"]), dtype=torch.int32, device="cuda")
        sel = lambda: self.binding.dsa_topk_select(self.scores, c["ctx_len"], c["k"], idx=idx, workspace=ws,
                                                   flags=self.binding.FLAG_FORCE_FALLBACK)
        sel()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)
        e0.record()
        for _ in range(calls):
            sel()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / calls

    def replay_stats(self, reps, flags=0):
        """Per-step mean of each replay of an R-step graph (HIP events between the replays on
        the replay stream): the distribution over replays of the graph-replayed step time."""
        torch = self.torch
        full = self.capture(range(self.R), flags)
        stream = torch.cuda.Stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        with torch.cuda.stream(stream):
            torch.cuda._sleep(20_000_000)  # lets the host queue the replays ahead of the GPU
            ev[0].record()
            for i in range(reps):
                full.replay()
                ev[i + 1].record()
        torch.cuda.synchronize()
        del full
        return summary([ev[i].elapsed_time(ev[i + 1]) * 1e3 / self.R for i in range(reps)])

    def kernel_us(self, steps, flags=0, chunk=30):
        """Mean duration of each stage's kernels (us): score, select+attend, combine,
        from events the runtime stamps with each dispatch's own start and end; and per
        step the span from its first kernel's start to its last kernel's end."""
        torch = self.torch
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(self.layers)]
               for _ in range(steps)]
        for per_step in evs:  # torch creates the HIP event on first record
            for per_layer in per_step:
                for e in per_layer:
                    e.record()
        torch.cuda.synchronize()
        # the host takes longer to issue an eager step than the GPU takes to run it: each
        # chunk is queued behind a sleep kernel and then runs back to back
        for i0 in range(0, steps, chunk):
            torch.cuda._sleep(16_000_000)
            for i in range(i0, min(steps, i0 + chunk)):
                self.step(i % self.R, flags, evs[i])
        torch.cuda.synchronize()
        st = np.array([[[e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3]), e[4].elapsed_time(e[5])]
                        for e in per_step] for per_step in evs]) * 1e3  # [steps][layers][3]
        spans = [per_step[0][0].elapsed_time(per_step[-1][5]) * 1e3 for per_step in evs]
        self.last_spans = spans
        return [float(st[:, :, i].mean()) for i in range(3)]

    def host_issue_us(self, calls=300):
        """Host time to issue one eager dsa_decode_step: the C entry point called through
        ctypes with arguments marshalled once, `calls` times in a row behind a sleep kernel
        (the GPU runs none of them meanwhile, so the wall time is the host's own: argument
        checks, launch planning and three kernel launches)."""
        torch, c = self.torch, self.c
        d = self.data[0][0]
        if self.paged:
            return None
        step = self.binding.prepared_decode_step(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], c["ctx_len"], c["k"],
                                                 c["Dv"], c["scale"], self.scores, self.idx, self.out, self.ws)
        step()
        torch.cuda.synchronize()
        torch.cuda._sleep(50_000_000)
        t0 = time.perf_counter()
        for _ in range(calls):
            step()
        us = (time.perf_counter() - t0) * 1e6 / calls
        torch.cuda.synchronize()
        return us

    def paths(self):
        return [s["path"] for s in self.binding.dsa_read_stats(self.ws, self.c["B"])]


def describe(c, name, layers):
    return ("%s: %d cached positions, k=%d, %d query row(s), %d layer(s)/step; indexer %d heads x %d int8, "
            "one shared key per position; attention %d heads over a %d-value %s latent row (%d output values)"
            % (name, c["N"], c["k"], c["B"], layers, c["Hi"], c["Di"], c["Hq"], c["Dk"],
               "fp8 e4m3 (bf16 queries)" if c["dtype"] == "fp8" else c["dtype"], c["Dv"]))


def summary(t):
    t = np.array(t)
    return {"median_us": round(float(np.median(t)), 3), "p10_us": round(float(np.percentile(t, 10)), 3),
            "p90_us": round(float(np.percentile(t, 90)), 3), "mean_us": round(float(t.mean()), 3),
            "n": int(t.size)}


def measured_traffic(config):
    """HBM bytes per launch of each libdsa kernel from the committed counter summary, or
    {} when a kernel source changed since the counters were taken."""
    from sparse_attention_decode_scores_amd.profsum import library_source_sha
    if not os.path.exists(PMC_SUMMARY):
        return {}
    with open(PMC_SUMMARY) as f:
        pmc = json.load(f)
    if pmc.get("kernel_source_sha") != library_source_sha() or pmc.get("config") != config:
        return {}
    return {k: v.get("hbm_bytes_per_launch") for k, v in pmc.get("kernels", {}).items()}


# ---------------------------------------------------------------- CPU baseline

def cpu_model():
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(name, reps=5):
    """The oracle on one layer of the workload: per stage and whole step, median of
    `reps` runs after one warm-up, single-threaded and with the OpenMP build."""
    import oracle
    from sparse_attention_decode_scores_amd import inputs
    c = inputs.make(name, 0)
    out = {}
    for omp in (False, True):
        stages = {"index_scores": [], "topk_select": [], "sparse_attn": []}
        for r in range(reps + 1):
            t0 = time.perf_counter()
            s = oracle.index_scores(c["iq"], c["iw"], c["ik"], c["ctx_len"], omp=omp)
            t1 = time.perf_counter()
            i = oracle.topk_select(s, c["ctx_len"], c["k"], omp=omp)
            t2 = time.perf_counter()
            oracle.sparse_attn(c["q"], c["kv"], i, c["Dv"], c["scale"], omp=omp)
            t3 = time.perf_counter()
            if r > 0:  # run 0 warms up
                stages["index_scores"].append(t1 - t0)
                stages["topk_select"].append(t2 - t1)
                stages["sparse_attn"].append(t3 - t2)
        tot = np.sum([stages[k] for k in stages], axis=0)
        out[omp] = {"value": round(float(np.median(tot)) * 1e6, 1),
                    "stages_us": {k: round(float(np.median(v)) * 1e6, 1) for k, v in stages.items()},
                    "cores": oracle.threads(omp)}
    layers = inputs.CONFIGS[name]["layers"]
    single, allc = out[False], out[True]
    return {
        "value": single["value"] * layers, "unit": "us", "cores": single["cores"], "kind": "oracle",
        "sample": ("one layer of %s (%d positions, k=%d), each stage timed, median of %d runs after one "
                   "warm-up; value = that step time x %d layer(s)" % (name, c["N"], c["k"], reps, layers)),
        "stages_us": single["stages_us"],
        "all_cores": {"value": allc["value"] * layers, "unit": "us", "cores": allc["cores"],
                      "build": "the same oracle source with -fopenmp (positions and heads split over "
                               "threads; the sort sequential)", "stages_us": allc["stages_us"]},
        "cpu_model": cpu_model(), "nproc": os.cpu_count(),
    }


# ---------------------------------------------------------------- legs

def kernel_figures(c, score_us, select_us, combine_us):
    sb, gb = score_kernel_bytes(c), gather_pass_bytes(c)
    return {"score_us": round(score_us, 3), "select_attend_us": round(select_us, 3),
            "combine_us": round(combine_us, 3),
            "indexer_GBps": round(sb / (score_us * 1e-6) / 1e9, 1),
            "indexer_frac_of_hbm_peak": round(sb / (score_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "gather_GBps": round(gb / (select_us * 1e-6) / 1e9, 1),
            "gather_frac_of_hbm_peak": round(gb / (select_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def leg(torch, binding, name, steps, sets, paged=False):
    log("leg", name, "(paged pools)" if paged else "")
    r = Runner(torch, binding, name, sets, host_set0=False, paged=paged)
    for i in range(2 * sets):
        r.step(i % sets)
    torch.cuda.synchronize()
    us, n = r.graph_us(steps)
    k = r.kernel_us(max(8, steps // 2))
    c = r.c
    res = {"workload": describe(c, name, r.layers) + (
               "; each input set's caches in pools of %d 256-position pages (the 1,048,576-token pool), "
               "laid out by one page table (the sets stand for the layers of one sequence), the "
               "sequence's pages in a seeded random order over the pool" % r.pool_pages
               if paged else ""), "us_per_step": round(us, 3),
           "us_per_layer": round(us / r.layers, 3), "steps": n,
           "cache": "cold: %d rotating input sets of %.0f MB" % (sets, r.bytes_per_set() / 1e6),
           "kernels_per_layer": kernel_figures(c, *k),
           "step_essential_GBps": round(r.layers * step_essential_bytes(c) / (us * 1e-6) / 1e9, 1)}
    if c["B"] > 1:
        ops = indexer_int_ops(c)
        tops = ops / (k[0] * 1e-6) / 1e12
        res["indexer_int8_TOPS"] = round(tops, 1)
        res["indexer_frac_of_int8_peak"] = round(tops / INT8_PEAK_TOPS, 4)
        res["indexer_int_ops_per_launch"] = ops
    log("leg %s: %.2f us/step" % (name, us))
    del r
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--config", default="ctx300k",
                    choices=["ctx16k", "ctx62k_11layers", "ctx300k", "verify8_ctx131k", "verify16_ctx131k",
                             "ctx300k_fp8kv"])
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = default per workload)")
    ap.add_argument("--legs", default="fallback,ctx62k_11layers,verify8_ctx131k,verify16_ctx131k,ctx300k_fp8kv,"
                                      "ctx300k_paged,verify8_ctx131k_paged",
                    help="comma list of extra legs, or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy kernel of 256 MiB (scale reference for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (DESIGN.md describes how "
              "the path would shard by position over RCCL). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from sparse_attention_decode_scores_amd import binding, inputs

    binding.load_library()
    torch.cuda.set_device(0)
    cfg = inputs.CONFIGS[args.config]
    R = args.sets or (4 if cfg["layers"] > 1 else 12)
    log("workload", args.config, "layers", cfg["layers"], "sets", R)
    run = Runner(torch, binding, args.config, R)
    c = run.c
    log("inputs resident: %.2f GB" % (torch.cuda.memory_allocated() / 1e9))

    for i in range(args.warmup):
        run.step(i % R)
    torch.cuda.synchronize()

    # ---- timed region: K graph-replayed steps
    K = args.steps
    full = run.capture(range(R))
    tail = run.capture(range(K % R)) if K % R else None
    graphs = [full] * (K // R) + ([tail] if tail is not None else [])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    us_step = (time.perf_counter() - t0) * 1e6 / K
    log("timed %d steps: %.2f us/step" % (K, us_step))
    del graphs, full, tail

    replays = run.replay_stats(max(20, K // R))
    log("graph replays: per-step median %.2f us (p10 %.2f, p90 %.2f) over %d replays of %d steps"
        % (replays["median_us"], replays["p10_us"], replays["p90_us"], replays["n"], R))
    score_us, select_us, combine_us = run.kernel_us(K)
    spans = summary(run.last_spans)
    log("kernel durations (eager, dispatch-stamped events): score %.2f us, select+attend %.2f us, "
        "combine %.2f us; per-step span median %.2f us (p10 %.2f, p90 %.2f)"
        % (score_us, select_us, combine_us, spans["median_us"], spans["p10_us"], spans["p90_us"]))
    paths = run.paths()
    issue_us = run.host_issue_us()
    log("host time to issue one eager step: %.2f us" % issue_us)

    fallback = None
    legs = [x for x in args.legs.split(",") if x and x != "none"]
    if "fallback" in legs:
        f_us, f_n = run.graph_us(max(R, K // 5), flags=binding.FLAG_FORCE_FALLBACK)
        f_paths = run.paths()
        fk = run.kernel_us(max(R, K // 10), flags=binding.FLAG_FORCE_FALLBACK)
        full_us = run.full_row_select_us(max(R, K // 10))
        fallback = {"us_per_step": round(f_us, 3), "steps": f_n, "ratio_to_candidate_path": round(f_us / us_step, 3),
                    "paths": f_paths, "select_attend_us": round(fk[1], 3),
                    "what": "the same workload with DSA_FLAG_FORCE_FALLBACK, graph replay: the exhaustive "
                            "path for every row (threshold from the candidate union, the union's keys plus "
                            "rescans of the chunks whose best dropped key reaches it, exact top-k, the "
                            "attention window from that list)",
                    "full_row_select_us": round(full_us, 3),
                    "full_row_what": "dsa_topk_select with DSA_FLAG_FORCE_FALLBACK on the same scores (no "
                                     "candidate pass: sampled threshold, one streamed pass over every "
                                     "position, exact top-k, ranking; the path of rows without "
                                     "candidates), mean per call of back-to-back calls queued behind a "
                                     "sleep kernel between two HIP events (launch gaps included)"}
        log("forced fallback: %.2f us/step; full-row exhaustive selection %.2f us" % (f_us, full_us))

    # reference read rate: a vendor streaming reduction over the same key caches, in the same
    # cold rotation (context for the roofline fraction, not part of the metric)
    rd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4 * R)]
    for i, (r0, r1) in enumerate(rd):
        ikf = run.data[i % R][0]["ik"].view(torch.float32)  # the same bytes; values are irrelevant
        r0.record()
        torch.sum(ikf)
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
        del src, dst

    layers = run.layers
    cache = ("cold: %d rotating input sets of %.0f MB each" % (R, run.bytes_per_set() / 1e6))
    del run
    torch.cuda.empty_cache()

    leg_out = {}
    for name in legs:
        if name in ("ctx62k_11layers", "verify8_ctx131k", "verify16_ctx131k", "ctx300k_fp8kv") and name != args.config:
            leg_out[name] = leg(torch, binding, name, max(16, K // 8), 4)
        elif name == "ctx300k_paged":
            leg_out[name] = leg(torch, binding, "ctx300k", max(16, K // 8), R, paged=True)
        elif name == "verify8_ctx131k_paged":
            leg_out[name] = leg(torch, binding, "verify8_ctx131k", max(16, K // 8), 4, paged=True)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: the oracle, single-threaded and all-core, median of 5")
        cpu = cpu_baseline(args.config)

    kb = score_kernel_bytes(c)
    achieved = kb / (score_us * 1e-6) / 1e9
    traffic = measured_traffic(args.config)
    gb = gather_pass_bytes(c)
    g_achieved = gb / (select_us * 1e-6) / 1e9
    sb = layers * step_essential_bytes(c)
    budget_us = sb / (0.7 * HBM_PEAK_GBPS * 1e9) * 1e6
    timing_note = ("duration: mean over the eager pass of dispatch-stamped HIP events on the launch stream "
                   "(kernels run back to back as in the graph; the rocprofv3 kernel trace of the same "
                   "command lists the graph-replayed launches beside them)")
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
        "dtype": ("int8 indexer (int32 accumulate) + bf16 attention (fp32 accumulate)"
                  + (" over an FP8 E4M3 latent cache" if c["dtype"] == "fp8" else "")),
        "data": "synthetic (seeded; no model weights or caches)",
        "config": {"workload": describe(c, args.config, layers), "cache": cache,
                   "launch": "HIP graph replay of %d step(s) per graph" % R},
        "step_stats": dict(replays, how="per-step mean of each replay of the %d-step graph (HIP events "
                                        "between replays queued behind a sleep kernel; events recorded "
                                        "inside a graph are not restamped on replay)" % R),
        "eager_step_span": dict(spans, how="per step of the eager kernel pass: first kernel's start to last "
                                           "kernel's end, dispatch-stamped events (includes the eager "
                                           "launch gaps that the graph removes)"),
        "roofline": {
            "bound": "hbm",
            "kernel": "indexer score pass (k_score_row: int8 MFMA, per-chunk top-m candidates)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic.get("k_score"),
            "algorithmic_bytes_per_launch": kb,
            "algorithmic_bytes": "every indexer key once (N*Di) + queries and head weights (B*Hi*(Di+1))",
            "as_built_score_write_bytes": c["B"] * c["N"] * 4,
            "launch_us": round(score_us, 3),
            "timing": timing_note,
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
        "roofline_step": {
            "bound": "hbm",
            "essential_bytes": sb,
            "achieved": round(sb / (us_step * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(sb / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "us_at_70pct_of_peak": round(budget_us, 3),
            "x_over_that": round(us_step / budget_us, 2),
        },
        "kernel_us_events": {"score": round(score_us, 3), "select_attend": round(select_us, 3),
                             "combine": round(combine_us, 3)},
        "fallback": fallback,
        "legs": leg_out,
        "cpu_baseline": cpu,
        "read_reference": {
            "what": "torch.sum over one layer's key cache (its bytes viewed as fp32), same cold rotation, "
                    "eager, HIP events around each launch (dispatch latency included): a streaming-read "
                    "rate for this buffer",
            "bytes": read_bytes,
            "us": round(read_us, 3),
            "GBps": round(read_bytes / (read_us * 1e-6) / 1e9, 1),
        },
        "host_issue_us": {"us": round(issue_us, 2),
                          "how": "dsa_decode_step called through ctypes with its arguments marshalled "
                                 "once, 300 calls in a row while the GPU runs a sleep kernel: the host's "
                                 "own cost per eager step (checks, planning, three launches)"},
        "selection_paths": paths,
        "context": CONTEXT,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
