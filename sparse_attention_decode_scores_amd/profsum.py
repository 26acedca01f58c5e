"""Summaries of rocprofv3 results for the libdsa kernels (host-side, no GPU needed).

Reads the rocpd SQLite databases that `rocprofv3 -d DIR -o NAME` writes
(DIR/NAME_results.db) and writes short text summaries:

  stats     per-kernel dispatch count and duration of a --kernel-trace --stats run
  counters  HBM bytes per dispatch of each libdsa kernel from two --pmc runs (FETCH_SIZE,
            then WRITE_SIZE), each scaled by what the same counter reads for a plain
            copy kernel of known size run in the same process (torch.neg over 64 Mi fp32
            values: 256 MiB read, 256 MiB written)
  mfma      matrix-core work and busy time per dispatch of each libdsa kernel from one
            --pmc run of SQ_INSTS_VALU_MFMA_MOPS_I8, SQ_VALU_MFMA_BUSY_CYCLES and
            GRBM_GUI_ACTIVE

The counter summary records a hash of the kernel sources (csrc/) it was taken from;
a reader treats it as stale once they change.
"""
import argparse
import glob
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = sorted(
    os.path.relpath(p, ROOT) for p in glob.glob(os.path.join(ROOT, "sparse_attention_decode_scores_amd", "csrc", "*"))
    if p.endswith((".hip", ".h")))
LIB_KERNELS = ("k_score", "k_select", "k_combine", "k_chunk_cand", "k_attend_idx")
COPY_MATCH = "neg_kernel"
COPY_BYTES = 64 * 1024 * 1024 * 4  # read and written by one calibration dispatch


def library_source_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(p.encode())
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _db(path):
    if os.path.isdir(path):
        found = sorted(glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True))
        if not found:
            raise SystemExit("no *_results.db under %s" % path)
        path = found[-1]
    return sqlite3.connect("file:%s?mode=ro" % path, uri=True)


def short_name(name):
    for k in LIB_KERNELS:
        if "dsa::" + k in name:
            return k
    return None


def kernel_stats(db):
    """Per (kernel, grid) rows: one kernel launched with different grids (different
    workloads in one run) is listed once per grid."""
    con = _db(db)
    rows = con.execute("SELECT name, grid_x * grid_y * grid_z, workgroup_x * workgroup_y * workgroup_z, "
                       "COUNT(*), AVG(end - start), MIN(end - start), MAX(end - start), SUM(end - start) "
                       "FROM kernels GROUP BY name, grid_x, grid_y, grid_z "
                       "ORDER BY SUM(end - start) DESC").fetchall()
    total = sum(r[7] for r in rows) or 1
    return [{"name": r[0], "grid": r[1], "block": r[2], "calls": r[3], "avg_us": r[4] / 1e3,
             "min_us": r[5] / 1e3, "max_us": r[6] / 1e3, "pct": 100.0 * r[7] / total} for r in rows]


def kernel_passes(db, split):
    """Per library kernel (and grid), the mean duration of consecutive groups of its
    calls in start order: split is [(label, count), ...], the passes of the command
    in the order they ran."""
    con = _db(db)
    calls = {}
    for name, grid, dur in con.execute("SELECT name, grid_x * grid_y * grid_z, end - start FROM kernels "
                                       "ORDER BY start"):
        if short_name(name) is not None:
            calls.setdefault((name, grid), []).append(dur)
    out = []
    for (name, grid), durs in calls.items():
        i = 0
        for label, n in split:
            part = durs[i:i + n]
            i += n
            if part:
                out.append({"name": name, "grid": grid, "pass": label, "calls": len(part),
                            "avg_us": sum(part) / len(part) / 1e3})
    return out


def counter_per_kernel(db, counter):
    """{kernel name: (dispatches, mean value per dispatch)} for one counter (KiB for *_SIZE)."""
    con = _db(db)
    rows = con.execute("SELECT kernel_name, dispatch_id, SUM(value) FROM counters_collection "
                       "WHERE counter_name = ? GROUP BY kernel_name, dispatch_id", (counter,)).fetchall()
    acc = {}
    for name, _, v in rows:
        n, s = acc.get(name, (0, 0.0))
        acc[name] = (n + 1, s + float(v))
    return {k: (n, s / n) for k, (n, s) in acc.items()}


def _copy_value(per_kernel, counter):
    cands = [(n, v) for k, (n, v) in per_kernel.items() if COPY_MATCH in k]
    if not cands:
        raise SystemExit("no %s dispatch (%s) in the %s run; kernels seen: %s"
                         % (COPY_MATCH, "calibration copy", counter, sorted(per_kernel)[:20]))
    n = sum(c[0] for c in cands)
    return n, sum(c[0] * c[1] for c in cands) / n


def cmd_stats(args):
    rows = kernel_stats(args.db)
    lines = ["# Kernel durations: %s" % args.title, "",
             "Command (from the repository root on the GPU host):", "", "```", args.command, "```", "",
             "| kernel | grid threads | calls | avg us | min us | max us | % of kernel time |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows[:args.top]:
        nm = r["name"] if len(r["name"]) <= 90 else r["name"][:87] + "..."
        lines.append("| `%s` | %d | %d | %.2f | %.2f | %.2f | %.1f |"
                     % (nm.replace("|", "\\|"), r["grid"], r["calls"], r["avg_us"], r["min_us"], r["max_us"],
                        r["pct"]))
    lines.append("")
    if args.split:
        split = []
        for item in args.split.split(","):
            label, n = item.rsplit(":", 1)
            split.append((label, int(n)))
        lines += ["Library kernels by pass (each kernel's calls in start order: %s):"
                  % ", ".join("%s %d" % s_ for s_ in split), "",
                  "| kernel | grid threads | pass | calls | avg us |", "|---|---:|---|---:|---:|"]
        for r in kernel_passes(args.db, split):
            nm = r["name"] if len(r["name"]) <= 90 else r["name"][:87] + "..."
            lines.append("| `%s` | %d | %s | %d | %.2f |"
                         % (nm.replace("|", "\\|"), r["grid"], r["pass"], r["calls"], r["avg_us"]))
        lines.append("")
    if args.note:
        lines += [args.note, ""]
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def cmd_counters(args):
    fetch = counter_per_kernel(args.fetch_db, "FETCH_SIZE")
    write = counter_per_kernel(args.write_db, "WRITE_SIZE")
    nf, cf = _copy_value(fetch, "FETCH_SIZE")
    nw, cw = _copy_value(write, "WRITE_SIZE")
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    kernels = {}
    for name in sorted(set(fetch) | set(write)):
        k = short_name(name)
        if k is None:
            continue
        fn, fv = fetch.get(name, (0, 0.0))
        wn, wv = write.get(name, (0, 0.0))
        ent = kernels.setdefault(k, {"names": [], "fetch_dispatches": 0, "write_dispatches": 0,
                                     "_f": 0.0, "_w": 0.0})
        ent["names"].append(name)
        ent["fetch_dispatches"] += fn
        ent["write_dispatches"] += wn
        ent["_f"] += fn * fv
        ent["_w"] += wn * wv
    for k, ent in kernels.items():
        fkib = ent.pop("_f") / max(ent["fetch_dispatches"], 1)
        wkib = ent.pop("_w") / max(ent["write_dispatches"], 1)
        ent["fetch_kib_per_dispatch"] = round(fkib, 1)
        ent["write_kib_per_dispatch"] = round(wkib, 1)
        ent["hbm_read_bytes_per_launch"] = int(fkib * 1024 * f_scale)
        ent["hbm_write_bytes_per_launch"] = int(wkib * 1024 * w_scale)
        ent["hbm_bytes_per_launch"] = ent["hbm_read_bytes_per_launch"] + ent["hbm_write_bytes_per_launch"]
    out = {
        "config": args.config,
        "kernel_source_sha": library_source_sha(),
        "command_fetch": args.command_fetch,
        "command_write": args.command_write,
        "summary_command": "python3 -m sparse_attention_decode_scores_amd.profsum " + " ".join(
            "'%s'" % x if " " in x else x for x in sys.argv[1:]),
        "copy_calibration": {
            "kernel": "torch.neg over 64 Mi fp32 values (%d bytes read, %d written per dispatch)"
                      % (COPY_BYTES, COPY_BYTES),
            "fetch_kib_per_dispatch": round(cf, 1), "fetch_dispatches": nf,
            "write_kib_per_dispatch": round(cw, 1), "write_dispatches": nw,
            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        },
        "kernels": kernels,
    }
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


MI355X_CUS, SIMDS_PER_CU, CLOCK_GHZ, INT8_PEAK_TOPS = 256, 4, 2.4, 5000.0


def cmd_mfma(args):
    """Per library kernel: int8 matrix ops per dispatch (MOPS_I8 counts ops / 512), the
    matrix-core busy cycles per SIMD (the counter sums over every SIMD), and that as a
    fraction of the dispatch's cycles at the nominal clock; the rate those ops reach
    over the dispatch (counters run serialises dispatches, so durations run longer
    than in the timed bench)."""
    con = _db(args.db)
    rows = con.execute("SELECT kernel_name, dispatch_id, counter_name, SUM(value), MAX(end) - MIN(start) "
                       "FROM counters_collection GROUP BY kernel_name, dispatch_id, counter_name").fetchall()
    acc = {}
    for name, did, counter, value, dur in rows:
        k = short_name(name)
        if k is None:
            continue
        d = acc.setdefault(name, {}).setdefault(did, {"dur_ns": dur})
        d[counter] = float(value)
    out = {"command": args.command, "kernel_source_sha": library_source_sha(),
           "summary_command": "python3 -m sparse_attention_decode_scores_amd.profsum " + " ".join(
               "'%s'" % x if " " in x else x for x in sys.argv[1:]),
           "assumptions": {"simds": MI355X_CUS * SIMDS_PER_CU, "clock_GHz": CLOCK_GHZ,
                           "int8_peak_TOPS": INT8_PEAK_TOPS},
           "kernels": {}}
    for name, per in acc.items():
        n = len(per)
        mean = lambda key: sum(d.get(key, 0.0) for d in per.values()) / n
        dur_us = mean("dur_ns") / 1e3
        ops = mean("SQ_INSTS_VALU_MFMA_MOPS_I8") * 512
        busy_simd = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (MI355X_CUS * SIMDS_PER_CU)
        ent = {"name": name, "dispatches": n, "dispatch_us_under_counters": round(dur_us, 2),
               "int8_ops_per_dispatch": int(ops), "mfma_busy_cycles_per_simd": round(busy_simd, 1),
               "grbm_gui_active_per_dispatch": round(mean("GRBM_GUI_ACTIVE"), 1)}
        if dur_us > 0:
            ent["mfma_busy_frac_of_dispatch"] = round(busy_simd / (dur_us * 1e3 * CLOCK_GHZ), 4)
            ent["int8_TOPS_over_dispatch"] = round(ops / (dur_us * 1e-6) / 1e12, 1)
        if busy_simd > 0:
            ent["int8_ops_per_busy_cycle_per_simd"] = round(ops / (busy_simd * MI355X_CUS * SIMDS_PER_CU), 1)
        out["kernels"].setdefault(short_name(name), []).append(ent)
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--db", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--top", type=int, default=14)
    s.add_argument("--split", default="", help="label:count,... the passes of the command, in order")
    c = sub.add_parser("counters")
    c.add_argument("--fetch-db", required=True)
    c.add_argument("--write-db", required=True)
    c.add_argument("--config", required=True)
    c.add_argument("--command-fetch", required=True)
    c.add_argument("--command-write", required=True)
    c.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--db", required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    {"stats": cmd_stats, "counters": cmd_counters, "mfma": cmd_mfma}[args.cmd](args)


if __name__ == "__main__":
    main()
