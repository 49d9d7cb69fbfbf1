"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

Two summaries:

* ``stats``: per-kernel call count and average / min / max duration from a
  ``rocprofv3 --kernel-trace --stats --output-format csv`` run
  (``*_kernel_stats.csv``).
* ``traffic``: HBM bytes per dispatch from two counter runs
  (``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, KiB per dispatch),
  each scaled by what the same counter reads for a plain device copy of known
  size (``bench.py --copy-calibration``: b = -a over 1 GiB of float32, 1 GiB
  read + 1 GiB written per launch).  The summary carries the machine-readable lines
  ``kernel_source_sha:``, ``hbm_read_bytes_per_launch:`` and
  ``hbm_write_bytes_per_launch:`` that bench.py reads back.

* ``counters``: instruction mix and matrix-core occupancy from ``rocprofv3 --pmc`` runs of
  ``SQ_*`` counters (at most 8 per run): per kernel, instructions per 32x32 score tile (MFMA,
  VALU, of which transcendental, LDS, scalar, vector memory) and the MFMA pipe's busy fraction,
  ``SQ_INSTS_MFMA`` x 32 cycles (one 32x32x16 MFMA occupies a SIMD's matrix core 32 cycles) over
  the dispatch's duration x 2.4 GHz x 1024 SIMDs.

Usage (on the CPU, after the GPU runs have written their CSVs)::

    python -m vision_transformer_windowed_amd.profiling stats DIR --command CMD --out FILE
    python -m vision_transformer_windowed_amd.profiling counters DIR [DIR ...] --kernels REGEX[,REGEX] \\
        --tiles N --title TITLE --command CMD --out FILE
    python -m vision_transformer_windowed_amd.profiling traffic --fetch DIR --write DIR \\
        --copy-fetch DIR --copy-write DIR --kernels REGEX[,REGEX] --tag TAG --workload NAME \\
        --command CMD --out FILE
"""

import argparse
import csv
import glob
import os
import re
import statistics


def _find(dirpath, suffix):
    hits = sorted(glob.glob(os.path.join(dirpath, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {dirpath}")
    return hits[0]


def short_name(name):
    """Kernel name without its argument list: 'ns::kernel<8, 32>'."""
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def read_stats(dirpath):
    rows = []
    for r in csv.DictReader(open(_find(dirpath, "kernel_stats.csv"))):
        rows.append({"kernel": short_name(r["Name"]), "calls": int(r["Calls"]),
                     "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                     "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return rows


def stats_markdown(dirpath, command, title):
    rows = read_stats(dirpath)
    out = [f"# {title}", "", "Command (from the repository root; `cd /tmp && export TMPDIR=/tmp` first):", "",
           "```", command, "```", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['kernel']}` | {r['calls']} | {r['avg_us']:.1f} | {r['min_us']:.1f} | {r['max_us']:.1f} "
                   f"| {r['pct']:.1f} |")
    return "\n".join(out) + "\n"


def read_counter(dirpath, counter):
    """{kernel short name: [value per dispatch]} for one counter (summed over its instances)."""
    per = {}
    for r in csv.DictReader(open(_find(dirpath, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        key = (short_name(r["Kernel_Name"]), r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (k, _), v in per.items():
        out.setdefault(k, []).append(v)
    return out


def read_counters_with_time(dirpaths):
    """{kernel: {counter: mean per dispatch, '_dur_ns': mean duration}} over several counter runs."""
    acc, dur = {}, {}
    for d in dirpaths:
        per = {}
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            k = short_name(r["Kernel_Name"])
            key = (k, r["Dispatch_Id"], r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            dur.setdefault(k, {})[(d, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for (k, _, c), v in per.items():
            acc.setdefault(k, {}).setdefault(c, []).append(v)
    out = {}
    for k, cs in acc.items():
        out[k] = {c: statistics.mean(vs) for c, vs in cs.items()}
        out[k]["_dur_ns"] = statistics.mean(dur[k].values())
    return out


MFMA_CYCLES = 32        # cycles one v_mfma_f32_32x32x16 occupies a SIMD's matrix core
SIMDS = 1024            # 256 CUs x 4 SIMDs
CLOCK_HZ = 2.4e9        # peak engine clock


def counters_markdown(dirpaths, kernels, tiles, title, command):
    data = read_counters_with_time(dirpaths)
    pats = [re.compile(p) for p in kernels]
    per_tile = [("MFMA", "SQ_INSTS_MFMA"), ("VALU", "SQ_INSTS_VALU"), ("of which transcendental",
                "SQ_INSTS_VALU_TRANS_F32"), ("LDS", "SQ_INSTS_LDS"), ("SALU", "SQ_INSTS_SALU"),
                ("VMEM read", "SQ_INSTS_VMEM_RD"), ("VMEM write", "SQ_INSTS_VMEM_WR")]
    lines = [f"# {title}", "",
             "Commands (from the repository root; `cd /tmp && export TMPDIR=/tmp` first), one run per counter set:",
             "", "```", command, "```", "",
             f"Instructions are counted per wave instruction and divided by the {tiles:.6g} score tiles (32 queries x "
             "32 keys) of one launch.  MFMA busy = SQ_INSTS_MFMA x 32 cycles / (dispatch duration x 2.4 GHz x 1024 "
             "SIMDs); SQ_VALU_MFMA_BUSY_CYCLES / (MFMA x 32) checks the 32 cycles.  Durations are those of the "
             "counter runs.", "",
             "| kernel | duration us | " + " | ".join(n + "/tile" for n, _ in per_tile) +
             " | MFMA busy | busy cycles / (MFMA x 32) |",
             "|---|---|" + "---|" * len(per_tile) + "---|---|"]
    for k in sorted(data):
        if not any(p.search(k) for p in pats):
            continue
        d = data[k]
        cells = [f"{d.get(c, float('nan')) / tiles:.2f}" for _, c in per_tile]
        mfma = d.get("SQ_INSTS_MFMA", float("nan"))
        busy = mfma * MFMA_CYCLES / (d["_dur_ns"] * 1e-9 * CLOCK_HZ * SIMDS)
        chk = d.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (mfma * MFMA_CYCLES)
        lines.append(f"| `{k}` | {d['_dur_ns'] / 1e3:.1f} | " + " | ".join(cells) + f" | {busy:.1%} | {chk:.3f} |")
    return "\n".join(lines) + "\n"


def _copy_factor(dirpath, counter, nbytes):
    vals = [v for k, vs in read_counter(dirpath, counter).items() for v in vs if "neg" in k.lower()]
    if not vals:
        raise RuntimeError(f"no calibration (neg) kernel dispatch with {counter} under {dirpath}")
    measured = statistics.median(vals) * 1024.0  # KiB -> bytes
    return measured / nbytes, measured


def traffic_markdown(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, kernels, tag, workload, sha, command,
                     copy_bytes=1 << 30):
    fr, fmeas = _copy_factor(copy_fetch_dir, "FETCH_SIZE", copy_bytes)
    wr, wmeas = _copy_factor(copy_write_dir, "WRITE_SIZE", copy_bytes)
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")
    pats = [re.compile(p) for p in kernels]
    lines = [f"# HBM traffic: {tag}, workload {workload}", "",
             "Commands (from the repository root; `cd /tmp && export TMPDIR=/tmp` first), one counter per run:", "",
             "```", command, "```", "",
             f"Copy calibration (`bench.py --copy-calibration`: b = -a, {copy_bytes} bytes read and written per launch): "
             f"FETCH_SIZE reads {fmeas:.4g} bytes (factor {fr:.4f}), WRITE_SIZE reads {wmeas:.4g} bytes "
             f"(factor {wr:.4f}).  Kernel figures below are divided by these factors.", "",
             "| kernel | dispatches | FETCH KiB/dispatch | WRITE KiB/dispatch | read bytes (calibrated) "
             "| write bytes (calibrated) |", "|---|---|---|---|---|---|"]
    tot_r = tot_w = 0.0
    for k in sorted(set(fetch) | set(write)):
        if not any(p.search(k) for p in pats):
            continue
        f = statistics.mean(fetch.get(k, [0.0]))
        w = statistics.mean(write.get(k, [0.0]))
        rb, wb = f * 1024.0 / fr, w * 1024.0 / wr
        tot_r += rb
        tot_w += wb
        lines.append(f"| `{k}` | {len(fetch.get(k, []))} | {f:.6g} | {w:.6g} | {rb:.6g} | {wb:.6g} |")
    lines += ["", f"kernel_source_sha: {sha}", f"hbm_read_bytes_per_launch: {tot_r:.6g}",
              f"hbm_write_bytes_per_launch: {tot_w:.6g}", ""]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for name in ("fetch", "write", "copy-fetch", "copy-write", "kernels", "tag", "workload", "command", "out"):
        t.add_argument("--" + name, required=True)
    t.add_argument("--sha", default=None)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernels", required=True)
    c.add_argument("--tiles", type=float, required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.mode == "stats":
        text = stats_markdown(a.dir, a.command, a.title)
    elif a.mode == "counters":
        text = counters_markdown(a.dirs, a.kernels.split(","), a.tiles, a.title, a.command)
    else:
        sha = a.sha
        if sha is None:
            import importlib.util
            spec = importlib.util.spec_from_file_location(
                "bench", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
            bench = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(bench)
            sha = bench.kernel_source_sha()
        text = traffic_markdown(a.fetch, a.write, a.copy_fetch, a.copy_write, a.kernels.split(","), a.tag,
                                a.workload, sha, a.command)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
