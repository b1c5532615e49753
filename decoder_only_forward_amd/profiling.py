"""Text summaries of rocprofv3 output for the benchmark.

Three kinds of run are summarised (all write CSV with ``--output-format csv``):

* kernel trace with statistics (``--kernel-trace --stats``): per kernel class, the number
  of dispatches, total and average duration;
* hardware counters (``--pmc FETCH_SIZE`` and, in a second run, ``--pmc WRITE_SIZE``):
  HBM kilobytes read / written per dispatch.  The raw counter is scaled by what it reads
  for a plain elementwise copy of known size, run first in the same process
  (``bench.py --copy-gib``), so the figure is in real bytes;
* matrix-core counters (``--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16
  SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE``): per kernel class, the
  fp16 and bf16 MFMA work executed (each MOPS unit is 512 flops) and the share of SIMD
  cycles the matrix cores were busy.

The traffic table is keyed by profile tag and stamped with a hash of the sources the
kernel is built from; ``bench.py`` reports it only while those sources are unchanged.

Usage (after the rocprofv3 runs):
  python -m decoder_only_forward_amd.profiling stats <dir> <workload> <command> <out.md>
  python -m decoder_only_forward_amd.profiling traffic <fetch_dir> <write_dir> <workload>
         <copy_gib> <command_fetch> <command_write> <traffic.json>
  python -m decoder_only_forward_amd.profiling mfma <out.md> <command> <workload>=<dir> ...
  python -m decoder_only_forward_amd.profiling counters <out.md> <command> <workload>=<dir> ...
"""
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# profile tag -> (substring of the demangled kernel name, source files of that kernel)
_GEMM = ["gemm_kernel.h", "gemm.hip", "common.h"]
KERNELS = {
    "qkv_gemm": ("gemm_kernel<", _GEMM),
    "qk_norm_rope_cache": ("qkv_rope_", ["norm_rope.hip", "common.h"]),
    "attn_prefill": ("attn_prefill_kernel", ["attention.hip", "common.h"]),
    "attn_decode": ("attn_decode_kernel", ["attention.hip", "common.h"]),
    "gate_up_gemm": ("gemm_kernel<", _GEMM),
    "lm_head_gemm": ("gemm_kernel<", _GEMM),
    "moe_gate_up_gemm": ("gemm_kernel<", _GEMM),
    "moe_down_gemm": ("gemm_kernel<", _GEMM),
    # decode-size products (<= 256 rows): one 16-column block per output slice
    "decode_qkv_gemm": ("decode_gemm_kernel<1, 6, false>", _GEMM),
    "decode_gate_up_gemm": ("decode_gemm_kernel<2, 5, false>", _GEMM),
    "decode_res_gemm": ("decode_gemm_kernel<0, 2, true>", _GEMM),
}

# Template signatures that single out one GEMM use (fp16 A, B mode, epilogue, grouped).
# o_proj and down share one instantiation and are not told apart here.
GEMM_SIGNATURE = {
    "qkv_gemm": "true, 1, 7, false>",  # prefill: q/k-norm + RoPE + cache writes fused
    "gate_up_gemm": "true, 2, 5, false>",
    "lm_head_gemm": "true, 0, 1, false>",
    "moe_gate_up_gemm": ", 2, 5, true>",
    "moe_down_gemm": ", 0, 1, true>",
}


def source_hash(tag):
    h = hashlib.sha256()
    for f in KERNELS[tag][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _csv_rows(pattern):
    rows = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def short_name(name):
    """Demangled kernel name without its argument list and anonymous namespaces."""
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i][:110]
    return n[:110]


def stats_markdown(rocprof_dir, workload, command):
    rows = _csv_rows(os.path.join(rocprof_dir, "**", "*kernel_stats.csv"))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {rocprof_dir}")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"# rocprofv3 kernel statistics: {workload}", "",
           "Command (run from the repository root):", "", "```", command, "```", "",
           "| kernel | calls | total ms | avg us | % time |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        t = float(r["TotalDurationNs"])
        if t / total < 0.002:
            continue
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {t / 1e6:.3f} | "
                   f"{float(r['AverageNs']) / 1e3:.2f} | {100 * t / total:.1f} |")
    out.append("")
    out.append(f"All kernels: {total / 1e6:.3f} ms in total (setup kernels included).")
    return "\n".join(out) + "\n"


def _per_dispatch(rocprof_dir, counter):
    rows = _csv_rows(os.path.join(rocprof_dir, "**", "*counter_collection.csv"))
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return [(name, v) for (_, name), v in per.items()]


def _select(dispatches, tag):
    sub, _ = KERNELS[tag]
    sig = GEMM_SIGNATURE.get(tag)
    vals = [v for n, v in dispatches if sub in n and (sig is None or sig in n)]
    return vals


def _copy_scale(dispatches, copy_bytes):
    # the calibration copy is the largest elementwise dispatch of the run
    cands = [v for n, v in dispatches if "elementwise" in n]
    if not cands:
        raise SystemExit("calibration copy dispatch not found")
    return copy_bytes / 1024.0 / max(cands)


def traffic_json(fetch_dir, write_dir, workload, copy_gib, cmd_fetch, cmd_write, tags,
                 existing=None):
    fd = _per_dispatch(fetch_dir, "FETCH_SIZE")
    wd = _per_dispatch(write_dir, "WRITE_SIZE")
    copy_bytes = copy_gib * (1 << 30)
    fscale, wscale = _copy_scale(fd, copy_bytes), _copy_scale(wd, copy_bytes)
    table = dict(existing or {})
    for tag in tags:
        fv, wv = _select(fd, tag), _select(wd, tag)
        if not fv or not wv:
            continue
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        table[f"{workload}/{tag}"] = {
            "fetch_kib_raw": round(f_kib, 1), "write_kib_raw": round(w_kib, 1),
            "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
            "bytes_per_launch": round((f_kib * fscale + w_kib * wscale) * 1024.0),
            "dispatches": [len(fv), len(wv)], "source_sha": source_hash(tag),
            "commands": [cmd_fetch, cmd_write]}
    return table


def traffic_for(workload, tag, path=None):
    """HBM bytes per launch from the committed counter table, or None when absent or
    when the kernel's sources changed since the counters were taken."""
    path = path or os.path.join(os.path.dirname(HERE), "profiles", "traffic.json")
    try:
        with open(path) as fh:
            e = json.load(fh).get(f"{workload}/{tag}")
    except (OSError, ValueError):
        return None
    if not e or tag not in KERNELS or e.get("source_sha") != source_hash(tag):
        return None
    return float(e["bytes_per_launch"])


def traffic_markdown(table):
    out = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
           "Raw counters are KiB per dispatch; each is scaled by (known bytes / counter "
           "reading) of a plain elementwise copy run first in the same process.", "",
           "| workload/tag | fetch KiB (raw) | write KiB (raw) | fetch scale | write scale | "
           "HBM bytes / launch | dispatches | source sha |",
           "|---|---:|---:|---:|---:|---:|---|---|"]
    for k, e in sorted(table.items()):
        out.append(f"| {k} | {e['fetch_kib_raw']} | {e['write_kib_raw']} | "
                   f"{e['fetch_scale']} | {e['write_scale']} | {e['bytes_per_launch']:.0f} | "
                   f"{e['dispatches']} | {e['source_sha']} |")
    out.append("")
    out.append("Commands:")
    for k, e in sorted(table.items()):
        out.append(f"- {k}: `{e['commands'][0]}` then `{e['commands'][1]}`")
    return "\n".join(out) + "\n"


MFMA_PEAK_F16 = 2.5e15  # dense fp16/bf16 MFMA flops per second at the 2.4 GHz peak clock


def _gpu_agent(rocprof_dir):
    for r in _csv_rows(os.path.join(rocprof_dir, "**", "*agent_info.csv")):
        if r["Agent_Type"] == "GPU":
            return int(r["Simd_Count"]), int(r["Num_Xcc"])
    raise SystemExit(f"no GPU agent in {rocprof_dir}")


def mfma_rows(rocprof_dir):
    """Per kernel class: dispatches, mean duration, executed fp16 MFMA flops per dispatch,
    MFMA busy share and the shader clock implied by the active-cycle count.

    GRBM_GUI_ACTIVE comes back summed over the XCDs, so one XCD's active cycles are the sum
    over Num_Xcc; SQ_VALU_MFMA_BUSY_CYCLES is summed over every SIMD of the chip."""
    simds, xcc = _gpu_agent(rocprof_dir)
    per, meta = {}, {}
    for r in _csv_rows(os.path.join(rocprof_dir, "**", "*counter_collection.csv")):
        d = per.setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        meta[r["Dispatch_Id"]] = (r["Kernel_Name"],
                                  int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    groups = {}
    for k, c in per.items():
        name, dur = meta[k]
        g = groups.setdefault(name, [0, 0.0, 0.0, 0.0, 0.0])
        g[0] += 1
        g[1] += dur
        g[2] += (c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) +
                 c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)) * 512.0
        g[3] += c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        g[4] += c.get("GRBM_GUI_ACTIVE", 0.0) / xcc
    out = []
    for name, (n, dur, flops, busy, active) in groups.items():
        if flops == 0.0:
            continue
        label = short_name(name)
        for tag, sig in GEMM_SIGNATURE.items():
            if "gemm_kernel<" in name and sig in name:
                label += f" ({tag})"
        out.append({"kernel": label, "dispatches": n, "avg_us": dur / n / 1e3,
                    "gflop": flops / n / 1e9, "tflops": flops / dur / 1e3,
                    "busy_pct": 100.0 * busy / (active * simds),
                    "clock_ghz": active / dur, "total_us": dur / 1e3})
    out.sort(key=lambda e: -e["total_us"])
    return out


def mfma_markdown(runs, command):
    out = ["# MFMA utilisation per kernel (rocprofv3 matrix-core counters)", "",
           "Command (run from the repository root, once per workload):", "", "```",
           command, "```", "",
           "Executed flops are (SQ_INSTS_VALU_MFMA_MOPS_F16 + SQ_INSTS_VALU_MFMA_MOPS_BF16) "
           "x 512 per dispatch (a run without the bf16 counter counts fp16 work only); the rate is "
           "that over the dispatch's own duration; the fraction is of the 2.5 PFLOP/s dense "
           "fp16/bf16 peak (2.4 GHz).  MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES over (one XCD's "
           "GRBM_GUI_ACTIVE x 1024 SIMDs): the share of SIMD cycles the matrix cores were "
           "busy at the clock the chip actually ran, which is given beside it "
           "(active cycles of one XCD / duration).  Counter runs serialise dispatches, so "
           "durations are a little longer than in the timed benchmark.", ""]
    for workload, rows in runs:
        out += [f"## {workload}", "",
                "| kernel | dispatches | avg us | GFLOP / dispatch | TFLOP/s | of peak | "
                "MFMA busy % | clock GHz |", "|---|---:|---:|---:|---:|---:|---:|---:|"]
        for e in rows:
            out.append(f"| `{e['kernel']}` | {e['dispatches']} | {e['avg_us']:.1f} | "
                       f"{e['gflop']:.2f} | {e['tflops']:.0f} | "
                       f"{1e12 * e['tflops'] / MFMA_PEAK_F16:.3f} | {e['busy_pct']:.1f} | "
                       f"{e['clock_ghz']:.2f} |")
        out.append("")
    return "\n".join(out)


def counter_rows(rocprof_dir):
    """Per kernel class: dispatches, mean duration and the mean of every collected counter
    per dispatch (counters summed over the chip's instances)."""
    per, meta = {}, {}
    for r in _csv_rows(os.path.join(rocprof_dir, "**", "*counter_collection.csv")):
        d = per.setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        meta[r["Dispatch_Id"]] = (r["Kernel_Name"],
                                  int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    groups = {}
    for k, c in per.items():
        name, dur = meta[k]
        g = groups.setdefault(short_name(name), {"n": 0, "dur": 0.0, "c": {}})
        g["n"] += 1
        g["dur"] += dur
        for cn, v in c.items():
            g["c"][cn] = g["c"].get(cn, 0.0) + v
    out = [{"kernel": name, "dispatches": g["n"], "avg_us": g["dur"] / g["n"] / 1e3,
            "total_us": g["dur"] / 1e3,
            "counters": {cn: v / g["n"] for cn, v in g["c"].items()}}
           for name, g in groups.items()]
    out.sort(key=lambda e: -e["total_us"])
    return out


def counters_markdown(runs, command, top=12):
    out = ["# Memory-hierarchy counters per kernel (rocprofv3)", "",
           "Command (run from the repository root, once per workload):", "", "```",
           command, "```", "",
           "Each counter is the mean per dispatch over the kernel class's dispatches (summed "
           "over the chip's counter instances).  Counter runs serialise dispatches, so "
           "durations are a little longer than in the timed benchmark.", ""]
    for workload, rows in runs:
        names = sorted({cn for e in rows for cn in e["counters"]})
        out += [f"## {workload}", "",
                "| kernel | dispatches | avg us | " + " | ".join(names) + " |",
                "|---|---:|---:|" + "---:|" * len(names)]
        for e in rows[:top]:
            vals = " | ".join(f"{e['counters'].get(cn, 0.0):.4g}" for cn in names)
            out.append(f"| `{e['kernel']}` | {e['dispatches']} | {e['avg_us']:.1f} | {vals} |")
        out.append("")
    return "\n".join(out)


def main(argv):
    if argv[0] == "stats":
        d, workload, cmd, out = argv[1:5]
        with open(out, "w") as fh:
            fh.write(stats_markdown(d, workload, cmd))
    elif argv[0] == "traffic":
        fdir, wdir, workload, gib, cf, cw, out = argv[1:8]
        tags = argv[8].split(",") if len(argv) > 8 else list(KERNELS)
        existing = None
        if os.path.exists(out):
            with open(out) as fh:
                existing = json.load(fh)
        table = traffic_json(fdir, wdir, workload, float(gib), cf, cw, tags, existing)
        with open(out, "w") as fh:
            json.dump(table, fh, indent=1, sort_keys=True)
        with open(os.path.splitext(out)[0] + ".md", "w") as fh:
            fh.write(traffic_markdown(table))
    elif argv[0] == "counters":
        out, cmd = argv[1:3]
        runs = [(a.split("=", 1)[0], counter_rows(a.split("=", 1)[1])) for a in argv[3:]]
        with open(out, "w") as fh:
            fh.write(counters_markdown(runs, cmd))
    elif argv[0] == "mfma":
        out, cmd = argv[1:3]
        runs = [(a.split("=", 1)[0], mfma_rows(a.split("=", 1)[1])) for a in argv[3:]]
        with open(out, "w") as fh:
            fh.write(mfma_markdown(runs, cmd))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
