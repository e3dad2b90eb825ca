"""Kernel-duration summary of a bench.py run under the rocprofv3 kernel
trace, written as the markdown file kept under profiles/.

  python bench_trace.py summarize TRACE_DIR BENCH_JSON OUT.md
  python bench_trace.py steps TRACE_DIR BENCH_JSON OUT.md TITLE COMMAND

TRACE_DIR holds the csv output of

  rocprofv3 --kernel-trace --stats --output-format csv -d TRACE_DIR -o bench \\
      -- python bench.py --no-cpu --no-extra

and BENCH_JSON the JSON line that same run printed. The summary has
  * the per-kernel statistics of the whole run (rocprofv3's stats file);
  * the block step: every kernel of the timed block fwd+bwd loop, per step;
  * the GEMM replay behind the roofline entry: each repetition starts after
    the spin kernel bench.py queues in front of it, so the trace's GEMM
    dispatches (split-K reduces included) between two spins are one
    repetition; their mean duration per launch is set beside the figure
    bench.py measured with HIP events in the same run.
"""
import csv
import glob
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))



def _rel(path):
    """A path as given on the command line, relative to the repository root."""
    return os.path.relpath(os.path.abspath(path), ROOT)

def _csv(d, suffix):
    f = glob.glob(os.path.join(d, f"*{suffix}"))
    if not f:
        raise SystemExit(f"no *{suffix} under {d}")
    return list(csv.DictReader(open(f[0])))


def short(n):
    n = re.sub(r"qblk::\(anonymous namespace\)::", "", n)
    n = re.sub(r"\(qblk::GemmDesc, qblk::Grid\)", "", n)
    return n[:120]


def is_gemm(n):
    return "gemm_pp_kernel" in n or "gemm_dma_kernel" in n or "gemm_kernel" in n or "splitk_reduce" in n


def groups(trace):
    """Dispatches in order, split at each spin kernel: [[(name, ns)], ...]."""
    rows = sorted(trace, key=lambda r: int(r["Start_Timestamp"]))
    out, cur = [], None
    for r in rows:
        n = r["Kernel_Name"]
        if "spin_kernel" in n:
            cur = []
            out.append(cur)
            continue
        if cur is not None:
            cur.append((n, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def summarize(trace_dir, bench_json, out_path):
    stats = _csv(trace_dir, "kernel_stats.csv")
    trace = _csv(trace_dir, "kernel_trace.csv")
    bench = json.loads(open(bench_json).read().strip().splitlines()[-1])
    roof = bench["roofline"]
    steps = bench["steps"]
    nlaunch = len(roof["per_launch_us"])
    gs = groups(trace)

    # GEMM replay: groups made of GEMM dispatches only, nlaunch products each
    reps = []
    for g in gs:
        if g and all(is_gemm(n) for n, _ in g):
            launches = []
            for n, ns in g:
                if "splitk_reduce" in n and launches:
                    launches[-1] += ns
                else:
                    launches.append(ns)
            if len(launches) == nlaunch:
                reps.append(launches)
    if not reps:
        raise SystemExit("no GEMM replay found in the trace")
    per = [sum(r[i] for r in reps) / len(reps) / 1e3 for i in range(nlaunch)]
    avg = sum(per) / nlaunch

    # block step: the group holding `steps` QK-norm/RoPE backward launches
    blk = next((g for g in gs if sum("qk_rope_bwd" in n for n, _ in g) == steps), None)
    if blk:
        blk = [(n, ns) for n, ns in blk if "at::" not in n]

    lines = [
        "# Kernel durations: Qwen3-4B-shaped block fwd+bwd (h2560, 32/8 heads, d128, I9728, S512, fp16 GEMM operands)",
        "",
        "Commands (repository root, one MI355X):",
        "",
        "```",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d {_rel(trace_dir)} -o bench "
        f"-- python bench.py --no-cpu --no-extra > {_rel(bench_json)}",
        f"python bench_trace.py summarize {_rel(trace_dir)} {_rel(bench_json)} " + os.path.relpath(out_path, ROOT),
        "```",
        "",
        "## GEMM replay (the roofline entry)",
        "",
        f"{len(reps)} repetitions of the block's {nlaunch} GEMM launches found in the trace.",
        "",
        "| launch | trace mean us | bench events us |",
        "|---:|---:|---:|",
    ]
    for i, (a, b) in enumerate(zip(per, roof["per_launch_us"])):
        lines.append(f"| {i} | {a:.1f} | {b:.1f} |")
    lines += [
        "",
        f"Mean per launch: trace {avg:.2f} us; bench, one event pair around the sequence, "
        f"{roof['avg_launch_us']:.2f} us (it also holds the gaps between kernels). The per-launch event "
        f"column brackets each launch alone and so also holds the event packets' own time.",
        "",
    ]
    if blk:
        agg = {}
        for n, ns in blk:
            c, t = agg.get(n, (0, 0))
            agg[n] = (c + 1, t + ns)
        busy = sum(t for _, t in agg.values()) / steps / 1e3
        lines += [
            "## Block step (timed loop, per step)",
            "",
            f"{steps} steps; kernel busy time {busy:.1f} us per step; bench: {bench['ms_per_step'] * 1e3:.1f} us "
            f"per step by events.",
            "",
            "| kernel | launches/step | us/step |",
            "|---|---:|---:|",
        ]
        for n, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
            lines.append(f"| `{short(n)}` | {c / steps:.0f} | {t / steps / 1e3:.1f} |")
        lines.append("")
    lines += [
        "## Whole run (rocprofv3 --stats)",
        "",
        "| kernel | calls | total us | avg us | min us | max us | % |",
        "|---|---:|---:|---:|---:|---:|---:|",
    ]
    for r in stats:
        if float(r["Percentage"]) < 0.05:
            continue
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines += ["", "Bench line of the same run:", "", "```", json.dumps(bench), "```", ""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out_path}: replay {avg:.2f} us/launch (events {roof['avg_launch_us']})")


def summarize_steps(trace_dir, bench_json, out_path, title, command):
    """Per-step kernel table of a `bench.py --only NAME` run: its timed loop
    is the group of dispatches between the spin kernel queued in front of
    it and the end-marker spin (the group with the most dispatches)."""
    stats = _csv(trace_dir, "kernel_stats.csv")
    trace = _csv(trace_dir, "kernel_trace.csv")
    bench = json.loads(open(bench_json).read().strip().splitlines()[-1])
    steps = bench["steps"]
    loop = max(groups(trace), key=len)
    agg = {}
    for n, ns in loop:
        c, t = agg.get(n, (0, 0))
        agg[n] = (c + 1, t + ns)
    busy = sum(t for _, t in agg.values()) / steps / 1e3
    lines = [f"# Kernel durations: {title}", "", "Commands (repository root, one MI355X):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d {_rel(trace_dir)} -o bench -- " + command
             + f" > {_rel(bench_json)}",
             f"python bench_trace.py steps {_rel(trace_dir)} {_rel(bench_json)} "
             f"{os.path.relpath(out_path, ROOT)} \"{title}\" \"{command}\"", "```", "",
             "## Timed loop, per step", "",
             f"{steps} steps; kernel busy time {busy:.1f} us per step; bench: {bench['ms_per_step'] * 1e3:.1f} us "
             f"per step by events.", "",
             "| kernel | launches/step | us/step | % of busy |", "|---|---:|---:|---:|"]
    for n, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| `{short(n)}` | {c / steps:.2f} | {t / steps / 1e3:.1f} | "
                     f"{100.0 * t / steps / 1e3 / busy:.1f} |")
    lines += ["", "## Whole run (rocprofv3 --stats)", "",
              "| kernel | calls | total us | avg us | min us | max us | % |",
              "|---|---:|---:|---:|---:|---:|---:|"]
    for r in stats:
        if float(r["Percentage"]) < 0.05:
            continue
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines += ["", "Bench output of the same run:", "", "```", json.dumps(bench), "```", ""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out_path}: {busy:.1f} us kernel time per step")


if __name__ == "__main__":
    if len(sys.argv) == 5 and sys.argv[1] == "summarize":
        summarize(*sys.argv[2:5])
    elif len(sys.argv) == 7 and sys.argv[1] == "steps":
        summarize_steps(*sys.argv[2:7])
    else:
        raise SystemExit(__doc__)
