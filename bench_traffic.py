"""HBM traffic and MFMA busy time of the block's GEMM launches, from
rocprofv3 hardware counters, for bench.py's roofline entry.

  python bench_traffic.py run
      One 256 MiB fp32 device-to-device copy (the calibration kernel, the
      runtime's plain copy: 256 MiB read, 256 MiB written), then the 12 GEMM
      launches of one Qwen3-4B-shaped block
      forward + backward (same kernels, shapes and operand types as
      bench.py's replay), each once; then, each after a marker (a short
      spin kernel), one forward + backward of the Qwen3-4B-shaped block
      (seq 512), of the NF4 + LoRA block (seq 2048) and of one layer of the
      36-layer stack's block (fp32, seq 1024), whose attention kernels the
      summary reports. Meant to run under `rocprofv3 --pmc <counter>`, one
      counter set per run.

  python bench_traffic.py summarize FETCH_DIR WRITE_DIR MFMA_DIR OUT.md
      Reads the three counter runs (FETCH_SIZE; WRITE_SIZE; GRBM_GUI_ACTIVE
      with SQ_VALU_MFMA_BUSY_CYCLES) and writes the summary: per launch the
      counter bytes scaled by the calibration factor (known bytes of the copy
      / what the same counter reads for it), and the MFMA busy fraction.
      The summary records a digest of the GEMM sources; bench.py uses its
      traffic figure only while the sources still match.
"""
import csv
import glob
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

COPY_BYTES = 256 << 20


def _attn_workloads():
    from bwd_rmsnorm_qkv_amd import synth
    return [("qwen3_4b block, seq 512 (fp16)", synth.QWEN3_4B_BLOCK),
            ("nf4 + LoRA qwen3_4b block, seq 2048 (fp16)", synth.NF4_LORA_QWEN3_4B),
            ("36-layer stack block, seq 1024 (fp32)", synth.STACK36_SMALL)]

GEMM_SOURCES = ["bwd_rmsnorm_qkv_amd/csrc/gemm.hip", "bwd_rmsnorm_qkv_amd/csrc/gemm.h",
                "bwd_rmsnorm_qkv_amd/csrc/common.h"]


ATTENTION_SOURCES = ["bwd_rmsnorm_qkv_amd/csrc/attention.hip", "bwd_rmsnorm_qkv_amd/csrc/attention.h",
                     "bwd_rmsnorm_qkv_amd/csrc/common.h"]


def _rel(path):
    """A path as given on the command line, relative to the repository root."""
    return os.path.relpath(os.path.abspath(path), ROOT)


def source_digest(files=None):
    h = hashlib.sha1()
    for rel in files or GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def run():
    import torch
    import bench
    from bwd_rmsnorm_qkv_amd import qblk, synth
    torch.cuda.set_device(0)
    qblk.lib()
    src = torch.ones(COPY_BYTES // 4, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    c = synth.QWEN3_4B_BLOCK
    specs = bench.block_gemms(c)
    bufs = []
    for (lay, M, N, K, acc) in specs:
        a_shape = (M, K) if lay in (0, 1) else (K, M)
        b_shape = (N, K) if lay == 0 else (K, N)
        A = (torch.randn(a_shape, device="cuda") * 0.02).half()
        B = torch.randn(b_shape, device="cuda").half()
        C = torch.zeros((M, N), device="cuda")
        bufs.append((lay, M, N, K, acc, A, a_shape[1], B, b_shape[1], C))
    ws = max(qblk.gemm_workspace_size(lay, 1, M, N, K) for (lay, M, N, K, _) in specs)
    scratch = torch.empty(max(ws, 16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for (lay, M, N, K, acc, A, lda, B, ldb, C) in bufs:
        qblk.gemm(lay, 1, M, N, K, A, lda, B, ldb, C, N, acc, scratch=scratch)
        torch.cuda.synchronize()
    del bufs, scratch, src, dst
    from bwd_rmsnorm_qkv_amd.runtime import Block, Nf4Block, dev, empty
    for name, cfg in _attn_workloads():
        torch.cuda._sleep(1)  # marker
        torch.cuda.synchronize()
        if name.startswith("nf4"):
            blk = Nf4Block(cfg, synth.LORA_RANK, synth.LORA_ALPHA)
            blk.load(synth.nf4_lora_inputs(cfg, b_std=1e-3))
            blk.fwd_bwd()
        else:
            inp = synth.block_inputs(cfg)
            P = {k: dev(v) for k, v in inp["params"].items()}
            blk = Block(cfg)
            blk.forward(P, dev(inp["x"]))
            blk.backward(P, dev(inp["x"]), dev(inp["dy"]), {k: empty(v.shape) for k, v in inp["params"].items()})
        torch.cuda.synchronize()
        del blk
    print("done", flush=True)


def _rows(d):
    f = glob.glob(os.path.join(d, "*counter_collection.csv"))
    if not f:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = list(csv.DictReader(open(f[0])))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _per_dispatch(rows, counter):
    out = {}
    for r in rows:
        if r["Counter_Name"] == counter:
            out[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
    return [out[k] for k in sorted(out)]


def _groups(disp):
    """Dispatches split at the marker spins: [before the first marker, then
    one group per attention workload]."""
    out = [[]]
    for n, v in disp:
        if "spin_kernel" in n:
            out.append([])
        else:
            out[-1].append((n, v))
    return out


def _split(disp):
    """(copy, launches): the calibration copy and the 12 GEMM launches, each a
    list of dispatches (the product, then its split-K reduce if any)."""
    disp = _groups(disp)[0]
    copy = [v for (n, v) in disp if "copyBuffer" in n]  # the runtime's plain copy kernel
    gemm = [(n, v) for (n, v) in disp if "gemm" in n or "splitk_reduce" in n]
    launches = []
    for n, v in gemm:
        if "splitk_reduce" in n and launches:
            launches[-1].append((n, v))
        else:
            launches.append([(n, v)])
    if len(copy) != 1 or len(launches) != 12:
        raise SystemExit(f"expected 1 copy and 12 GEMM launches, got {len(copy)} and {len(launches)}")
    return copy[0], launches


def summarize(fetch_dir, write_dir, mfma_dir, out_path):
    import bench
    from bwd_rmsnorm_qkv_amd import synth
    fcopy, fl = _split(_per_dispatch(_rows(fetch_dir), "FETCH_SIZE"))
    wcopy, wl = _split(_per_dispatch(_rows(write_dir), "WRITE_SIZE"))
    mrows = _rows(mfma_dir)
    _, busy = _split(_per_dispatch(mrows, "SQ_VALU_MFMA_BUSY_CYCLES"))
    _, gui = _split(_per_dispatch(mrows, "GRBM_GUI_ACTIVE"))
    # counters are in KiB per dispatch; the copy moved COPY_BYTES each way
    f_fac = COPY_BYTES / (fcopy * 1024.0)
    w_fac = COPY_BYTES / (wcopy * 1024.0)
    specs = bench.block_gemms(synth.QWEN3_4B_BLOCK)
    lines = [
        "# HBM traffic and MFMA busy time of the block GEMM launches (Qwen3-4B shape, S 512)",
        "",
        "Commands (repository root; one counter set per run):",
        "",
        "```",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {_rel(fetch_dir)} -o f -- python bench_traffic.py run",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {_rel(write_dir)} -o w -- python bench_traffic.py run",
        f"rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES --output-format csv -d {_rel(mfma_dir)} -o m "
        "-- python bench_traffic.py run",
        f"python bench_traffic.py summarize {_rel(fetch_dir)} {_rel(write_dir)} {_rel(mfma_dir)} "
        + os.path.relpath(out_path, ROOT),
        "```",
        "",
        f"Calibration: a 256 MiB fp32 copy reads FETCH_SIZE {fcopy:.0f} KiB and writes WRITE_SIZE {wcopy:.0f} KiB; "
        f"scale factors {f_fac:.4f} (fetch) and {w_fac:.4f} (write) turn the counters into bytes.",
        "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 128): the first sums over the 1024 SIMDs, the",
        "second over the 8 XCDs, so this is the busy fraction of an average SIMD over the launch.",
        "",
        "| launch | layout M x N x K | dispatches | read MB | written MB | MFMA busy |",
        "|---|---|---:|---:|---:|---:|",
    ]
    total = 0.0
    names = ["NT", "NN", "TN"]
    for i, (spec, fd, wd, bd, gd) in enumerate(zip(specs, fl, wl, busy, gui)):
        rd = sum(v for _, v in fd) * 1024 * f_fac
        wr = sum(v for _, v in wd) * 1024 * w_fac
        total += rd + wr
        util = bd[0][1] / max(gd[0][1] * 128.0, 1.0)
        lay, M, N, K, _ = spec
        lines.append(f"| {i} | {names[lay]} {M} x {N} x {K} | {len(fd)} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{util:.3f} |")
    per = total / len(specs)
    lines += [
        "",
        f"traffic_bytes_per_launch: {per:.0f}",
        f"gemm_source_sha1: {source_digest()}",
        f"attention_source_sha1: {source_digest(ATTENTION_SOURCES)}",
        "",
        "## Attention kernels (MFMA busy and HBM traffic per dispatch)",
        "",
        "| workload | kernel | read MB | written MB | MFMA busy |",
        "|---|---|---:|---:|---:|",
    ]
    fg = _groups(_per_dispatch(_rows(fetch_dir), "FETCH_SIZE"))[1:]
    wg = _groups(_per_dispatch(_rows(write_dir), "WRITE_SIZE"))[1:]
    bg = _groups(_per_dispatch(mrows, "SQ_VALU_MFMA_BUSY_CYCLES"))[1:]
    gg = _groups(_per_dispatch(mrows, "GRBM_GUI_ACTIVE"))[1:]
    for (wname, _), f_, w_, b_, g_ in zip(_attn_workloads(), fg, wg, bg, gg):
        for (n, fv), (_, wv), (_, bv), (_, gv) in zip(f_, w_, b_, g_):
            if "attn_" not in n:
                continue
            short = n.split("attn_", 1)[1].split("(")[0].split("Ev")[0][:40]
            lines.append(f"| {wname} | attn_{short} | {fv * f_fac / 1e3 * 1.024:.1f} | {wv * w_fac / 1e3 * 1.024:.1f} | "
                         f"{bv / max(gv * 128.0, 1.0):.3f} |")
    lines.append("")
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out_path}: {per / 1e6:.1f} MB per launch")


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) == 6 and sys.argv[1] == "summarize":
        summarize(*sys.argv[2:6])
    else:
        raise SystemExit(__doc__)
