"""Benchmark of the decoder-block training step on one MI355X.

Headline: train tokens/s of one Qwen3-4B-shaped block forward + backward
(hidden 2560, 32 heads, 8 KV heads, head_dim 128, intermediate 9728,
seq 512, batch 1; fp32 master weights, fp16 GEMM operands with fp32
accumulate), inputs resident in HBM, timed with HIP events over exactly
--steps steps after --warmup untimed ones.

Also reported in the same JSON line:
  roofline      the GEMM kernels of one step (the dominant cost), replayed
                launch by launch with HIP events on the launch stream:
                algorithmic FLOPs / summed launch durations vs the dense
                fp16 MFMA peak;
  hbm           the memory-bound steps exported as calls (AdamW, the clip's
                squared sum, RMSNorm, NF4 dequantize), each timed alone:
                algorithmic bytes / time vs the HBM peak;
  cpu_baseline  the CPU oracle (numpy float64) on a bounded sample of the
                same workload, on this host's cores;
  extra         the 36-layer stack training step (fused CE, global clip,
                AdamW), also with activation checkpointing (6 segments),
                the frozen-NF4 + LoRA block at seq 2048 (each with its
                roofline fraction), and the Qwen3-4B block's whole training
                step (fwd + bwd + clip + AdamW writing the fp16 weights).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu] [--only NAME]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK = 2516.6   # TFLOP/s, dense
MFMA_F8_PEAK = 5033.2    # TFLOP/s, dense
MFMA_F32_PEAK = 157.3    # TFLOP/s
HBM_PEAK = 8000.0        # GB/s
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "block_gemm_hbm_traffic_qwen3_4b_s512.md")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["stack36_train_step", "stack36_train_step_checkpointed", "nf4_lora_block",
                                       "qwen3_4b_block_train_step", "qwen3_4b_block_bf16", "qwen3_4b_gemm_fp8"],
                    help="time only this workload (for kernel traces) and print its JSON object")
    return ap.parse_args()


_SPIN_PER_MS = None


def front_run(torch, ms):
    """Queue a spin kernel that keeps the GPU busy for about `ms` so the
    launches queued behind it are all on the GPU's queue when it ends: the
    events that follow then time the GPU work, not the host's launch
    latency on an idle queue (a training loop runs ahead of the GPU the
    same way). The spin's rate is measured once with events."""
    global _SPIN_PER_MS
    if _SPIN_PER_MS is None:
        torch.cuda._sleep(1000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1 << 20)
        e1.record()
        torch.cuda.synchronize()
        _SPIN_PER_MS = (1 << 20) / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(_SPIN_PER_MS * ms))


def timed(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    front_run(torch, min(20.0, 1.0 + 0.05 * steps))
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda._sleep(1)  # end marker for kernel traces, outside the timed region
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per step


def step_percentiles(fn, steps, torch):
    """p10 / p50 / p90 of per-step times: one event pair around each step,
    all queued behind one spin (the pairs' own packets add a few us)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    fn()
    torch.cuda.synchronize()
    front_run(torch, min(20.0, 1.0 + 0.05 * steps))
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = np.sort([e0.elapsed_time(e1) for e0, e1 in evs])
    pick = lambda q: round(float(t[min(len(t) - 1, int(q * (len(t) - 1) + 0.5))]), 4)
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "steps": steps}


def block_gemms(c):
    """(layout, M, N, K, accumulate) of every GEMM launch of one block
    forward + backward as the block entry points issue them on the fp16
    path: fp16 operands throughout (activation copies written by their
    producers, weights from the packed fp16 set); forward NT, dX NN, dW TN;
    accumulate stands in for the residual read of the O-projection and
    down epilogues."""
    T, h, q, kv, I = c.tokens, c.hidden, c.q_dim, c.kv_dim, c.intermediate
    qkv = q + 2 * kv
    return [
        (0, T, qkv, h, 0), (0, T, h, q, 1), (0, T, 2 * I, h, 0), (0, T, h, I, 1),   # forward
        (1, T, I, h, 0), (2, h, I, T, 0),                                         # down: dX, dW
        (1, T, h, 2 * I, 0), (2, 2 * I, h, T, 0),                                 # gate/up
        (1, T, q, h, 0), (2, h, q, T, 0),                                         # o
        (1, T, h, qkv, 0), (2, qkv, h, T, 0),                                     # qkv
    ]


def gemm_traffic():
    """HBM bytes per GEMM launch from the committed counter summary (see
    bench_traffic.py), or None when it is missing or was taken on GEMM
    sources other than the current ones."""
    import bench_traffic
    try:
        with open(TRAFFIC_SUMMARY) as f:
            txt = f.read()
    except OSError:
        return None
    vals = {}
    for line in txt.splitlines():
        if ": " in line and line.split(": ", 1)[0] in ("traffic_bytes_per_launch", "gemm_source_sha1"):
            k, v = line.split(": ", 1)
            vals[k] = v.strip()
    if vals.get("gemm_source_sha1") != bench_traffic.source_digest() or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def mfma_counters():
    """MFMA busy fractions (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x
    SIMDs) of the block's GEMM launches and of the attention kernels, from
    the same committed counter summary as `traffic` (a rocprofv3 --pmc run
    of bench_traffic.py); each part is None when its kernels' sources
    changed since the counters were taken."""
    import bench_traffic
    try:
        with open(TRAFFIC_SUMMARY) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    gemm, attn, sha, asha = [], [], None, None
    for line in lines:
        if line.startswith("gemm_source_sha1: "):
            sha = line.split(": ", 1)[1].strip()
        if line.startswith("attention_source_sha1: "):
            asha = line.split(": ", 1)[1].strip()
        cells = [x.strip() for x in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[0].isdigit():
            gemm.append({"launch": int(cells[0]), "shape": cells[1], "mfma_busy": float(cells[5])})
        elif len(cells) == 5 and "attn" in cells[1]:
            attn.append({"workload": cells[0], "kernel": cells[1].strip("`"), "mfma_busy": float(cells[4])})
    fresh_attn = asha == bench_traffic.source_digest(bench_traffic.ATTENTION_SOURCES)
    return {"source": TRAFFIC_SUMMARY.replace(ROOT + os.sep, ""),
            "gemm": gemm if sha == bench_traffic.source_digest() else None,
            "attention": attn if fresh_attn else None}


def gemm_roofline(c, torch, qblk, reps):
    """Replay the step's GEMMs (same kernels, shapes, layouts and operand
    types as the block), timed with HIP events on the current stream, the
    stream the launches go to, all queued behind a spin kernel so that the
    events time the GPU work alone. `achieved` = the 12 products' FLOPs
    over the time of the whole sequence (one event pair around it, so the
    figure holds the short gaps between kernels); `per_launch_us` from
    launches bracketed one by one (each figure also holds the event
    packets' own few microseconds)."""
    specs = block_gemms(c)
    bufs = []
    for (lay, M, N, K, acc) in specs:
        a_shape = (M, K) if lay in (0, 1) else (K, M)
        b_shape = (N, K) if lay == 0 else (K, N)
        A = (torch.randn(a_shape, device="cuda") * 0.02).half()
        B = torch.randn(b_shape, device="cuda").half()
        C = torch.zeros((M, N), device="cuda")
        bufs.append((lay, M, N, K, acc, A, a_shape[1], B, b_shape[1], C))
    flops = sum(2.0 * M * N * K for (_, M, N, K, _) in specs)
    ws = max(qblk.gemm_workspace_size(lay, 1, M, N, K) for (lay, M, N, K, _) in specs)
    scratch = torch.empty(max(ws, 16), dtype=torch.uint8, device="cuda")

    def run_all(events=None):
        for i, (lay, M, N, K, acc, A, lda, B, ldb, C) in enumerate(bufs):
            if events:
                events[i][0].record()
            qblk.gemm(lay, 1, M, N, K, A, lda, B, ldb, C, N, acc, scratch=scratch)
            if events:
                events[i][1].record()

    for _ in range(3):
        run_all()
    torch.cuda.synchronize()
    # the sequence: one event pair around the 12 launches (no event packets
    # between kernels); per launch: each bracketed by its own pair, which
    # adds the event packets' few microseconds to every figure
    total_ms, per = 0.0, np.zeros(len(bufs))
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        front_run(torch, 3.0)
        e0.record()
        run_all()
        e1.record()
        torch.cuda._sleep(1)
        torch.cuda.synchronize()
        total_ms += e0.elapsed_time(e1)
    for _ in range(reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in bufs]
        front_run(torch, 3.0)
        run_all(ev)
        torch.cuda._sleep(1)
        torch.cuda.synchronize()
        per += np.array([a.elapsed_time(b) for a, b in ev])
    step_ms = total_ms / reps
    achieved = flops / (step_ms * 1e-3) / 1e12
    return {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK, "unit": "TFLOP/s",
        "frac": round(achieved / MFMA_F16_PEAK, 4), "traffic": gemm_traffic(),
        "traffic_source": "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of the same 12 launches, scaled by a 256 MiB "
                          "copy (profiles/block_gemm_hbm_traffic_qwen3_4b_s512.md; null when the GEMM sources "
                          "changed since)",
        "kernel": "gemm_dma_kernel (the 12 GEMM launches of one block fwd+bwd, split-K reduce included)",
        "flops_per_step": flops, "gemm_ms_per_step": round(step_ms, 4),
        "avg_launch_us": round(1e3 * step_ms / len(bufs), 2),
        "per_launch_us": [round(1e3 * x / reps, 1) for x in per],
    }


def stack_param_count(synth):
    c, L, V = synth.STACK36_SMALL, synth.STACK_LAYERS, synth.STACK_VOCAB
    h, qd, kvd, I, d = c.hidden, c.heads * c.head_dim, c.kv_heads * c.head_dim, c.intermediate, c.head_dim
    per_layer = h * qd + 2 * h * kvd + qd * h + 3 * h * I + 2 * h + 2 * d
    return L * per_layer + V * h + h


def hbm_kernels(torch, qblk, synth, reps=10):
    """The memory-bound steps the library exports as calls, each timed alone
    with HIP events on the current stream (reps calls after two warm-ups):
    algorithmic bytes / time against the HBM peak. Working sets are sized
    well beyond the 256 MB last-level cache (the `shape` of each row), so
    the rate is HBM's; the norms are also timed at the Qwen3-4B block shape
    the block step runs (512 rows: 10-16 MB, cache-resident and
    launch-latency bound)."""
    out = []

    def add(name, workload, nbytes, fn):
        ms = timed(fn, reps, 2, torch)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out.append({"kernel": name, "workload": workload, "bytes": int(nbytes), "us": round(ms * 1e3, 2),
                    "GB/s": round(gbps, 1), "frac": round(gbps / HBM_PEAK, 4)})

    n = stack_param_count(synth)
    w = torch.randn(n, device="cuda") * 0.02
    g = torch.randn(n, device="cuda") * 1e-3
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    add("adamw_step", f"{n} fp32 parameters (36-layer stack): w, g, m, v read; w, m, v written", 28 * n,
        lambda: qblk.adamw_step([w], [g], [m], [v], 1e-3, 0.9, 0.999, 1e-8, 0.01, 1))
    w16 = torch.empty(n, dtype=torch.float16, device="cuda")
    add("adamw_step_pack16", f"{n} fp32 parameters: as adamw_step plus the fp16 copy of w written", 30 * n,
        lambda: qblk.adamw_step_pack16([w], [g], [m], [v], [w16], 1e-3, 0.9, 0.999, 1e-8, 0.01, 1))
    del w16
    norm = torch.zeros(1, device="cuda")
    scale = torch.zeros(1, device="cuda")
    cs = torch.empty(max(qblk.clip_workspace_size([g]), 16), dtype=torch.uint8, device="cuda")
    add("clip_grad_norm (squared sum)", f"{n} fp32 gradients read once", 4 * n,
        lambda: qblk.clip_grad_norm([g], 1.0, 0, norm, scale, cs))
    del w, m, v, cs, g
    c = synth.QWEN3_4B_BLOCK
    h = c.hidden
    for T, tag in ((c.tokens, "block shape"), (16384, "HBM-resident")):
        x = torch.randn(T, h, device="cuda")
        dy = torch.randn(T, h, device="cuda")
        gam = torch.ones(h, device="cuda")
        y = torch.empty_like(x)
        rho = torch.empty(T, device="cuda")
        add("rmsnorm_forward", f"[{T}, {h}] fp32 ({tag}): x read, y written", 2 * 4 * T * h,
            lambda: qblk.rmsnorm_forward(T, h, 1e-6, x, None, gam, y, None, rho))
        dx = torch.empty_like(x)
        dgam = torch.empty(h, device="cuda")
        rs = torch.empty(max(qblk.rmsnorm_workspace_size(T, h), 16), dtype=torch.uint8, device="cuda")
        add("rmsnorm_backward", f"[{T}, {h}] fp32 ({tag}): x, dy read, dx written", 3 * 4 * T * h,
            lambda: qblk.rmsnorm_backward(T, h, 1e-6, x, gam, dy, None, dx, dgam, rs))
        del x, dy, y, dx, rs
    T, I = 4096, c.intermediate
    gu = torch.randn(T, 2 * I, device="cuda")
    sw = torch.empty(T, I, device="cuda")
    add("swiglu_forward", f"gu [{T}, {2 * I}] read, s [{T}, {I}] written (fp32)", 3 * 4 * T * I,
        lambda: qblk.swiglu_forward(T, I, gu, sw))
    dgu = torch.empty_like(gu)
    add("swiglu_backward", f"gu [{T}, {2 * I}], ds [{T}, {I}] read, dgu written (fp32)", 5 * 4 * T * I,
        lambda: qblk.swiglu_backward(T, I, gu, sw, dgu))
    del gu, sw, dgu
    T, S, H, KV, d = 8192, 512, c.heads, c.kv_heads, c.head_dim
    ld = (H + 2 * KV) * d
    qkv = torch.randn(T, ld, device="cuda")
    gq, gk = torch.ones(d, device="cuda"), torch.ones(d, device="cuda")
    qr, kr = torch.empty(T, H * d, device="cuda"), torch.empty(T, KV * d, device="cuda")
    rq, rk = torch.empty(T, H, device="cuda"), torch.empty(T, KV, device="cuda")
    qs = torch.empty(max(qblk.qk_norm_rope_workspace_size(T, S, H, KV, d), 16), dtype=torch.uint8, device="cuda")
    add("qk_norm_rope_forward", f"q, k of qkv [{T}, {ld}] read, qr, kr written (fp32, 32/8 heads, d128)",
        2 * 4 * T * (H + KV) * d,
        lambda: qblk.qk_norm_rope_forward(T, S, H, KV, d, 1, 1e-6, 1e6, qkv, ld, gq, gk, qr, kr, rq, rk, qs))
    dqkv = torch.empty_like(qkv)
    dg1, dg2 = torch.empty(d, device="cuda"), torch.empty(d, device="cuda")
    add("qk_norm_rope_backward", f"q, k of qkv, dqr, dkr read; dq, dk written (fp32, [{T}] tokens)",
        3 * 4 * T * (H + KV) * d,
        lambda: qblk.qk_norm_rope_backward(T, S, H, KV, d, 1, 1e-6, 1e6, qkv, ld, gq, gk, qr, kr, dqkv, dg1, dg2,
                                           qs))
    del qkv, qr, kr, dqkv, qs
    T, V = synth.STACK36_SMALL.tokens, synth.STACK_VOCAB
    z = torch.randn(T, V, device="cuda")
    tgt = torch.randint(0, V, (T,), dtype=torch.int32, device="cuda")
    lp, am = torch.empty(T, device="cuda"), torch.empty(T, dtype=torch.int32, device="cuda")
    add("cross_entropy_rows", f"logits [{T}, {V}] fp32 read and overwritten by their gradient", 2 * 4 * T * V,
        lambda: qblk.cross_entropy_rows(T, V, z, tgt, 1.0 / T, lp, am))
    del z
    T = 16384
    x = torch.randn(T, h, device="cuda")
    q8 = torch.empty(T, h, dtype=torch.uint8, device="cuda")
    inv = torch.empty(1, device="cuda")
    fs = torch.empty(qblk.fp8_quantize_workspace_size(T, h), dtype=torch.uint8, device="cuda")
    add("fp8_quantize", f"[{T}, {h}] fp32 -> E4M3 codes: x read twice (max, then convert), codes written",
        9 * T * h, lambda: qblk.fp8_quantize(T, h, x, h, 0, q8, h, inv, fs))
    del x, q8
    numel = 2 * c.intermediate * h
    codes = torch.randint(0, 256, (numel // 2,), dtype=torch.uint8, device="cuda")
    absmax = torch.rand(numel // 64, device="cuda")
    wout = torch.empty(numel, device="cuda")
    add("nf4_dequantize", f"gate+up weights [{2 * c.intermediate}, {h}]: codes and absmax read, fp32 written",
        numel // 2 + 4 * (numel // 64) + 4 * numel, lambda: qblk.nf4_dequantize(codes, absmax, numel, wout))
    return out


def host_cores():
    """(threads the BLAS pool runs, cores in this process's affinity mask,
    CPU model)."""
    aff = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [aff])
    except Exception:
        blas = aff
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return blas, aff, model


def cpu_baseline(c, inp, budget_s=10.0):
    import oracle
    blas, aff, model = host_cores()
    n, t0 = 0, time.perf_counter()
    while True:
        y, cache = oracle.block_forward(c, inp["params"], inp["x"])
        oracle.block_backward(c, inp["params"], cache, inp["dy"])
        n += 1
        if time.perf_counter() - t0 > budget_s or n >= 5:
            break
    dt = (time.perf_counter() - t0) / n
    return {"value": round(c.tokens / dt, 2), "unit": "tokens/s", "cores": blas, "kind": "oracle",
            "sample": f"{n} x full Qwen3-4B-shaped block fwd+bwd (512 tokens), numpy float64, "
                      f"{dt:.2f} s each", "affinity_cores": aff, "cpu_model": model}


def cpu_baselines_other(synth):
    """The oracle on the other workloads, each on a bounded sample scaled to
    the workload's unit (tokens/s of a block or of a stack step)."""
    import oracle
    blas, aff, model = host_cores()
    out = []

    def tm(fn, reps=1):
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t0) / reps

    def block_fb(c, inp):
        _, cache = oracle.block_forward(c, inp["params"], inp["x"])
        return oracle.block_backward(c, inp["params"], cache, inp["dy"])

    c = synth.TINY_BLOCK
    inp = synth.block_inputs(c)
    dt = tm(lambda: block_fb(c, inp), 20)
    out.append({"workload": "tiny block fwd+bwd (32 tokens, fp32)", "value": round(c.tokens / dt, 1),
                "unit": "tokens/s", "sample": f"20 runs, {dt * 1e3:.1f} ms each"})
    c = synth.SMALL_BLOCK
    inp = synth.block_inputs(c)

    def small_step():
        _, g = block_fb(c, inp)
        names = list(g)
        _, _, cl = oracle.global_clip([g[k] for k in names], synth.CLIP_MAX_NORM)
        for k, gg in zip(names, cl):
            z = np.zeros(np.shape(gg))
            oracle.adamw_update(inp["params"][k], gg, z, z, step=1, **synth.ADAMW)
    dt = tm(small_step, 2)
    out.append({"workload": "small block fwd+bwd + clip + AdamW (1024 tokens, fp32)",
                "value": round(c.tokens / dt, 1), "unit": "tokens/s", "sample": f"2 runs, {dt:.2f} s each"})
    # 36-layer stack step: one layer fwd+bwd, the LM head + CE and AdamW over
    # 1/16 of the parameters, each timed once and scaled to the whole step
    c = synth.STACK36_SMALL
    inp = synth.block_inputs(c)
    t_layer = tm(lambda: block_fb(c, inp))
    rng = np.random.default_rng(0)
    V = synth.STACK_VOCAB
    w_lm = (rng.standard_normal((V, c.hidden)) * 0.02).astype(np.float32)
    tgt = rng.integers(0, V, c.tokens)
    t_lm = tm(lambda: oracle.lm_head_cross_entropy(inp["x"], np.ones(c.hidden, np.float32), w_lm, tgt, c.eps))
    del w_lm
    n_par = stack_param_count(synth)
    part = n_par // 16
    wp, gp = rng.standard_normal(part) * 0.02, rng.standard_normal(part) * 1e-3
    t_adam = 16 * tm(lambda: oracle.adamw_update(wp, gp, np.zeros(part), np.zeros(part), step=1, **synth.ADAMW))
    step_s = synth.STACK_LAYERS * t_layer + t_lm + t_adam
    out.append({"workload": "36-layer stack training step (1024 tokens, vocab 151936, fp32)",
                "value": round(c.tokens / step_s, 2), "unit": "tokens/s",
                "sample": f"1 layer fwd+bwd {t_layer:.2f} s x 36 + LM head/CE {t_lm:.2f} s + AdamW "
                          f"{t_adam:.2f} s (1/16 of the parameters, x 16) = {step_s:.1f} s per step"})
    # NF4 + LoRA block at seq 2048: one forward + backward
    c = synth.NF4_LORA_QWEN3_4B
    inp = synth.nf4_lora_inputs(c, b_std=1e-3)
    deq = {}
    for k in synth.PROJ_NAMES:
        packed, scales, _ = oracle.nf4_quantize(inp["params"][k])
        deq[k] = oracle.nf4_dequantize(packed, scales, inp["params"][k].shape)
    gam = {k: inp["params"][k] for k in ("g_in", "g_post", "g_q", "g_k")}
    sc = synth.LORA_ALPHA / synth.LORA_RANK

    def nf4_fb():
        _, cache = oracle.nf4_block_forward(c, gam, deq, inp["lora_a"], inp["lora_b"], inp["x"], sc)
        oracle.nf4_block_backward(c, gam, deq, inp["lora_a"], inp["lora_b"], cache, inp["dy"], sc)
    dt = tm(nf4_fb)
    out.append({"workload": "NF4 + LoRA Qwen3-4B-shaped block fwd+bwd (2048 tokens)",
                "value": round(c.tokens / dt, 1), "unit": "tokens/s", "sample": f"1 run, {dt:.2f} s"})
    for o in out:
        o.update({"cores": blas, "kind": "oracle", "affinity_cores": aff, "cpu_model": model})
    return out


def stack_flops(synth):
    """Algorithmic FLOPs of one 36-layer stack step: per layer 6 T P of the
    projections (fwd, dX, dW) plus the causal attention (fwd 2 2 S^2/2 d
    per head, backward twice that), and the LM head's 6 T V h."""
    c, L, V = synth.STACK36_SMALL, synth.STACK_LAYERS, synth.STACK_VOCAB
    T, h, qd, kvd, I, d = c.tokens, c.hidden, c.q_dim, c.kv_dim, c.intermediate, c.head_dim
    P = h * (qd + 2 * kvd) + qd * h + 3 * h * I
    attn = 3 * 2 * 2 * (c.seq * c.seq / 2) * d * c.heads * c.batch
    return L * (6 * T * P + attn) + 6 * T * V * h


def nf4_flops(synth):
    """fwd + dX of the 7 projections (4 T P; no base dW), causal attention
    fwd + bwd, and the rank-r LoRA products (h, dh, dA, dB and their share
    of the fused products: 2 T r (in + out) per projection, x 4)."""
    c, r = synth.NF4_LORA_QWEN3_4B, synth.LORA_RANK
    T, h, qd, kvd, I, d = c.tokens, c.hidden, c.q_dim, c.kv_dim, c.intermediate, c.head_dim
    P = h * (qd + 2 * kvd) + qd * h + 3 * h * I
    attn = 3 * 2 * 2 * (c.seq * c.seq / 2) * d * c.heads * c.batch
    io = [(h, qd), (h, kvd), (h, kvd), (qd, h), (h, I), (h, I), (I, h)]
    lora = sum(4 * 2 * T * r * (i + o) for i, o in io)
    return 4 * T * P + attn + lora


def extra_stack(torch, qblk, synth, steps, warmup, checkpoint_segments=None):
    from bwd_rmsnorm_qkv_amd.stack import StackStep
    st = StackStep(synth.STACK36_SMALL, synth.STACK_LAYERS, synth.STACK_VOCAB,
                   checkpoint_segments=checkpoint_segments)
    st.load(synth.stack_inputs())
    ms = timed(st.step, steps, warmup, torch)
    flops = stack_flops(synth)
    adam_bytes = 28 * stack_param_count(synth)
    ideal_ms = (flops / (MFMA_F32_PEAK * 1e12) + adam_bytes / (HBM_PEAK * 1e9)) * 1e3
    out = {"workload": "36-layer stack (h512, 8 heads, 2 kv, d64, I1408), seq 1024, vocab 151936, fp32: "
                       "fwd + fused CE + bwd + global clip + AdamW, loss partials to host",
           "ms_per_step": round(ms, 3), "tokens_per_s": round(synth.STACK36_SMALL.tokens / ms * 1e3, 1),
           "activation_bytes": st.workspace_bytes(),
           "roofline": {"bound": "mfma fp32 + hbm", "gflop": round(flops / 1e9, 1),
                        "adamw_gb": round(adam_bytes / 1e9, 3), "ideal_ms": round(ideal_ms, 3),
                        "peak": f"{MFMA_F32_PEAK} TFLOP/s fp32, {HBM_PEAK} GB/s",
                        "frac": round(ideal_ms / ms, 4)}}
    if checkpoint_segments:
        out["checkpoint_segments"] = checkpoint_segments
    return out


def extra_stack_ckpt(torch, qblk, synth, steps, warmup):
    return extra_stack(torch, qblk, synth, steps, warmup, checkpoint_segments=6)


def extra_nf4(torch, qblk, synth, steps, warmup):
    from bwd_rmsnorm_qkv_amd.runtime import Nf4Block
    c = synth.NF4_LORA_QWEN3_4B
    blk = Nf4Block(c, synth.LORA_RANK, synth.LORA_ALPHA)
    blk.load(synth.nf4_lora_inputs(c, b_std=1e-3))
    ms = timed(blk.fwd_bwd, steps, warmup, torch)
    flops = nf4_flops(synth)
    ideal_ms = flops / (MFMA_F16_PEAK * 1e12) * 1e3
    return {"workload": "frozen NF4 + LoRA r16 Qwen3-4B block, seq 2048, fp16 operands, NF4 decoded inside the "
                        "GEMMs: fwd + bwd (dx, LoRA grads)",
            "ms_per_step": round(ms, 3), "tokens_per_s": round(c.tokens / ms * 1e3, 1),
            "roofline": {"bound": "mfma fp16", "gflop": round(flops / 1e9, 1), "ideal_ms": round(ideal_ms, 4),
                         "peak": f"{MFMA_F16_PEAK} TFLOP/s", "frac": round(ideal_ms / ms, 4)}}


def extra_block_train(torch, qblk, synth, steps, warmup):
    """One Qwen3-4B-shaped block's whole training step: fwd + bwd + global
    clip + AdamW, AdamW writing the fp16 weight copies the next step's GEMMs
    read (no separate cast)."""
    from bwd_rmsnorm_qkv_amd.runtime import BlockTrainStep, dev
    c = synth.QWEN3_4B_BLOCK
    inp = synth.block_inputs(c)
    st = BlockTrainStep(c)
    st.load(inp["params"])
    X, DY = dev(inp["x"]), dev(inp["dy"])
    ms = timed(lambda: st.step(X, DY), steps, warmup, torch)
    return {"workload": "Qwen3-4B-shaped block training step (seq 512): fwd + bwd + global clip + AdamW with the "
                        "fp16 weight copies written by AdamW", "ms_per_step": round(ms, 4),
            "tokens_per_s": round(c.tokens / ms * 1e3, 1)}


def extra_block_bf16(torch, qblk, synth, steps, warmup):
    """The headline block with bfloat16 GEMM and attention operands."""
    from dataclasses import replace
    from bwd_rmsnorm_qkv_amd.runtime import Block, dev, empty
    c = replace(synth.QWEN3_4B_BLOCK, gemm_precision=2)
    inp = synth.block_inputs(c)
    blk = Block(c)
    P = blk.pack_f16({k: dev(v) for k, v in inp["params"].items()})
    X, DY = dev(inp["x"]), dev(inp["dy"])
    G = {k: empty(v.shape) for k, v in inp["params"].items()}

    def step():
        blk.forward(P, X)
        blk.backward(P, X, DY, G)
    ms = timed(step, steps, warmup, torch)
    return {"workload": "Qwen3-4B-shaped block fwd+bwd (seq 512) with bfloat16 operands, fp32 accumulate",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(c.tokens / ms * 1e3, 1)}


def extra_gemm_fp8(torch, qblk, synth, steps, warmup):
    """The 12 products of one Qwen3-4B block step (seq 512) as fp8 NT
    products (qblk_gemm_fp8): activations and weights E4M3, gradients E5M2,
    every operand already quantized with K contiguous (the backward's dX and
    dW take transposed copies), against the fp8 MFMA peak; beside it the
    quantizer at the block's activation shapes, the work an fp8 step adds
    per product."""
    c = synth.QWEN3_4B_BLOCK
    bufs, flops = [], 0.0
    for i, (_, M, N, K, acc) in enumerate(block_gemms(c)):
        A = torch.randint(0, 0x70, (M, K), dtype=torch.uint8, device="cuda")
        B = torch.randint(0, 0x70, (N, K), dtype=torch.uint8, device="cuda")
        Cm = torch.empty(M, N, device="cuda")
        ws = qblk.gemm_fp8_workspace_size(M, N, K)
        sc = torch.empty(ws, dtype=torch.uint8, device="cuda") if ws else None
        bufs.append((M, N, K, A, int(i >= 4), B, Cm, acc, sc))
        flops += 2.0 * M * N * K
    one = torch.ones(1, device="cuda")

    def seq():
        for M, N, K, A, a5, B, Cm, acc, sc in bufs:
            qblk.gemm_fp8(M, N, K, A, K, a5, B, K, 0, one, one, Cm, N, accumulate=acc, scratch=sc)
    ms = timed(seq, steps, warmup, torch)
    tf = flops / (ms * 1e-3) / 1e12
    quant = []
    for rows, cols in ((c.tokens, c.hidden), (c.tokens, c.intermediate), (c.tokens, 2 * c.intermediate)):
        x = torch.randn(rows, cols, device="cuda")
        q8 = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
        inv = torch.empty(1, device="cuda")
        fs = torch.empty(qblk.fp8_quantize_workspace_size(rows, cols), dtype=torch.uint8, device="cuda")
        qms = timed(lambda: qblk.fp8_quantize(rows, cols, x, cols, 1, q8, cols, inv, fs), steps, warmup, torch)
        quant.append({"shape": [rows, cols], "us": round(qms * 1e3, 2)})
    return {"workload": "the 12 GEMM products of one Qwen3-4B block fwd+bwd (seq 512) as fp8 NT products, "
                        "operands pre-quantized", "ms_per_step": round(ms, 4), "gflop": round(flops / 1e9, 2),
            "roofline": {"bound": "mfma fp8", "achieved": round(tf, 1), "peak": MFMA_F8_PEAK, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_F8_PEAK, 4)},
            "fp8_quantize": quant}


EXTRAS = {"stack36_train_step": extra_stack, "stack36_train_step_checkpointed": extra_stack_ckpt,
          "nf4_lora_block": extra_nf4, "qwen3_4b_block_train_step": extra_block_train,
          "qwen3_4b_block_bf16": extra_block_bf16, "qwen3_4b_gemm_fp8": extra_gemm_fp8}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); nothing here shards across GPUs.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from bwd_rmsnorm_qkv_amd import qblk, synth
    from bwd_rmsnorm_qkv_amd.runtime import Block, dev, empty

    torch.cuda.set_device(0)
    qblk.lib()
    if args.only:
        fn = EXTRAS[args.only]
        print(json.dumps({"only": args.only, "steps": args.steps, **fn(torch, qblk, synth, args.steps, args.warmup)}),
              flush=True)
        return
    c = synth.QWEN3_4B_BLOCK
    log("generating Qwen3-4B-shaped block inputs")
    inp = synth.block_inputs(c)
    P = {k: dev(v) for k, v in inp["params"].items()}
    X, DY = dev(inp["x"]), dev(inp["dy"])
    G = {k: empty(v.shape) for k, v in inp["params"].items()}
    blk = Block(c)
    # the fp16 weight copies the GEMMs read: packed once at load here; in a
    # training step AdamW writes them as it updates the fp32 masters
    # (qblk_adamw_step_pack16, timed in the qwen3_4b_block_train_step extra)
    P = blk.pack_f16(P)

    def step():
        blk.forward(P, X)
        blk.backward(P, X, DY, G)

    log("timing block fwd+bwd")
    ms = timed(step, args.steps, args.warmup, torch)
    value = c.tokens / (ms * 1e-3)
    log(f"block fwd+bwd {ms:.4f} ms/step, {value:.0f} tokens/s")
    pct = step_percentiles(step, max(10, args.steps), torch)
    roof = gemm_roofline(c, torch, qblk, reps=max(5, args.steps // 2))
    log(f"GEMM roofline {roof['achieved']} TFLOP/s ({roof['frac']*100:.1f}% of peak)")
    out = {
        "metric": "train tokens/s per block fwd+bwd (Qwen3-4B shape); % MFMA peak, % HBM BW",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "step_ms_percentiles": pct,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16 GEMM operands, fp32 accumulate/master",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights)",
        "config": {"workload": "Qwen3-4B-shaped decoder block fwd+bwd", "hidden": c.hidden, "heads": c.heads,
                   "kv_heads": c.kv_heads, "head_dim": c.head_dim, "intermediate": c.intermediate,
                   "seq": c.seq, "batch": c.batch, "global_batch": c.batch, "seq_len": c.seq,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "mfma_busy_counters": mfma_counters(),
        "fp16_weights": "packed once at load; a training step refreshes them inside AdamW "
                        "(qblk_adamw_step_pack16), see extra.qwen3_4b_block_train_step",
    }
    log("memory-bound kernels")
    out["hbm"] = hbm_kernels(torch, qblk, synth)
    if not args.no_extra:
        extra = {}
        for name, fn in EXTRAS.items():
            try:
                log(f"extra: {name}")
                extra[name] = fn(torch, qblk, synth, max(3, args.steps // 10), 2)
            except Exception as e:  # reported, never silently dropped
                extra[name] = {"error": repr(e)}
        out["extra"] = extra
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(c, inp)
        out["cpu_baseline_other_workloads"] = cpu_baselines_other(synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
