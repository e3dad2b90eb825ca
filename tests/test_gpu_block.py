"""Block-level parity on the GPU: qblk_block_forward / qblk_block_backward
against the oracle's block on the same seeded inputs, at the tiny, small
and Qwen3-4B-shaped configurations (full sizes) and at ragged shapes."""
import numpy as np
import pytest
import torch

import oracle
from bwd_rmsnorm_qkv_amd import qblk, synth
from bwd_rmsnorm_qkv_amd.runtime import Block, dev, empty
from gpu_util import BF16_TOL, FP16_TOL, FP32_TOL, announce, check, need_gpu

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": synth.TINY_BLOCK,
    "tiny_ragged": synth.TINY_BLOCK.with_tokens(seq=45, batch=3),
    "small": synth.SMALL_BLOCK,
    "small_ragged_fp16": synth.BlockShape(hidden=512, heads=8, kv_heads=2, head_dim=64, intermediate=1408,
                                          seq=77, batch=2, rope_theta=1e4, gemm_precision=1),
    # fp16 operands with T a multiple of 64 (every product on the direct-to-LDS
    # kernel) and of 8 only (the weight-gradient products on the general one)
    "small_fp16_t192": synth.BlockShape(hidden=512, heads=8, kv_heads=2, head_dim=64, intermediate=1408,
                                        seq=96, batch=2, rope_theta=1e4, gemm_precision=1),
    "small_fp16_t200": synth.BlockShape(hidden=512, heads=8, kv_heads=2, head_dim=64, intermediate=1408,
                                        seq=100, batch=2, rope_theta=1e4, gemm_precision=1),
    # few tokens and a wide hidden size: the long-K products split K, the
    # down projection's dX among them, so its split-K reduce applies the
    # fused SwiGLU backward
    "fp16_wide_split": synth.BlockShape(hidden=4096, heads=8, kv_heads=2, head_dim=64, intermediate=512,
                                        seq=64, batch=1, rope_theta=1e4, gemm_precision=1),
    # head_dim 32: QK-norm/RoPE with four heads per wave, ragged token count
    "small_d32_ragged": synth.BlockShape(hidden=256, heads=8, kv_heads=2, head_dim=32, intermediate=512,
                                         seq=37, batch=2, rope_theta=1e4),
    # no QK-norm (RoPE only; the q/k gamma gradients are zero)
    "small_fp16_no_qk_norm": synth.BlockShape(hidden=512, heads=8, kv_heads=2, head_dim=64, intermediate=1408,
                                              seq=96, batch=2, rope_theta=1e4, qk_norm=0, gemm_precision=1),
    "qwen3_4b": synth.QWEN3_4B_BLOCK,
    # bfloat16 operands (gemm_precision 2)
    "small_bf16_t192": synth.BlockShape(hidden=512, heads=8, kv_heads=2, head_dim=64, intermediate=1408,
                                        seq=96, batch=2, rope_theta=1e4, gemm_precision=2),
    "qwen3_4b_bf16": synth.BlockShape(hidden=2560, heads=32, kv_heads=8, head_dim=128, intermediate=9728,
                                      seq=512, batch=1, rope_theta=1e6, gemm_precision=2),
}


def _tol(c):
    return {0: FP32_TOL, 1: FP16_TOL, 2: BF16_TOL}[c.gemm_precision]


def _gammas_perturbed(p, seed):
    """Non-unit gammas so every gamma path is exercised (the configs use 1)."""
    rng = np.random.default_rng(seed)
    p = dict(p)
    for n in ("g_in", "g_post", "g_q", "g_k"):
        p[n] = (1.0 + 0.25 * rng.standard_normal(p[n].shape)).astype(np.float32)
    return p


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("unit_gammas", [True, False])
def test_block_forward_backward(name, unit_gammas):
    need_gpu()
    c = CASES[name]
    if name.startswith("qwen3_4b") and not unit_gammas:
        pytest.skip("one gamma variant at full Qwen3-4B size")
    announce(f"block {name} T={c.tokens} unit_gammas={unit_gammas}")
    inp = synth.block_inputs(c)
    params = inp["params"] if unit_gammas else _gammas_perturbed(inp["params"], 3)
    P = {k: dev(v) for k, v in params.items()}
    X, DY = dev(inp["x"]), dev(inp["dy"])
    blk = Block(c)
    if name.startswith("qwen3_4b"):
        P = blk.pack_f16(P)  # weights cast once, as the benchmark runs it
    y = blk.forward(P, X)
    grads = {k: empty(v.shape) for k, v in params.items()}
    dx = blk.backward(P, X, DY, grads)
    torch.cuda.synchronize()
    y_ref, cache = oracle.block_forward(c, params, inp["x"])
    dx_ref, g_ref = oracle.block_backward(c, params, cache, inp["dy"])
    tol = _tol(c)
    rep = {}
    check("y", y, y_ref, tol, rep)
    check("dx", dx, dx_ref, tol, rep)
    for k in qblk.PARAMS:
        check("d" + k, grads[k], g_ref[k], tol, rep)
    announce("  " + " ".join(f"{k}={v:.1e}" for k, v in rep.items()))


@pytest.mark.parametrize("name", ["small_fp16_t192", "small_fp16_t200", "small_bf16_t192", "qwen3_4b"])
def test_block_packed_weights_match(name):
    """Caller-packed fp16 weights and the per-call cast into scratch are the
    same numbers, so the results are bitwise equal (at the full Qwen3-4B
    shape this ties the benchmark's launch configuration, packed weights,
    to the oracle-checked per-call path)."""
    need_gpu()
    c = CASES[name]
    announce(f"block packed vs per-call cast {name}")
    inp = synth.block_inputs(c)
    P = {k: dev(v) for k, v in inp["params"].items()}
    X, DY = dev(inp["x"]), dev(inp["dy"])
    blk = Block(c)
    outs = []
    for params in (P, blk.pack_f16(P)):
        y = blk.forward(params, X).clone()
        grads = {k: empty(v.shape) for k, v in inp["params"].items()}
        dx = blk.backward(params, X, DY, grads).clone()
        torch.cuda.synchronize()
        outs.append((y, dx, grads))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
    for k in qblk.PARAMS:
        assert torch.equal(outs[0][2][k], outs[1][2][k]), k


def test_block_backward_deterministic():
    need_gpu()
    c = synth.SMALL_BLOCK
    announce("block determinism (small)")
    inp = synth.block_inputs(c)
    P = {k: dev(v) for k, v in inp["params"].items()}
    X, DY = dev(inp["x"]), dev(inp["dy"])
    blk = Block(c)
    outs = []
    for _ in range(2):
        blk.forward(P, X)
        grads = {k: empty(v.shape) for k, v in inp["params"].items()}
        dx = blk.backward(P, X, DY, grads).clone()
        torch.cuda.synchronize()
        outs.append((dx, grads))
    assert torch.equal(outs[0][0], outs[1][0])
    for k in qblk.PARAMS:
        assert torch.equal(outs[0][1][k], outs[1][1][k]), k


@pytest.mark.parametrize("name", ["small", "small_fp16_t192", "fp16_wide_split", "small_d32_ragged",
                                  "small_fp16_no_qk_norm", "small_bf16_t192"])
def test_block_backward_accumulate(name):
    """Two micro-batches through qblk_block_backward_accumulate: every
    parameter gradient matches the sum of the oracle's gradients of the two
    micro-batches (the tolerance of the configuration), and equals, bit for
    bit, the sum of the two gradients the overwriting backward gives (one
    fp32 addition per element); dx is the second micro-batch's and matches
    the oracle's."""
    need_gpu()
    c = CASES[name]
    announce(f"block backward accumulate {name} T={c.tokens}")
    inp1, inp2 = synth.block_inputs(c, seed=1), synth.block_inputs(c, seed=2)
    params = _gammas_perturbed(inp1["params"], 5)
    P = {k: dev(v) for k, v in params.items()}
    blk = Block(c)
    if c.gemm_precision:
        P = blk.pack_f16(P)
    mb = [(dev(i["x"]), dev(i["dy"])) for i in (inp1, inp2)]
    single = []
    for X, DY in mb:
        blk.forward(P, X)
        g = {k: empty(v.shape) for k, v in inp1["params"].items()}
        dx = blk.backward(P, X, DY, g).clone()
        single.append((dx, g))
    acc = {k: v.clone() for k, v in single[0][1].items()}
    X, DY = mb[1]
    blk.forward(P, X)
    dx = blk.backward(P, X, DY, acc, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dx, single[1][0])
    for k in qblk.PARAMS:
        assert torch.equal(acc[k], single[0][1][k] + single[1][1][k]), k
    ref, dx_ref = None, None
    for i in (inp1, inp2):
        _, cache = oracle.block_forward(c, params, i["x"])
        dx_ref, g = oracle.block_backward(c, params, cache, i["dy"])
        ref = g if ref is None else {k: ref[k] + g[k] for k in ref}
    tol = _tol(c)
    rep = {}
    check("dx", dx, dx_ref, tol, rep)
    for k in qblk.PARAMS:
        check("sum d" + k, acc[k], ref[k], tol, rep)
    announce("  " + " ".join(f"{k}={v:.1e}" for k, v in rep.items()))


def test_block_rejects_bad_config():
    need_gpu()
    c = synth.TINY_BLOCK
    bad = qblk.make_config(c)
    bad.kv_heads = 3
    with pytest.raises(qblk.QblkError) as e:
        qblk.block_workspace_size(bad)
    assert e.value.code == qblk.QBLK_EINVAL
