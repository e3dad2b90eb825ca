"""Parity of the frozen-NF4 + LoRA block on the GPU: the GPU encodes the base
weights itself (codes checked bit-exact against the oracle's encoding), then
forward and the LoRA-only backward against the oracle block built on the
oracle's dequantized weights."""
import numpy as np
import pytest
import torch

import oracle
from bwd_rmsnorm_qkv_amd import qblk, synth
from bwd_rmsnorm_qkv_amd.runtime import Nf4Block
from gpu_util import FP16_TOL, announce, check, need_gpu

pytestmark = pytest.mark.gpu

SMALL = synth.BlockShape(hidden=256, heads=4, kv_heads=2, head_dim=64, intermediate=512, seq=70, batch=2,
                         rope_theta=1e6, gemm_precision=1)

# T = 72 (a multiple of 8): the fp16 copies path with contractions whose K is
# not a multiple of 64 (general GEMM kernel); T = 140: the fused-decode path
SMALL_T72 = synth.BlockShape(hidden=256, heads=4, kv_heads=2, head_dim=64, intermediate=480, seq=36, batch=2,
                             rope_theta=1e6, gemm_precision=1)
# T = 600: the fused kernel's 256 x 256 tiles (M >= 512), ragged in M and N
MID_T600 = synth.BlockShape(hidden=256, heads=4, kv_heads=2, head_dim=64, intermediate=576, seq=300, batch=2,
                            rope_theta=1e6, gemm_precision=1)
CASES = [("small_ragged", SMALL, 8), ("small_t72", SMALL_T72, 8), ("mid_t600", MID_T600, 8),
         ("qwen3_4b_seq2048", synth.NF4_LORA_QWEN3_4B, synth.LORA_RANK)]


@pytest.mark.parametrize("name,c,rank", CASES)
@pytest.mark.parametrize("b_std", [0.0, 1e-3])
def test_nf4_lora_block(name, c, rank, b_std):
    need_gpu()
    announce(f"nf4 lora block {name} T={c.tokens} rank={rank} b_std={b_std}")
    alpha = 2.0 * rank
    inp = synth.nf4_lora_inputs(c, rank=rank, b_std=b_std)
    blk = Nf4Block(c, rank, alpha)
    blk.load(inp)
    y = blk.forward()
    dx = blk.backward()
    torch.cuda.synchronize()
    deq = {}
    for n in synth.PROJ_NAMES:
        packed, scales, _ = oracle.nf4_quantize(inp["params"][n])
        assert np.array_equal(blk.codes[n].cpu().numpy(), packed), n
        assert np.array_equal(blk.absmax[n].cpu().numpy().view(np.uint32), scales.view(np.uint32)), n
        deq[n] = oracle.nf4_dequantize(packed, scales, inp["params"][n].shape)
    gam = {n: inp["params"][n] for n in ("g_in", "g_post", "g_q", "g_k")}
    scale = alpha / rank
    y_ref, cache = oracle.nf4_block_forward(c, gam, deq, inp["lora_a"], inp["lora_b"], inp["x"], scale)
    dx_ref, da_ref, db_ref = oracle.nf4_block_backward(c, gam, deq, inp["lora_a"], inp["lora_b"], cache,
                                                       inp["dy"], scale)
    rep = {}
    check("y", y, y_ref, FP16_TOL, rep)
    check("dx", dx, dx_ref, FP16_TOL, rep)
    for n in synth.PROJ_NAMES:
        if b_std == 0.0:
            assert torch.count_nonzero(blk.grad_a[n]).item() == 0, f"dA_{n} must be exactly 0 when B = 0"
        else:
            check("dA_" + n, blk.grad_a[n], da_ref[n], FP16_TOL, rep)
        check("dB_" + n, blk.grad_b[n], db_ref[n], FP16_TOL, rep)
    announce("  " + " ".join(f"{k}={v:.1e}" for k, v in rep.items()))


def test_nf4_backward_recompute_bitwise():
    """backward(recompute=True) re-runs the forward into the workspace first:
    with the workspace overwritten after the forward, dx and the LoRA
    gradients equal those of the plain forward + backward bit for bit."""
    need_gpu()
    c = SMALL.with_tokens(seq=64, batch=2)
    announce(f"nf4 lora block recompute T={c.tokens}")
    inp = synth.nf4_lora_inputs(c, rank=8, b_std=1e-3)
    blk = Nf4Block(c, 8, 16.0)
    blk.load(inp)
    blk.forward()
    dx0 = blk.backward().clone()
    ga0 = {n: t.clone() for n, t in blk.grad_a.items()}
    gb0 = {n: t.clone() for n, t in blk.grad_b.items()}
    blk.saved.fill_(0x7F)  # the saved activations are gone
    dx1 = blk.backward(recompute=True)
    torch.cuda.synchronize()
    assert torch.equal(dx0, dx1)
    for n in synth.PROJ_NAMES:
        assert torch.equal(ga0[n], blk.grad_a[n]), n
        assert torch.equal(gb0[n], blk.grad_b[n]), n
