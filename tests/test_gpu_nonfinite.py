"""Non-finite values are data: a NaN in the input reaches the loss partials
of its own token, never crosses into another sequence of the batch, and the
step's guard (the clip's NaN scale) leaves every weight, moment and 16-bit
weight copy as it was, as the trainer skips its optimizer step on a
non-finite loss or gradient (cuda_trainer.rs page, train_step_inner)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from bwd_rmsnorm_qkv_amd import qblk, synth
from bwd_rmsnorm_qkv_amd.runtime import BlockTrainStep, dev, empty
from gpu_util import FP16_TOL, FP32_TOL, announce, check, need_gpu

pytestmark = pytest.mark.gpu


def test_stack_step_nan_input():
    """2-layer stack, two sequences of 128, vocab 2048; x[last token of the
    first sequence, 3] = NaN. The oracle on the same input fixes what each
    partial must be: that token's partial is NaN, the second sequence's
    partials are finite and match; the loss is NaN, and after the step the
    weights are bitwise the loaded ones and the moments still zero."""
    need_gpu()
    from bwd_rmsnorm_qkv_amd.stack import StackStep
    c = synth.STACK36_SMALL.with_tokens(seq=128, batch=2)
    layers, vocab = 2, 2048
    inp = synth.stack_inputs(c, layers=layers, vocab=vocab, seed=5)
    x = inp["x"].copy()
    x[c.seq - 1, 3] = np.nan
    announce("stack step with a NaN input element (2 layers, vocab 2048)")
    ref = oracle.stack_step(c, inp["layers"], x, inp["g_final"], inp["w_lm"], inp["targets"],
                            synth.CLIP_MAX_NORM, synth.ADAMW)
    assert ref["skipped"]
    st = StackStep(c, layers, vocab)
    st.load(inp, x=x)
    w0 = st.w.buf.clone()
    st.step()
    loss = st.loss()
    part = st.loss_host.numpy().astype(np.float64)
    second = slice(c.seq, 2 * c.seq)
    assert np.isnan(part[c.seq - 1])
    assert np.isfinite(part[second]).all()
    check("second sequence loss partials", part[second], ref["loss_partials"][second], FP32_TOL)
    assert np.isnan(loss)
    assert not np.isfinite(st.norm.item()) and np.isnan(st.scale.item())
    assert torch.equal(st.w.buf, w0), "weights moved on a non-finite step"
    assert not st.m.buf.any().item() and not st.v.buf.any().item(), "moments moved on a non-finite step"


def test_block_train_step_nan_fp16_copies_unchanged():
    """fp16-operand block training step (AdamW writes the packed fp16
    weights): with a NaN in dY the gradients are NaN, the step is skipped,
    and the fp32 masters and the packed fp16 set keep their bytes."""
    need_gpu()
    c = synth.SMALL_BLOCK.with_tokens(seq=96, batch=2)
    c = dataclasses.replace(c, gemm_precision=1)
    announce(f"block train step fp16 with NaN dY T={c.tokens}")
    inp = synth.block_inputs(c)
    ts = BlockTrainStep(c)
    ts.load(inp["params"])
    w0, p0 = ts.w.buf.clone(), ts.packed.clone()
    dy = inp["dy"].copy()
    dy[5, 7] = np.nan
    ts.step(dev(inp["x"]), dev(dy))
    torch.cuda.synchronize()
    assert np.isnan(ts.scale.item())
    assert torch.equal(ts.w.buf, w0) and torch.equal(ts.packed, p0)
    assert not ts.m.buf.any().item() and not ts.v.buf.any().item()


def test_block_forward_nan_stays_in_its_sequence():
    """fp16 operands, two sequences of 96: a NaN in the first sequence's
    last token makes that token's output row NaN; the second sequence's
    rows are finite and match the oracle."""
    need_gpu()
    c = synth.SMALL_BLOCK.with_tokens(seq=96, batch=2)
    c = dataclasses.replace(c, gemm_precision=1)
    announce(f"block forward with a NaN input element T={c.tokens}")
    inp = synth.block_inputs(c)
    x = inp["x"].copy()
    x[c.seq - 1, 0] = np.nan
    from bwd_rmsnorm_qkv_amd.runtime import Block
    blk = Block(c)
    y = blk.forward({k: dev(v) for k, v in inp["params"].items()}, dev(x)).cpu().numpy().astype(np.float64)
    ref = oracle.block_forward(c, inp["params"], x)[0]
    assert np.isnan(y[c.seq - 1]).all()
    second = slice(c.seq, 2 * c.seq)
    assert np.isfinite(y[second]).all()
    check("second sequence y", y[second], ref[second], FP16_TOL)


def test_fused_cross_entropy_nan_row():
    """One NaN hidden row: its loss partial is NaN, every other partial
    finite and equal to the oracle's."""
    need_gpu()
    T, h, V = 64, 128, 1000
    announce(f"fused CE with a NaN row T={T} V={V}")
    rng = np.random.default_rng(21)
    y = rng.standard_normal((T, h)).astype(np.float32)
    y[9, 4] = np.nan
    gf = (1 + 0.2 * rng.standard_normal(h)).astype(np.float32)
    w = (rng.standard_normal((V, h)) * 0.02).astype(np.float32)
    tgt = rng.integers(0, V, T).astype(np.int32)
    loss, am = empty(T), torch.empty(T, dtype=torch.int32, device="cuda")
    dy, dgf, dw = empty((T, h)), empty(h), empty((V, h))
    from bwd_rmsnorm_qkv_amd.runtime import byte_buffer
    scratch = byte_buffer(qblk.cross_entropy_workspace_size(T, h, V))
    qblk.fused_cross_entropy(T, h, V, 1e-6, dev(y), dev(gf), dev(w), dev(tgt), 1.0 / T, loss, am, dy, dgf, dw,
                             scratch)
    ref = oracle.lm_head_cross_entropy(y, gf, w, tgt, 1e-6)
    lp = loss.cpu().numpy().astype(np.float64)
    ok = np.ones(T, bool)
    ok[9] = False
    assert np.isnan(lp[9]) and np.isnan(ref["loss_partials"][9])
    assert np.isfinite(lp[ok]).all()
    check("finite loss partials", lp[ok], ref["loss_partials"][ok], FP32_TOL)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_clip_marks_non_finite_and_adamw_skips(bad):
    """The clip over gradients holding a NaN or an infinity writes a
    non-finite norm and a NaN scale; AdamW and AdamW with the fp16 copy,
    given that scale, write nothing. A finite scale still updates."""
    need_gpu()
    announce(f"clip + AdamW with a {bad} gradient")
    rng = np.random.default_rng(4)
    n = 5000
    w = dev(rng.standard_normal(n).astype(np.float32))
    g_np = rng.standard_normal(n).astype(np.float32)
    g_np[1234] = bad
    g = dev(g_np)
    m, v = torch.zeros_like(w), torch.zeros_like(w)
    w16 = w.half()
    norm, scale = empty(1), empty(1)
    from bwd_rmsnorm_qkv_amd.runtime import byte_buffer
    qblk.clip_grad_norm([g], 1.0, 0, norm, scale, byte_buffer(qblk.clip_workspace_size([g])))
    torch.cuda.synchronize()
    assert not np.isfinite(norm.item()) and np.isnan(scale.item())
    w0, w160 = w.clone(), w16.clone()
    hp = synth.ADAMW
    qblk.adamw_step([w], [g], [m], [v], hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], 1,
                    grad_scale_dev=scale)
    qblk.adamw_step_pack16([w], [g], [m], [v], [w16], hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                           hp["weight_decay"], 1, grad_scale_dev=scale)
    torch.cuda.synchronize()
    assert torch.equal(w, w0) and torch.equal(w16, w160)
    assert not m.any().item() and not v.any().item()
    one = torch.ones(1, device="cuda")
    g_np[1234] = 0.0
    qblk.adamw_step([w], [dev(g_np)], [m], [v], hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], 1,
                    grad_scale_dev=one)
    torch.cuda.synchronize()
    assert not torch.equal(w, w0)
