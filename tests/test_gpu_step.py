"""Parity of the step entry points on the GPU: cross-entropy (rows and
fused with the LM head), the global clip, AdamW, one training step of the
small block, and one full 36-layer stack step with vocab 151936."""
import numpy as np
import pytest
import torch

import oracle
from bwd_rmsnorm_qkv_amd import qblk, synth
from bwd_rmsnorm_qkv_amd.runtime import Block, FlatParams, block_shapes, byte_buffer, dev, empty
from gpu_util import BF16_TOL, FP16_TOL, FP32_TOL, announce, check, need_gpu, rel_err

pytestmark = pytest.mark.gpu


def test_cross_entropy_rows_bit_exact_argmax():
    """Both sides get the same fp32 logits: argmax bit-exact, loss and
    gradient within the fp32 tolerance. Ties and a NaN-free extreme row
    included."""
    need_gpu()
    announce("cross_entropy_rows T=67 V=1000")
    rng = np.random.default_rng(11)
    T, V = 67, 1000
    z = (rng.standard_normal((T, V)) * 3).astype(np.float32)
    z[5, 17] = z[5, 400] = z[5].max() + 1.0          # tie: first index wins
    z[6] = 0.0                                      # all equal
    z[7] *= 30.0                                    # large logits
    tgt = rng.integers(0, V, T).astype(np.int32)
    Z = dev(z)
    loss, am = empty(T), torch.empty(T, dtype=torch.int32, device="cuda")
    qblk.cross_entropy_rows(T, V, Z, dev(tgt), 1.0 / T, loss, am)
    ref = oracle.lm_head_cross_entropy(z, None, np.eye(V), tgt, 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(am.cpu().numpy(), ref["argmax"])
    check("loss_partials", loss, ref["loss_partials"], FP32_TOL)
    zr = ref["logits"]
    p = np.exp(zr - zr.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    p[np.arange(T), tgt] -= 1
    check("dz", Z, p / T, FP32_TOL)


@pytest.mark.parametrize("T,h,V,final_norm", [(40, 64, 1000, True), (256, 512, 4096, False),
                                               (1024, 512, 151936, True)])
def test_fused_cross_entropy(T, h, V, final_norm):
    need_gpu()
    announce(f"fused CE T={T} h={h} V={V} final_norm={final_norm}")
    rng = np.random.default_rng(T + V)
    y = rng.standard_normal((T, h)).astype(np.float32)
    gf = (1 + 0.2 * rng.standard_normal(h)).astype(np.float32) if final_norm else None
    w = (rng.standard_normal((V, h)) * 0.02).astype(np.float32)
    tgt = rng.integers(0, V, T).astype(np.int32)
    Y, W, TG = dev(y), dev(w), dev(tgt)
    GF = dev(gf) if final_norm else None
    loss, am = empty(T), torch.empty(T, dtype=torch.int32, device="cuda")
    dy, dgf, dw = empty((T, h)), empty(h), empty((V, h))
    scratch = byte_buffer(qblk.cross_entropy_workspace_size(T, h, V))
    qblk.fused_cross_entropy(T, h, V, 1e-6, Y, GF, W, TG, 1.0 / T, loss, am, dy, dgf if final_norm else None,
                             dw, scratch)
    ref = oracle.lm_head_cross_entropy(y, gf, w, tgt, 1e-6)
    torch.cuda.synchronize()
    check("loss_partials", loss, ref["loss_partials"], FP32_TOL)
    assert abs(float(loss.double().sum()) / T - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    check("dy_last", dy, ref["dy_last"], FP32_TOL)
    check("dw_lm", dw, ref["dw_lm"], FP32_TOL)
    if final_norm:
        check("dg_final", dgf, ref["dg_final"], FP32_TOL)
    agree = float(np.mean(am.cpu().numpy() == ref["argmax"]))
    announce(f"  argmax agreement {agree:.4f}")
    assert agree >= 0.99


def test_clip_and_adamw_against_oracle():
    need_gpu()
    announce("clip + adamw multi-tensor")
    rng = np.random.default_rng(2)
    sizes = [(37,), (64, 33), (5000,), (4097,), (1, 3), (300, 300)] * 7   # 42 tensors: two chunks
    gs = [rng.standard_normal(s).astype(np.float32) for s in sizes]
    ws = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in sizes]
    ms = [(rng.standard_normal(s) * 1e-3).astype(np.float32) for s in sizes]
    vs = [np.abs(rng.standard_normal(s) * 1e-4).astype(np.float32) for s in sizes]
    G, W, M, Vv = ([dev(a) for a in arrs] for arrs in (gs, ws, ms, vs))
    norm, scale = empty(1), empty(1)
    scratch = byte_buffer(qblk.clip_workspace_size(G))
    qblk.clip_grad_norm(G, 1.0, 0, norm, scale, scratch)
    n_ref, s_ref, clipped = oracle.global_clip(gs, 1.0)
    torch.cuda.synchronize()
    assert abs(norm.item() - n_ref) <= 1e-6 * n_ref
    assert abs(scale.item() - s_ref) <= 1e-6 * s_ref
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    qblk.adamw_step(W, G, M, Vv, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], 3,
                    grad_scale_dev=scale)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        w2, m2, v2 = oracle.adamw_update(ws[i], clipped[i], ms[i], vs[i], step=3, **hp)
        check(f"w{i}", W[i], w2, FP32_TOL)
        check(f"m{i}", M[i], m2, FP32_TOL)
        check(f"v{i}", Vv[i], v2, FP32_TOL)
    # apply = 1 rescales in place; a second norm is then max_norm
    qblk.clip_grad_norm(G, 1.0, 1, norm, scale, scratch)
    qblk.clip_grad_norm(G, 1.0, 0, norm, scale, scratch)
    torch.cuda.synchronize()
    assert abs(norm.item() - 1.0) < 1e-5 and scale.item() == 1.0


def _adamw_weight_check(name, w_gpu, w_ref, g_ref, report):
    """Updated weights at step 1: elements whose reference gradient is within
    the gradient tolerance of zero may legitimately take the other sign of
    the ~lr-sized step; they are excluded and counted."""
    g = np.abs(np.asarray(g_ref, np.float64))
    keep = g > FP32_TOL * g.max()
    wg = w_gpu.detach().cpu().double().numpy()
    err = np.max(np.abs(wg - w_ref)[keep]) / np.max(np.abs(w_ref)) if keep.any() else 0.0
    report[name] = (err, int((~keep).sum()))
    assert err <= FP32_TOL, f"{name}: {err:.3e}"


def test_small_block_train_step():
    """Small block: fwd + bwd + global clip (1.0) + AdamW (step 1) on the 11
    block tensors, held in one flat buffer."""
    need_gpu()
    c = synth.SMALL_BLOCK
    announce("small block train step")
    inp = synth.block_inputs(c)
    shapes = block_shapes(c)
    Wf, Gf, Mf, Vf = FlatParams(shapes), FlatParams(shapes), FlatParams(shapes), FlatParams(shapes)
    Wf.load(inp["params"])
    X, DY = dev(inp["x"]), dev(inp["dy"])
    blk = Block(c)
    blk.forward(Wf.views, X)
    blk.backward(Wf.views, X, DY, Gf.views)
    norm, scale = empty(1), empty(1)
    scratch = byte_buffer(qblk.clip_workspace_size([Gf.buf]))
    qblk.clip_grad_norm([Gf.buf], synth.CLIP_MAX_NORM, 0, norm, scale, scratch)
    hp = synth.ADAMW
    qblk.adamw_step([Wf.buf], [Gf.buf], [Mf.buf], [Vf.buf], hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                    hp["weight_decay"], 1, grad_scale_dev=scale)
    torch.cuda.synchronize()
    _, cache = oracle.block_forward(c, inp["params"], inp["x"])
    _, g_ref = oracle.block_backward(c, inp["params"], cache, inp["dy"])
    names = list(qblk.PARAMS)
    n_ref, s_ref, clipped = oracle.global_clip([g_ref[n] for n in names], synth.CLIP_MAX_NORM)
    assert abs(norm.item() - n_ref) <= FP32_TOL * n_ref
    assert abs(scale.item() - s_ref) <= FP32_TOL * s_ref
    rep = {}
    for n, g in zip(names, clipped):
        z = np.zeros(g.shape)
        w2, m2, v2 = oracle.adamw_update(inp["params"][n], g, z, z, step=1, **hp)
        _adamw_weight_check(n, Wf[n], w2, g, rep)
        check("m_" + n, Mf[n], m2, FP32_TOL)
        check("v_" + n, Vf[n], v2, FP32_TOL)
    announce("  excluded near-zero-gradient elements: " + str({k: v[1] for k, v in rep.items()}))


@pytest.fixture(scope="module")
def stack_case():
    from bwd_rmsnorm_qkv_amd.stack import StackStep
    c = synth.STACK36_SMALL
    inp = synth.stack_inputs()
    st = StackStep(c, synth.STACK_LAYERS, synth.STACK_VOCAB)
    st.load(inp)
    return c, inp, st


def test_stack36_train_step(stack_case):
    need_gpu()
    c, inp, st = stack_case
    announce("36-layer stack train step (vocab 151936)")
    st.step()
    loss = st.loss()
    ref = oracle.stack_step(c, inp["layers"], inp["x"], inp["g_final"], inp["w_lm"], inp["targets"],
                            synth.CLIP_MAX_NORM, synth.ADAMW)
    announce(f"  loss gpu={loss:.6f} ref={ref['loss']:.6f} norm gpu={st.norm.item():.6f} ref={ref['norm']:.6f}")
    assert abs(loss - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    check("loss_partials", st.loss_host.numpy(), ref["loss_partials"], FP32_TOL)
    assert abs(st.norm.item() - ref["norm"]) <= FP32_TOL * ref["norm"]
    assert abs(st.scale.item() - ref["scale"]) <= FP32_TOL * ref["scale"]
    check("dx", st.dx, ref["dx"], FP32_TOL)
    names = [f"{l}.{n}" for l in range(synth.STACK_LAYERS) for n in qblk.PARAMS] + ["g_final", "w_lm"]
    rep, worst = {}, 0.0
    for i, n in enumerate(names):
        worst = max(worst, check("g_" + n, st.g[n], ref["grads"][i], FP32_TOL))
        _adamw_weight_check(n, st.w[n], ref["new_w"][i], ref["grads"][i] * ref["scale"], rep)
        check("m_" + n, st.m[n], ref["new_m"][i], FP32_TOL)
        check("v_" + n, st.v[n], ref["new_v"][i], FP32_TOL)
    agree = float(np.mean(st.argmax.cpu().numpy() == ref["argmax"]))
    announce(f"  worst grad err {worst:.2e}; argmax agreement {agree:.4f}; "
             f"excluded {sum(v[1] for v in rep.values())} near-zero-gradient weights")


def test_stack_micro_batches():
    """A batch of 4 sequences as 1, 2 and 4 micro-batches (accumulating
    backward and cross-entropy, one clip and AdamW) against oracle.stack_step
    on the whole 4-sequence batch: loss, gradient norm, clip scale, every
    gradient, the updated weights (first-step sign rule) and moments; the
    three runs also agree with each other."""
    need_gpu()
    from bwd_rmsnorm_qkv_amd.stack import StackStep
    c = synth.STACK36_SMALL.with_tokens(seq=128, batch=4)
    layers, vocab = 2, 2048
    inp = synth.stack_inputs(c, layers=layers, vocab=vocab, seed=3)
    ref = oracle.stack_step(c, inp["layers"], inp["x"], inp["g_final"], inp["w_lm"], inp["targets"],
                            synth.CLIP_MAX_NORM, synth.ADAMW)
    names = [f"{l}.{n}" for l in range(layers) for n in qblk.PARAMS] + ["g_final", "w_lm"]
    out = []
    for k in (1, 2, 4):
        announce(f"stack micro-batches k={k}")
        st = StackStep(c, layers, vocab, micro_batches=k)
        st.load(inp)
        st.step()
        loss = st.loss()
        assert abs(loss - ref["loss"]) <= 1e-5 * abs(ref["loss"]), (k, loss, ref["loss"])
        assert abs(st.norm.item() - ref["norm"]) <= FP32_TOL * ref["norm"], (k, st.norm.item(), ref["norm"])
        assert abs(st.scale.item() - ref["scale"]) <= FP32_TOL * ref["scale"]
        rep, worst = {}, 0.0
        for i, n in enumerate(names):
            worst = max(worst, check(f"k={k} g_{n}", st.g[n], ref["grads"][i], FP32_TOL))
            _adamw_weight_check(f"k={k} w_{n}", st.w[n], ref["new_w"][i], ref["grads"][i] * ref["scale"], rep)
            check(f"k={k} m_{n}", st.m[n], ref["new_m"][i], FP32_TOL)
            check(f"k={k} v_{n}", st.v[n], ref["new_v"][i], FP32_TOL)
        announce(f"  k={k}: loss {loss:.6f} (ref {ref['loss']:.6f}), worst grad err {worst:.2e}, "
                 f"excluded {sum(v[1] for v in rep.values())} near-zero-gradient weights")
        out.append((loss, st.norm.item(), st.g.buf.clone()))
    loss0, norm0, g0 = out[0]
    for k, (loss, norm, g) in zip((2, 4), out[1:]):
        assert abs(loss - loss0) <= 1e-5 * abs(loss0), (k, loss, loss0)
        assert abs(norm - norm0) <= FP32_TOL * norm0, (k, norm, norm0)
        check(f"grads k={k} vs k=1", g, g0.cpu().numpy().astype(np.float64), FP32_TOL)


@pytest.mark.parametrize("segments", [1, 2, 4])
def test_stack_checkpoint_segments(segments):
    """Activation checkpointing: a 4-layer stack with its layers in 1, 2 or
    4 segments, recomputed from their checkpoints in the backward (all but
    the last segment). Loss, norm, every gradient and
    the updated weights equal those of the step that keeps every layer's
    activations bit for bit, and match oracle.stack_step; the kept
    activations shrink with the segment length."""
    need_gpu()
    from bwd_rmsnorm_qkv_amd.stack import StackStep
    c = synth.STACK36_SMALL.with_tokens(seq=128, batch=2)
    layers, vocab = 4, 2048
    inp = synth.stack_inputs(c, layers=layers, vocab=vocab, seed=5)
    announce(f"stack checkpoint segments={segments}")
    runs = []
    for seg in (None, segments):
        st = StackStep(c, layers, vocab, checkpoint_segments=seg)
        st.load(inp)
        st.step()
        torch.cuda.synchronize()
        runs.append((st, st.loss(), st.norm.clone(), st.g.buf.clone(), st.w.buf.clone(), st.dx.clone()))
    (s0, l0, n0, g0, w0, dx0), (s1, l1, n1, g1, w1, dx1) = runs
    assert l0 == l1 and torch.equal(n0, n1)
    assert torch.equal(g0, g1) and torch.equal(w0, w1) and torch.equal(dx0, dx1)
    announce(f"  kept activations: {s0.workspace_bytes() / 2**20:.1f} MiB without, "
             f"{s1.workspace_bytes() / 2**20:.1f} MiB with {segments} segment(s)")
    if segments > 1:
        assert s1.workspace_bytes() < s0.workspace_bytes()
    ref = oracle.stack_step(c, inp["layers"], inp["x"], inp["g_final"], inp["w_lm"], inp["targets"],
                            synth.CLIP_MAX_NORM, synth.ADAMW)
    assert abs(l1 - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    names = [f"{l}.{n}" for l in range(layers) for n in qblk.PARAMS] + ["g_final", "w_lm"]
    for i, n in enumerate(names):
        check("g_" + n, s1.g[n], ref["grads"][i], FP32_TOL)
    check("dx", dx1, ref["dx"], FP32_TOL)


@pytest.mark.parametrize("shape", ["small_fp16", "qwen3_4b", "small_bf16"])
def test_block_train_step_fp16_pack_in_adamw(shape):
    """Two training steps of one fp16-operand block in which AdamW writes the
    packed fp16 weight set (qblk_adamw_step_pack16): after each step the
    packed set equals, bit for bit, qblk_block_pack_f16 of the updated fp32
    masters, and the masters and moments equal those of qblk_adamw_step on
    the same gradients; step 1's loss-free quantities (gradient norm, clip
    scale) match the oracle."""
    need_gpu()
    from bwd_rmsnorm_qkv_amd.runtime import BlockTrainStep
    c = (synth.QWEN3_4B_BLOCK if shape == "qwen3_4b" else
         synth.BlockShape(hidden=512, heads=8, kv_heads=2, head_dim=64, intermediate=1408, seq=96, batch=2,
                          rope_theta=1e4, gemm_precision=2 if shape == "small_bf16" else 1))
    announce(f"block train step with fp16 pack in AdamW ({shape}, T={c.tokens})")
    inp = synth.block_inputs(c)
    st = BlockTrainStep(c)
    st.load(inp["params"])
    X, DY = dev(inp["x"]), dev(inp["dy"])
    ref_pack = byte_buffer(st.packed.numel())
    for step in (1, 2):
        w0, m0, v0 = st.w.buf.clone(), st.m.buf.clone(), st.v.buf.clone()
        st.step(X, DY)
        torch.cuda.synchronize()
        # the same update by the plain AdamW from the same state and gradients
        w1, m1, v1 = w0.clone(), m0.clone(), v0.clone()
        hp = synth.ADAMW
        qblk.adamw_step([w1], [st.g.buf], [m1], [v1], hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                        hp["weight_decay"], step, grad_scale_dev=st.scale)
        qblk.block_pack_f16(st.blk.c, st.w.views, ref_pack)
        torch.cuda.synchronize()
        assert torch.equal(w1, st.w.buf) and torch.equal(m1, st.m.buf) and torch.equal(v1, st.v.buf)
        assert torch.equal(ref_pack, st.packed), f"packed fp16 set differs after step {step}"
        if step == 1:
            _, cache = oracle.block_forward(c, inp["params"], inp["x"])
            _, g_ref = oracle.block_backward(c, inp["params"], cache, inp["dy"])
            n_ref, s_ref, _ = oracle.global_clip([g_ref[n] for n in qblk.PARAMS], synth.CLIP_MAX_NORM)
            tol = BF16_TOL if c.gemm_precision == 2 else FP16_TOL
            assert abs(st.norm.item() - n_ref) <= tol * n_ref
            assert abs(st.scale.item() - s_ref) <= tol * s_ref
