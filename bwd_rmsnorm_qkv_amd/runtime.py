"""Device-side bookkeeping for the block step: workspaces, flat parameter
buffers, and call sequences over the C ABI (no arithmetic here; every step
runs in libqblk's kernels through ``qblk``)."""
from __future__ import annotations

import numpy as np
import torch

from . import qblk
from .qblk import PARAMS, PROJ


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def empty(n_or_shape, dtype=torch.float32):
    shape = (n_or_shape,) if isinstance(n_or_shape, int) else tuple(n_or_shape)
    return torch.empty(shape, dtype=dtype, device="cuda")


def byte_buffer(nbytes: int):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device="cuda")


class FlatParams:
    """One contiguous fp32 buffer carved into named tensors (16-byte aligned
    views), so a whole model's parameters, gradients or moments can be
    handed to the multi-tensor clip and AdamW as a few large tensors."""

    def __init__(self, shapes: list, zero=True):
        self.shapes = shapes  # list of (name, shape)
        offs, off = [], 0
        for _, shp in shapes:
            n = int(np.prod(shp))
            offs.append((off, n))
            off += (n + 63) // 64 * 64
        self.total = off
        self.buf = (torch.zeros if zero else torch.empty)(off, dtype=torch.float32, device="cuda")
        self.views = {}
        self.order = []
        for (name, shp), (o, n) in zip(shapes, offs):
            self.views[name] = self.buf[o:o + n].view(*shp)
            self.order.append(name)

    def __getitem__(self, k):
        return self.views[k]

    def tensors(self):
        return [self.views[k] for k in self.order]

    def load(self, arrays: dict):
        for k, a in arrays.items():
            self.views[k].copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)))


def block_shapes(c, prefix=""):
    h, q, kv, i, d = c.hidden, c.q_dim, c.kv_dim, c.intermediate, c.head_dim
    s = {"w_q": (q, h), "w_k": (kv, h), "w_v": (kv, h), "w_o": (h, q), "w_gate": (i, h), "w_up": (i, h),
         "w_down": (h, i), "g_in": (h,), "g_post": (h,), "g_q": (d,), "g_k": (d,)}
    return [(prefix + n, s[n]) for n in PARAMS]


class Block:
    """Workspaces for one block configuration."""

    def __init__(self, cfg):
        self.cfg = cfg
        self.c = qblk.make_config(cfg)
        self.saved_bytes, self.scratch_bytes = qblk.block_workspace_size(self.c)
        T, h = cfg.tokens, cfg.hidden
        self.saved = byte_buffer(self.saved_bytes)
        self.scratch = byte_buffer(self.scratch_bytes)
        self.y = empty((T, h))
        self.dx = empty((T, h))

    def pack_f16(self, params, stream=None):
        """params plus "w16": the packed fp16 weight copies (fp16-operand
        configurations), refreshed from params' fp32 weights now."""
        if not hasattr(self, "packed"):
            self.packed = byte_buffer(qblk.block_pack_f16_size(self.c))
        qblk.block_pack_f16(self.c, params, self.packed, stream)
        return {**params, "w16": self.packed}

    def forward(self, params, x, saved=None, y=None, stream=None):
        qblk.block_forward(self.c, params, x, self.y if y is None else y,
                           self.saved if saved is None else saved, self.scratch, stream)
        return self.y if y is None else y

    def backward(self, params, x, dy, grads, saved=None, dx=None, stream=None, accumulate=False):
        qblk.block_backward(self.c, params, x, dy, self.saved if saved is None else saved,
                            self.dx if dx is None else dx, grads, self.scratch, stream, accumulate)
        return self.dx if dx is None else dx


class BlockTrainStep:
    """One training step of a single block: forward, backward, the global
    clip and AdamW over its 11 tensors (flat fp32 buffers). With fp16
    operands (gemm_precision 1) the packed fp16 weight set the GEMMs read is
    written by AdamW itself (qblk_adamw_step_pack16) as it updates the
    fp32 masters, so no separate cast runs between steps; it is packed once
    at load."""

    def __init__(self, cfg, adamw=None, max_norm=1.0):
        from .synth import ADAMW
        self.cfg, self.blk = cfg, Block(cfg)
        self.hp = dict(ADAMW if adamw is None else adamw)
        self.max_norm = max_norm
        shapes = block_shapes(cfg)
        self.w, self.g, self.m, self.v = (FlatParams(shapes) for _ in range(4))
        self.fp16 = cfg.gemm_precision in (1, 2)  # 16-bit operands: fp16 (1) or bfloat16 (2)
        self.params = self.w.views
        if self.fp16:
            self.packed = byte_buffer(qblk.block_pack_f16_size(self.blk.c))
            off = qblk.block_pack_f16_offsets(self.blk.c)
            base = self.packed.data_ptr()
            self.w16 = [base + 2 * off[n] if n in off else None for n in PARAMS]
            self.params = {**self.w.views, "w16": self.packed}
        self.norm, self.scale = empty(1), empty(1)
        self.clip_scratch = byte_buffer(qblk.clip_workspace_size([self.g.buf]))
        self.t = 0

    def load(self, params: dict):
        self.w.load(params)
        self.m.buf.zero_()
        self.v.buf.zero_()
        if self.fp16:
            qblk.block_pack_f16(self.blk.c, self.w.views, self.packed)
        self.t = 0

    def step(self, x, dy):
        self.blk.forward(self.params, x)
        self.blk.backward(self.params, x, dy, self.g.views)
        qblk.clip_grad_norm([self.g.buf], self.max_norm, 0, self.norm, self.scale, self.clip_scratch)
        self.t += 1
        hp = self.hp
        if self.fp16:
            qblk.adamw_step_pack16(self.w.tensors(), self.g.tensors(), self.m.tensors(), self.v.tensors(), self.w16,
                                   hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], self.t,
                                   grad_scale_dev=self.scale, bf16=self.cfg.gemm_precision == 2)
        else:
            qblk.adamw_step([self.w.buf], [self.g.buf], [self.m.buf], [self.v.buf], hp["lr"], hp["beta1"],
                            hp["beta2"], hp["eps"], hp["weight_decay"], self.t, grad_scale_dev=self.scale)


class Nf4Block:
    """A frozen-NF4 + LoRA block: base weights encoded on the device by
    qblk_nf4_quantize, LoRA A/B and their gradients, and workspaces."""

    def __init__(self, cfg, rank, alpha):
        from .synth import proj_shapes
        self.cfg, self.rank, self.alpha = cfg, rank, float(alpha)
        self.c = qblk.make_config(cfg)
        self.saved_bytes, self.scratch_bytes = qblk.nf4_block_workspace_size(self.c, rank)
        self.saved = byte_buffer(self.saved_bytes)
        self.scratch = byte_buffer(self.scratch_bytes)
        ps = proj_shapes(cfg)
        self.shapes = ps
        self.codes = {n: torch.empty(ps[n][0] * ps[n][1] // 2, dtype=torch.uint8, device="cuda") for n in PROJ}
        self.absmax = {n: empty(ps[n][0] * ps[n][1] // 64) for n in PROJ}
        self.lora_a = {n: empty((rank, ps[n][1])) for n in PROJ}
        self.lora_b = {n: empty((ps[n][0], rank)) for n in PROJ}
        self.grad_a = {n: empty((rank, ps[n][1])) for n in PROJ}
        self.grad_b = {n: empty((ps[n][0], rank)) for n in PROJ}
        T, h = cfg.tokens, cfg.hidden
        self.x, self.dy = empty((T, h)), empty((T, h))
        self.y, self.dx = empty((T, h)), empty((T, h))
        self.gammas = {}

    def load(self, inp: dict):
        for n in PROJ:
            w = dev(inp["params"][n])
            qblk.nf4_quantize(w, self.codes[n], self.absmax[n])
            self.lora_a[n].copy_(torch.from_numpy(inp["lora_a"][n]))
            self.lora_b[n].copy_(torch.from_numpy(inp["lora_b"][n]))
        self.gammas = {n: dev(inp["params"][n]) for n in ("g_in", "g_post", "g_q", "g_k")}
        self.x.copy_(torch.from_numpy(inp["x"]))
        self.dy.copy_(torch.from_numpy(inp["dy"]))
        torch.cuda.synchronize()

    def forward(self):
        qblk.block_forward_nf4_lora(self.c, self.codes, self.absmax, self.lora_a, self.lora_b, self.gammas,
                                    self.rank, self.alpha, self.x, self.y, self.saved, self.scratch)
        return self.y

    def backward(self, recompute=False):
        """recompute=True: the forward's activations are not taken from an
        earlier forward call; the forward is re-run first (into the same
        `saved` workspace), as [block] CudaNf4TransformerBlock::backward
        re-runs the forward before its backward, so one workspace can serve
        many blocks. The results are the same bit for bit."""
        if recompute:
            self.forward()
        qblk.block_backward_nf4_lora(self.c, self.codes, self.absmax, self.lora_a, self.lora_b, self.gammas,
                                     self.rank, self.alpha, self.x, self.dy, self.saved, self.dx, self.grad_a,
                                     self.grad_b, self.scratch)
        return self.dx

    def fwd_bwd(self):
        self.forward()
        self.backward()
