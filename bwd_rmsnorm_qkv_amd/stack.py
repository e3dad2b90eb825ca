"""One training step of a stack of decoder blocks with the LM head, on one
GPU, as a sequence of libqblk calls (no arithmetic here).

cuda_trainer.rs page, train_step_inner: gpu_forward over the blocks (each
block's input kept for its backward), fused cross-entropy with loss scale
1/T, gpu_backward in reverse block order. Different from the page: every
gradient of the step is kept (one flat fp32 buffer) so that ONE global L2
clip over all of them precedes any AdamW, and the clip scale is folded into
the AdamW read instead of rewriting the gradients. The only device-to-host
transfer of a step is the T loss partials.
"""
from __future__ import annotations

import numpy as np
import torch

from . import qblk
from .qblk import PARAMS
from .runtime import FlatParams, block_shapes, byte_buffer, empty


class StackStep:
    """micro_batches = k > 1: the batch is taken as k micro-batches of
    cfg.batch / k sequences, each run forward and backward with the
    accumulating backward and cross-entropy (loss scale 1/T of the whole
    batch), then one clip and one AdamW step ([trainer] GPU-resident
    gradient accumulation).

    checkpoint_segments = S >= 1: activation checkpointing ([trainer]
    checkpoint segments and recompute_segment in gpu_backward). The layers
    are cut into S consecutive segments of ceil(L / S) layers; the forward
    keeps only each segment's input (its checkpoint) and runs every layer of
    a segment through one shared set of ceil(L / S) `saved` workspaces; the
    backward, segment by segment from the last, first re-runs the segment's
    forward from its checkpoint with the same kernels (all but the last
    segment, whose activations are still in place), then its backward. The
    forward is deterministic, so the gradients equal those of the step
    without checkpointing bit for bit. None: every layer's activations are
    kept (no recompute)."""

    def __init__(self, cfg, layers, vocab, adamw=None, max_norm=1.0, micro_batches=1,
                 checkpoint_segments=None):
        from .synth import ADAMW
        if micro_batches < 1 or cfg.batch % micro_batches:
            raise ValueError(f"micro_batches={micro_batches} must divide batch={cfg.batch}")
        self.full = cfg
        self.k = micro_batches
        cfg = cfg.with_tokens(seq=cfg.seq, batch=cfg.batch // micro_batches)
        self.cfg, self.L, self.V = cfg, layers, vocab
        self.hp = dict(ADAMW if adamw is None else adamw)
        self.max_norm = max_norm
        self.c = qblk.make_config(cfg)
        T, h = cfg.tokens, cfg.hidden
        self.x_all = empty((micro_batches, T, h))
        self.targets_all = torch.zeros((micro_batches, T), dtype=torch.int32, device="cuda")
        shapes = []
        for l in range(layers):
            shapes += block_shapes(cfg, prefix=f"{l}.")
        shapes += [("g_final", (h,)), ("w_lm", (vocab, h))]
        self.w = FlatParams(shapes)
        self.g = FlatParams(shapes)  # zeroed: the padding between tensors stays 0 for the norm
        self.m = FlatParams(shapes)
        self.v = FlatParams(shapes)
        self.saved_bytes, self.scratch_bytes = qblk.block_workspace_size(self.c)
        if checkpoint_segments is None:
            self.segs = [(0, layers)]
            n_saved, n_acts = layers, layers + 1
        else:
            if not 1 <= checkpoint_segments <= layers:
                raise ValueError(f"checkpoint_segments={checkpoint_segments} must be in 1..{layers}")
            per = -(-layers // checkpoint_segments)
            self.segs = [(a, min(layers, a + per)) for a in range(0, layers, per)]
            n_saved, n_acts = per, per
        self.checkpointed = checkpoint_segments is not None
        self.saved = [byte_buffer(self.saved_bytes) for _ in range(n_saved)]
        self.scratch = byte_buffer(self.scratch_bytes)
        # block inputs of the segment in flight (all layers without
        # checkpointing); the checkpoints: each segment's input and the
        # last block's output
        self.acts = empty((n_acts, T, h))
        self.ckpt = empty((len(self.segs) + 1, T, h)) if self.checkpointed else None
        self.dh = [empty((T, h)), empty((T, h))]
        self.ce_scratch = byte_buffer(qblk.cross_entropy_workspace_size(T, h, vocab))
        self.targets = torch.zeros(T, dtype=torch.int32, device="cuda")
        self.loss_partials = empty(T)
        self.argmax = torch.empty(T, dtype=torch.int32, device="cuda")
        self.loss_host = torch.empty(micro_batches * T, dtype=torch.float32, pin_memory=True)
        self.norm = empty(1)
        self.scale = empty(1)
        self.clip_scratch = byte_buffer(qblk.clip_workspace_size([self.g.buf]))
        self.t = 0

    def load(self, inp: dict, x=None):
        for l, p in enumerate(inp["layers"]):
            self.w.load({f"{l}.{n}": p[n] for n in PARAMS})
        self.w.load({"g_final": inp["g_final"], "w_lm": inp["w_lm"]})
        T = self.cfg.tokens
        self.x_all.copy_(torch.from_numpy(inp["x"] if x is None else x).reshape(self.k, T, -1))
        self.targets_all.copy_(torch.from_numpy(inp["targets"]).reshape(self.k, T))
        self.x_in().copy_(self.x_all[0])
        self.targets.copy_(self.targets_all[0])
        self.m.buf.zero_()
        self.v.buf.zero_()
        self.t = 0

    def _layer(self, fp: FlatParams, l):
        return {n: fp[f"{l}.{n}"] for n in PARAMS}

    def x_in(self):
        """The stack's input buffer (the first block's input)."""
        return self.ckpt[0] if self.checkpointed else self.acts[0]

    def workspace_bytes(self):
        """Device bytes of the activations kept between forward and backward
        (the per-layer `saved` workspaces and the block inputs/checkpoints)."""
        n = len(self.saved) * self.saved_bytes + self.acts.numel() * 4
        return n + (self.ckpt.numel() * 4 if self.checkpointed else 0)

    def _io(self, si, l):
        """Input and output buffers of block l of segment si: without
        checkpointing acts[l] and acts[l + 1]; with it, the segment's
        checkpoint feeds its first block, its last block writes the next
        checkpoint, and the blocks in between use acts[l - a]."""
        a, b = self.segs[si]
        if not self.checkpointed:
            return self.acts[l], self.acts[l + 1]
        x = self.ckpt[si] if l == a else self.acts[l - a]
        y = self.ckpt[si + 1] if l == b - 1 else self.acts[l - a + 1]
        return x, y

    def _forward_segment(self, si):
        a, b = self.segs[si]
        for l in range(a, b):
            x, y = self._io(si, l)
            qblk.block_forward(self.c, self._layer(self.w, l), x, y, self.saved[l - a], self.scratch)

    def step(self):
        """Forward, loss, backward, global clip and AdamW; returns the loss
        (the host sum of the partials) lazily as a callable."""
        cfg, T, h, V = self.cfg, self.cfg.tokens, self.cfg.hidden, self.V
        last = len(self.segs) - 1
        for mb in range(self.k):
            acc = mb > 0
            if self.k > 1:
                self.x_in().copy_(self.x_all[mb])
                self.targets.copy_(self.targets_all[mb])
            for si in range(len(self.segs)):
                self._forward_segment(si)
            y_last = self._io(last, self.L - 1)[1]
            qblk.fused_cross_entropy(T, h, V, cfg.eps, y_last, self.w["g_final"], self.w["w_lm"],
                                     self.targets, 1.0 / (T * self.k), self.loss_partials, self.argmax,
                                     self.dh[0], self.g["g_final"], self.g["w_lm"], self.ce_scratch,
                                     accumulate=acc)
            self.loss_host[mb * T:(mb + 1) * T].copy_(self.loss_partials, non_blocking=True)
            cur = 0
            for si in range(last, -1, -1):
                a, b = self.segs[si]
                if si != last:  # recompute: the segment's activations were overwritten
                    self._forward_segment(si)
                for l in range(b - 1, a - 1, -1):
                    qblk.block_backward(self.c, self._layer(self.w, l), self._io(si, l)[0], self.dh[cur],
                                        self.saved[l - a], self.dh[cur ^ 1], self._layer(self.g, l), self.scratch,
                                        accumulate=acc)
                    cur ^= 1
            self.dx = self.dh[cur]
        qblk.clip_grad_norm([self.g.buf], self.max_norm, 0, self.norm, self.scale, self.clip_scratch)
        self.t += 1
        hp = self.hp
        qblk.adamw_step([self.w.buf], [self.g.buf], [self.m.buf], [self.v.buf], hp["lr"], hp["beta1"],
                        hp["beta2"], hp["eps"], hp["weight_decay"], self.t, grad_scale_dev=self.scale)

    def loss(self):
        torch.cuda.current_stream().synchronize()
        return float(np.sum(self.loss_host.numpy().astype(np.float64))) / self.full.tokens
