"""NF4 encoding of frozen weights and the NF4 + LoRA block (test infrastructure).

cuda_block.rs page: ``CudaNf4TransformerBlock`` (``quantize_nf4`` over blocks
of ``NF4_BLOCK_SIZE`` elements of each flattened [out, in] projection, with a
per-block scale), its forward and its LoRA-only backward. wgpu_trainer.rs
page: ``lora_forward`` / ``lora_backward`` (LoRA on a dequantized base weight,
A [r, in], B [out, r], scale alpha/r).

Neither page prints the codebook, the quantizer or the nibble order. The
readings taken: the 16-level NormalFloat4 codebook of the QLoRA paper
(Dettmers et al., 2023) built from normal quantiles in float64 and rounded
once to float32; blocks of 64 with an fp32 absmax scale; the nearest level
chosen in float32 (the kernel's precision) with ties to the lower code; a zero
block gets scale 0 and the zero level; element 2i in the low nibble of byte i.
"""
from __future__ import annotations

import numpy as np
from scipy.special import ndtri

from . import ops
from .block import block_forward, block_backward

NF4_BLOCK = 64


def nf4_codebook():
    """The 16 NormalFloat4 levels, ascending, as float32.

    QLoRA's construction: take the standard-normal quantiles at 8 evenly
    spaced probabilities from delta to 1/2 (the 1/2 end excluded) for the
    positive side and at 7 such probabilities for the negative side, where
    delta is the mean of 1 - 1/(2*15) and 1 - 1/(2*16); add an exact zero;
    divide by the largest value so the range is [-1, 1].
    """
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    pos = ndtri(np.linspace(delta, 0.5, 9)[:-1])
    neg = -ndtri(np.linspace(delta, 0.5, 8)[:-1])
    levels = np.sort(np.concatenate([neg, [0.0], pos]))
    levels = levels / levels.max()
    return levels.astype(np.float32)


def nf4_quantize(w):
    """Encode a float32 tensor (numel divisible by 64) into packed NF4 codes.

    Per block of 64 consecutive elements of the flattened tensor:
    a = max |w| (float32); if a == 0 every code is the zero level; otherwise,
    in float32, x = w / a and code = the number of level midpoints
    (L[c] + L[c+1]) / 2 lying strictly below x (the nearest level, ties to
    the lower code). Returns (packed uint8 [numel/2], scales float32
    [numel/64], codes uint8 [numel]).
    """
    w = np.asarray(w, np.float32).reshape(-1)
    if w.size % NF4_BLOCK:
        raise ValueError("numel must be a multiple of 64")
    blocks = w.reshape(-1, NF4_BLOCK)
    absmax = np.max(np.abs(blocks), axis=1).astype(np.float32)
    levels = nf4_codebook()
    mids = ((levels[:-1] + levels[1:]) * np.float32(0.5)).astype(np.float32)
    zero_code = int(np.flatnonzero(levels == 0.0)[0])
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)
    codes = np.searchsorted(mids, x, side="left").astype(np.uint8)
    codes[absmax == 0] = zero_code
    codes = codes.reshape(-1)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return packed, absmax, codes


def nf4_unpack(packed):
    packed = np.asarray(packed, np.uint8)
    codes = np.empty(packed.size * 2, np.uint8)
    codes[0::2] = packed & 0x0F
    codes[1::2] = packed >> 4
    return codes


def nf4_dequantize(packed, absmax, shape):
    """w~ = L[code] * a_block, in float64 (exact product of two float32)."""
    codes = nf4_unpack(packed)
    levels = nf4_codebook().astype(np.float64)
    vals = levels[codes].reshape(-1, NF4_BLOCK) * np.asarray(absmax, np.float64)[:, None]
    return vals.reshape(shape)


def lora_linear_fwd(x, w_base, a, b, scale):
    """y = x W~^T + scale * (x A^T) B^T (wgpu_trainer.rs page, ``lora_forward``)."""
    x = np.asarray(x, np.float64)
    h = x @ np.asarray(a, np.float64).T
    return ops.linear_fwd(x, w_base) + scale * (h @ np.asarray(b, np.float64).T)


def lora_linear_bwd(x, w_base, a, b, dy, scale):
    """Gradients of ``lora_linear_fwd`` for x, A and B; the base is frozen.

    wgpu_trainer.rs page, ``lora_backward``: h = x A^T; dh = scale * dy B;
    dB = scale * dy^T h; dA = dh^T x; dx = dy W~ + dh A.
    Returns (dx, dA, dB).
    """
    x, dy = np.asarray(x, np.float64), np.asarray(dy, np.float64)
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    h = x @ a.T
    dh = scale * (dy @ b)
    db = scale * (dy.T @ h)
    da = dh.T @ x
    dx = dy @ np.asarray(w_base, np.float64) + dh @ a
    return dx, da, db


def nf4_block_forward(c, gammas, w_deq, lora_a, lora_b, x, scale):
    """The block of ``oracle.block`` with every projection replaced by the
    frozen dequantized base plus its LoRA branch (all seven projections)."""
    lin = lambda name, a: lora_linear_fwd(a, w_deq[name], lora_a[name], lora_b[name], scale)
    return block_forward(c, gammas, x, linear=lin)


def nf4_block_backward(c, gammas, w_deq, lora_a, lora_b, cache, dy, scale):
    """dx and the 14 LoRA gradients (dA, dB per projection) of the NF4 block;
    the base weights and the norm gammas are frozen. Returns (dx, dA, dB)."""
    da, db = {}, {}

    def lb(name, a, g):
        dx_, da[name], db[name] = lora_linear_bwd(a, w_deq[name], lora_a[name],
                                                  lora_b[name], g, scale)
        return dx_, None

    dx, _ = block_backward(c, gammas, cache, dy, linear_bwd=lb)
    return dx, da, db
