"""Seeded synthetic workloads for the decoder-block training step.

This module only draws random numbers in a fixed order and names the five
workload shapes. It holds none of the method's arithmetic, so both the CPU
oracle (through the tests) and the HIP path (through the binding, the tests
and the bench) can take their inputs from it.

Every tensor is drawn with ``numpy.random.Generator(PCG64(seed))`` as float64
``standard_normal`` scaled by its standard deviation, then cast once to
float32. Weights are ``[out, in]`` row-major; activations are ``[T, C]`` with
token ``t = b * seq + s``.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict, replace

import numpy as np


@dataclass(frozen=True)
class BlockShape:
    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    intermediate: int
    seq: int
    batch: int
    eps: float = 1e-6
    rope_theta: float = 1e4
    qk_norm: int = 1
    gemm_precision: int = 0  # 0: fp32 contractions, 1: fp16 operands with fp32 accumulate

    @property
    def tokens(self) -> int:
        return self.seq * self.batch

    @property
    def q_dim(self) -> int:
        return self.heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.kv_heads * self.head_dim

    def as_dict(self) -> dict:
        return asdict(self)

    def with_tokens(self, seq: int, batch: int = 1) -> "BlockShape":
        return replace(self, seq=seq, batch=batch)


# The five workloads, named by what they are.
TINY_BLOCK = BlockShape(hidden=64, heads=4, kv_heads=2, head_dim=16, intermediate=176,
                        seq=32, batch=1, rope_theta=1e4)
SMALL_BLOCK = BlockShape(hidden=512, heads=8, kv_heads=2, head_dim=64, intermediate=1408,
                         seq=256, batch=4, rope_theta=1e4)
QWEN3_4B_BLOCK = BlockShape(hidden=2560, heads=32, kv_heads=8, head_dim=128, intermediate=9728,
                            seq=512, batch=1, rope_theta=1e6, gemm_precision=1)
STACK36_SMALL = BlockShape(hidden=512, heads=8, kv_heads=2, head_dim=64, intermediate=1408,
                           seq=1024, batch=1, rope_theta=1e4)
NF4_LORA_QWEN3_4B = BlockShape(hidden=2560, heads=32, kv_heads=8, head_dim=128, intermediate=9728,
                               seq=2048, batch=1, rope_theta=1e6, gemm_precision=1)

STACK_LAYERS = 36
STACK_VOCAB = 151936
LORA_RANK = 16
LORA_ALPHA = 32.0
ADAMW = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
CLIP_MAX_NORM = 1.0

# Projection names in draw order, with (out, in) as a function of the shape.
PROJ_NAMES = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")


def proj_shapes(c: BlockShape) -> dict:
    h, q, kv, i = c.hidden, c.q_dim, c.kv_dim, c.intermediate
    return {"w_q": (q, h), "w_k": (kv, h), "w_v": (kv, h), "w_o": (h, q),
            "w_gate": (i, h), "w_up": (i, h), "w_down": (h, i)}


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(shape) * std).astype(np.float32)


def _gammas(c: BlockShape) -> dict:
    return {"g_in": np.ones(c.hidden, np.float32), "g_post": np.ones(c.hidden, np.float32),
            "g_q": np.ones(c.head_dim, np.float32), "g_k": np.ones(c.head_dim, np.float32)}


def draw_weights(rng: np.random.Generator, c: BlockShape, std: float = 0.02) -> dict:
    ps = proj_shapes(c)
    w = {n: _normal(rng, ps[n], std) for n in PROJ_NAMES}
    w.update(_gammas(c))
    return w


def block_inputs(c: BlockShape, seed: int = 0) -> dict:
    """x, dy, then the seven projections (N(0, 0.02)); every gamma is 1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (c.tokens, c.hidden), 1.0)
    dy = _normal(rng, (c.tokens, c.hidden), 1.0)
    params = draw_weights(rng, c)
    return {"x": x, "dy": dy, "params": params}


def stack_inputs(c: BlockShape = STACK36_SMALL, layers: int = STACK_LAYERS,
                 vocab: int = STACK_VOCAB, seed: int = 0) -> dict:
    """Embedding output x, then per layer the seven projections, then the
    LM head [V, h], then the integer targets in [0, V)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (c.tokens, c.hidden), 1.0)
    layer_params = [draw_weights(rng, c) for _ in range(layers)]
    w_lm = _normal(rng, (vocab, c.hidden), 0.02)
    targets = rng.integers(0, vocab, c.tokens).astype(np.int32)
    return {"x": x, "layers": layer_params, "w_lm": w_lm,
            "g_final": np.ones(c.hidden, np.float32), "targets": targets}


def nf4_lora_inputs(c: BlockShape = NF4_LORA_QWEN3_4B, rank: int = LORA_RANK,
                    b_std: float = 0.0, seed: int = 0) -> dict:
    """x, dy, the seven fp32 base weights (to be quantized by each side),
    LoRA A_p [r, in] N(0, 0.02) for every projection, then B_p [out, r]:
    zeros when ``b_std == 0`` (the initial state), else N(0, b_std)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (c.tokens, c.hidden), 1.0)
    dy = _normal(rng, (c.tokens, c.hidden), 1.0)
    base = draw_weights(rng, c)
    ps = proj_shapes(c)
    lora_a = {n: _normal(rng, (rank, ps[n][1]), 0.02) for n in PROJ_NAMES}
    if b_std == 0.0:
        lora_b = {n: np.zeros((ps[n][0], rank), np.float32) for n in PROJ_NAMES}
    else:
        lora_b = {n: _normal(rng, (ps[n][0], rank), b_std) for n in PROJ_NAMES}
    return {"x": x, "dy": dy, "params": base, "lora_a": lora_a, "lora_b": lora_b}


def uniform_targets(rng: np.random.Generator, tokens: int, vocab: int) -> np.ndarray:
    return rng.integers(0, vocab, tokens).astype(np.int32)
