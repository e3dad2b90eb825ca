"""CPU oracle for the decoder-block training step — TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 restatement of what the pages compute, written from
their definitions and sharing no code with the HIP path. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does.

Pages cited (docs.rs source pages of the Rust crate aprender-train, module
``entrenar``):

* "cuda_block.rs page" — ``entrenar/transformer/cuda_block.rs`` (0.32.0): the
  GPU decoder block, its forward, backward, AdamW call sequence and NF4 block.
* "cuda_trainer.rs page" — ``entrenar/train/transformer_trainer/cuda_trainer.rs``
  (0.34.0): the training step, LM head, fused cross-entropy, gradient clipping.
* "wgpu_trainer.rs page" — ``entrenar/train/transformer_trainer/wgpu_trainer.rs``
  (0.38.0): CPU/WGPU restatements of RMSNorm, cross-entropy, the FFN backward
  and the LoRA forward/backward.

``fp8`` follows the OCP 8-bit floating point specification (the 8-bit
operand variant; the pages name no 8-bit format).

Inputs are float32 arrays widened exactly to float64; every step runs in
float64 with numpy matmul as the only library primitive. Where the pages leave
a step open, the reading taken is named in the function's docstring.

Parity status: every public function is pinned by a CPU test under ``tests/``
(closed forms, invariants, library special cases or finite differences); none
is "parity unpinned".
"""
from .ops import (rmsnorm_fwd, rmsnorm_bwd, head_rmsnorm_fwd, head_rmsnorm_bwd,
                  rope_angles, rope_fwd, rope_bwd, attention_fwd, attention_bwd,
                  swiglu_fwd, swiglu_bwd, linear_fwd, linear_bwd)
from .block import block_forward, block_backward, PARAM_NAMES
from .step import (lm_head_cross_entropy, global_clip, adamw_update, stack_step)
from .nf4 import (nf4_codebook, nf4_quantize, nf4_dequantize, lora_linear_fwd,
                  lora_linear_bwd, nf4_block_forward, nf4_block_backward)
from . import fp8
