"""CPU checks of the C ABI: the library loads, exports every function that
include/*.h declares, its host-only entry points behave, and invalid
arguments are rejected on the host before any device work."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from bwd_rmsnorm_qkv_amd import qblk, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(qblk_\w+)\s*\(", text, re.M))
    return names


def test_library_exports_every_declared_function():
    lib = qblk.lib()
    decl = declared_functions()
    assert len(decl) >= 20
    for name in sorted(decl):
        assert hasattr(lib, name), name
    assert decl == set(qblk.exported_symbols())


def test_codebook_matches_oracle_bitwise():
    a = np.array(qblk.nf4_codebook(), np.float32)
    assert np.array_equal(a.view(np.uint32), oracle.nf4_codebook().view(np.uint32))


def test_workspace_queries_and_validation():
    saved, scratch = qblk.block_workspace_size(synth.QWEN3_4B_BLOCK)
    assert saved > 0 and scratch > 0
    s2, w2 = qblk.block_workspace_size(synth.QWEN3_4B_BLOCK.with_tokens(seq=1024))
    assert s2 > saved and w2 > scratch
    for field, value in (("kv_heads", 3), ("head_dim", 48), ("hidden", 60), ("seq", 0)):
        cfg = qblk.make_config(synth.TINY_BLOCK)
        setattr(cfg, field, value)
        with pytest.raises(qblk.QblkError) as e:
            qblk.block_workspace_size(cfg)
        assert e.value.code in (qblk.QBLK_EINVAL, qblk.QBLK_EUNSUPPORTED), field
    with pytest.raises(qblk.QblkError):
        qblk.nf4_block_workspace_size(synth.NF4_LORA_QWEN3_4B, 6)
    assert qblk.cross_entropy_workspace_size(1024, 512, 151936) >= 1024 * 151936 * 4


def test_invalid_arguments_fail_before_device_work():
    lib = qblk.lib()
    # bad layout, null operands, misaligned lda: all rejected on the host
    # (only NULL pointers are passed: nothing here can reach a launch)
    assert lib.qblk_gemm(5, 0, 4, 4, 4, None, 4, None, 4, None, 4, 0, None, 0, None) == qblk.QBLK_EINVAL
    assert lib.qblk_gemm(0, 0, 4, 4, 4, None, 6, None, 4, None, 4, 0, None, 0, None) == qblk.QBLK_EINVAL
    assert b"lda" in lib.qblk_last_error()
    assert lib.qblk_gemm(0, 0, 4, 4, 4, None, 4, None, 4, None, 4, 0, None, 0, None) == qblk.QBLK_EINVAL
    assert b"null" in lib.qblk_last_error()
    assert lib.qblk_nf4_quantize(None, 100, None, None, None) == qblk.QBLK_EINVAL
    assert b"multiple of 64" in lib.qblk_last_error()
    assert lib.qblk_adamw_step(1, None, None, None, None, None, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None,
                               None) == qblk.QBLK_EINVAL
    cfg = qblk.make_config(synth.TINY_BLOCK)
    assert lib.qblk_block_forward(C.byref(cfg), None, None, None, None, 0, None, 0, None) == qblk.QBLK_EINVAL


def test_bf16_config_needs_direct_to_lds_shapes():
    """bfloat16 operands run only on the direct-to-LDS kernels: a token
    count that is not a multiple of 64 is refused on the host (no device
    work); the Qwen3-4B shape is accepted."""
    c = synth.BlockShape(hidden=512, heads=8, kv_heads=2, head_dim=64, intermediate=1408, seq=100, batch=2,
                         rope_theta=1e4, gemm_precision=2)
    with pytest.raises(qblk.QblkError) as e:
        qblk.block_workspace_size(qblk.make_config(c))
    assert e.value.code == qblk.QBLK_EUNSUPPORTED
    ok = synth.BlockShape(hidden=2560, heads=32, kv_heads=8, head_dim=128, intermediate=9728, seq=512, batch=1,
                          rope_theta=1e6, gemm_precision=2)
    saved, scratch = qblk.block_workspace_size(qblk.make_config(ok))
    assert saved > 0 and scratch > 0
    bad = qblk.make_config(ok)
    bad.gemm_precision = 3
    with pytest.raises(qblk.QblkError) as e:
        qblk.block_workspace_size(bad)
    assert e.value.code == qblk.QBLK_EINVAL


def test_size_limits_are_refused_on_the_host():
    """The limits of the row kernels and of the LoRA tile, refused before
    any device work: hidden above 4096 (one RMSNorm row per wave's
    registers) is unsupported; LoRA ranks must be multiples of 4 up to 20
    (three ranks of a projection group in one 64-wide tile); 4096 and 20
    themselves are accepted."""
    import dataclasses
    big = dataclasses.replace(synth.QWEN3_4B_BLOCK, hidden=4160)
    with pytest.raises(qblk.QblkError) as e:
        qblk.block_workspace_size(qblk.make_config(big))
    assert e.value.code == qblk.QBLK_EUNSUPPORTED
    assert b"4096" in qblk.lib().qblk_last_error()
    edge = dataclasses.replace(synth.QWEN3_4B_BLOCK, hidden=4096)
    assert min(qblk.block_workspace_size(qblk.make_config(edge))) > 0
    for rank in (0, 24, 6):
        with pytest.raises(qblk.QblkError) as e:
            qblk.nf4_block_workspace_size(synth.NF4_LORA_QWEN3_4B, rank)
        assert e.value.code == qblk.QBLK_EINVAL, rank
    assert min(qblk.nf4_block_workspace_size(synth.NF4_LORA_QWEN3_4B, 20)) > 0
