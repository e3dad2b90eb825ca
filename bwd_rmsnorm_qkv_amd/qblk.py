"""Python binding of libqblk (ctypes; argument marshalling only).

Every function here forwards to the C entry point of the same name in
``include/qblk.h`` / ``include/qblk_ops.h``; all arithmetic runs in the HIP
kernels of the library. Tensors are torch tensors on the current HIP device
and must be contiguous; PyTorch is used only for memory and streams. If the
library is not built, loading fails loudly (there is no CPU fallback).
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqblk.so")

QBLK_OK, QBLK_EINVAL, QBLK_EHIP, QBLK_EUNSUPPORTED = 0, -1, -2, -3

PROJ = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")
GAMMAS = ("g_in", "g_post", "g_q", "g_k")
PARAMS = PROJ + GAMMAS


class QblkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libqblk error {code}: {msg}")
        self.code = code


class Config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("heads", C.c_int32), ("kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("intermediate", C.c_int32), ("seq", C.c_int32),
                ("batch", C.c_int32), ("eps", C.c_float), ("rope_theta", C.c_float),
                ("qk_norm", C.c_int32), ("gemm_precision", C.c_int32)]


class BlockParams(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in PARAMS] + [("w16", C.c_void_p)]


class BlockGrads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in PARAMS]


class Nf4BlockParams(C.Structure):
    _fields_ = [("codes", C.c_void_p * 7), ("absmax", C.c_void_p * 7), ("lora_a", C.c_void_p * 7),
                ("lora_b", C.c_void_p * 7), ("g_in", C.c_void_p), ("g_post", C.c_void_p),
                ("g_q", C.c_void_p), ("g_k", C.c_void_p), ("rank", C.c_int32), ("alpha", C.c_float)]


class LoraGrads(C.Structure):
    _fields_ = [("lora_a", C.c_void_p * 7), ("lora_b", C.c_void_p * 7)]


_lib = None

_SIGS = {
    "qblk_last_error": ([], C.c_char_p),
    "qblk_clear_error": ([], None),
    "qblk_block_workspace_size": ([C.c_void_p, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_block_forward": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                            C.c_void_p, C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_block_backward": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                             C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_block_backward_accumulate": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                        C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_attention_forward_f16": ([C.c_int32] * 5 + [C.c_void_p] * 5 + [C.c_void_p], C.c_int32),
    "qblk_attention_backward_f16": ([C.c_int32] * 5 + [C.c_void_p] * 11 + [C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_block_pack_f16_size": ([C.c_void_p, C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_block_pack_f16": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_cross_entropy_workspace_size": ([C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_fused_cross_entropy": ([C.c_int32, C.c_int32, C.c_int32, C.c_float, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_float, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_fused_cross_entropy_accumulate": ([C.c_int32, C.c_int32, C.c_int32, C.c_float, C.c_void_p, C.c_void_p,
                                             C.c_void_p, C.c_void_p, C.c_float, C.c_void_p, C.c_void_p,
                                             C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                             C.c_void_p], C.c_int32),
    "qblk_cross_entropy_rows": ([C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_float, C.c_void_p,
                                 C.c_void_p, C.c_void_p], C.c_int32),
    "qblk_clip_workspace_size": ([C.c_int32, C.c_void_p, C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_clip_grad_norm": ([C.c_int32, C.c_void_p, C.c_void_p, C.c_float, C.c_int32, C.c_void_p,
                             C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_clip_grad_norm_noalloc": ([C.c_int32, C.c_void_p, C.c_void_p, C.c_float, C.c_int32, C.c_void_p,
                                     C.c_void_p, C.c_void_p], C.c_int32),
    "qblk_adamw_step": ([C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                         C.c_float, C.c_float, C.c_float, C.c_float, C.c_float, C.c_int32, C.c_void_p,
                         C.c_void_p], C.c_int32),
    "qblk_adamw_step_pack16": ([C.c_int32] + [C.c_void_p] * 6 + [C.c_int32] + [C.c_float] * 5
                               + [C.c_int32, C.c_void_p, C.c_void_p], C.c_int32),
    "qblk_block_pack_f16_offsets": ([C.c_void_p, C.c_void_p], C.c_int32),
    "qblk_nf4_codebook": ([C.c_void_p], C.c_int32),
    "qblk_nf4_quantize": ([C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int32),
    "qblk_nf4_dequantize": ([C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p], C.c_int32),
    "qblk_nf4_block_workspace_size": ([C.c_void_p, C.c_int32, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)],
                                      C.c_int32),
    "qblk_block_forward_nf4_lora": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                     C.c_void_p, C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_block_backward_nf4_lora": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_size_t, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                      C.c_void_p], C.c_int32),
    "qblk_gemm": ([C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_int64,
                   C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_size_t,
                   C.c_void_p], C.c_int32),
    "qblk_gemm_workspace_size": ([C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                  C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_gemm_ex": ([C.c_int32] * 5 + [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_int64, C.c_int32,
                                        C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p],
                     C.c_int32),
    "qblk_fp8_quantize_workspace_size": ([C.c_int32, C.c_int32, C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_fp8_quantize": ([C.c_int32, C.c_int32, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_int64,
                           C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_gemm_fp8_workspace_size": ([C.c_int32] * 3 + [C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_gemm_fp8": ([C.c_int32] * 3 + [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_int64, C.c_int32,
                                         C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p,
                                         C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_swiglu_forward": ([C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int32),
    "qblk_swiglu_backward": ([C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int32),
    "qblk_qk_norm_rope_workspace_size": ([C.c_int32] * 5 + [C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_qk_norm_rope_forward": ([C.c_int32] * 6 + [C.c_float, C.c_float, C.c_void_p, C.c_int64]
                                  + [C.c_void_p] * 7 + [C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_qk_norm_rope_backward": ([C.c_int32] * 6 + [C.c_float, C.c_float, C.c_void_p, C.c_int64]
                                   + [C.c_void_p] * 8 + [C.c_size_t, C.c_void_p], C.c_int32),
    "qblk_rmsnorm_workspace_size": ([C.c_int32, C.c_int32, C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_rmsnorm_forward": ([C.c_int32, C.c_int32, C.c_float, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p],
                             C.c_int32),
    "qblk_rmsnorm_backward": ([C.c_int32, C.c_int32, C.c_float, C.c_void_p, C.c_void_p, C.c_void_p,
                               C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p],
                              C.c_int32),
    "qblk_attention_forward": ([C.c_int32] * 6 + [C.c_void_p, C.c_int64] * 4 + [C.c_void_p, C.c_void_p],
                               C.c_int32),
    "qblk_attention_workspace_size": ([C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_size_t)], C.c_int32),
    "qblk_attention_backward": ([C.c_int32] * 6 + [C.c_void_p, C.c_int64] * 4 + [C.c_void_p]
                                + [C.c_void_p, C.c_int64] * 4 + [C.c_void_p, C.c_size_t, C.c_void_p],
                                C.c_int32),
}


def exported_symbols():
    """Names of every C entry point this binding expects the library to export."""
    return sorted(_SIGS)


def lib():
    """Load libqblk.so (built in-tree by ``bwd_rmsnorm_qkv_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        h = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def _check(rc: int):
    if rc != QBLK_OK:
        raise QblkError(rc, lib().qblk_last_error().decode(errors="replace"))


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_config(shape) -> Config:
    """Config from any object/dict with the BlockShape fields."""
    g = (lambda k: shape[k]) if isinstance(shape, dict) else (lambda k: getattr(shape, k))
    return Config(g("hidden"), g("heads"), g("kv_heads"), g("head_dim"), g("intermediate"), g("seq"),
                  g("batch"), float(g("eps")), float(g("rope_theta")), int(g("qk_norm")),
                  int(g("gemm_precision")))


def _cfg(cfg):
    return cfg if isinstance(cfg, Config) else make_config(cfg)


# ------------------------------------------------------------------ block

def block_workspace_size(cfg):
    c = _cfg(cfg)
    a, b = C.c_size_t(), C.c_size_t()
    _check(lib().qblk_block_workspace_size(C.byref(c), C.byref(a), C.byref(b)))
    return a.value, b.value


def _params(p: dict) -> BlockParams:
    """p: the 11 tensors by name, plus an optional packed fp16 set under "w16"."""
    return BlockParams(*[_p(p[n]) for n in PARAMS], _p(p.get("w16")))


def block_pack_f16_size(cfg):
    c = _cfg(cfg)
    n = C.c_size_t()
    _check(lib().qblk_block_pack_f16_size(C.byref(c), C.byref(n)))
    return n.value


def block_pack_f16(cfg, params: dict, packed, stream=None):
    c = _cfg(cfg)
    bp = _params({**params, "w16": None})
    _check(lib().qblk_block_pack_f16(C.byref(c), C.byref(bp), _p(packed), packed.numel() * packed.element_size(),
                                     _stream(stream)))


def block_forward(cfg, params: dict, x, y, saved, scratch=None, stream=None):
    c = _cfg(cfg)
    bp = _params(params)
    _check(lib().qblk_block_forward(C.byref(c), C.byref(bp), _p(x), _p(y), _p(saved), saved.numel() * saved.element_size(),
                                    _p(scratch), 0 if scratch is None else scratch.numel() * scratch.element_size(),
                                    _stream(stream)))


def block_backward(cfg, params: dict, x, dy, saved, dx, grads: dict, scratch, stream=None, accumulate=False):
    """accumulate: qblk_block_backward_accumulate (parameter gradients added
    into `grads`) instead of qblk_block_backward (overwritten)."""
    c = _cfg(cfg)
    bp = _params(params)
    gp = BlockGrads(*[_p(grads[n]) for n in PARAMS])
    fn = lib().qblk_block_backward_accumulate if accumulate else lib().qblk_block_backward
    _check(fn(C.byref(c), C.byref(bp), _p(x), _p(dy), _p(saved),
              saved.numel() * saved.element_size(), _p(dx), C.byref(gp), _p(scratch),
              scratch.numel() * scratch.element_size(), _stream(stream)))


# ----------------------------------------------------------- LM head + CE

def cross_entropy_workspace_size(tokens, hidden, vocab):
    n = C.c_size_t()
    _check(lib().qblk_cross_entropy_workspace_size(tokens, hidden, vocab, C.byref(n)))
    return n.value


def fused_cross_entropy(tokens, hidden, vocab, eps, y_last, g_final, w_lm, targets, loss_scale,
                        loss_partials, argmax, dy_last, dg_final, dw_lm, scratch, stream=None, accumulate=False):
    """accumulate: qblk_fused_cross_entropy_accumulate (dw_lm, dg_final added into)."""
    fn = lib().qblk_fused_cross_entropy_accumulate if accumulate else lib().qblk_fused_cross_entropy
    _check(fn(tokens, hidden, vocab, eps, _p(y_last), _p(g_final), _p(w_lm), _p(targets), loss_scale,
              _p(loss_partials), _p(argmax), _p(dy_last), _p(dg_final), _p(dw_lm), _p(scratch),
              scratch.numel() * scratch.element_size(), _stream(stream)))


def cross_entropy_rows(tokens, vocab, z, targets, loss_scale, loss_partials, argmax, stream=None):
    _check(lib().qblk_cross_entropy_rows(tokens, vocab, _p(z), _p(targets), loss_scale, _p(loss_partials),
                                         _p(argmax), _stream(stream)))


# ---------------------------------------------------------- clip + AdamW

def _ptr_array(ts):
    return (C.c_void_p * len(ts))(*[_p(t) for t in ts])


def _numel_array(ts):
    return (C.c_int64 * len(ts))(*[t.numel() for t in ts])


def clip_workspace_size(tensors):
    n = C.c_size_t()
    _check(lib().qblk_clip_workspace_size(len(tensors), _numel_array(tensors), C.byref(n)))
    return n.value


def clip_grad_norm(grads, max_norm, apply, norm_dev, scale_dev, scratch, stream=None):
    _check(lib().qblk_clip_grad_norm(len(grads), _ptr_array(grads), _numel_array(grads), max_norm, int(apply),
                                     _p(norm_dev), _p(scale_dev), _p(scratch),
                                     scratch.numel() * scratch.element_size(), _stream(stream)))


def clip_grad_norm_noalloc(grads, max_norm, apply, norm_dev, scale_dev, stream=None):
    _check(lib().qblk_clip_grad_norm_noalloc(len(grads), _ptr_array(grads), _numel_array(grads), max_norm,
                                             int(apply), _p(norm_dev), _p(scale_dev), _stream(stream)))


def adamw_step(w, g, m, v, lr, beta1, beta2, eps, weight_decay, step, grad_scale_dev=None, stream=None):
    assert len(w) == len(g) == len(m) == len(v)
    _check(lib().qblk_adamw_step(len(w), _ptr_array(w), _ptr_array(g), _ptr_array(m), _ptr_array(v),
                                 _numel_array(w), lr, beta1, beta2, eps, weight_decay, int(step),
                                 _p(grad_scale_dev), _stream(stream)))


def swiglu_forward(tokens, inter, gu, s, stream=None):
    _check(lib().qblk_swiglu_forward(tokens, inter, _p(gu), _p(s), _stream(stream)))


def swiglu_backward(tokens, inter, gu, ds, dgu, stream=None):
    _check(lib().qblk_swiglu_backward(tokens, inter, _p(gu), _p(ds), _p(dgu), _stream(stream)))


def qk_norm_rope_workspace_size(tokens, seq, heads, kv_heads, head_dim):
    n = C.c_size_t()
    _check(lib().qblk_qk_norm_rope_workspace_size(tokens, seq, heads, kv_heads, head_dim, C.byref(n)))
    return n.value


def qk_norm_rope_forward(tokens, seq, heads, kv_heads, head_dim, qk_norm, eps, theta, qkv, ld_qkv, g_q, g_k,
                         qr, kr, rho_q, rho_k, scratch, stream=None):
    _check(lib().qblk_qk_norm_rope_forward(tokens, seq, heads, kv_heads, head_dim, int(qk_norm), eps, theta,
                                           _p(qkv), ld_qkv, _p(g_q), _p(g_k), _p(qr), _p(kr), _p(rho_q),
                                           _p(rho_k), _p(scratch), scratch.numel() * scratch.element_size(),
                                           _stream(stream)))


def qk_norm_rope_backward(tokens, seq, heads, kv_heads, head_dim, qk_norm, eps, theta, qkv, ld_qkv, g_q, g_k,
                          dqr, dkr, dqkv, dg_q, dg_k, scratch, stream=None):
    _check(lib().qblk_qk_norm_rope_backward(tokens, seq, heads, kv_heads, head_dim, int(qk_norm), eps, theta,
                                            _p(qkv), ld_qkv, _p(g_q), _p(g_k), _p(dqr), _p(dkr), _p(dqkv),
                                            _p(dg_q), _p(dg_k), _p(scratch),
                                            scratch.numel() * scratch.element_size(), _stream(stream)))


def adamw_step_pack16(w, g, m, v, w16, lr, beta1, beta2, eps, weight_decay, step, grad_scale_dev=None,
                      stream=None, bf16=False):
    """w16: per tensor a 16-bit device address (int) or tensor for the copy,
    or None; bf16: the copies are bfloat16 (else fp16)."""
    assert len(w) == len(g) == len(m) == len(v) == len(w16)
    ptrs = (C.c_void_p * len(w16))(*[(x if isinstance(x, int) else _p(x)) if x is not None else None
                                     for x in w16])
    _check(lib().qblk_adamw_step_pack16(len(w), _ptr_array(w), _ptr_array(g), _ptr_array(m), _ptr_array(v),
                                        _numel_array(w), ptrs, int(bool(bf16)), lr, beta1, beta2, eps, weight_decay,
                                        int(step), _p(grad_scale_dev), _stream(stream)))


def block_pack_f16_offsets(cfg):
    c = cfg if isinstance(cfg, Config) else make_config(cfg)
    off = (C.c_int64 * 7)()
    _check(lib().qblk_block_pack_f16_offsets(C.byref(c), off))
    return dict(zip(PROJ, list(off)))


# ------------------------------------------------------------------- NF4

def nf4_codebook():
    out = (C.c_float * 16)()
    _check(lib().qblk_nf4_codebook(out))
    return list(out)


def nf4_quantize(w, codes, absmax, stream=None):
    _check(lib().qblk_nf4_quantize(_p(w), w.numel(), _p(codes), _p(absmax), _stream(stream)))


def nf4_dequantize(codes, absmax, numel, w, stream=None):
    _check(lib().qblk_nf4_dequantize(_p(codes), _p(absmax), numel, _p(w), _stream(stream)))


def nf4_block_workspace_size(cfg, rank):
    c = _cfg(cfg)
    a, b = C.c_size_t(), C.c_size_t()
    _check(lib().qblk_nf4_block_workspace_size(C.byref(c), rank, C.byref(a), C.byref(b)))
    return a.value, b.value


def _nf4_params(codes, absmax, lora_a, lora_b, gammas, rank, alpha):
    arr = lambda d: (C.c_void_p * 7)(*[_p(d[n]) for n in PROJ])
    return Nf4BlockParams(arr(codes), arr(absmax), arr(lora_a), arr(lora_b), _p(gammas["g_in"]),
                          _p(gammas["g_post"]), _p(gammas["g_q"]), _p(gammas["g_k"]), rank, alpha)


def block_forward_nf4_lora(cfg, codes, absmax, lora_a, lora_b, gammas, rank, alpha, x, y, saved, scratch,
                           stream=None):
    c = _cfg(cfg)
    p = _nf4_params(codes, absmax, lora_a, lora_b, gammas, rank, alpha)
    _check(lib().qblk_block_forward_nf4_lora(C.byref(c), C.byref(p), _p(x), _p(y), _p(saved),
                                             saved.numel() * saved.element_size(), _p(scratch),
                                             scratch.numel() * scratch.element_size(), _stream(stream)))


def block_backward_nf4_lora(cfg, codes, absmax, lora_a, lora_b, gammas, rank, alpha, x, dy, saved, dx,
                            grad_a, grad_b, scratch, stream=None):
    c = _cfg(cfg)
    p = _nf4_params(codes, absmax, lora_a, lora_b, gammas, rank, alpha)
    g = LoraGrads((C.c_void_p * 7)(*[_p(grad_a[n]) for n in PROJ]),
                  (C.c_void_p * 7)(*[_p(grad_b[n]) for n in PROJ]))
    _check(lib().qblk_block_backward_nf4_lora(C.byref(c), C.byref(p), _p(x), _p(dy), _p(saved),
                                              saved.numel() * saved.element_size(), _p(dx), C.byref(g),
                                              _p(scratch), scratch.numel() * scratch.element_size(),
                                              _stream(stream)))


# ---------------------------------------------------------- single steps

def gemm_workspace_size(layout, precision, M, N, K):
    n = C.c_size_t()
    _check(lib().qblk_gemm_workspace_size(layout, precision, M, N, K, C.byref(n)))
    return n.value


def gemm(layout, precision, M, N, K, A, lda, B, ldb, Cm, ldc, accumulate=0, scratch=None, stream=None):
    """fp32, fp16 or bfloat16 operand tensors (the storage type is taken from the tensors)."""
    nbytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    code = lambda t: {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[t.dtype]
    _check(lib().qblk_gemm_ex(layout, precision, M, N, K, _p(A), lda, code(A), _p(B), ldb, code(B), _p(Cm), ldc,
                              accumulate, _p(scratch), nbytes, _stream(stream)))


def fp8_quantize_workspace_size(rows, cols):
    n = C.c_size_t()
    _check(lib().qblk_fp8_quantize_workspace_size(rows, cols, C.byref(n)))
    return n.value


def fp8_quantize(rows, cols, x, ldx, e5m2, q, ldq, inv_scale, scratch, stream=None):
    """x fp32 [rows, ldx] -> q uint8 [rows, ldq] (E4M3, or E5M2 with
    e5m2 = 1) and inv_scale (device fp32 [1]) = 1 / the per-tensor scale."""
    _check(lib().qblk_fp8_quantize(rows, cols, _p(x), ldx, int(e5m2), _p(q), ldq, _p(inv_scale), _p(scratch),
                                   scratch.numel() * scratch.element_size(), _stream(stream)))


def gemm_fp8_workspace_size(M, N, K):
    n = C.c_size_t()
    _check(lib().qblk_gemm_fp8_workspace_size(M, N, K, C.byref(n)))
    return n.value


def gemm_fp8(M, N, K, A, lda, a_e5m2, B, ldb, b_e5m2, a_inv_scale, b_inv_scale, Cm, ldc, accumulate=0,
             scratch=None, stream=None):
    """C[M, N] (+)= (A8 [M, K] B8 [N, K]^T) * a_inv_scale[0] * b_inv_scale[0]."""
    nbytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    _check(lib().qblk_gemm_fp8(M, N, K, _p(A), lda, int(a_e5m2), _p(B), ldb, int(b_e5m2), _p(a_inv_scale),
                               _p(b_inv_scale), _p(Cm), ldc, accumulate, _p(scratch), nbytes, _stream(stream)))


def rmsnorm_workspace_size(rows, n):
    s = C.c_size_t()
    _check(lib().qblk_rmsnorm_workspace_size(rows, n, C.byref(s)))
    return s.value


def rmsnorm_forward(rows, n, eps, x, res, gamma, y, sum_out, rho, stream=None):
    _check(lib().qblk_rmsnorm_forward(rows, n, eps, _p(x), _p(res), _p(gamma), _p(y), _p(sum_out), _p(rho),
                                      None, 0, _stream(stream)))


def rmsnorm_backward(rows, n, eps, x, gamma, dy, dres, dx, dgamma, scratch, stream=None):
    _check(lib().qblk_rmsnorm_backward(rows, n, eps, _p(x), _p(gamma), _p(dy), _p(dres), _p(dx), _p(dgamma),
                                       _p(scratch), scratch.numel() * scratch.element_size(), _stream(stream)))


def attention_forward(batch, seq, heads, kv_heads, head_dim, precision, q, ldq, k, ldk, v, ldv, o, ldo, lse,
                      stream=None):
    _check(lib().qblk_attention_forward(batch, seq, heads, kv_heads, head_dim, precision, _p(q), ldq, _p(k), ldk,
                                        _p(v), ldv, _p(o), ldo, _p(lse), _stream(stream)))


def attention_workspace_size(batch, seq, heads):
    s = C.c_size_t()
    _check(lib().qblk_attention_workspace_size(batch, seq, heads, C.byref(s)))
    return s.value


def attention_forward_f16(batch, seq, heads, kv_heads, head_dim, q16, k16, v16, o, lse, stream=None):
    _check(lib().qblk_attention_forward_f16(batch, seq, heads, kv_heads, head_dim, _p(q16), _p(k16), _p(v16),
                                            _p(o), _p(lse), _stream(stream)))


def attention_backward_f16(batch, seq, heads, kv_heads, head_dim, q16, k16, v16, o, lse, do16, do32, dq, dk, dv,
                           scratch, stream=None):
    _check(lib().qblk_attention_backward_f16(batch, seq, heads, kv_heads, head_dim, _p(q16), _p(k16), _p(v16),
                                             _p(o), _p(lse), _p(do16), _p(do32), _p(dq), _p(dk), _p(dv),
                                             _p(scratch), scratch.numel() * scratch.element_size(),
                                             _stream(stream)))


def attention_backward(batch, seq, heads, kv_heads, head_dim, precision, q, ldq, k, ldk, v, ldv, o, ldo, lse,
                       d_o, lddo, dq, lddq, dk, lddk, dv, lddv, scratch, stream=None):
    _check(lib().qblk_attention_backward(batch, seq, heads, kv_heads, head_dim, precision, _p(q), ldq, _p(k), ldk,
                                         _p(v), ldv, _p(o), ldo, _p(lse), _p(d_o), lddo, _p(dq), lddq, _p(dk),
                                         lddk, _p(dv), lddv, _p(scratch),
                                         scratch.numel() * scratch.element_size(), _stream(stream)))
