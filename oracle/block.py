"""Float64 decoder block forward and backward (test infrastructure).

Composition of the steps in ``oracle.ops`` in the order of
``CudaTransformerBlock::forward`` and ``CudaTransformerBlock::backward`` on the
cuda_block.rs page. Every intermediate is kept; nothing is recomputed.

Parameters (11 tensors): w_q [H*d, h], w_k [KV*d, h], w_v [KV*d, h],
w_o [h, H*d], w_gate [I, h], w_up [I, h], w_down [h, I] (all [out, in]),
g_in [h], g_post [h], g_q [d], g_k [d].
"""
from __future__ import annotations

import numpy as np

from . import ops

PARAM_NAMES = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down",
               "g_in", "g_post", "g_q", "g_k")


def _get(c, name):
    return c[name] if isinstance(c, dict) else getattr(c, name)


def _dims(c):
    names = ("hidden", "heads", "kv_heads", "head_dim", "intermediate", "seq", "batch",
             "eps", "rope_theta")
    out = {n: _get(c, n) for n in names}
    try:
        out["qk_norm"] = int(_get(c, "qk_norm"))
    except (KeyError, AttributeError):
        out["qk_norm"] = 1
    return out


def positions(seq, batch):
    """Position of token t = b*seq + s is s: every batch element is its own
    sequence starting at 0 (the ``rope_positions`` buffer 0..seq-1 of the
    cuda_block.rs page, one sequence per call)."""
    return np.tile(np.arange(seq), batch)


def block_forward(c, p, x, linear=None):
    """y = block(x). ``linear(name, x)`` may replace the projection x W^T (the
    NF4+LoRA block uses this); by default it is ``ops.linear_fwd``.

    cuda_block.rs page, ``CudaTransformerBlock::forward`` and
    ``compute_attention_cuda``: RMSNorm -> Q/K/V -> per-head QK RMSNorm ->
    NeoX RoPE -> GQA causal attention -> O-projection -> residual ->
    RMSNorm -> gate/up -> SwiGLU -> down -> residual.
    Returns (y, cache).
    """
    d = _dims(c)
    H, KV, hd, eps = d["heads"], d["kv_heads"], d["head_dim"], d["eps"]
    lin = linear or (lambda name, a: ops.linear_fwd(a, p[name]))
    x = np.asarray(x, np.float64)
    pos = positions(d["seq"], d["batch"])

    n1, rho1 = ops.rmsnorm_fwd(x, p["g_in"], eps)
    q = lin("w_q", n1)
    k = lin("w_k", n1)
    v = lin("w_v", n1)
    if d["qk_norm"]:
        qn, rho_q = ops.head_rmsnorm_fwd(q, p["g_q"], H, eps)
        kn, rho_k = ops.head_rmsnorm_fwd(k, p["g_k"], KV, eps)
    else:
        qn, kn, rho_q, rho_k = q, k, None, None
    qr = ops.rope_fwd(qn, pos, H, d["rope_theta"])
    kr = ops.rope_fwd(kn, pos, KV, d["rope_theta"])
    o = ops.attention_fwd(qr, kr, v, d["batch"], d["seq"], H, KV, hd)
    a = lin("w_o", o)
    r1 = x + a
    n2, rho2 = ops.rmsnorm_fwd(r1, p["g_post"], eps)
    g = lin("w_gate", n2)
    u = lin("w_up", n2)
    s = ops.swiglu_fwd(g, u)
    y = r1 + lin("w_down", s)
    cache = dict(x=x, n1=n1, rho1=rho1, q=q, k=k, v=v, qn=qn, kn=kn, rho_q=rho_q,
                 rho_k=rho_k, qr=qr, kr=kr, o=o, a=a, r1=r1, n2=n2, rho2=rho2,
                 g=g, u=u, s=s, pos=pos)
    return y, cache


def block_backward(c, p, cache, dy, linear_bwd=None):
    """dx and the 11 parameter gradients of ``block_forward``.

    cuda_block.rs page, ``CudaTransformerBlock::backward`` and its parts
    ``backward_ffn`` -> ``backward_post_attn_norm`` -> add the upstream
    gradient (second residual) -> ``backward_attention`` (O-proj, attention,
    GQA reduction, RoPE backward, Q/K/V projection backward) ->
    ``backward_residual_and_input_norm`` (norm backward, then add the first
    residual's gradient). The QK-norm backward that the page lacks is
    inserted between the RoPE backward and the projection backward.

    ``linear_bwd(name, x, dy) -> (dx, dW or None)`` may replace the projection
    backward. Returns (dx, grads) with grads keyed like the parameters.
    """
    d = _dims(c)
    H, KV, hd, eps = d["heads"], d["kv_heads"], d["head_dim"], d["eps"]
    lb = linear_bwd or (lambda name, a, g: ops.linear_bwd(a, p[name], g))
    ch = cache
    dy = np.asarray(dy, np.float64)
    grads = {}

    ds, grads["w_down"] = lb("w_down", ch["s"], dy)
    dg, du = ops.swiglu_bwd(ch["g"], ch["u"], ds)
    dn2_g, grads["w_gate"] = lb("w_gate", ch["n2"], dg)
    dn2_u, grads["w_up"] = lb("w_up", ch["n2"], du)
    dn2 = dn2_g + dn2_u
    dr1, grads["g_post"] = ops.rmsnorm_bwd(ch["r1"], p["g_post"], dn2, eps)
    dr1 = dr1 + dy
    do, grads["w_o"] = lb("w_o", ch["o"], dr1)
    dqr, dkr, dv = ops.attention_bwd(ch["qr"], ch["kr"], ch["v"], do, d["batch"], d["seq"],
                                     H, KV, hd)
    dqn = ops.rope_bwd(dqr, ch["pos"], H, d["rope_theta"])
    dkn = ops.rope_bwd(dkr, ch["pos"], KV, d["rope_theta"])
    if d["qk_norm"]:
        dq, grads["g_q"] = ops.head_rmsnorm_bwd(ch["q"], p["g_q"], dqn, H, eps)
        dk, grads["g_k"] = ops.head_rmsnorm_bwd(ch["k"], p["g_k"], dkn, KV, eps)
    else:
        dq, dk = dqn, dkn
        grads["g_q"] = np.zeros(hd)
        grads["g_k"] = np.zeros(hd)
    dn1_q, grads["w_q"] = lb("w_q", ch["n1"], dq)
    dn1_k, grads["w_k"] = lb("w_k", ch["n1"], dk)
    dn1_v, grads["w_v"] = lb("w_v", ch["n1"], dv)
    dn1 = dn1_q + dn1_k + dn1_v
    dx, grads["g_in"] = ops.rmsnorm_bwd(ch["x"], p["g_in"], dn1, eps)
    dx = dx + dr1
    return dx, grads
