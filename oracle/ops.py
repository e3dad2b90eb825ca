"""Float64 restatements of the single steps of the block (test infrastructure).

Each function is the plain definition of one step; the page passage it follows
is named in its docstring. Arrays may be float32 on entry and are widened to
float64 before any arithmetic.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- RMSNorm ---

def rmsnorm_fwd(x, gamma, eps):
    """RMSNorm over the last axis: rho = (mean(x^2) + eps)^(-1/2), y = x*rho*gamma.

    cuda_block.rs page, ``CudaTransformerBlock::forward`` (pre-attention and
    post-attention RMSNorm). The pages do not print the kernel; eps sits inside
    the square root as in the inline RMSNorm helper of ``full_train_step`` on
    the wgpu_trainer.rs page. Returns (y, rho) with rho of shape x.shape[:-1].
    """
    x = _f64(x)
    rho = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    y = x * rho[..., None] * _f64(gamma)
    return y, rho


def rmsnorm_bwd(x, gamma, dy, eps):
    """Gradient of ``rmsnorm_fwd`` for x and gamma.

    cuda_block.rs page, ``backward_post_attn_norm`` and
    ``backward_residual_and_input_norm`` (the ``rms_norm_backward`` calls).
    With xhat = x*rho and e = gamma*dy:
    dx = rho * (e - xhat * mean(e * xhat)), dgamma = sum over rows of dy*xhat.
    """
    x, dy, gamma = _f64(x), _f64(dy), _f64(gamma)
    rho = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    xhat = x * rho[..., None]
    e = dy * gamma
    dx = rho[..., None] * (e - xhat * np.mean(e * xhat, axis=-1, keepdims=True))
    dgamma = (dy * xhat).reshape(-1, x.shape[-1]).sum(axis=0)
    return dx, dgamma


def head_rmsnorm_fwd(x, gamma, n_heads, eps):
    """Per-head RMSNorm (QK-norm): RMSNorm over each head's head_dim slice of a
    [T, n_heads*head_dim] row, with one gamma [head_dim] shared by all heads.

    cuda_block.rs page, ``compute_attention_cuda`` (the per-head RMSNorm
    applied to Q and K before RoPE) and the q_norm / k_norm weight fields.
    Returns (y [T, n_heads*d], rho [T, n_heads]).
    """
    x = _f64(x)
    t = x.shape[0]
    d = x.shape[1] // n_heads
    y, rho = rmsnorm_fwd(x.reshape(t, n_heads, d), gamma, eps)
    return y.reshape(t, n_heads * d), rho


def head_rmsnorm_bwd(x, gamma, dy, n_heads, eps):
    """Gradient of ``head_rmsnorm_fwd``. The pages have no QK-norm backward
    (their RoPE-backward output feeds the projection backward directly); this
    is the true derivative, since the backward chain mirrors the forward.
    Returns (dx [T, n_heads*d], dgamma [d])."""
    x, dy = _f64(x), _f64(dy)
    t = x.shape[0]
    d = x.shape[1] // n_heads
    dx, dgamma = rmsnorm_bwd(x.reshape(t, n_heads, d), gamma, dy.reshape(t, n_heads, d), eps)
    return dx.reshape(t, n_heads * d), dgamma


# ------------------------------------------------------------------- RoPE ---

def rope_angles(positions, head_dim, theta):
    """Angle a[t, i] = pos_t * theta^(-2i/head_dim) for i < head_dim/2.

    cuda_block.rs page, ``batched_rope_neox_forward`` call with the
    ``rope_positions`` buffer (0, 1, ..., seq-1) and ``rope_theta``. The
    frequency formula is not printed; this is the standard NeoX/Llama one.
    """
    pos = _f64(positions)[:, None]
    i = np.arange(head_dim // 2, dtype=np.float64)[None, :]
    return pos * float(theta) ** (-2.0 * i / head_dim)


def rope_fwd(x, positions, n_heads, theta):
    """NeoX half rotation of every head: for i < d/2, with c, s = cos, sin(a),
    (x_i, x_{i+d/2}) -> (x_i c - x_{i+d/2} s, x_{i+d/2} c + x_i s).

    cuda_block.rs page, ``compute_attention_cuda`` (RoPE on Q and K). The
    forward rotation is the inverse of the one the page states for the RoPE
    backward in ``backward_attention``.
    """
    x = _f64(x)
    t = x.shape[0]
    d = x.shape[1] // n_heads
    a = rope_angles(positions, d, theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    xh = x.reshape(t, n_heads, d)
    x0, x1 = xh[..., : d // 2], xh[..., d // 2:]
    y = np.concatenate([x0 * c - x1 * s, x1 * c + x0 * s], axis=-1)
    return y.reshape(t, n_heads * d)


def rope_bwd(dy, positions, n_heads, theta):
    """Transpose of the RoPE rotation: dx_i = dy_i c + dy_{i+d/2} s,
    dx_{i+d/2} = dy_{i+d/2} c - dy_i s.

    cuda_block.rs page, ``backward_attention`` (the RoPE backward step, which
    states this inverse rotation)."""
    dy = _f64(dy)
    t = dy.shape[0]
    d = dy.shape[1] // n_heads
    a = rope_angles(positions, d, theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    gh = dy.reshape(t, n_heads, d)
    g0, g1 = gh[..., : d // 2], gh[..., d // 2:]
    dx = np.concatenate([g0 * c + g1 * s, g1 * c - g0 * s], axis=-1)
    return dx.reshape(t, n_heads * d)


# -------------------------------------------------------------- Attention ---

def _group(h, heads, kv_heads):
    """GQA: query head h reads KV head floor(h / (heads/kv_heads)).
    cuda_block.rs page, ``expand_kv_heads`` and the GQA gradient reduction
    (contiguous groups of heads/kv_heads query heads)."""
    return h // (heads // kv_heads)


def _causal_probs(qh, kh, d):
    """Scores q.k/sqrt(d) for j <= i, -inf above the diagonal; row softmax
    with the row maximum subtracted; exact zeros above the diagonal."""
    s = (qh @ kh.T) / np.sqrt(d)
    n = s.shape[0]
    mask = np.triu(np.ones((n, n), dtype=bool), k=1)
    s = np.where(mask, -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= p.sum(axis=1, keepdims=True)
    p[mask] = 0.0
    return p


def attention_fwd(q, k, v, batch, seq, heads, kv_heads, head_dim, return_probs=False):
    """GQA causal softmax attention, one independent sequence per batch element.

    cuda_block.rs page, ``compute_attention_cuda`` (QK^T, 1/sqrt(d) scale,
    causal mask keeping key j <= query i, row softmax, times V, with the KV
    head of each query head chosen by ``expand_kv_heads``). Positions and the
    mask restart for every batch element (each is its own sequence).
    q: [T, heads*d]; k, v: [T, kv_heads*d]; returns o [T, heads*d]
    (and probs [batch, heads, seq, seq] if asked).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    d = head_dim
    o = np.zeros_like(q)
    probs = np.zeros((batch, heads, seq, seq)) if return_probs else None
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for h in range(heads):
            g = _group(h, heads, kv_heads)
            qh = q[rows, h * d:(h + 1) * d]
            kh = k[rows, g * d:(g + 1) * d]
            vh = v[rows, g * d:(g + 1) * d]
            p = _causal_probs(qh, kh, d)
            o[rows, h * d:(h + 1) * d] = p @ vh
            if return_probs:
                probs[b, h] = p
    return (o, probs) if return_probs else o


def attention_bwd(q, k, v, do, batch, seq, heads, kv_heads, head_dim):
    """Gradient of ``attention_fwd`` for q, k, v.

    cuda_block.rs page, ``backward_attention``: dP = dO V^T; the softmax
    backward dS = P * (dP - rowsum(P * dP)); the 1/sqrt(d) scale; dQ = dS K;
    dK = dS^T Q; dV = P^T dO; then the GQA reduction that sums dK and dV over
    the query heads sharing a KV head. Probabilities are recomputed from q, k.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    d = head_dim
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for h in range(heads):
            g = _group(h, heads, kv_heads)
            qc, kc = slice(h * d, (h + 1) * d), slice(g * d, (g + 1) * d)
            qh, kh, vh, doh = q[rows, qc], k[rows, kc], v[rows, kc], do[rows, qc]
            p = _causal_probs(qh, kh, d)
            dp = doh @ vh.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True)) / np.sqrt(d)
            dq[rows, qc] = ds @ kh
            dk[rows, kc] += ds.T @ qh
            dv[rows, kc] += p.T @ doh
    return dq, dk, dv


# ----------------------------------------------------------------- SwiGLU ---

def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def swiglu_fwd(g, u):
    """s = silu(g) * u = g * sigmoid(g) * u.
    cuda_block.rs page, ``fused_swiglu_forward`` call in ``forward``."""
    g, u = _f64(g), _f64(u)
    return g * _sigmoid(g) * u


def swiglu_bwd(g, u, ds):
    """dg = ds * u * silu'(g) with silu'(g) = sigma(g) * (1 + g - g*sigma(g)),
    du = ds * silu(g).
    wgpu_trainer.rs page, ``ffn_backward`` (the SiLU-backward loop); the same
    chain as ``backward_ffn`` on the cuda_block.rs page."""
    g, u, ds = _f64(g), _f64(u), _f64(ds)
    sg = _sigmoid(g)
    silu = g * sg
    dsilu = sg * (1.0 + g - silu)
    return ds * u * dsilu, ds * silu


# ----------------------------------------------------------------- Linear ---

def linear_fwd(x, w):
    """y = x W^T with W stored [out, in] row-major (HF layout, as the NF4 block
    and the wgpu_trainer.rs page ``lora_forward`` use)."""
    return _f64(x) @ _f64(w).T


def linear_bwd(x, w, dy):
    """dx = dy W, dW = dy^T x (the ``gemm_backward_a`` / ``gemm_backward_b``
    pair on the cuda_block.rs page, in the [out, in] layout)."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    return dy @ w, dy.T @ x
