"""Float64 LM head + cross-entropy, global clip, AdamW and the stack training
step (test infrastructure)."""
from __future__ import annotations

import numpy as np

from . import ops
from .block import block_forward, block_backward, PARAM_NAMES


def lm_head_cross_entropy(y_last, g_final, w_lm, targets, eps, loss_scale=None):
    """Final RMSNorm, LM head and cross-entropy, forward and backward.

    cuda_trainer.rs page: ``gpu_forward`` (final ``rms_norm_forward_with_eps``
    then the LM-head GEMM), ``train_step_inner`` (``fused_cross_entropy_cuda``
    with loss scale 1/seq), ``gpu_backward`` (LM-head ``gemm_backward_a`` and
    ``gemm_backward_b``, then the final-norm ``rms_norm_backward``). The logit
    product is z = hf W_lm^T as written out in ``train_step`` on the
    wgpu_trainer.rs page, with W_lm [V, h].

    Per token: l_t = logsumexp(z_t) - z_t[target_t] (max-subtracted);
    loss = loss_scale * sum_t l_t with loss_scale = 1/T by default;
    dz = loss_scale * (softmax(z) - onehot(target)). The argmax is the first
    index of the row maximum. ``g_final`` None skips the final norm.
    """
    y = np.asarray(y_last, np.float64)
    t_count = y.shape[0]
    scale = 1.0 / t_count if loss_scale is None else float(loss_scale)
    if g_final is not None:
        hf, _ = ops.rmsnorm_fwd(y, g_final, eps)
    else:
        hf = y
    w = np.asarray(w_lm, np.float64)
    z = hf @ w.T
    tgt = np.asarray(targets, np.int64)
    rows = np.arange(t_count)
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    sez = ez.sum(axis=1, keepdims=True)
    lse = (np.log(sez) + m)[:, 0]
    partials = lse - z[rows, tgt]
    dz = ez / sez
    dz[rows, tgt] -= 1.0
    dz *= scale
    argmax = z.argmax(axis=1).astype(np.int32)
    del ez
    dhf = dz @ w
    dw_lm = dz.T @ hf
    if g_final is not None:
        dy_last, dg_final = ops.rmsnorm_bwd(y, g_final, dhf, eps)
    else:
        dy_last, dg_final = dhf, None
    return dict(loss_partials=partials, loss=scale * partials.sum(), argmax=argmax,
                dy_last=dy_last, dg_final=dg_final, dw_lm=dw_lm, logits=z)


def global_clip(grads, max_norm):
    """One L2 norm over every gradient: N = sqrt(sum g^2); scale
    c = max_norm / N when N > max_norm, else 1; every gradient times c.

    cuda_trainer.rs page, the squared-sum clip helper (host fp64 sum of the
    squared-sum partials, square root, then max_norm / norm above the limit).
    The reading taken: a single global norm over all trainable gradients of
    the step, without the +1e-6 of the LoRA workspace clip.
    Returns (norm, scale, clipped grads).
    """
    total = 0.0
    for g in grads:
        g = np.asarray(g, np.float64)
        total += float(np.sum(g * g))
    norm = np.sqrt(total)
    scale = max_norm / norm if norm > max_norm else 1.0
    return norm, scale, [np.asarray(g, np.float64) * scale for g in grads]


def adamw_update(w, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """One AdamW step (decoupled weight decay, bias correction, eps outside
    the square root; decay uses the weight before the step).

    cuda_block.rs page, ``optimizer_step`` (``adamw_step_cuda`` on every block
    tensor, norm weights included, with step > 0 for the bias adjustment);
    the formula itself is not printed: this is Loshchilov and Hutter's AdamW.
    m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2; mh = m/(1-b1^t); vh = v/(1-b2^t);
    w = w - lr * (mh / (sqrt(vh) + eps) + weight_decay * w).
    Returns (w, m, v).
    """
    w, g, m, v = (np.asarray(a, np.float64) for a in (w, g, m, v))
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mh = m / (1.0 - beta1 ** step)
    vh = v / (1.0 - beta2 ** step)
    w_new = w - lr * (mh / (np.sqrt(vh) + eps) + weight_decay * w)
    return w_new, m, v


def stack_step(c, layers, x, g_final, w_lm, targets, max_norm, adamw, step=1):
    """One training step of a stack of blocks with the LM head.

    cuda_trainer.rs page, ``train_step_inner``: ``gpu_forward`` over every
    block, fused cross-entropy, ``gpu_backward`` in reverse block order. The
    reading taken for the optimizer: one global clip over every gradient
    (all block tensors, the final-norm gamma and the LM head) before any
    AdamW, then AdamW on every tensor with zero initial moments.
    Returns a dict with the loss, per-token partials, the norm, the clip
    scale, the updated parameters and moments, and whether the guard
    against non-finite values skipped the update.
    """
    eps = c["eps"] if isinstance(c, dict) else c.eps
    h = np.asarray(x, np.float64)
    caches = []
    for p in layers:
        h, ch = block_forward(c, p, h)
        caches.append(ch)
    ce = lm_head_cross_entropy(h, g_final, w_lm, targets, eps)
    dh = ce["dy_last"]
    layer_grads = [None] * len(layers)
    for li in range(len(layers) - 1, -1, -1):
        dh, layer_grads[li] = block_backward(c, layers[li], caches[li], dh)
    flat = []
    for gr in layer_grads:
        flat += [gr[n] for n in PARAM_NAMES]
    flat += [ce["dg_final"], ce["dw_lm"]]
    norm, scale, clipped = global_clip(flat, max_norm)
    params = []
    for p in layers:
        params += [p[n] for n in PARAM_NAMES]
    params += [g_final, w_lm]
    # The trainer's guard (same page, train_step_inner): a non-finite loss
    # ends the step before the optimizer, and its accumulated-gradient path
    # skips the optimizer when any gradient is NaN or infinite; either way
    # the parameters and moments stay as they were.
    skipped = not (np.isfinite(ce["loss"]) and all(np.all(np.isfinite(g)) for g in flat))
    new_w, new_m, new_v = [], [], []
    for w, g in zip(params, clipped):
        z = np.zeros(np.shape(w))
        if skipped:
            w2, m2, v2 = np.array(w, np.float64), z, z
        else:
            w2, m2, v2 = adamw_update(w, g, z, z, step=step, **adamw)
        new_w.append(w2)
        new_m.append(m2)
        new_v.append(v2)
    return dict(loss=ce["loss"], loss_partials=ce["loss_partials"], argmax=ce["argmax"],
                norm=norm, scale=scale, grads=flat, new_w=new_w, new_m=new_m, new_v=new_v,
                dx=dh, skipped=skipped)
