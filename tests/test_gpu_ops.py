"""Step-level parity on the GPU: each single-step entry point of libqblk
against the CPU oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from oracle import ops
from bwd_rmsnorm_qkv_amd import qblk
from bwd_rmsnorm_qkv_amd.runtime import dev, empty, byte_buffer
from gpu_util import BF16_TOL, FP16_TOL, FP32_TOL, announce, check, need_gpu

pytestmark = pytest.mark.gpu

# (M, N, K): several tiles plus ragged tails in every dimension
GEMM_SHAPES = [(32, 64, 64), (200, 136, 104), (300, 392, 260), (37, 20, 12),
               (64, 96, 4096), (520, 264, 3000)]   # long K: split over workgroups


@pytest.mark.parametrize("precision", [0, 1])
@pytest.mark.parametrize("layout", [0, 1, 2])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm(layout, precision, shape):
    need_gpu()
    M, N, K = shape
    announce(f"gemm layout={layout} precision={precision} M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    if layout == 2 and M % 4:
        pytest.skip("TN needs M % 4 == 0")
    a_shape = (M, K) if layout in (0, 1) else (K, M)
    b_shape = (N, K) if layout == 0 else (K, N)
    A = rng.standard_normal(a_shape).astype(np.float32)
    B = rng.standard_normal(b_shape).astype(np.float32)
    Cref = (A.astype(np.float64) if layout != 2 else A.astype(np.float64).T) @ \
           (B.astype(np.float64).T if layout == 0 else B.astype(np.float64))
    dA, dB = dev(A), dev(B)
    Cg = torch.full((M, N), 7.0, device="cuda")
    ws = qblk.gemm_workspace_size(layout, precision, M, N, K)
    scratch = byte_buffer(ws) if ws else None
    qblk.gemm(layout, precision, M, N, K, dA, a_shape[1], dB, b_shape[1], Cg, N, scratch=scratch)
    torch.cuda.synchronize()
    check("C", Cg, Cref, FP16_TOL if precision else FP32_TOL)
    # accumulate mode adds to the existing C
    qblk.gemm(layout, precision, M, N, K, dA, a_shape[1], dB, b_shape[1], Cg, N, accumulate=1, scratch=scratch)
    torch.cuda.synchronize()
    check("C+C", Cg, 2 * Cref, FP16_TOL if precision else FP32_TOL)
    if ws:
        # without the workspace the same product runs unsplit
        C1 = torch.empty((M, N), device="cuda")
        qblk.gemm(layout, precision, M, N, K, dA, a_shape[1], dB, b_shape[1], C1, N)
        torch.cuda.synchronize()
        check("C unsplit", C1, Cref, FP16_TOL if precision else FP32_TOL)


# fp32 products with K a multiple of 32 and 16-byte rows run on the
# direct-to-LDS kernel: 128 x 128 tiles with two rounds of workgroups or
# >= 4096 K per workgroup, 64 x 64 tiles otherwise; ragged M and N, K
# splits, all three layouts (NN and TN read M/N-contiguous fp32 tiles);
# layout, M, N, K
GEMM32_DMA_SHAPES = [(0, 2048, 4096, 96), (2, 2048, 4096, 96), (1, 264, 520, 73728),  # 128 x 128
                     (0, 1000, 2952, 96), (0, 1288, 2056, 1408), (1, 1000, 2952, 96), (1, 1024, 512, 2816),
                     (2, 1000, 2952, 96), (2, 2816, 512, 1024), (2, 520, 1400, 1024), (0, 72, 40, 64)]


@pytest.mark.parametrize("layout,M,N,K", GEMM32_DMA_SHAPES)
def test_gemm_fp32_direct(layout, M, N, K):
    need_gpu()
    announce(f"gemm fp32 direct-to-LDS layout={layout} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 5 * N + 11 * K + layout)
    a_shape = (M, K) if layout in (0, 1) else (K, M)
    b_shape = (N, K) if layout == 0 else (K, N)
    A = rng.standard_normal(a_shape).astype(np.float32)
    B = rng.standard_normal(b_shape).astype(np.float32)
    Cref = (A.astype(np.float64) if layout != 2 else A.astype(np.float64).T) @ \
           (B.astype(np.float64).T if layout == 0 else B.astype(np.float64))
    dA, dB = dev(A), dev(B)
    Cg = torch.full((M, N), 7.0, device="cuda")
    ws = qblk.gemm_workspace_size(layout, 0, M, N, K)
    scratch = byte_buffer(ws) if ws else None
    qblk.gemm(layout, 0, M, N, K, dA, a_shape[1], dB, b_shape[1], Cg, N, scratch=scratch)
    torch.cuda.synchronize()
    check("C", Cg, Cref, FP32_TOL)
    qblk.gemm(layout, 0, M, N, K, dA, a_shape[1], dB, b_shape[1], Cg, N, accumulate=1, scratch=scratch)
    torch.cuda.synchronize()
    check("C+C", Cg, 2 * Cref, FP32_TOL)
    if ws:
        # without the workspace: unsplit, on whichever kernel then applies
        C1 = torch.empty((M, N), device="cuda")
        qblk.gemm(layout, 0, M, N, K, dA, a_shape[1], dB, b_shape[1], C1, N)
        torch.cuda.synchronize()
        check("C unsplit", C1, Cref, FP32_TOL)


# fp16-stored operands: K a multiple of 64 takes the NT direct-to-LDS kernel,
# the others the general one
GEMM16_SHAPES = [(200, 136, 128), (37, 24, 64), (300, 392, 256), (130, 130, 192),
                 (64, 96, 4096), (520, 264, 3008), (520, 264, 3000), (72, 40, 104)]


@pytest.mark.parametrize("storage", ["h16", "f32h16", "h16f32"])
@pytest.mark.parametrize("layout", [0, 1, 2])
@pytest.mark.parametrize("shape", GEMM16_SHAPES)
def test_gemm_fp16_storage(layout, storage, shape):
    """Operands held as IEEE half. Both sides contract the same fp16 values
    (fp32 operands are rounded to nearest even), so the only difference is
    fp32 accumulation order: the fp32 tolerance applies."""
    need_gpu()
    M, N, K = shape
    announce(f"gemm16 layout={layout} storage={storage} M={M} N={N} K={K}")
    a_cont = K if layout in (0, 1) else M
    b_cont = K if layout == 0 else N
    if (storage != "f32h16" and a_cont % 8) or (storage != "h16f32" and b_cont % 8) or a_cont % 4 or b_cont % 4:
        pytest.skip("fp16 operands need their contiguous dimension a multiple of 8")
    rng = np.random.default_rng(M * 5 + N * 11 + K)
    a_shape = (M, K) if layout in (0, 1) else (K, M)
    b_shape = (N, K) if layout == 0 else (K, N)
    A = rng.standard_normal(a_shape).astype(np.float32)
    B = rng.standard_normal(b_shape).astype(np.float32)
    A16 = A.astype(np.float16)
    B16 = B.astype(np.float16)
    a64 = A16.astype(np.float64)
    b64 = B16.astype(np.float64)
    Cref = (a64 if layout != 2 else a64.T) @ (b64.T if layout == 0 else b64)
    dA = dev(A16) if storage in ("h16", "h16f32") else dev(A)
    dB = dev(B16) if storage in ("h16", "f32h16") else dev(B)
    ws = qblk.gemm_workspace_size(layout, 1, M, N, K)
    scratch = byte_buffer(ws) if ws else None
    Cg = torch.full((M, N), 3.0, device="cuda")
    qblk.gemm(layout, 1, M, N, K, dA, a_shape[1], dB, b_shape[1], Cg, N, scratch=scratch)
    torch.cuda.synchronize()
    check("C", Cg, Cref, FP32_TOL)
    qblk.gemm(layout, 1, M, N, K, dA, a_shape[1], dB, b_shape[1], Cg, N, accumulate=1, scratch=scratch)
    torch.cuda.synchronize()
    check("C+C", Cg, 2 * Cref, FP32_TOL)


# fp16 operands with enough output tiles for the 256-row tiles (256 x 192
# for NT when that takes fewer rounds over the CUs, with a third B stage):
# one to five K tiles (every prologue/tail case of the copy pipeline), a
# ragged N, a ragged M, a 128-tile product that splits K, and a weight-
# gradient shape whose big tiles would underfill their last round (it
# takes the small tiles)
GEMM16_BIG = [(0, 512, 16376, 64), (0, 512, 16376, 128), (0, 512, 16376, 192), (0, 512, 16376, 256),
              (0, 512, 16376, 320), (0, 520, 16376, 256), (1, 512, 16384, 1024), (2, 4096, 4096, 64),
              (2, 4096, 4088, 192), (2, 2560, 9728, 128)]


@pytest.mark.parametrize("layout,M,N,K", GEMM16_BIG)
def test_gemm_fp16_big_tiles(layout, M, N, K):
    need_gpu()
    announce(f"gemm16 big layout={layout} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 3 * N + 7 * K + layout)
    a_shape = (M, K) if layout in (0, 1) else (K, M)
    b_shape = (N, K) if layout == 0 else (K, N)
    A16 = rng.standard_normal(a_shape).astype(np.float16)
    B16 = rng.standard_normal(b_shape).astype(np.float16)
    a64, b64 = A16.astype(np.float64), B16.astype(np.float64)
    Cref = (a64 if layout != 2 else a64.T) @ (b64.T if layout == 0 else b64)
    ws = qblk.gemm_workspace_size(layout, 1, M, N, K)
    scratch = byte_buffer(ws) if ws else None
    Cg = torch.full((M, N), 3.0, device="cuda")
    qblk.gemm(layout, 1, M, N, K, dev(A16), a_shape[1], dev(B16), b_shape[1], Cg, N, scratch=scratch)
    torch.cuda.synchronize()
    check("C", Cg, Cref, FP32_TOL)


# (512, 2560), (5, 4096), (3000, 1028): one workgroup per row (run of rows), the
# last with more rows than partials; (4100, 1024) and the narrow rows: one wave per row
@pytest.mark.parametrize("rows,n", [(32, 64), (77, 512), (512, 2560), (5, 4096), (3000, 1028), (4100, 1024)])
def test_rmsnorm(rows, n):
    need_gpu()
    announce(f"rmsnorm rows={rows} n={n}")
    rng = np.random.default_rng(rows + n)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    r = rng.standard_normal((rows, n)).astype(np.float32)
    g = (1 + 0.2 * rng.standard_normal(n)).astype(np.float32)
    dy = rng.standard_normal((rows, n)).astype(np.float32)
    dr = rng.standard_normal((rows, n)).astype(np.float32)
    eps = 1e-6
    X, R, G, DY, DR = (dev(a) for a in (x, r, g, dy, dr))
    y, s, rho = empty((rows, n)), empty((rows, n)), empty(rows)
    qblk.rmsnorm_forward(rows, n, eps, X, R, G, y, s, rho)
    y_ref, rho_ref = ops.rmsnorm_fwd(x.astype(np.float64) + r, g, eps)
    torch.cuda.synchronize()
    check("y", y, y_ref, FP32_TOL)
    check("sum", s, x.astype(np.float64) + r, 1e-7)
    check("rho", rho, rho_ref, FP32_TOL)
    dx, dg = empty((rows, n)), empty(n)
    scratch = byte_buffer(qblk.rmsnorm_workspace_size(rows, n))
    qblk.rmsnorm_backward(rows, n, eps, X, G, DY, DR, dx, dg, scratch)
    dx_ref, dg_ref = ops.rmsnorm_bwd(x, g, dy, eps)
    torch.cuda.synchronize()
    check("dx", dx, dx_ref + dr, FP32_TOL)
    check("dgamma", dg, dg_ref, FP32_TOL)
    # deterministic: a second run is bitwise equal
    dg2 = empty(n)
    qblk.rmsnorm_backward(rows, n, eps, X, G, DY, DR, dx, dg2, scratch)
    torch.cuda.synchronize()
    assert torch.equal(dg, dg2)


ATTN_SHAPES = [  # batch, seq, heads, kv_heads, head_dim, precision
    (1, 32, 4, 2, 16, 0),
    (2, 45, 4, 2, 16, 0),
    (3, 100, 8, 2, 64, 0),
    (1, 160, 8, 8, 64, 0),
    (1, 130, 8, 2, 128, 1),
    (2, 96, 4, 1, 64, 1),
]


@pytest.mark.parametrize("shape", ATTN_SHAPES)
def test_attention(shape):
    need_gpu()
    B, S, H, KV, D, prec = shape
    announce(f"attention batch={B} seq={S} heads={H} kv={KV} d={D} prec={prec}")
    rng = np.random.default_rng(S * H + D)
    T = B * S
    q = rng.standard_normal((T, H * D)).astype(np.float32)
    k = rng.standard_normal((T, KV * D)).astype(np.float32)
    v = rng.standard_normal((T, KV * D)).astype(np.float32)
    do = rng.standard_normal((T, H * D)).astype(np.float32)
    Q, K_, V, DO = dev(q), dev(k), dev(v), dev(do)
    o, lse = empty((T, H * D)), empty(B * H * S)
    qblk.attention_forward(B, S, H, KV, D, prec, Q, H * D, K_, KV * D, V, KV * D, o, H * D, lse)
    o_ref = ops.attention_fwd(q, k, v, B, S, H, KV, D)
    tol = FP16_TOL if prec else FP32_TOL
    torch.cuda.synchronize()
    check("o", o, o_ref, tol)
    # lse against the definition
    lse_ref = np.zeros((B, H, S))
    for b in range(B):
        for h in range(H):
            g = h // (H // KV)
            s = q[b * S:(b + 1) * S, h * D:(h + 1) * D].astype(np.float64) @ \
                k[b * S:(b + 1) * S, g * D:(g + 1) * D].astype(np.float64).T / np.sqrt(D)
            s[np.triu_indices(S, 1)] = -np.inf
            m = s.max(1)
            lse_ref[b, h] = m + np.log(np.exp(s - m[:, None]).sum(1))
    assert np.max(np.abs(lse.cpu().numpy().reshape(B, H, S) - lse_ref)) < (5e-2 if prec else 1e-4)
    dq, dk, dv = empty((T, H * D)), empty((T, KV * D)), empty((T, KV * D))
    scratch = byte_buffer(qblk.attention_workspace_size(B, S, H))
    qblk.attention_backward(B, S, H, KV, D, prec, Q, H * D, K_, KV * D, V, KV * D, o, H * D, lse, DO, H * D,
                            dq, H * D, dk, KV * D, dv, KV * D, scratch)
    dq_ref, dk_ref, dv_ref = ops.attention_bwd(q, k, v, do, B, S, H, KV, D)
    torch.cuda.synchronize()
    check("dq", dq, dq_ref, tol)
    check("dk", dk, dk_ref, tol)
    check("dv", dv, dv_ref, tol)


ATTN16_SHAPES = [  # batch, seq, heads, kv_heads, head_dim: fp16 copies, direct-to-LDS tiles
    (1, 32, 4, 2, 64),
    (2, 96, 4, 1, 64),      # G = 4, several tiles per sequence
    (1, 144, 8, 2, 128),    # ragged last tile (144 = 4.5 tiles)
    (3, 40, 8, 8, 128),     # G = 1, ragged, batch > 1
    (1, 512, 32, 8, 128),   # the Qwen3-4B-shaped attention
    (1, 64, 8, 1, 64),      # G = 8: two dQ workgroups per group
    (1, 640, 24, 24, 64),   # tile pairs without a key-range split
    (2, 48, 12, 2, 64),     # G = 6: dQ workgroups of 3 waves
    # tile pairs x KV heads x batch >= 128: the forward shares each K/V tile
    # among the G query heads of its group (one wave per head)
    (1, 1024, 32, 8, 128),  # G = 4
    (2, 1024, 16, 8, 64),   # G = 2, batch > 1
    (1, 1000, 64, 8, 64),   # G = 8, ragged last tile
    # (tile, head) units >= 512, one key-range split, no group kernel: one
    # tile per 2-wave workgroup instead of causal tile pairs
    (1, 504, 32, 8, 64),    # G = 4, ragged last tile
    (2, 328, 24, 24, 128),  # G = 1, ragged, batch > 1
    (1, 1024, 16, 2, 64),   # G = 8
]


@pytest.mark.parametrize("shape", ATTN16_SHAPES)
def test_attention_f16(shape):
    """The fp16 kernels take fp16 copies; the oracle gets the same fp16
    values widened to float64. P and dS are rounded to fp16 inside, so the
    fp16-operand tolerance applies."""
    need_gpu()
    B, S, H, KV, D = shape
    announce(f"attention16 batch={B} seq={S} heads={H} kv={KV} d={D}")
    rng = np.random.default_rng(S * H + D + 1)
    T = B * S
    q, k, v, do = (rng.standard_normal((T, n * D)).astype(np.float16) for n in (H, KV, KV, H))
    q64, k64, v64, do64 = (x.astype(np.float64) for x in (q, k, v, do))
    o, lse = empty((T, H * D)), empty(B * H * S)
    qblk.attention_forward_f16(B, S, H, KV, D, dev(q), dev(k), dev(v), o, lse)
    o_ref = ops.attention_fwd(q64, k64, v64, B, S, H, KV, D)
    torch.cuda.synchronize()
    check("o", o, o_ref, FP16_TOL)
    dq, dk, dv = empty((T, H * D)), empty((T, KV * D)), empty((T, KV * D))
    scratch = byte_buffer(qblk.attention_workspace_size(B, S, H))
    # dO in fp32 for the row term; its fp16 copy for the products
    qblk.attention_backward_f16(B, S, H, KV, D, dev(q), dev(k), dev(v), o, lse, dev(do),
                                dev(do.astype(np.float32)), dq, dk, dv, scratch)
    dq_ref, dk_ref, dv_ref = ops.attention_bwd(q64, k64, v64, do64, B, S, H, KV, D)
    torch.cuda.synchronize()
    check("dq", dq, dq_ref, FP16_TOL)
    check("dk", dk, dk_ref, FP16_TOL)
    check("dv", dv, dv_ref, FP16_TOL)


def test_nf4_quantize_bit_exact():
    need_gpu()
    announce("nf4 quantize")
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((256, 320)) * 0.02).astype(np.float32)
    w[7, :64] = 0.0                        # zero block
    w[9, 64:128] = w[9, 64]                # constant block
    w[11, 0:64] = np.float32(0.0123)       # all equal positive
    packed, scales, _ = oracle.nf4_quantize(w)
    W = dev(w)
    codes = torch.empty(w.size // 2, dtype=torch.uint8, device="cuda")
    absmax = empty(w.size // 64)
    qblk.nf4_quantize(W, codes, absmax)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), packed)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), scales.view(np.uint32))
    deq = empty(w.size)
    qblk.nf4_dequantize(codes, absmax, w.size, deq)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(deq.cpu().numpy().reshape(w.shape),
                                  oracle.nf4_dequantize(packed, scales, w.shape).astype(np.float32))


@pytest.mark.parametrize("T,I", [(37, 176), (256, 1408), (512, 9728)])
def test_swiglu(T, I):
    need_gpu()
    announce(f"swiglu T={T} I={I}")
    rng = np.random.default_rng(T + I)
    gu = (rng.standard_normal((T, 2 * I)) * 2).astype(np.float32)
    ds = rng.standard_normal((T, I)).astype(np.float32)
    GU, DS = dev(gu), dev(ds)
    s, dgu = empty((T, I)), empty((T, 2 * I))
    qblk.swiglu_forward(T, I, GU, s)
    qblk.swiglu_backward(T, I, GU, DS, dgu)
    torch.cuda.synchronize()
    g, u = gu[:, :I].astype(np.float64), gu[:, I:].astype(np.float64)
    check("s", s, ops.swiglu_fwd(g, u), FP32_TOL)
    dg, du = ops.swiglu_bwd(g, u, ds.astype(np.float64))
    check("dg", dgu[:, :I], dg, FP32_TOL)
    check("du", dgu[:, I:], du, FP32_TOL)


# (batch, seq, heads, kv_heads, head_dim, qk_norm, theta)
QK_CASES = [(1, 32, 4, 2, 16, 1, 1e4), (3, 13, 4, 2, 16, 1, 1e4), (2, 48, 8, 2, 64, 1, 1e4),
            (2, 48, 8, 2, 64, 0, 1e4), (1, 37, 8, 2, 32, 1, 1e4), (1, 512, 32, 8, 128, 1, 1e6)]


@pytest.mark.parametrize("case", QK_CASES)
def test_qk_norm_rope(case):
    """QK-norm + RoPE forward and backward (the true QK-norm derivative)
    against the oracle's per-head RMSNorm and RoPE, with non-unit gammas and
    the v columns of the packed projection output left alone."""
    need_gpu()
    B, S, H, KV, d, qk, theta = case
    T = B * S
    announce(f"qk_norm_rope T={T} H={H} KV={KV} d={d} qk_norm={qk}")
    rng = np.random.default_rng(T * d + H)
    ld = (H + 2 * KV) * d
    qkv = rng.standard_normal((T, ld)).astype(np.float32)
    gq = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    gk = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    dqr = rng.standard_normal((T, H * d)).astype(np.float32)
    dkr = rng.standard_normal((T, KV * d)).astype(np.float32)
    eps = 1e-6
    QKV, GQ, GK = dev(qkv), dev(gq), dev(gk)
    qr, kr = empty((T, H * d)), empty((T, KV * d))
    rq, rk = empty((T, H)), empty((T, KV))
    scratch = byte_buffer(qblk.qk_norm_rope_workspace_size(T, S, H, KV, d))
    qblk.qk_norm_rope_forward(T, S, H, KV, d, qk, eps, theta, QKV, ld, GQ, GK, qr, kr, rq, rk, scratch)
    dqkv = torch.full((T, ld), 5.0, device="cuda")
    dgq, dgk = empty(d), empty(d)
    qblk.qk_norm_rope_backward(T, S, H, KV, d, qk, eps, theta, QKV, ld, GQ, GK, dev(dqr), dev(dkr), dqkv, dgq,
                               dgk, scratch)
    torch.cuda.synchronize()
    pos = np.tile(np.arange(S), B)
    q = qkv[:, :H * d].astype(np.float64)
    k = qkv[:, H * d:(H + KV) * d].astype(np.float64)
    if qk:
        qn, rho_q = ops.head_rmsnorm_fwd(q, gq, H, eps)
        kn, rho_k = ops.head_rmsnorm_fwd(k, gk, KV, eps)
        check("rho_q", rq, rho_q, FP32_TOL)
        check("rho_k", rk, rho_k, FP32_TOL)
    else:
        qn, kn = q, k
    check("qr", qr, ops.rope_fwd(qn, pos, H, theta), FP32_TOL)
    check("kr", kr, ops.rope_fwd(kn, pos, KV, theta), FP32_TOL)
    dqn = ops.rope_bwd(dqr.astype(np.float64), pos, H, theta)
    dkn = ops.rope_bwd(dkr.astype(np.float64), pos, KV, theta)
    if qk:
        dq, dg_q = ops.head_rmsnorm_bwd(q, gq, dqn, H, eps)
        dk, dg_k = ops.head_rmsnorm_bwd(k, gk, dkn, KV, eps)
        check("dg_q", dgq, dg_q, FP32_TOL)
        check("dg_k", dgk, dg_k, FP32_TOL)
    else:
        dq, dk = dqn, dkn
        assert torch.count_nonzero(dgq).item() == 0 and torch.count_nonzero(dgk).item() == 0
    out = dqkv.cpu().numpy()
    check("dq", out[:, :H * d], dq, FP32_TOL)
    check("dk", out[:, H * d:(H + KV) * d], dk, FP32_TOL)
    assert np.all(out[:, (H + KV) * d:] == 5.0), "v columns must be left alone"


# bfloat16 operands (precision 2): shapes the direct-to-LDS kernels take
# (K a multiple of 64), small and big tiles, split K, ragged M and N
GEMM_BF16_SHAPES = [(200, 136, 128), (300, 392, 256), (64, 96, 4096), (512, 2560, 4096), (512, 19456, 2560),
                    (2560, 9728, 512)]


@pytest.mark.parametrize("layout", [0, 1, 2])
@pytest.mark.parametrize("shape", GEMM_BF16_SHAPES)
def test_gemm_bf16(layout, shape):
    """The operands are rounded to bfloat16 on the host (torch, nearest
    even) and handed over as bfloat16 storage: the reference is the exact
    fp64 product of those same values, so the only difference is the fp32
    accumulation order (the fp32 tolerance applies). The fp32 originals
    against the same product stay within the bfloat16 tolerance."""
    need_gpu()
    M, N, K = shape
    if layout == 2 and M % 8:
        pytest.skip("TN needs M % 8 == 0")
    announce(f"gemm bf16 layout={layout} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 3 * N + 7 * K + layout)
    a_shape = (M, K) if layout in (0, 1) else (K, M)
    b_shape = (N, K) if layout == 0 else (K, N)
    A32 = torch.from_numpy(rng.standard_normal(a_shape).astype(np.float32))
    B32 = torch.from_numpy(rng.standard_normal(b_shape).astype(np.float32))
    A16, B16 = A32.to(torch.bfloat16), B32.to(torch.bfloat16)
    Ar, Br = A16.double().numpy(), B16.double().numpy()
    ref = (Ar if layout != 2 else Ar.T) @ (Br.T if layout == 0 else Br)
    ref32 = (A32.double().numpy() if layout != 2 else A32.double().numpy().T) @ \
            (B32.double().numpy().T if layout == 0 else B32.double().numpy())
    C = torch.full((M, N), 3.0, device="cuda")
    ws = qblk.gemm_workspace_size(layout, 2, M, N, K)
    scratch = byte_buffer(ws) if ws else None
    qblk.gemm(layout, 2, M, N, K, A16.cuda(), a_shape[1], B16.cuda(), b_shape[1], C, N, scratch=scratch)
    torch.cuda.synchronize()
    check("C (same bfloat16 inputs)", C, ref, FP32_TOL)
    check("C (fp32 originals)", C, ref32, BF16_TOL)


def test_gemm_bf16_needs_bf16_storage():
    need_gpu()
    A = torch.zeros((64, 64), device="cuda")
    with pytest.raises(qblk.QblkError):
        qblk.gemm(0, 2, 64, 64, 64, A, 64, A, 64, torch.empty((64, 64), device="cuda"), 64)
