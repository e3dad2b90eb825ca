/*
 * qblk_ops.h — single-step entry points of libqblk, exported for step-level
 * parity tests and measurement. Each runs one step of the block path with
 * the same kernels the block entry points use. Conventions are those of
 * qblk.h (device pointers owned by the caller, row-major, return codes).
 */
#ifndef QBLK_OPS_H
#define QBLK_OPS_H

#include "qblk.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Dense contraction on MFMA ([block] gemm_forward, gemm_backward_a,
 * gemm_backward_b): layout 0 NT: C[M,N] = A[M,K] B[N,K]^T;
 * 1 NN: C = A[M,K] B[K,N]; 2 TN: C = A[K,M]^T B[K,N]. All fp32 row-major
 * with leading dimensions lda/ldb/ldc (elements). precision 0: fp32
 * contraction; 1: operands rounded to fp16 (nearest even), fp32 accumulate.
 * With accumulate = 1, C += result. The contiguous dimension of each
 * operand must be a multiple of 4. `scratch` (optional, may be NULL) lets
 * a long-K, few-tile product split K over more workgroups; its useful size
 * comes from qblk_gemm_workspace_size (a smaller one disables the split).
 * Results do not depend on whether the split is taken beyond fp32
 * rounding order, and are bitwise reproducible for a given scratch size. */
int32_t qblk_gemm(int32_t layout, int32_t precision, int32_t M, int32_t N, int32_t K,
                  const float* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                  int32_t accumulate, void* scratch, size_t scratch_bytes, qblk_stream_t stream);

/* Split-K scratch bytes for this shape, enough whichever storage type
 * (fp32 or fp16) the operands are given in. */
int32_t qblk_gemm_workspace_size(int32_t layout, int32_t precision, int32_t M, int32_t N, int32_t K,
                                 size_t* scratch_bytes);

/* qblk_gemm with the storage type of each operand given: a_dtype/b_dtype
 * 0 = fp32, 1 = fp16 (IEEE binary16), 2 = bfloat16. 16-bit storage is how
 * the block keeps activations that only feed contractions. precision 2
 * (bfloat16 operands, fp32 accumulate) takes bfloat16 storage of both
 * operands, K a multiple of 64 and 16-byte aligned rows (the direct-to-LDS
 * kernels), else QBLK_EUNSUPPORTED. */
int32_t qblk_gemm_ex(int32_t layout, int32_t precision, int32_t M, int32_t N, int32_t K, const void* A,
                     int64_t lda, int32_t a_dtype, const void* B, int64_t ldb, int32_t b_dtype, float* C,
                     int64_t ldc, int32_t accumulate, void* scratch, size_t scratch_bytes,
                     qblk_stream_t stream);

/* 8-bit floating-point operands (the 8-bit counterpart of [block]'s
 * fp16 GEMM tier and set_fp16_weights copies; the formats are those of the
 * OCP 8-bit floating point specification: E4M3 with largest finite 448,
 * no infinities; E5M2 with largest finite 57344).
 *
 * qblk_fp8_quantize: per-tensor scaled conversion of an fp32 matrix x
 * [rows, cols] (row stride ldx elements) into q [rows, cols] bytes (row
 * stride ldq), E4M3 (e5m2 = 0) or E5M2 (e5m2 = 1):
 *   s = FMAX / max|x| (fp32, correctly rounded; 1 if x is all zero),
 *   q = round_to_nearest_even(clamp(fp32(x * s), -FMAX, FMAX)),
 * and inv_scale_dev[0] = 1 / s (device fp32). A NaN element stays NaN;
 * infinite inputs are outside the contract. scratch: device memory of
 * qblk_fp8_quantize_workspace_size bytes (the partial maxima). Two
 * launches on `stream`, no host synchronisation. */
int32_t qblk_fp8_quantize_workspace_size(int32_t rows, int32_t cols, size_t* scratch_bytes);
int32_t qblk_fp8_quantize(int32_t rows, int32_t cols, const float* x, int64_t ldx, int32_t e5m2, uint8_t* q,
                          int64_t ldq, float* inv_scale_dev, void* scratch, size_t scratch_bytes,
                          qblk_stream_t stream);

/* fp8 contraction on v_mfma_f32_32x32x64_f8f6f4, fp32 accumulate:
 *   C[M, N] (+)= (A8[M, K] B8[N, K]^T) * a_inv_scale[0] * b_inv_scale[0]
 * A8, B8 row-major bytes (K contiguous, strides lda / ldb >= K, multiples
 * of 16, 16-byte aligned), each E4M3 or E5M2 (a_e5m2 / b_e5m2); the two
 * scales are device fp32 scalars (NULL: 1), as qblk_fp8_quantize leaves
 * them. K a multiple of 128 (else QBLK_EINVAL). C fp32 [M, ldc]; with
 * accumulate = 1, C += result. `scratch` (optional) enables split K; its
 * useful size comes from qblk_gemm_fp8_workspace_size. */
int32_t qblk_gemm_fp8_workspace_size(int32_t M, int32_t N, int32_t K, size_t* scratch_bytes);
int32_t qblk_gemm_fp8(int32_t M, int32_t N, int32_t K, const uint8_t* A, int64_t lda, int32_t a_e5m2,
                      const uint8_t* B, int64_t ldb, int32_t b_e5m2, const float* a_inv_scale,
                      const float* b_inv_scale, float* C, int64_t ldc, int32_t accumulate, void* scratch,
                      size_t scratch_bytes, qblk_stream_t stream);

/* RMSNorm forward over rows of x [rows, n] ([block] rms_norm_forward):
 * y = x * rho * gamma with rho[r] = (mean x^2 + eps)^(-1/2) written to rho.
 * When `res` is not NULL, x is first replaced by x + res and that sum is
 * written to `sum_out` ([block] fused residual + RMSNorm). */
int32_t qblk_rmsnorm_forward(int32_t rows, int32_t n, float eps, const float* x, const float* res,
                             const float* gamma, float* y, float* sum_out, float* rho,
                             void* scratch, size_t scratch_bytes, qblk_stream_t stream);

/* RMSNorm backward ([block] rms_norm_backward): dx = rho (e - xhat
 * mean(e xhat)), e = gamma dy, plus `dres` when not NULL (the residual
 * gradient); dgamma = sum over rows of dy xhat (overwritten; deterministic
 * two-stage reduction in scratch). */
int32_t qblk_rmsnorm_backward(int32_t rows, int32_t n, float eps, const float* x,
                              const float* gamma, const float* dy, const float* dres, float* dx,
                              float* dgamma, void* scratch, size_t scratch_bytes,
                              qblk_stream_t stream);

/* Scratch bytes for the RMSNorm entry points above. */
int32_t qblk_rmsnorm_workspace_size(int32_t rows, int32_t n, size_t* scratch_bytes);

/* SwiGLU ([block] fused_swiglu_forward): s [T, I] = silu(g) * u with
 * g = gu[:, :I], u = gu[:, I:] of gu [T, 2I] (fp32, dense). I a multiple
 * of 4; buffers 16-byte aligned. */
int32_t qblk_swiglu_forward(int32_t tokens, int32_t inter, const float* gu, float* s, qblk_stream_t stream);

/* Its backward ([block] SwiGLU backward; [wgpu] ffn_backward):
 * dgu = [ds * u * silu'(g) | ds * silu(g)], silu'(g) = sigmoid(g) (1 + g
 * (1 - sigmoid(g))). dgu [T, 2I] overwritten. */
int32_t qblk_swiglu_backward(int32_t tokens, int32_t inter, const float* gu, const float* ds, float* dgu,
                             qblk_stream_t stream);

/* Scratch bytes of the two QK-norm + RoPE entry points below (the RoPE
 * table and the gamma-gradient partial sums). */
int32_t qblk_qk_norm_rope_workspace_size(int32_t tokens, int32_t seq, int32_t heads, int32_t kv_heads,
                                         int32_t head_dim, size_t* scratch_bytes);

/* Per-head RMSNorm of q and k (when qk_norm; gammas g_q, g_k [head_dim]
 * shared by the heads) then NeoX RoPE at position s = t % seq with angle
 * s * theta^(-2i/head_dim) ([block] compute_attention_cuda). qkv [T,
 * ld_qkv] holds q | k | v (heads, kv_heads, kv_heads heads of head_dim);
 * writes qr [T, heads*d], kr [T, kv_heads*d] (dense), rho_q [T, heads],
 * rho_k [T, kv_heads] (the inverse RMS, when qk_norm). */
int32_t qblk_qk_norm_rope_forward(int32_t tokens, int32_t seq, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                  int32_t qk_norm, float eps, float rope_theta, const float* qkv, int64_t ld_qkv,
                                  const float* g_q, const float* g_k, float* qr, float* kr, float* rho_q,
                                  float* rho_k, void* scratch, size_t scratch_bytes, qblk_stream_t stream);

/* Its backward: from dqr, dkr (gradients at the attention inputs) the
 * gradients at the projection outputs, written into the q and k columns of
 * dqkv [T, ld_qkv] (v columns untouched), and dg_q, dg_k [head_dim]
 * (overwritten; zero without qk_norm). The QK-norm backward is the true
 * derivative (absent on the page). */
int32_t qblk_qk_norm_rope_backward(int32_t tokens, int32_t seq, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                   int32_t qk_norm, float eps, float rope_theta, const float* qkv, int64_t ld_qkv,
                                   const float* g_q, const float* g_k, const float* dqr, const float* dkr,
                                   float* dqkv, float* dg_q, float* dg_k, void* scratch, size_t scratch_bytes,
                                   qblk_stream_t stream);

/* GQA causal softmax attention forward over q [T, heads*d], k, v
 * [T, kv_heads*d] (rows strided by ldq/ldk/ldv elements) for `batch`
 * independent sequences of length seq: o [T, heads*d] (ldo) and the
 * row log-sum-exp lse [batch, heads, seq] (natural log, of the scaled
 * scores). precision as in qblk_gemm. */
int32_t qblk_attention_forward(int32_t batch, int32_t seq, int32_t heads, int32_t kv_heads,
                               int32_t head_dim, int32_t precision, const float* q, int64_t ldq,
                               const float* k, int64_t ldk, const float* v, int64_t ldv, float* o,
                               int64_t ldo, float* lse, qblk_stream_t stream);

/* Attention backward: given q, k, v, o, lse of the forward and do, writes
 * dq [T, heads*d], dk, dv [T, kv_heads*d] (overwritten; dk and dv summed
 * over the heads that share a KV head). scratch: qblk_attention_workspace_size. */
int32_t qblk_attention_backward(int32_t batch, int32_t seq, int32_t heads, int32_t kv_heads,
                                int32_t head_dim, int32_t precision, const float* q, int64_t ldq,
                                const float* k, int64_t ldk, const float* v, int64_t ldv,
                                const float* o, int64_t ldo, const float* lse, const float* d_o,
                                int64_t lddo, float* dq, int64_t lddq, float* dk, int64_t lddk,
                                float* dv, int64_t lddv, void* scratch, size_t scratch_bytes,
                                qblk_stream_t stream);

int32_t qblk_attention_workspace_size(int32_t batch, int32_t seq, int32_t heads,
                                      size_t* scratch_bytes);

/* The attention the fp16-operand block runs (head_dim 64 or 128, seq a
 * multiple of 8), on fp16 (IEEE half) copies of its inputs, all dense
 * row-major: q16 [T, heads*d], k16, v16 [T, kv_heads*d]. Writes o
 * [T, heads*d] (fp32) and lse [batch, heads, seq]. Same computation as
 * qblk_attention_forward with precision 1. */
int32_t qblk_attention_forward_f16(int32_t batch, int32_t seq, int32_t heads, int32_t kv_heads,
                                   int32_t head_dim, const void* q16, const void* k16,
                                   const void* v16, float* o, float* lse, qblk_stream_t stream);

/* Its backward: fp16 copies q16, k16, v16 and do16 [T, heads*d]; fp32 o and
 * do32 (for rowsum(dO o)) and the forward's lse. Writes dq, dk, dv (fp32,
 * dense, overwritten; dk and dv summed over each KV group). scratch:
 * qblk_attention_workspace_size bytes. */
int32_t qblk_attention_backward_f16(int32_t batch, int32_t seq, int32_t heads, int32_t kv_heads,
                                    int32_t head_dim, const void* q16, const void* k16,
                                    const void* v16, const float* o, const float* lse,
                                    const void* do16, const float* do32, float* dq, float* dk,
                                    float* dv, void* scratch, size_t scratch_bytes,
                                    qblk_stream_t stream);

/* Cross-entropy over materialised logits z [tokens, vocab] (fp32, row
 * stride vocab), in place ([trainer] fused_cross_entropy_cuda):
 * loss_partials[t] = logsumexp(z_t) - z_t[targets[t]]; argmax[t] = first
 * index of the row maximum (NULL: skipped); z_t is overwritten with
 * loss_scale * (softmax(z_t) - onehot(targets[t])). A target outside
 * [0, vocab) yields a NaN partial and no onehot term. */
int32_t qblk_cross_entropy_rows(int32_t tokens, int32_t vocab, float* z, const int32_t* targets,
                                float loss_scale, float* loss_partials, int32_t* argmax,
                                qblk_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QBLK_OPS_H */
