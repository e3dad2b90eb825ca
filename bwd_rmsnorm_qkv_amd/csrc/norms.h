// Internal interface of the memory-bound kernels: RMSNorm, QK-norm + RoPE,
// SwiGLU, and the column-sum used by every deterministic gamma gradient.
#pragma once

#include "common.h"

namespace qblk {

int rmsnorm_check(int rows, int n);
int rmsnorm_bwd_parts(int rows, int n);
size_t rmsnorm_bwd_scratch(int rows, int n);

// y (fp32) and/or y16 (fp16) = RMSNorm(x [+ res]) * gamma; sum_out = x + res.
// With `tab` the same launch also writes that RoPE table.
struct RopeTabJob;
// bf16: the 16-bit copies (y16, dx16, s16, ...) of every producer below hold
// bfloat16 instead of fp16.
int rmsnorm_forward(int rows, int n, float eps, const float* x, const float* res,
                    const float* gamma, float* y, f16* y16, float* sum_out, float* rho,
                    hipStream_t st, const RopeTabJob* tab = nullptr, bool bf16 = false);
// dx = RMSNorm backward (+ dres); dgamma overwritten; scratch: rmsnorm_bwd_scratch.
int rmsnorm_backward(int rows, int n, float eps, const float* x, const float* gamma,
                     const float* dy, const float* dres, float* dx, f16* dx16, float* dgamma, float* scratch,
                     hipStream_t st, bool bf16 = false);
// The same, leaving dgamma's per-block partial sums ([rmsnorm_bwd_parts,
// n]) in `partial` for a later column sum.
int rmsnorm_backward_partials(int rows, int n, float eps, const float* x, const float* gamma, const float* dy,
                              const float* dres, float* dx, f16* dx16, float* partial, hipStream_t st,
                              bool bf16 = false);
// out[c] = sum_p partial[p][c], fixed order.
int colsum(int parts, int n, const float* partial, float* out, hipStream_t st);
// Up to four such sums in one launch.
struct ColsumJob {
  int parts, n;
  const float* partial;
  float* out;
  int accumulate = 0;  // 1: out[c] += the sum
};
constexpr int kMaxColsumJobs = 4;
int colsum_jobs(int njobs, const ColsumJob* jobs, hipStream_t st);

// RoPE table: tab[s][i] = (cos, sin)(s * theta^(-2i/d)), computed in fp64.
int rope_table(int seq, int head_dim, float theta, float2* tab, hipStream_t st);
// The same table as extra workgroups of another launch (it depends on no
// other data): entry idx < seq * half of the job.
struct RopeTabJob {
  int seq = 0, half = 0, d = 0;
  double log_theta = 0.0;
  float2* tab = nullptr;
};
RopeTabJob rope_table_job(int seq, int head_dim, float theta, float2* tab);
__device__ __forceinline__ void rope_entry(const RopeTabJob& j, int idx) {
  if (idx >= j.seq * j.half) return;
  const int s = idx / j.half, i = idx % j.half;
  const double f = exp(-2.0 * (double)i / (double)j.d * j.log_theta);
  const double a = (double)s * f;
  j.tab[idx] = make_float2((float)cos(a), (float)sin(a));
}

// Per-head RMSNorm (optional) + NeoX RoPE of the q and k heads of a packed
// [T, (H + 2KV) d] projection output. Writes qr [T, H d], kr [T, KV d]
// (fp32), rho_q [T, H], rho_k [T, KV] (when qk_norm).
struct QkRopeArgs {
  int T, seq, heads, kv_heads, head_dim, qk_norm;
  float eps;
  const float* qkv;  // [T, ld_qkv]
  int64_t ld_qkv;
  const float *g_q, *g_k;
  const float2* tab;
  float *qr, *kr, *rho_q, *rho_k;  // qr, kr may be null (fp16 outputs only)
  // optional fp16 copies of the attention operands [T, heads d] and
  // [T, kv_heads d] (v16 copies V from qkv unchanged)
  f16 *q16 = nullptr, *k16 = nullptr, *v16 = nullptr;
  int bf16 = 0;  // the 16-bit copies hold bfloat16
};
int qk_norm_rope_forward(const QkRopeArgs& a, hipStream_t st);

// Backward: dqr/dkr (gradients at the attention inputs) -> dq/dk at the
// projection outputs, written into dqkv (same packing as qkv), and
// dg_q/dg_k (overwritten). scratch: qk_norm_rope_bwd_scratch floats.
struct QkRopeBwdArgs {
  int T, seq, heads, kv_heads, head_dim, qk_norm;
  float eps;
  const float* qkv;
  int64_t ld_qkv;
  const float *g_q, *g_k;
  const float2* tab;
  const float *dqr, *dkr;  // [T, H d], [T, KV d]
  float* dqkv;             // [T, ld_qkv] (may be null)
  float *dg_q, *dg_k;
  f16* dqkv16 = nullptr;   // optional fp16 copy of the q and k columns of dqkv
  int accumulate_dg = 0;   // 1: dg_q, dg_k receive += (and stay as they are without QK-norm)
  int bf16 = 0;            // dqkv16 holds bfloat16
};
size_t qk_norm_rope_bwd_scratch(int T, int heads, int kv_heads, int head_dim);
int qk_norm_rope_backward(const QkRopeBwdArgs& a, float* scratch, hipStream_t st);
// The same with dg_q, dg_k left as per-block partial sums in `scratch`;
// `jobs` receives the column sums that finish them (none without QK-norm,
// when dg_q and dg_k are zero-filled here).
int qk_norm_rope_backward_partials(const QkRopeBwdArgs& a, float* scratch, ColsumJob* jobs, int& njobs,
                                   hipStream_t st);

// s = silu(g) * u with g, u the two halves of gu [T, 2I]; s fp32 and/or fp16.
int swiglu_forward(int T, int I, const float* gu, float* s, f16* s16, hipStream_t st, bool bf16 = false);
// dgu = [ds * u * silu'(g) | ds * silu(g)].
int swiglu_backward(int T, int I, const float* gu, const float* ds, float* dgu, f16* dgu16, hipStream_t st,
                    bool bf16 = false);

// fp16 copies of an fp32 matrix in [R, C] (row stride ldi): out [R, C]
// (stride ldo) and/or outT [C, R] (stride ldt); either may be NULL.
// C and every stride must be multiples of 4.
int cast_f16(int R, int C, const float* in, int64_t ldi, f16* out, int64_t ldo, f16* outT, int64_t ldt,
             hipStream_t st, bool bf16 = false);

}  // namespace qblk
