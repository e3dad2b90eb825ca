// QK-norm + NeoX RoPE (forward and backward) and SwiGLU (forward and
// backward): the memory-bound steps between the projections and attention.
//
// cuda_block.rs page, compute_attention_cuda: per-head RMSNorm of Q and K
// with one gamma of size head_dim shared by the heads, applied before the
// NeoX half rotation with positions 0..seq-1 and rope_theta; backward_attention
// gives the inverse rotation for the backward. The page has no QK-norm
// backward; here it is the true derivative. SwiGLU is fused_swiglu_forward;
// its backward follows backward_ffn (and ffn_backward of the wgpu_trainer.rs
// page): dg = ds * u * silu'(g), du = ds * silu(g).
//
// One wave handles one (token, head) row of head_dim <= 128 elements: lane
// i < d/2 owns the rotation pair (i, i + d/2), so the norm's reduction and
// the rotation stay in registers. The cos/sin table is built once per call
// in fp64 and rounded to fp32.
#include "norms.h"

#include "../../include/qblk.h"

namespace qblk {
namespace {

__global__ void rope_table_kernel(const RopeTabJob j) { rope_entry(j, blockIdx.x * blockDim.x + threadIdx.x); }

// Forward: one wave per (t, head) over the H + KV heads (plus the KV value
// heads when their fp16 copy is requested).
__global__ __launch_bounds__(256) void qk_rope_fwd_kernel(QkRopeArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nqk = a.heads + a.kv_heads;
  const int nh = nqk + (a.v16 ? a.kv_heads : 0);
  if (item >= a.T * nh) return;
  const int t = item / nh, head = item % nh;
  const int d = a.head_dim, half = d >> 1;
  if (head >= nqk) {  // value head: fp16 copy only
    const int hh = head - nqk;
    const float* src = a.qkv + (int64_t)t * a.ld_qkv + (int64_t)nqk * d + hh * d;
    f16* dst = a.v16 + ((int64_t)t * a.kv_heads + hh) * d;
    for (int c = lane; c < d; c += 64) dst[c] = (f16)src[c];
    return;
  }
  const bool is_q = head < a.heads;
  const int hh = is_q ? head : head - a.heads;
  const int64_t orow = is_q ? ((int64_t)t * a.heads + hh) * d : ((int64_t)t * a.kv_heads + hh) * d;
  const float* src = a.qkv + (int64_t)t * a.ld_qkv + (is_q ? 0 : a.heads * d) + hh * d;
  float* dst = is_q ? a.qr : a.kr;
  f16* dst16 = is_q ? a.q16 : a.k16;
  const float* g = is_q ? a.g_q : a.g_k;
  const bool act = lane < half;
  const int li = act ? lane : 0;
  float x0 = src[li], x1 = src[li + half];
  const float2 cs = a.tab[(t % a.seq) * half + li];
  if (!act) x0 = x1 = 0.f;
  if (a.qk_norm) {
    const float ga = g[li], gb = g[li + half];
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float rho = 1.0f / sqrtf(ss / (float)d + a.eps);
    if (lane == 0) (is_q ? a.rho_q[(int64_t)t * a.heads + hh] : a.rho_k[(int64_t)t * a.kv_heads + hh]) = rho;
    x0 = x0 * rho * ga;
    x1 = x1 * rho * gb;
  }
  if (act) {
    const float o0 = x0 * cs.x - x1 * cs.y, o1 = x1 * cs.x + x0 * cs.y;
    if (dst) {
      dst[orow + lane] = o0;
      dst[orow + lane + half] = o1;
    }
    if (dst16) {
      dst16[orow + lane] = (f16)o0;
      dst16[orow + lane + half] = (f16)o1;
    }
  }
}

// Backward: blocks [0, nbq) take the q heads, the rest the k heads; each
// wave takes kQkRows consecutive (t, head) rows with all their loads issued
// before any arithmetic (rows past the end load the last row and are
// skipped). dgamma partials: one row per workgroup, in a fixed order.
constexpr int kQkRows = 8;

__global__ __launch_bounds__(256) void qk_rope_bwd_kernel(QkRopeBwdArgs a, int nbq, float* __restrict__ part_q,
                                                          float* __restrict__ part_k) {
  __shared__ float red[4][128];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool is_q = (int)blockIdx.x < nbq;
  const int blk = is_q ? blockIdx.x : blockIdx.x - nbq;
  const int nh = is_q ? a.heads : a.kv_heads;
  const int d = a.head_dim, half = d >> 1;
  const int col0 = is_q ? 0 : a.heads * d;
  const float* __restrict__ dsrc = is_q ? a.dqr : a.dkr;
  const float* __restrict__ g = is_q ? a.g_q : a.g_k;
  const bool act = lane < half;
  const int li = act ? lane : 0;
  const int rows = a.T * nh;
  const int r0 = (blk * 4 + w) * kQkRows;
  float y0[kQkRows], y1[kQkRows], x0[kQkRows], x1[kQkRows];
  float2 cs[kQkRows];
#pragma unroll
  for (int j = 0; j < kQkRows; ++j) {
    const int row = min(r0 + j, rows - 1), t = row / nh, hh = row % nh;
    y0[j] = dsrc[(int64_t)row * d + li];
    y1[j] = dsrc[(int64_t)row * d + li + half];
    cs[j] = a.tab[(t % a.seq) * half + li];
    if (a.qk_norm) {
      const float* xr = a.qkv + (int64_t)t * a.ld_qkv + col0 + hh * d;
      x0[j] = xr[li];
      x1[j] = xr[li + half];
    }
  }
  const float ga = a.qk_norm ? g[li] : 0.f, gb = a.qk_norm ? g[li + half] : 0.f;
  float dg0 = 0.f, dg1 = 0.f;
#pragma unroll
  for (int j = 0; j < kQkRows; ++j) {
    const int row = r0 + j;
    if (row >= rows) break;
    const int t = row / nh, hh = row % nh;
    // transpose of the rotation
    const float g0 = y0[j] * cs[j].x + y1[j] * cs[j].y;
    const float g1 = y1[j] * cs[j].x - y0[j] * cs[j].y;
    float o0 = g0, o1 = g1;
    if (a.qk_norm) {
      const float xa = act ? x0[j] : 0.f, xb = act ? x1[j] : 0.f;
      const float ss = wave_sum(xa * xa + xb * xb);
      const float rho = 1.0f / sqrtf(ss / (float)d + a.eps);
      const float xh0 = xa * rho, xh1 = xb * rho;
      const float e0 = act ? ga * g0 : 0.f, e1 = act ? gb * g1 : 0.f;
      const float dot = wave_sum(e0 * xh0 + e1 * xh1) / (float)d;
      o0 = rho * (e0 - xh0 * dot);
      o1 = rho * (e1 - xh1 * dot);
      if (act) {
        dg0 += g0 * xh0;
        dg1 += g1 * xh1;
      }
    }
    if (act) {
      const int64_t o = (int64_t)t * a.ld_qkv + col0 + hh * d + lane;
      if (a.dqkv) {
        a.dqkv[o] = o0;
        a.dqkv[o + half] = o1;
      }
      if (a.dqkv16) {
        a.dqkv16[o] = (f16)o0;
        a.dqkv16[o + half] = (f16)o1;
      }
    }
  }
  if (!a.qk_norm) return;
  if (act) {
    red[w][lane] = dg0;
    red[w][lane + half] = dg1;
  }
  __syncthreads();
  if (threadIdx.x < d) {
    const int c = threadIdx.x;
    (is_q ? part_q : part_k)[(int64_t)blk * d + c] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
  }
}

__global__ void fill_kernel(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

int qk_parts(int T, int nh) { return (int)ceil_div((int64_t)T * nh, 4 * kQkRows); }

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

__global__ void swiglu_fwd_kernel(int T, int I, const float* __restrict__ gu, float* __restrict__ s,
                                  f16* __restrict__ s16) {
  const int64_t n4 = (int64_t)T * I / 4;
  const int i4 = I / 4;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = e / i4, j = e % i4;
    const float4 g = ((const float4*)(gu + t * 2 * I))[j];
    const float4 u = ((const float4*)(gu + t * 2 * I + I))[j];
    float4 o;
    o.x = g.x * sigmoidf_(g.x) * u.x;
    o.y = g.y * sigmoidf_(g.y) * u.y;
    o.z = g.z * sigmoidf_(g.z) * u.z;
    o.w = g.w * sigmoidf_(g.w) * u.w;
    if (s) ((float4*)s)[e] = o;
    if (s16) ((half4*)s16)[e] = to_half4(o);
  }
}

__device__ __forceinline__ void swiglu_grad(float g, float u, float ds, float& dg, float& du) {
  const float sg = sigmoidf_(g);
  const float silu = g * sg;
  dg = ds * u * (sg * (1.0f + g - silu));
  du = ds * silu;
}

__global__ void swiglu_bwd_kernel(int T, int I, const float* __restrict__ gu,
                                  const float* __restrict__ ds, float* __restrict__ dgu,
                                  f16* __restrict__ dgu16) {
  const int64_t n4 = (int64_t)T * I / 4;
  const int i4 = I / 4;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = e / i4, j = e % i4;
    const float4 g = ((const float4*)(gu + t * 2 * I))[j];
    const float4 u = ((const float4*)(gu + t * 2 * I + I))[j];
    const float4 d = ((const float4*)ds)[e];
    float4 dg, du;
    swiglu_grad(g.x, u.x, d.x, dg.x, du.x);
    swiglu_grad(g.y, u.y, d.y, dg.y, du.y);
    swiglu_grad(g.z, u.z, d.z, dg.z, du.z);
    swiglu_grad(g.w, u.w, d.w, dg.w, du.w);
    if (dgu) {
      ((float4*)(dgu + t * 2 * I))[j] = dg;
      ((float4*)(dgu + t * 2 * I + I))[j] = du;
    }
    if (dgu16) {
      ((half4*)(dgu16 + t * 2 * I))[j] = to_half4(dg);
      ((half4*)(dgu16 + t * 2 * I + I))[j] = to_half4(du);
    }
  }
}

unsigned grid_for(int64_t n4) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n4, 256), 4096)); }

}  // namespace

RopeTabJob rope_table_job(int seq, int head_dim, float theta, float2* tab) {
  RopeTabJob j;
  j.seq = seq;
  j.half = head_dim / 2;
  j.d = head_dim;
  j.log_theta = log((double)theta);
  j.tab = tab;
  return j;
}

int rope_table(int seq, int head_dim, float theta, float2* tab, hipStream_t st) {
  const RopeTabJob j = rope_table_job(seq, head_dim, theta, tab);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)ceil_div((int64_t)seq * j.half, 256)), dim3(256), 0,
                     st, j);
  return check_launch("rope_table_kernel");
}

int qk_norm_rope_forward(const QkRopeArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.T * (a.heads + a.kv_heads + (a.v16 ? a.kv_heads : 0));
  hipLaunchKernelGGL(qk_rope_fwd_kernel, dim3((unsigned)ceil_div(items, 4)), dim3(256), 0, st, a);
  return check_launch("qk_rope_fwd_kernel");
}

size_t qk_norm_rope_bwd_scratch(int T, int heads, int kv_heads, int head_dim) {
  return (size_t)(qk_parts(T, heads) + qk_parts(T, kv_heads)) * head_dim * sizeof(float);
}

int qk_norm_rope_backward(const QkRopeBwdArgs& a, float* scratch, hipStream_t st) {
  ColsumJob jobs[2];
  int nj = 0;
  QBLK_TRY(qk_norm_rope_backward_partials(a, scratch, jobs, nj, st));
  return nj ? colsum_jobs(nj, jobs, st) : 0;
}

int qk_norm_rope_backward_partials(const QkRopeBwdArgs& a, float* scratch, ColsumJob* jobs, int& njobs,
                                   hipStream_t st) {
  const int d = a.head_dim;
  const int pq = qk_parts(a.T, a.heads), pk = qk_parts(a.T, a.kv_heads);
  float* part_q = scratch;
  float* part_k = scratch + (size_t)pq * d;
  hipLaunchKernelGGL(qk_rope_bwd_kernel, dim3((unsigned)(pq + pk)), dim3(256), 0, st, a, pq, part_q, part_k);
  QBLK_TRY(check_launch("qk_rope_bwd_kernel"));
  if (a.qk_norm) {
    jobs[njobs++] = ColsumJob{pq, d, part_q, a.dg_q};
    jobs[njobs++] = ColsumJob{pk, d, part_k, a.dg_k};
  } else {
    if (a.dg_q) hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(256), 0, st, a.dg_q, d, 0.f);
    if (a.dg_k) hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(256), 0, st, a.dg_k, d, 0.f);
    QBLK_TRY(check_launch("fill_kernel"));
  }
  return 0;
}

int swiglu_forward(int T, int I, const float* gu, float* s, f16* s16, hipStream_t st) {
  const int64_t n4 = (int64_t)T * I / 4;
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(grid_for(n4)), dim3(256), 0, st, T, I, gu, s, s16);
  return check_launch("swiglu_fwd_kernel");
}

int swiglu_backward(int T, int I, const float* gu, const float* ds, float* dgu, f16* dgu16, hipStream_t st) {
  const int64_t n4 = (int64_t)T * I / 4;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid_for(n4)), dim3(256), 0, st, T, I, gu, ds, dgu, dgu16);
  return check_launch("swiglu_bwd_kernel");
}

}  // namespace qblk
