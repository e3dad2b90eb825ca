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
    for (int c = lane; c < d; c += 64) dst[c] = to_16(src[c], a.bf16);
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
      dst16[orow + lane] = to_16(o0, a.bf16);
      dst16[orow + lane + half] = to_16(o1, a.bf16);
    }
  }
}

// Backward: blocks [0, nbq) take the q heads, the rest the k heads; each
// wave takes kQkRows consecutive (t, head) rows with all their loads issued
// before any arithmetic (rows past the end load the last row and are
// skipped). dgamma partials: one row per workgroup, in a fixed order.
constexpr int kQkRows = 2;
// Waves per workgroup of the paired backward: each workgroup leaves one
// gamma-gradient partial row, so more waves mean fewer rows to sum after.
constexpr int kQkBwdWaves = 4;

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
        a.dqkv16[o] = to_16(o0, a.bf16);
        a.dqkv16[o + half] = to_16(o1, a.bf16);
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

// The same two passes with 64 / LPH heads side by side in one wave (head_dim
// = 4 LPH): LPH lanes per head, each holding elements 2j, 2j+1 of both
// halves, so that every load and store moves 8 (fp32) or 4 (fp16) bytes per
// lane; each wave takes kQkRows tokens of its heads with every load issued
// before any arithmetic (tokens past the end load the last token and are
// skipped). Heads past the last of a group's range are computed on head 0
// and not stored.
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2v to_h2(float a, float b, bool bf) {
  h2v h;
  h[0] = to_16(a, bf);
  h[1] = to_16(b, bf);
  return h;
}

template <int LPH>
__global__ __launch_bounds__(256) void qk_rope_fwd_pair_kernel(QkRopeArgs a) {
  constexpr int HPW = 64 / LPH, D = 4 * LPH, HALF = 2 * LPH, R = kQkRows;
  const int lane = threadIdx.x & 63, j = lane % LPH;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nqk = a.heads + a.kv_heads;
  const int nh = nqk + (a.v16 ? a.kv_heads : 0);
  const int ng = (nh + HPW - 1) / HPW;
  const int t0 = (wid / ng) * R;
  if (t0 >= a.T) return;
  const int head = (wid % ng) * HPW + lane / LPH;
  const bool valid = head < nh;
  const int hc = valid ? head : 0;
  const bool is_v = hc >= nqk, is_q = hc < a.heads;
  float2 x0[R], x1[R];
  float4 cs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = min(t0 + r, a.T - 1);
    const float* src = a.qkv + (int64_t)t * a.ld_qkv + (int64_t)hc * D + 2 * j;
    x0[r] = *(const float2*)src;
    x1[r] = *(const float2*)(src + HALF);
    cs[r] = *(const float4*)(a.tab + (t % a.seq) * HALF + 2 * j);
  }
  const float* g = is_q ? a.g_q : a.g_k;
  float2 ga = make_float2(1.f, 1.f), gb = ga;
  if (a.qk_norm) {
    ga = *(const float2*)(g + 2 * j);
    gb = *(const float2*)(g + HALF + 2 * j);
  }
  const int hh = is_v ? hc - nqk : is_q ? hc : hc - a.heads;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r;
    if (t >= a.T) break;
    float2 p = x0[r], q = x1[r];
    if (a.qk_norm) {
      const float ss = group_sum<LPH>(p.x * p.x + p.y * p.y + q.x * q.x + q.y * q.y);
      const float rho = 1.0f / sqrtf(ss / (float)D + a.eps);
      if (valid && !is_v && j == 0) (is_q ? a.rho_q[(int64_t)t * a.heads + hh] : a.rho_k[(int64_t)t * a.kv_heads + hh]) = rho;
      if (!is_v) {
        p = make_float2(p.x * rho * ga.x, p.y * rho * ga.y);
        q = make_float2(q.x * rho * gb.x, q.y * rho * gb.y);
      }
    }
    if (!valid) continue;
    if (is_v) {
      f16* dst = a.v16 + ((int64_t)t * a.kv_heads + hh) * D + 2 * j;
      *(h2v*)dst = to_h2(p.x, p.y, a.bf16);
      *(h2v*)(dst + HALF) = to_h2(q.x, q.y, a.bf16);
      continue;
    }
    // NeoX rotation of the pairs (2j, HALF + 2j) and (2j + 1, HALF + 2j + 1)
    const float2 o0 = make_float2(p.x * cs[r].x - q.x * cs[r].y, p.y * cs[r].z - q.y * cs[r].w);
    const float2 o1 = make_float2(q.x * cs[r].x + p.x * cs[r].y, q.y * cs[r].z + p.y * cs[r].w);
    const int64_t orow = ((int64_t)t * (is_q ? a.heads : a.kv_heads) + hh) * D + 2 * j;
    float* dst = is_q ? a.qr : a.kr;
    f16* dst16 = is_q ? a.q16 : a.k16;
    if (dst) {
      *(float2*)(dst + orow) = o0;
      *(float2*)(dst + orow + HALF) = o1;
    }
    if (dst16) {
      *(h2v*)(dst16 + orow) = to_h2(o0.x, o0.y, a.bf16);
      *(h2v*)(dst16 + orow + HALF) = to_h2(o1.x, o1.y, a.bf16);
    }
  }
}

// Backward in the same layout: blocks [0, nbq) take the q heads, the rest
// the k heads; the gamma-gradient partials of a block (its kQkBwdWaves waves, each
// over its HPW heads and R tokens) form one row, summed in a fixed order.
template <int LPH>
__global__ __launch_bounds__(64 * kQkBwdWaves) void qk_rope_bwd_pair_kernel(QkRopeBwdArgs a, int nbq,
                                                                           float* __restrict__ part_q,
                                                                           float* __restrict__ part_k) {
  constexpr int HPW = 64 / LPH, D = 4 * LPH, HALF = 2 * LPH, R = kQkRows, WB = kQkBwdWaves;
  __shared__ float4 red[WB][LPH];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, j = lane % LPH;
  const bool is_q = (int)blockIdx.x < nbq;
  const int blk = is_q ? blockIdx.x : blockIdx.x - nbq;
  const int nh = is_q ? a.heads : a.kv_heads;
  const int ng = (nh + HPW - 1) / HPW;
  const int wid = blk * WB + w;
  const int t0 = (wid / ng) * R;
  const int head = (wid % ng) * HPW + lane / LPH;
  const bool valid = head < nh && t0 < a.T;
  const int hc = head < nh ? head : 0;
  const int col0 = (is_q ? 0 : a.heads * D) + hc * D + 2 * j;
  const float* __restrict__ dsrc = (is_q ? a.dqr : a.dkr) + (int64_t)hc * D + 2 * j;
  float2 y0[R], y1[R], x0[R], x1[R];
  float4 cs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = min(t0 + r, a.T - 1);
    y0[r] = *(const float2*)(dsrc + (int64_t)t * nh * D);
    y1[r] = *(const float2*)(dsrc + (int64_t)t * nh * D + HALF);
    cs[r] = *(const float4*)(a.tab + (t % a.seq) * HALF + 2 * j);
    if (a.qk_norm) {
      const float* xr = a.qkv + (int64_t)t * a.ld_qkv + col0;
      x0[r] = *(const float2*)xr;
      x1[r] = *(const float2*)(xr + HALF);
    }
  }
  float2 ga = make_float2(0.f, 0.f), gb = ga;
  if (a.qk_norm) {
    const float* g = is_q ? a.g_q : a.g_k;
    ga = *(const float2*)(g + 2 * j);
    gb = *(const float2*)(g + HALF + 2 * j);
  }
  float4 dg = make_float4(0.f, 0.f, 0.f, 0.f);  // elements 2j, 2j+1, HALF+2j, HALF+2j+1
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r;
    if (t >= a.T) break;
    // transpose of the rotation
    float2 o0 = make_float2(y0[r].x * cs[r].x + y1[r].x * cs[r].y, y0[r].y * cs[r].z + y1[r].y * cs[r].w);
    float2 o1 = make_float2(y1[r].x * cs[r].x - y0[r].x * cs[r].y, y1[r].y * cs[r].z - y0[r].y * cs[r].w);
    if (a.qk_norm) {
      const float2 p = x0[r], q = x1[r];
      const float ss = group_sum<LPH>(p.x * p.x + p.y * p.y + q.x * q.x + q.y * q.y);
      const float rho = 1.0f / sqrtf(ss / (float)D + a.eps);
      const float2 hp = make_float2(p.x * rho, p.y * rho), hq = make_float2(q.x * rho, q.y * rho);
      const float2 ep = make_float2(ga.x * o0.x, ga.y * o0.y), eq = make_float2(gb.x * o1.x, gb.y * o1.y);
      const float dot = group_sum<LPH>(ep.x * hp.x + ep.y * hp.y + eq.x * hq.x + eq.y * hq.y) / (float)D;
      if (valid) {
        dg.x += o0.x * hp.x;
        dg.y += o0.y * hp.y;
        dg.z += o1.x * hq.x;
        dg.w += o1.y * hq.y;
      }
      o0 = make_float2(rho * (ep.x - hp.x * dot), rho * (ep.y - hp.y * dot));
      o1 = make_float2(rho * (eq.x - hq.x * dot), rho * (eq.y - hq.y * dot));
    }
    if (!valid) continue;
    const int64_t o = (int64_t)t * a.ld_qkv + col0;
    if (a.dqkv) {
      *(float2*)(a.dqkv + o) = o0;
      *(float2*)(a.dqkv + o + HALF) = o1;
    }
    if (a.dqkv16) {
      *(h2v*)(a.dqkv16 + o) = to_h2(o0.x, o0.y, a.bf16);
      *(h2v*)(a.dqkv16 + o + HALF) = to_h2(o1.x, o1.y, a.bf16);
    }
  }
  if (!a.qk_norm) return;
  // the wave's heads, then the waves in order
  if constexpr (LPH < 64) {
    __shared__ float4 hs[WB][64];
    hs[w][lane] = dg;
    __syncthreads();
    if (lane < LPH) {
#pragma unroll
      for (int k = 1; k < HPW; ++k) {
        const float4 e = hs[w][k * LPH + lane];
        dg = make_float4(dg.x + e.x, dg.y + e.y, dg.z + e.z, dg.w + e.w);
      }
    }
  }
  if (lane < LPH) red[w][lane] = dg;
  __syncthreads();
  if (threadIdx.x < LPH) {
    const int c = threadIdx.x;
    float4 t = red[0][c];
#pragma unroll
    for (int ww = 1; ww < WB; ++ww) {
      const float4 e = red[ww][c];
      t = make_float4(t.x + e.x, t.y + e.y, t.z + e.z, t.w + e.w);
    }
    float* pr = (is_q ? part_q : part_k) + (int64_t)blk * D;
    *(float2*)(pr + 2 * c) = make_float2(t.x, t.y);
    *(float2*)(pr + HALF + 2 * c) = make_float2(t.z, t.w);
  }
}

// Lanes per head of the paired layout, or 0 where it does not apply.
int qk_pair_lph(int head_dim) {
  if (head_dim % 4) return 0;
  const int lph = head_dim / 4;
  return (lph == 8 || lph == 16 || lph == 32) ? lph : 0;  // head_dim 32, 64, 128
}
bool al(const void* p, int n) { return (uintptr_t)p % n == 0; }
// The paired kernels' 8- and 16-byte accesses need these alignments.
bool qk_pair_fits(int64_t ld_qkv, const float2* tab, const float* g_q, const float* g_k,
                  std::initializer_list<const void*> p8) {
  bool ok = ld_qkv % 2 == 0 && al(tab, 16) && al(g_q, 8) && al(g_k, 8);
  for (const void* q : p8) ok = ok && al(q, 8);
  return ok;
}

__global__ void fill_kernel(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Partial rows of the backward with the paired layout (lph > 0) or without.
int qk_parts(int T, int nh, int lph) {
  if (lph) return (int)ceil_div(ceil_div((int64_t)T, kQkRows) * ceil_div(nh, 64 / lph), kQkBwdWaves);
  return (int)ceil_div((int64_t)T * nh, 4 * kQkRows);
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// One row of gu per blockIdx.y step, float4 column j per thread (a 2-D
// grid: no index division per element).
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(int T, int I, const float* __restrict__ gu,
                                                         float* __restrict__ s, f16* __restrict__ s16, int bf16) {
  const int i4 = I / 4, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= i4) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    const float4 g = ((const float4*)(gu + (int64_t)t * 2 * I))[j];
    const float4 u = ((const float4*)(gu + (int64_t)t * 2 * I + I))[j];
    float4 o;
    o.x = g.x * sigmoidf_(g.x) * u.x;
    o.y = g.y * sigmoidf_(g.y) * u.y;
    o.z = g.z * sigmoidf_(g.z) * u.z;
    o.w = g.w * sigmoidf_(g.w) * u.w;
    const int64_t e = (int64_t)t * i4 + j;
    if (s) ((float4*)s)[e] = o;
    if (s16) ((half4*)s16)[e] = to_16x4(o, bf16);
  }
}

__device__ __forceinline__ void swiglu_grad(float g, float u, float ds, float& dg, float& du) {
  const float sg = sigmoidf_(g);
  const float silu = g * sg;
  dg = ds * u * (sg * (1.0f + g - silu));
  du = ds * silu;
}

__global__ __launch_bounds__(256) void swiglu_bwd_kernel(int T, int I, const float* __restrict__ gu,
                                                         const float* __restrict__ ds, float* __restrict__ dgu,
                                                         f16* __restrict__ dgu16, int bf16) {
  const int i4 = I / 4, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= i4) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    const float4 g = ((const float4*)(gu + (int64_t)t * 2 * I))[j];
    const float4 u = ((const float4*)(gu + (int64_t)t * 2 * I + I))[j];
    const float4 d = ((const float4*)ds)[(int64_t)t * i4 + j];
    float4 dg, du;
    swiglu_grad(g.x, u.x, d.x, dg.x, du.x);
    swiglu_grad(g.y, u.y, d.y, dg.y, du.y);
    swiglu_grad(g.z, u.z, d.z, dg.z, du.z);
    swiglu_grad(g.w, u.w, d.w, dg.w, du.w);
    if (dgu) {
      ((float4*)(dgu + (int64_t)t * 2 * I))[j] = dg;
      ((float4*)(dgu + (int64_t)t * 2 * I + I))[j] = du;
    }
    if (dgu16) {
      ((half4*)(dgu16 + (int64_t)t * 2 * I))[j] = to_16x4(dg, bf16);
      ((half4*)(dgu16 + (int64_t)t * 2 * I + I))[j] = to_16x4(du, bf16);
    }
  }
}

dim3 swiglu_grid(int T, int I) {
  return dim3((unsigned)ceil_div(I / 4, 256), (unsigned)std::min(T, 65535));
}


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

template <class K>
static void launch_pair(int lph, K k) {
  switch (lph) {
    case 8: k(std::integral_constant<int, 8>{}); break;
    case 16: k(std::integral_constant<int, 16>{}); break;
    default: k(std::integral_constant<int, 32>{}); break;
  }
}

int qk_norm_rope_forward(const QkRopeArgs& a, hipStream_t st) {
  const int nh = a.heads + a.kv_heads + (a.v16 ? a.kv_heads : 0);
  const int lph = qk_pair_lph(a.head_dim);
  if (lph && qk_pair_fits(a.ld_qkv, a.tab, a.g_q, a.g_k, {a.qkv, a.qr, a.kr, a.q16, a.k16, a.v16})) {
    const int64_t waves = ceil_div((int64_t)a.T, kQkRows) * ceil_div(nh, 64 / lph);
    launch_pair(lph, [&](auto L) {
      hipLaunchKernelGGL(qk_rope_fwd_pair_kernel<decltype(L)::value>, dim3((unsigned)ceil_div(waves, 4)), dim3(256),
                         0, st, a);
    });
    return check_launch("qk_rope_fwd_pair_kernel");
  }
  const int64_t items = (int64_t)a.T * nh;
  hipLaunchKernelGGL(qk_rope_fwd_kernel, dim3((unsigned)ceil_div(items, 4)), dim3(256), 0, st, a);
  return check_launch("qk_rope_fwd_kernel");
}

size_t qk_norm_rope_bwd_scratch(int T, int heads, int kv_heads, int head_dim) {
  const int lph = qk_pair_lph(head_dim);
  const int rows = std::max(qk_parts(T, heads, lph) + qk_parts(T, kv_heads, lph),
                            qk_parts(T, heads, 0) + qk_parts(T, kv_heads, 0));
  return (size_t)rows * head_dim * sizeof(float);
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
  int lph = qk_pair_lph(d);
  if (!qk_pair_fits(a.ld_qkv, a.tab, a.g_q, a.g_k, {a.qkv, a.dqr, a.dkr, a.dqkv, a.dqkv16})) lph = 0;
  const int pq = qk_parts(a.T, a.heads, lph), pk = qk_parts(a.T, a.kv_heads, lph);
  float* part_q = scratch;
  float* part_k = scratch + (size_t)pq * d;
  if (lph) {
    launch_pair(lph, [&](auto L) {
      hipLaunchKernelGGL(qk_rope_bwd_pair_kernel<decltype(L)::value>, dim3((unsigned)(pq + pk)),
                         dim3(64 * kQkBwdWaves), 0, st,
                         a, pq, part_q, part_k);
    });
    QBLK_TRY(check_launch("qk_rope_bwd_pair_kernel"));
  } else {
    hipLaunchKernelGGL(qk_rope_bwd_kernel, dim3((unsigned)(pq + pk)), dim3(256), 0, st, a, pq, part_q, part_k);
    QBLK_TRY(check_launch("qk_rope_bwd_kernel"));
  }
  if (a.qk_norm) {
    jobs[njobs++] = ColsumJob{pq, d, part_q, a.dg_q, a.accumulate_dg};
    jobs[njobs++] = ColsumJob{pk, d, part_k, a.dg_k, a.accumulate_dg};
  } else if (!a.accumulate_dg) {
    if (a.dg_q) hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(256), 0, st, a.dg_q, d, 0.f);
    if (a.dg_k) hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(256), 0, st, a.dg_k, d, 0.f);
    QBLK_TRY(check_launch("fill_kernel"));
  }
  return 0;
}

int swiglu_forward(int T, int I, const float* gu, float* s, f16* s16, hipStream_t st, bool bf16) {
  hipLaunchKernelGGL(swiglu_fwd_kernel, swiglu_grid(T, I), dim3(256), 0, st, T, I, gu, s, s16, (int)bf16);
  return check_launch("swiglu_fwd_kernel");
}

int swiglu_backward(int T, int I, const float* gu, const float* ds, float* dgu, f16* dgu16, hipStream_t st,
                    bool bf16) {
  hipLaunchKernelGGL(swiglu_bwd_kernel, swiglu_grid(T, I), dim3(256), 0, st, T, I, gu, ds, dgu, dgu16, (int)bf16);
  return check_launch("swiglu_bwd_kernel");
}

}  // namespace qblk
