// RMSNorm forward (optionally fused with the residual add) and backward.
//
// cuda_block.rs page: rms_norm_forward in CudaTransformerBlock::forward (the
// pre-attention and post-attention norms), the fused residual + RMSNorm of
// the NF4 forward, and rms_norm_backward in backward_post_attn_norm and
// backward_residual_and_input_norm. eps sits inside the square root.
//
// A row is read once with 16-byte loads into registers, reduced with DPP
// lane exchanges, then written: one 64-lane wave per row (VPL float4 per
// lane, n <= 256 * VPL), or for wide rows and few of them one 256-thread
// workgroup per row, whose four wave sums are added in a fixed order. The
// backward's dgamma uses no atomics: each workgroup (a fixed function of
// rows and n) reduces its rows into one partial row in scratch, and
// colsum_kernel adds the partials in a fixed order, so results are bitwise
// reproducible.
#include "norms.h"

#include "../../include/qblk.h"

namespace qblk {
namespace {

constexpr int kWavesPerBlock = 4;

template <int VPL>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(int rows, int n, float eps,
                                                          const float* __restrict__ x,
                                                          const float* __restrict__ res,
                                                          const float* __restrict__ gamma,
                                                          float* __restrict__ y,
                                                          f16* __restrict__ y16, int bf16,
                                                          float* __restrict__ sum_out,
                                                          float* __restrict__ rho_out,
                                                          const RopeTabJob tj) {
  const int nb = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  if ((int)blockIdx.x >= nb) {  // the RoPE table's workgroups
    rope_entry(tj, ((int)blockIdx.x - nb) * 256 + threadIdx.x);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int n4 = n >> 2;
  const float4* xr = (const float4*)(x + (int64_t)row * n);
  const float4* rr = res ? (const float4*)(res + (int64_t)row * n) : nullptr;
  // Loads go to clamped (always valid) columns and are masked afterwards,
  // so a row's loads (gamma's too) are all in flight together instead of
  // one branch each.
  const float4* gr = (const float4*)gamma;
  float4 gv[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) gv[j] = gr[min(lane + j * 64, n4 - 1)];
  float4 v[VPL];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = lane + j * 64, cc = min(c, n4 - 1);
    float4 a = xr[cc];
    if (rr) {
      const float4 b = rr[cc];
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    if (c >= n4) a = make_float4(0.f, 0.f, 0.f, 0.f);
    v[j] = a;
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
  }
  ss = wave_sum(ss);
  const float rho = 1.0f / sqrtf(ss / (float)n + eps);
  if (lane == 0 && rho_out) rho_out[row] = rho;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = lane + j * 64;
    if (c < n4) {
      if (sum_out) ((float4*)(sum_out + (int64_t)row * n))[c] = v[j];
      const float4 g = gv[j];
      float4 o;
      o.x = v[j].x * rho * g.x;
      o.y = v[j].y * rho * g.y;
      o.z = v[j].z * rho * g.z;
      o.w = v[j].w * rho * g.w;
      if (y) ((float4*)(y + (int64_t)row * n))[c] = o;
      if (y16) ((half4*)(y16 + (int64_t)row * n))[c] = to_16x4(o, bf16);
    }
  }
}

template <int VPL>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(int rows, int n, float eps,
                                                          const float* __restrict__ x,
                                                          const float* __restrict__ gamma,
                                                          const float* __restrict__ dy,
                                                          const float* __restrict__ dres,
                                                          float* __restrict__ dx,
                                                          f16* __restrict__ dx16, int bf16,
                                                          float* __restrict__ partial) {
  __shared__ float4 red[kWavesPerBlock][VPL * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n4 = n >> 2;
  const float4* gr = (const float4*)gamma;
  float4 dg[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) dg[j] = make_float4(0.f, 0.f, 0.f, 0.f);

  for (int row = blockIdx.x * kWavesPerBlock + w; row < rows; row += gridDim.x * kWavesPerBlock) {
    const float4* xr = (const float4*)(x + (int64_t)row * n);
    const float4* dr = (const float4*)(dy + (int64_t)row * n);
    // clamped loads, masked afterwards: all of a row's loads in flight at once
    float4 xv[VPL], e[VPL], dv[VPL], rv[VPL];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int cc = min(lane + j * 64, n4 - 1);
      xv[j] = xr[cc];
      dv[j] = dr[cc];
      e[j] = gr[cc];
      rv[j] = dres ? ((const float4*)(dres + (int64_t)row * n))[cc] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      if (lane + j * 64 >= n4) {
        xv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        dv[j] = xv[j];
      }
      e[j] = make_float4(e[j].x * dv[j].x, e[j].y * dv[j].y, e[j].z * dv[j].z, e[j].w * dv[j].w);
      ss += xv[j].x * xv[j].x + xv[j].y * xv[j].y + xv[j].z * xv[j].z + xv[j].w * xv[j].w;
    }
    ss = wave_sum(ss);
    const float rho = 1.0f / sqrtf(ss / (float)n + eps);
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = lane + j * 64;
      if (c < n4) {
        xv[j].x *= rho; xv[j].y *= rho; xv[j].z *= rho; xv[j].w *= rho;  // xhat
        dot += e[j].x * xv[j].x + e[j].y * xv[j].y + e[j].z * xv[j].z + e[j].w * xv[j].w;
      }
    }
    dot = wave_sum(dot) / (float)n;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = lane + j * 64;
      if (c < n4) {
        float4 o;
        o.x = rho * (e[j].x - xv[j].x * dot);
        o.y = rho * (e[j].y - xv[j].y * dot);
        o.z = rho * (e[j].z - xv[j].z * dot);
        o.w = rho * (e[j].w - xv[j].w * dot);
        o.x += rv[j].x; o.y += rv[j].y; o.z += rv[j].z; o.w += rv[j].w;
        ((float4*)(dx + (int64_t)row * n))[c] = o;
        if (dx16) ((half4*)(dx16 + (int64_t)row * n))[c] = to_16x4(o, bf16);
        dg[j].x += dv[j].x * xv[j].x;
        dg[j].y += dv[j].y * xv[j].y;
        dg[j].z += dv[j].z * xv[j].z;
        dg[j].w += dv[j].w * xv[j].w;
      }
    }
  }
  // Reduce the waves' dgamma partials in a fixed order.
#pragma unroll
  for (int j = 0; j < VPL; ++j) red[w][lane + j * 64] = dg[j];
  __syncthreads();
  for (int c = threadIdx.x; c < n4; c += blockDim.x) {
    float4 s = red[0][c];
#pragma unroll
    for (int ww = 1; ww < kWavesPerBlock; ++ww) {
      const float4 t = red[ww][c];
      s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
    }
    ((float4*)(partial + (int64_t)blockIdx.x * n))[c] = s;
  }
}

// Wide rows on few rows (n >= 1024, rows <= 4096, e.g. 512 tokens x 2560):
// one 256-thread workgroup per row (forward) or per run of rows (backward),
// VPT float4 per thread, so every SIMD of a CU takes part in a row and each
// lane holds a quarter of what a wave-per-row layout gives it. The row sums
// go through the waves' DPP sums and a fixed-order add of the four.
bool rms_rowwg(int rows, int n) { return n >= 1024 && n <= 4096 && rows <= 4096; }
constexpr int kRowWgMaxParts = 1024;
int rowwg_parts(int rows) { return (int)std::min<int64_t>(ceil_div(rows, 2), kRowWgMaxParts); }

__device__ __forceinline__ float sum4(const float* r) { return ((r[0] + r[1]) + r[2]) + r[3]; }
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

template <int VPT>
__global__ __launch_bounds__(256) void rmsnorm_fwd_row_kernel(int rows, int n, float eps, const float* __restrict__ x,
                                                              const float* __restrict__ res,
                                                              const float* __restrict__ gamma, float* __restrict__ y,
                                                              f16* __restrict__ y16, int bf16,
                                                              float* __restrict__ sum_out,
                                                              float* __restrict__ rho_out, const RopeTabJob tj) {
  __shared__ float red[4];
  if ((int)blockIdx.x >= rows) {  // the RoPE table's workgroups
    rope_entry(tj, ((int)blockIdx.x - rows) * 256 + threadIdx.x);
    return;
  }
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int n4 = n >> 2;
  const float4* xr = (const float4*)(x + (int64_t)row * n);
  const float4* rr = res ? (const float4*)(res + (int64_t)row * n) : nullptr;
  const float4* gr = (const float4*)gamma;
  float4 v[VPT], gv[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int cc = min(t + j * 256, n4 - 1);
    v[j] = xr[cc];
    gv[j] = gr[cc];
  }
  float4 rv[VPT];
  if (rr) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) rv[j] = rr[min(t + j * 256, n4 - 1)];
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    if (rr) v[j] = make_float4(v[j].x + rv[j].x, v[j].y + rv[j].y, v[j].z + rv[j].z, v[j].w + rv[j].w);
    if (t + j * 256 >= n4) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    ss += dot4(v[j], v[j]);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  const float rho = 1.0f / sqrtf(sum4(red) / (float)n + eps);
  if (t == 0 && rho_out) rho_out[row] = rho;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int c = t + j * 256;
    if (c < n4) {
      if (sum_out) ((float4*)(sum_out + (int64_t)row * n))[c] = v[j];
      const float4 o = make_float4(v[j].x * rho * gv[j].x, v[j].y * rho * gv[j].y, v[j].z * rho * gv[j].z,
                                   v[j].w * rho * gv[j].w);
      if (y) ((float4*)(y + (int64_t)row * n))[c] = o;
      if (y16) ((half4*)(y16 + (int64_t)row * n))[c] = to_16x4(o, bf16);
    }
  }
}

// Backward: workgroup b takes rows [b rpb, (b+1) rpb), two at a time with
// all their loads issued together; each thread keeps the dgamma sums of
// its own columns over those rows and writes them as partial row b.
template <int VPT>
__global__ __launch_bounds__(256) void rmsnorm_bwd_row_kernel(int rows, int n, float eps, const float* __restrict__ x,
                                                              const float* __restrict__ gamma,
                                                              const float* __restrict__ dy,
                                                              const float* __restrict__ dres, float* __restrict__ dx,
                                                              f16* __restrict__ dx16, int bf16,
                                                              float* __restrict__ partial, int rpb) {
  __shared__ float red[2][2][4];  // [row of the pair][row sum, dot][wave]
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int n4 = n >> 2;
  const float4* gr = (const float4*)gamma;
  float4 gv[VPT], dg[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    gv[j] = gr[min(t + j * 256, n4 - 1)];
    dg[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int rb = blockIdx.x * rpb, re = min(rows, rb + rpb);
  for (int r0 = rb; r0 < re; r0 += 2) {
    const bool two = r0 + 1 < re;
    float4 xv[2][VPT], dv[2][VPT], rv[2][VPT];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int row = two ? r0 + k : r0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int cc = min(t + j * 256, n4 - 1);
        xv[k][j] = ((const float4*)(x + (int64_t)row * n))[cc];
        dv[k][j] = ((const float4*)(dy + (int64_t)row * n))[cc];
        rv[k][j] = dres ? ((const float4*)(dres + (int64_t)row * n))[cc] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float ss[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (t + j * 256 >= n4) {
          xv[k][j] = make_float4(0.f, 0.f, 0.f, 0.f);
          dv[k][j] = xv[k][j];
        }
        ss[k] += dot4(xv[k][j], xv[k][j]);
      }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      ss[k] = wave_sum(ss[k]);
      if (lane == 0) red[k][0][w] = ss[k];
    }
    __syncthreads();
    float rho[2], dot[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      rho[k] = 1.0f / sqrtf(sum4(red[k][0]) / (float)n + eps);
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        xv[k][j] = make_float4(xv[k][j].x * rho[k], xv[k][j].y * rho[k], xv[k][j].z * rho[k], xv[k][j].w * rho[k]);
        const float4 e = make_float4(gv[j].x * dv[k][j].x, gv[j].y * dv[k][j].y, gv[j].z * dv[k][j].z,
                                     gv[j].w * dv[k][j].w);
        dot[k] += dot4(e, xv[k][j]);
      }
      dot[k] = wave_sum(dot[k]);
      if (lane == 0) red[k][1][w] = dot[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k == 1 && !two) break;
      const int row = r0 + k;
      const float dm = sum4(red[k][1]) / (float)n;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int c = t + j * 256;
        if (c >= n4) continue;
        const float4 xh = xv[k][j], d = dv[k][j], r = rv[k][j];
        float4 o;
        o.x = rho[k] * (gv[j].x * d.x - xh.x * dm) + r.x;
        o.y = rho[k] * (gv[j].y * d.y - xh.y * dm) + r.y;
        o.z = rho[k] * (gv[j].z * d.z - xh.z * dm) + r.z;
        o.w = rho[k] * (gv[j].w * d.w - xh.w * dm) + r.w;
        ((float4*)(dx + (int64_t)row * n))[c] = o;
        if (dx16) ((half4*)(dx16 + (int64_t)row * n))[c] = to_16x4(o, bf16);
        dg[j] = make_float4(dg[j].x + d.x * xh.x, dg[j].y + d.y * xh.y, dg[j].z + d.z * xh.z, dg[j].w + d.w * xh.w);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int c = t + j * 256;
    if (c < n4) ((float4*)(partial + (int64_t)blockIdx.x * n))[c] = dg[j];
  }
}

// Column sums of partial rows: cw columns per workgroup and 1024 / cw row
// groups per column (row p goes to group p % groups, summed in row order);
// the group sums are then added in group order, so results are bitwise
// reproducible. Narrow sums (n <= 256: the QK gammas, whose partial rows
// are many) take 16 columns and 64 groups, the rest 64 and 16.
__host__ __device__ __forceinline__ int colsum_width(int n) { return n <= 256 ? 16 : 64; }

__device__ __forceinline__ void colsum_cols(int parts, int n, const float* __restrict__ partial,
                                            float* __restrict__ out, int accumulate) {
  __shared__ float red[1024];
  const int cw = colsum_width(n), ng = 1024 / cw;
  const int cl = threadIdx.x % cw, rg = threadIdx.x / cw;
  const int c = blockIdx.x * cw + cl;
  float s = 0.f;
  if (c < n) {
#pragma unroll 8
    for (int p = rg; p < parts; p += ng) s += partial[(int64_t)p * n + c];
  }
  red[rg * cw + cl] = s;
  __syncthreads();
  if (rg == 0 && c < n) {
    float t = red[cl];
    for (int g = 1; g < ng; ++g) t += red[g * cw + cl];
    out[c] = accumulate ? out[c] + t : t;
  }
}

__global__ __launch_bounds__(1024) void colsum_kernel(int parts, int n, const float* __restrict__ partial,
                                                      float* __restrict__ out) {
  colsum_cols(parts, n, partial, out, 0);
}

// Independent column sums in one launch (blockIdx.y picks the job).
struct ColsumJobs {
  ColsumJob j[kMaxColsumJobs];
};
__global__ __launch_bounds__(1024) void colsum_jobs_kernel(const ColsumJobs jobs) {
  const ColsumJob& j = jobs.j[blockIdx.y];
  if ((int)blockIdx.x * colsum_width(j.n) < j.n) colsum_cols(j.parts, j.n, j.partial, j.out, j.accumulate);
}

int vpl_for(int n) {
  const int need = (int)ceil_div(n, 256);
  if (need <= 1) return 1;
  if (need <= 2) return 2;
  if (need <= 4) return 4;
  if (need <= 8) return 8;
  if (need <= 12) return 12;
  if (need <= 16) return 16;
  return -1;
}

}  // namespace

int rmsnorm_bwd_parts(int rows, int n) {
  if (rms_rowwg(rows, n)) return rowwg_parts(rows);
  return (int)std::min<int64_t>(ceil_div(rows, kWavesPerBlock), 240);
}

size_t rmsnorm_bwd_scratch(int rows, int n) {
  return (size_t)rmsnorm_bwd_parts(rows, n) * n * sizeof(float);
}

int rmsnorm_check(int rows, int n) {
  if (rows <= 0 || n <= 0) return fail(QBLK_EINVAL, "rmsnorm: rows=%d n=%d", rows, n);
  if (n % 4) return fail(QBLK_EINVAL, "rmsnorm: n=%d must be a multiple of 4", n);
  if (vpl_for(n) < 0) return fail(QBLK_EUNSUPPORTED, "rmsnorm: n=%d above 4096", n);
  return 0;
}

int rmsnorm_forward(int rows, int n, float eps, const float* x, const float* res,
                    const float* gamma, float* y, f16* y16, float* sum_out, float* rho,
                    hipStream_t st, const RopeTabJob* tab, bool bf16) {
  QBLK_TRY(rmsnorm_check(rows, n));
  const RopeTabJob tj = tab ? *tab : RopeTabJob{};
  const int64_t tab_blocks = ceil_div((int64_t)tj.seq * tj.half, 256);
  if (rms_rowwg(rows, n)) {
    const dim3 g((unsigned)(rows + tab_blocks));
    switch ((int)ceil_div(n / 4, 256)) {
#define QBLK_CASE(V)                                                                                       \
  case V:                                                                                                  \
    hipLaunchKernelGGL(rmsnorm_fwd_row_kernel<V>, g, dim3(256), 0, st, rows, n, eps, x, res, gamma, y, y16, \
                       (int)bf16, sum_out, rho, tj);                                                                  \
    break;
      QBLK_CASE(1) QBLK_CASE(2) QBLK_CASE(3) QBLK_CASE(4)
#undef QBLK_CASE
    }
    return check_launch("rmsnorm_fwd_row_kernel");
  }
  const dim3 grid((unsigned)(ceil_div(rows, kWavesPerBlock) + tab_blocks)), block(256);
  switch (vpl_for(n)) {
#define QBLK_CASE(V)                                                                          \
  case V:                                                                                     \
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<V>, grid, block, 0, st, rows, n, eps, x, res, gamma, \
                       y, y16, (int)bf16, sum_out, rho, tj);                                  \
    break;
    QBLK_CASE(1) QBLK_CASE(2) QBLK_CASE(4) QBLK_CASE(8) QBLK_CASE(12) QBLK_CASE(16)
#undef QBLK_CASE
  }
  return check_launch("rmsnorm_fwd_kernel");
}

int rmsnorm_backward(int rows, int n, float eps, const float* x, const float* gamma,
                     const float* dy, const float* dres, float* dx, f16* dx16, float* dgamma, float* scratch,
                     hipStream_t st, bool bf16) {
  QBLK_TRY(rmsnorm_backward_partials(rows, n, eps, x, gamma, dy, dres, dx, dx16, scratch, st, bf16));
  return colsum(rmsnorm_bwd_parts(rows, n), n, scratch, dgamma, st);
}

int rmsnorm_backward_partials(int rows, int n, float eps, const float* x, const float* gamma, const float* dy,
                              const float* dres, float* dx, f16* dx16, float* scratch, hipStream_t st, bool bf16) {
  QBLK_TRY(rmsnorm_check(rows, n));
  const int parts = rmsnorm_bwd_parts(rows, n);
  if (rms_rowwg(rows, n)) {
    const int rpb = (int)ceil_div(rows, parts);
    switch ((int)ceil_div(n / 4, 256)) {
#define QBLK_CASE(V)                                                                                         \
  case V:                                                                                                    \
    hipLaunchKernelGGL(rmsnorm_bwd_row_kernel<V>, dim3((unsigned)parts), dim3(256), 0, st, rows, n, eps, x, \
                       gamma, dy, dres, dx, dx16, (int)bf16, scratch, rpb);                                  \
    break;
      QBLK_CASE(1) QBLK_CASE(2) QBLK_CASE(3) QBLK_CASE(4)
#undef QBLK_CASE
    }
    return check_launch("rmsnorm_bwd_row_kernel");
  }
  const dim3 grid((unsigned)parts), block(256);
  switch (vpl_for(n)) {
#define QBLK_CASE(V)                                                                             \
  case V:                                                                                        \
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<V>, grid, block, 0, st, rows, n, eps, x, gamma, dy,     \
                       dres, dx, dx16, (int)bf16, scratch);                                      \
    break;
    QBLK_CASE(1) QBLK_CASE(2) QBLK_CASE(4) QBLK_CASE(8) QBLK_CASE(12) QBLK_CASE(16)
#undef QBLK_CASE
  }
  return check_launch("rmsnorm_bwd_kernel");
}

int colsum_jobs(int njobs, const ColsumJob* jobs, hipStream_t st) {
  if (njobs <= 0 || njobs > kMaxColsumJobs) return fail(QBLK_EINVAL, "colsum: %d jobs", njobs);
  ColsumJobs js{};
  int64_t nb = 0;
  for (int i = 0; i < njobs; ++i) {
    js.j[i] = jobs[i];
    nb = std::max<int64_t>(nb, ceil_div(jobs[i].n, colsum_width(jobs[i].n)));
  }
  hipLaunchKernelGGL(colsum_jobs_kernel, dim3((unsigned)nb, (unsigned)njobs), dim3(1024), 0, st, js);
  return check_launch("colsum_jobs_kernel");
}

int colsum(int parts, int n, const float* partial, float* out, hipStream_t st) {
  hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)ceil_div(n, colsum_width(n))), dim3(1024), 0, st, parts, n,
                     partial, out);
  return check_launch("colsum_kernel");
}

}  // namespace qblk
