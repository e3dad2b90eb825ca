// Global L2 gradient clip and AdamW over many tensors.
//
// cuda_trainer.rs page: the squared-sum clip (per-workgroup partial sums of
// g^2, a final reduction in fp64, scale = max_norm / norm above the limit)
// and the fused clip state that keeps the scale on the device.
// cuda_block.rs page: optimizer_step applies adamw_step_cuda to every block
// tensor, norm gammas included; the update is AdamW with decoupled weight
// decay and bias correction (the page does not print it).
//
// Tensors are processed in chunks whose descriptors travel as kernel
// arguments (no device-side tables, no allocation). A chunk's elements are
// cut into tiles of 4096 that never straddle tensors; a workgroup finds its
// tensor by scanning the chunk's tile prefix sums. The norm reduction has a
// fixed shape (a function of the sizes only) and no atomics, so it is
// bitwise reproducible.
#include "step.h"

#include <mutex>
#include <vector>

#include "../../include/qblk.h"

namespace qblk {
namespace {

constexpr int kTile = 4096;   // elements per tile (256 threads x 16)
constexpr int kChunk = 32;    // tensors per launch
constexpr int kSqGrid = 512;  // workgroups of a squared-sum launch

struct SqChunk {
  const float* p[kChunk];
  int64_t n[kChunk];
  int64_t tile_end[kChunk];  // prefix sums of tiles
  int count;
};

__device__ __forceinline__ int find_tensor(const int64_t* tile_end, int count, int64_t tile) {
  int j = 0;
  while (j < count - 1 && tile >= tile_end[j]) ++j;
  return j;
}

// Streaming access for AdamW: every element of w, g, m, v is read once and
// w, m, v written once per call, over GBs far beyond the caches, so its
// loads and stores carry the nontemporal hint (measured faster there; the
// squared sum's plain loads measured faster than hinted ones).
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float* p) {
  const f4v v = __builtin_nontemporal_load((const f4v*)p);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(float* p, const float4 x) {
  const f4v v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, (f4v*)p);
}

__global__ __launch_bounds__(256) void sqsum_kernel(const SqChunk c, double* partial) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int64_t ntiles = c.tile_end[c.count - 1];
  double acc = 0.0;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int j = find_tensor(c.tile_end, c.count, tile);
    const int64_t t0 = j ? c.tile_end[j - 1] : 0;
    const int64_t base = (tile - t0) * kTile;
    const float* p = c.p[j];
    const int64_t n = c.n[j];
    float s = 0.f;
    if (base + kTile <= n && ((uintptr_t)p & 15) == 0) {
      const float4* p4 = (const float4*)(p + base);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 v = p4[tid + 256 * u];
        s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    } else {
      for (int64_t e = base + tid; e < min(base + kTile, n); e += 256) s += p[e] * p[e];
    }
    acc += (double)s;
  }
  red[tid] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void clip_finalize_kernel(int nparts, const double* partial,
                                                            float max_norm, float* norm_dev,
                                                            float* scale_dev) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int i = tid; i < nparts; i += 256) s += partial[i];
  red[tid] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) {
    const double norm = sqrt(red[0]);
    // a non-finite norm (some gradient is NaN or infinite) gives a NaN scale:
    // AdamW then skips the step
    const double scale = !isfinite(norm)          ? (double)NAN
                         : norm > (double)max_norm ? (double)max_norm / norm
                                                   : 1.0;
    norm_dev[0] = (float)norm;
    scale_dev[0] = (float)scale;
  }
}

struct ScaleChunk {
  float* p[kChunk];
  int64_t n[kChunk];
  int64_t tile_end[kChunk];
  int count;
};

__global__ __launch_bounds__(256) void scale_kernel(const ScaleChunk c, const float* scale_dev) {
  const int64_t tile = blockIdx.x;
  const int j = find_tensor(c.tile_end, c.count, tile);
  const int64_t base = (tile - (j ? c.tile_end[j - 1] : 0)) * kTile;
  const float s = scale_dev[0];
  float* p = c.p[j];
  const int64_t end = min(base + (int64_t)kTile, c.n[j]);
  for (int64_t e = base + threadIdx.x; e < end; e += 256) p[e] *= s;
}

struct AdamChunk {
  float* w[kChunk];
  f16* w16[kChunk];  // optional 16-bit copy of the updated weight (NULL: none)
  int bf16;          // the copies are bfloat16 (else fp16)
  const float* g[kChunk];
  float* m[kChunk];
  float* v[kChunk];
  int64_t n[kChunk];
  int64_t tile_end[kChunk];
  int count;
};

struct AdamHp {
  float lr, b1, b2, eps, wd, bc1, bc2;
};

// Every rounding step spelled out (explicit fma, no contraction left to the
// compiler), so the vector and scalar paths give the same bits whatever
// tile or tensor split an element falls in.
__device__ __forceinline__ void adam1(float& w, float g, float& m, float& v, const AdamHp& h) {
#pragma clang fp contract(off)
  m = __builtin_fmaf(h.b1, m, (1.f - h.b1) * g);
  v = __builtin_fmaf(h.b2, v, (1.f - h.b2) * (g * g));
  const float mh = m / h.bc1, vh = v / h.bc2;
  const float upd = __builtin_fmaf(h.wd, w, mh / (sqrtf(vh) + h.eps));
  w = __builtin_fmaf(-h.lr, upd, w);
}

__global__ __launch_bounds__(256) void adamw_kernel(const AdamChunk c, const AdamHp h,
                                                    const float* scale_dev) {
  const int64_t tile = blockIdx.x;
  const int j = find_tensor(c.tile_end, c.count, tile);
  const int64_t base = (tile - (j ? c.tile_end[j - 1] : 0)) * kTile;
  const float sc = scale_dev ? scale_dev[0] : 1.f;
  // the trainer's guard: a step with non-finite gradients (the clip's NaN
  // scale) leaves weights, moments and 16-bit copies as they are
  if (!isfinite(sc)) return;
  float *w = c.w[j], *m = c.m[j], *v = c.v[j];
  f16* const w16 = c.w16[j];
  const float* g = c.g[j];
  const int64_t n = c.n[j];
  const bool vec = base + kTile <= n &&
                   (((uintptr_t)w | (uintptr_t)g | (uintptr_t)m | (uintptr_t)v) & 15) == 0 &&
                   ((uintptr_t)w16 & 7) == 0;
  if (vec) {
    // every load of the tile is issued before any store (the stores could
    // alias later loads as far as the compiler knows, which would otherwise
    // serialize the four groups)
    float4 W[4], G[4], M[4], V[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = base + 4 * (threadIdx.x + 256 * u);
      W[u] = load_stream(w + e);
      G[u] = load_stream(g + e);
      M[u] = load_stream(m + e);
      V[u] = load_stream(v + e);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = base + 4 * (threadIdx.x + 256 * u);
      adam1(W[u].x, G[u].x * sc, M[u].x, V[u].x, h);
      adam1(W[u].y, G[u].y * sc, M[u].y, V[u].y, h);
      adam1(W[u].z, G[u].z * sc, M[u].z, V[u].z, h);
      adam1(W[u].w, G[u].w * sc, M[u].w, V[u].w, h);
      store_stream(w + e, W[u]);
      store_stream(m + e, M[u]);
      store_stream(v + e, V[u]);
      if (w16) *(half4*)(w16 + e) = to_16x4(W[u], c.bf16);
    }
  } else {
    const int64_t end = min(base + (int64_t)kTile, n);
    for (int64_t e = base + threadIdx.x; e < end; e += 256) {
      float W = w[e], M = m[e], V = v[e];
      adam1(W, g[e] * sc, M, V, h);
      w[e] = W;
      m[e] = M;
      v[e] = V;
      if (w16) w16[e] = to_16(W, c.bf16);
    }
  }
}

int64_t tiles_of(int64_t n) { return (n + kTile - 1) / kTile; }

int nchunks(int n) { return (n + kChunk - 1) / kChunk; }

}  // namespace

size_t clip_scratch(int n, const int64_t* numel) {
  (void)numel;
  return (size_t)nchunks(n) * kSqGrid * sizeof(double);
}

int clip_grad_norm(int n, float* const* g, const int64_t* numel, float max_norm, int apply,
                   float* norm_dev, float* scale_dev, void* scratch, hipStream_t st) {
  double* partial = (double*)scratch;
  const int nc = nchunks(n);
  for (int ci = 0; ci < nc; ++ci) {
    SqChunk c{};
    c.count = 0;
    int64_t acc = 0;
    for (int j = ci * kChunk; j < std::min(n, (ci + 1) * kChunk); ++j) {
      c.p[c.count] = g[j];
      c.n[c.count] = numel[j];
      acc += tiles_of(numel[j]);
      c.tile_end[c.count] = acc;
      ++c.count;
    }
    hipLaunchKernelGGL(sqsum_kernel, dim3(kSqGrid), dim3(256), 0, st, c, partial + (size_t)ci * kSqGrid);
    QBLK_TRY(check_launch("sqsum_kernel"));
  }
  hipLaunchKernelGGL(clip_finalize_kernel, dim3(1), dim3(256), 0, st, nc * kSqGrid, (const double*)partial,
                     max_norm, norm_dev, scale_dev);
  QBLK_TRY(check_launch("clip_finalize_kernel"));
  if (!apply) return 0;
  for (int ci = 0; ci < nc; ++ci) {
    ScaleChunk c{};
    int64_t acc = 0;
    for (int j = ci * kChunk; j < std::min(n, (ci + 1) * kChunk); ++j) {
      c.p[c.count] = g[j];
      c.n[c.count] = numel[j];
      acc += tiles_of(numel[j]);
      c.tile_end[c.count] = acc;
      ++c.count;
    }
    if (acc == 0) continue;
    hipLaunchKernelGGL(scale_kernel, dim3((unsigned)acc), dim3(256), 0, st, c, (const float*)scale_dev);
    QBLK_TRY(check_launch("scale_kernel"));
  }
  return 0;
}

// ------------------------------------------ the clip without a workspace
// For callers that cannot allocate (graph capture, tight loops): the
// squared-sum partials live in a file-scope device array, one copy per GPU,
// whose address is looked up once per device with that device current.
// In host code `scratch` names a host-side stand-in, never device memory:
// only the looked-up pointer is passed to kernels.
constexpr int kStaticClipChunks = 64;  // 2048 tensors
static __device__ __align__(256) double scratch[kStaticClipChunks * kSqGrid];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};
}  // namespace

int static_clip_scratch(void** out) {
  int dev = 0;
  QBLK_TRY(check_hip(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(QBLK_EUNSUPPORTED, "clip (no workspace): device %d", dev);
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    QBLK_TRY(check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(clip scratch)"));
    if (!p) return fail(QBLK_EHIP, "hipGetSymbolAddress(clip scratch) returned NULL");
    g_static_ptr[dev] = p;
  }
  *out = g_static_ptr[dev];
  return QBLK_OK;
}

size_t static_clip_scratch_bytes() { return sizeof(double) * kStaticClipChunks * kSqGrid; }

int adamw(int n, float* const* w, const float* const* g, float* const* m, float* const* v,
          const int64_t* numel, float lr, float b1, float b2, float eps, float wd, int step,
          const float* scale_dev, hipStream_t st, f16* const* w16, bool bf16) {
  AdamHp h;
  h.lr = lr;
  h.b1 = b1;
  h.b2 = b2;
  h.eps = eps;
  h.wd = wd;
  h.bc1 = (float)(1.0 - pow((double)b1, (double)step));
  h.bc2 = (float)(1.0 - pow((double)b2, (double)step));
  for (int ci = 0; ci < nchunks(n); ++ci) {
    AdamChunk c{};
    c.bf16 = bf16;
    int64_t acc = 0;
    for (int j = ci * kChunk; j < std::min(n, (ci + 1) * kChunk); ++j) {
      c.w[c.count] = w[j];
      c.w16[c.count] = w16 ? w16[j] : nullptr;
      c.g[c.count] = g[j];
      c.m[c.count] = m[j];
      c.v[c.count] = v[j];
      c.n[c.count] = numel[j];
      acc += tiles_of(numel[j]);
      c.tile_end[c.count] = acc;
      ++c.count;
    }
    if (acc == 0) continue;
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)acc), dim3(256), 0, st, c, h, scale_dev);
    QBLK_TRY(check_launch("adamw_kernel"));
  }
  return 0;
}

}  // namespace qblk
