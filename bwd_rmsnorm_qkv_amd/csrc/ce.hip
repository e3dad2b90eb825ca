// Cross-entropy over materialised logits, in place.
//
// cuda_trainer.rs page, train_step_inner: fused_cross_entropy_cuda overwrites
// the [seq, vocab] logits with (softmax - onehot) * loss_scale and hands back
// the per-token loss partials (the only device-to-host transfer of the step).
// One workgroup owns a row at a time: pass 1 keeps an online max/sum of
// exp and the first index of the maximum; pass 2 writes the gradient. The
// row (vocab * 4 bytes) is re-read from L2/MALL in pass 2.
#include "step.h"

#include <algorithm>

#include "../../include/qblk.h"

namespace qblk {
namespace {

struct MS {
  float m, s;
  int idx;
};

__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  MS r;
  r.m = fmaxf(a.m, b.m);
  r.s = (a.m == -INFINITY ? 0.f : a.s * expf(a.m - r.m)) + (b.m == -INFINITY ? 0.f : b.s * expf(b.m - r.m));
  r.idx = (b.m > a.m || (b.m == a.m && b.idx < a.idx)) ? b.idx : a.idx;
  return r;
}

__device__ __forceinline__ void ms_add(MS& a, float z, int j) {
  if (z > a.m) {
    a.s = a.s * expf(a.m - z) + 1.f;
    a.m = z;
    a.idx = j;
  } else {
    a.s += expf(z - a.m);
  }
}

// Rows are taken grid-stride by CE_WGS workgroups of CE_THREADS threads
// (one per CU): at most CE_WGS rows are in flight, so pass 2 re-reads a row
// that pass 1 left in the 256 MB last-level cache (a 151936-wide fp32 row is
// 0.6 MB; 256 of them 156 MB) instead of fetching it again from HBM. On the
// [1024, 151936] logits: 396 us with a 256-thread workgroup per row, 367 us
// this way.
constexpr int CE_THREADS = 1024, CE_WGS = 256;

__global__ __launch_bounds__(CE_THREADS) void ce_rows_kernel(int T, int V, float* z, const int32_t* tgt, float scale,
                                                             float* loss, int32_t* argmax) {
  __shared__ MS red[CE_THREADS];
  const int tid = threadIdx.x;
  const bool vec = (V % 4) == 0;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    float* row = z + (int64_t)t * V;
    MS a{-INFINITY, 0.f, 0x7fffffff};
    if (vec) {
      const float4* r4 = (const float4*)row;
      for (int c = tid; c < V / 4; c += CE_THREADS) {
        const float4 q = r4[c];
        ms_add(a, q.x, 4 * c);
        ms_add(a, q.y, 4 * c + 1);
        ms_add(a, q.z, 4 * c + 2);
        ms_add(a, q.w, 4 * c + 3);
      }
    } else {
      for (int j = tid; j < V; j += CE_THREADS) ms_add(a, row[j], j);
    }
    red[tid] = a;
    __syncthreads();
    for (int o = CE_THREADS / 2; o > 0; o >>= 1) {
      if (tid < o) red[tid] = ms_merge(red[tid], red[tid + o]);
      __syncthreads();
    }
    const MS all = red[0];
    const float lse = all.m + logf(all.s);
    // A target outside [0, V) is reported as a NaN loss and gets no onehot
    // term (no out-of-range access).
    const int tg0 = tgt[t];
    const bool ok = tg0 >= 0 && tg0 < V;
    const int tg = ok ? tg0 : -8;
    if (tid == 0) {
      loss[t] = ok ? lse - row[tg] : __builtin_nanf("");
      if (argmax) argmax[t] = all.idx;
    }
    __syncthreads();  // row[tg] and red[0] read before they are overwritten
    if (vec) {
      float4* r4 = (float4*)row;
      for (int c = tid; c < V / 4; c += CE_THREADS) {
        float4 q = r4[c];
        q.x = expf(q.x - lse);
        q.y = expf(q.y - lse);
        q.z = expf(q.z - lse);
        q.w = expf(q.w - lse);
        if ((tg >> 2) == c) {
          const int k = tg & 3;
          if (k == 0) q.x -= 1.f;
          else if (k == 1) q.y -= 1.f;
          else if (k == 2) q.z -= 1.f;
          else q.w -= 1.f;
        }
        q.x *= scale; q.y *= scale; q.z *= scale; q.w *= scale;
        r4[c] = q;
      }
    } else {
      for (int j = tid; j < V; j += CE_THREADS) {
        float p = expf(row[j] - lse);
        if (j == tg) p -= 1.f;
        row[j] = p * scale;
      }
    }
  }
}

}  // namespace

int ce_rows(int T, int V, float* z, const int32_t* tgt, float scale, float* loss, int32_t* argmax,
            hipStream_t st) {
  const unsigned wgs = (unsigned)std::min(T, CE_WGS);
  hipLaunchKernelGGL(ce_rows_kernel, dim3(wgs), dim3(CE_THREADS), 0, st, T, V, z, tgt, scale, loss, argmax);
  return check_launch("ce_rows_kernel");
}

}  // namespace qblk
