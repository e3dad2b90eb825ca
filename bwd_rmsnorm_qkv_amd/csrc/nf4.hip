// NF4 encoding of frozen projection weights and its decoder.
//
// cuda_block.rs page, CudaNf4TransformerBlock: quantize_nf4 over blocks of
// NF4_BLOCK_SIZE elements of each flattened [out, in] weight, packed codes
// plus one scale per block. The page prints neither the codebook nor the
// quantizer; this follows the NormalFloat4 construction of the QLoRA paper
// (Dettmers et al., 2023) with an absmax scale per 64 elements, the nearest
// level taken in fp32 (ties to the lower level), the zero level for an
// all-zero block, and element 2i in the low nibble of byte i.
#include "step.h"

#include <cmath>

#include "gemm.h"
#include "../../include/qblk.h"

namespace qblk {
namespace {

// Standard normal quantile by bisection on erfc (fp64, to full precision).
double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 400; ++it) {
    const double mid = 0.5 * (lo + hi);
    const double cdf = 0.5 * std::erfc(-mid / std::sqrt(2.0));
    if (cdf < p)
      lo = mid;
    else
      hi = mid;
    if (hi - lo <= 0.0) break;
  }
  return 0.5 * (lo + hi);
}

struct Codebook {
  float level[16];
  float mid[15];
  Codebook() {
    // 8 positive quantiles at probabilities spaced evenly from delta towards
    // 1/2 (the 1/2 end excluded), 7 negative ones likewise, and an exact
    // zero; delta is the mean of 1 - 1/(2*15) and 1 - 1/(2*16); scaled so
    // the largest magnitude is 1.
    const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
    double v[16];
    int k = 0;
    for (int i = 0; i < 7; ++i) v[k++] = -normal_quantile(delta + (0.5 - delta) * i / 7.0);
    v[k++] = 0.0;
    for (int i = 0; i < 8; ++i) v[k++] = normal_quantile(delta + (0.5 - delta) * i / 8.0);
    const double top = normal_quantile(delta);
    // ascending order
    double s[16];
    for (int i = 0; i < 7; ++i) s[i] = v[i];  // v[0] = -top is the most negative
    s[7] = 0.0;
    for (int i = 0; i < 8; ++i) s[8 + i] = v[8 + (7 - i)];
    for (int i = 0; i < 16; ++i) level[i] = (float)(s[i] / top);
    for (int i = 0; i < 15; ++i) mid[i] = (level[i] + level[i + 1]) * 0.5f;  // fp32 arithmetic
  }
};

const Codebook& codebook() {
  static const Codebook cb;
  return cb;
}

struct QuantArgs {
  float mid[15];
};

__global__ __launch_bounds__(256) void nf4_quantize_kernel(const float* __restrict__ w, int64_t nblocks,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ absmax, QuantArgs q) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;
  const float x = w[blk * 64 + lane];
  const float a = wave_max(fabsf(x));
  int code = 7;
  if (a > 0.f) {
    const float r = x / a;
    code = 0;
#pragma unroll
    for (int c = 0; c < 15; ++c) code += (q.mid[c] < r) ? 1 : 0;
  }
  const int hi = __shfl_down(code, 1, kWave);
  if ((lane & 1) == 0) codes[blk * 32 + (lane >> 1)] = (uint8_t)(code | (hi << 4));
  if (lane == 0) absmax[blk] = a;
}

struct LevelArgs {
  float level[16];
};

// fp32 decode: 8 elements (4 code bytes, one scale) per thread, the 16
// levels from an LDS copy of the codebook; two 16-byte stores.
__global__ __launch_bounds__(256) void nf4_dequant_kernel(const uint32_t* __restrict__ codes,
                                                          const float* __restrict__ absmax, int64_t n8,
                                                          float4* __restrict__ w, LevelArgs L) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = L.level[threadIdx.x];
  __syncthreads();
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const uint32_t b = codes[i];
  const float a = absmax[i >> 3];
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = lv[(b >> (4 * j)) & 15] * a;
  w[2 * i] = make_float4(o[0], o[1], o[2], o[3]);
  w[2 * i + 1] = make_float4(o[4], o[5], o[6], o[7]);
}

// fp16 decode for the GEMMs: 8 elements (4 code bytes, one scale) per
// thread; L[c] * a in fp32, rounded once to fp16.
__global__ __launch_bounds__(256) void nf4_dequant_f16_kernel(const uint32_t* __restrict__ codes,
                                                              const float* __restrict__ absmax, int64_t n8,
                                                              half8* __restrict__ w, LevelArgs L) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = L.level[threadIdx.x];
  __syncthreads();
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const uint32_t b = codes[i];
  const float a = absmax[i >> 3];
  half8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = (f16)(lv[(b >> (4 * j)) & 15] * a);
  w[i] = o;
}

}  // namespace

const float* nf4_codebook_host() { return codebook().level; }

int nf4_dequantize_f16(const uint8_t* codes, const float* absmax, int64_t numel, f16* w, hipStream_t st) {
  if (numel <= 0 || numel % 64) return fail(QBLK_EINVAL, "nf4_dequantize_f16: numel %lld not a positive multiple of 64", (long long)numel);
  if (((uintptr_t)codes & 3) || ((uintptr_t)w & 15)) return fail(QBLK_EINVAL, "nf4_dequantize_f16: misaligned buffer");
  LevelArgs L;
  for (int i = 0; i < 16; ++i) L.level[i] = codebook().level[i];
  const int64_t n8 = numel / 8;
  hipLaunchKernelGGL(nf4_dequant_f16_kernel, dim3((unsigned)ceil_div(n8, 256)), dim3(256), 0, st,
                     (const uint32_t*)codes, absmax, n8, (half8*)w, L);
  return check_launch("nf4_dequant_f16_kernel");
}

int nf4_quantize(const float* w, int64_t numel, uint8_t* codes, float* absmax, hipStream_t st) {
  if (numel <= 0 || numel % 64) return fail(QBLK_EINVAL, "nf4_quantize: numel %lld not a positive multiple of 64", (long long)numel);
  QuantArgs q;
  for (int i = 0; i < 15; ++i) q.mid[i] = codebook().mid[i];
  const int64_t nb = numel / 64;
  hipLaunchKernelGGL(nf4_quantize_kernel, dim3((unsigned)ceil_div(nb, 4)), dim3(256), 0, st, w, nb, codes,
                     absmax, q);
  return check_launch("nf4_quantize_kernel");
}

int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t numel, float* w, hipStream_t st) {
  if (numel <= 0 || numel % 64) return fail(QBLK_EINVAL, "nf4_dequantize: numel %lld not a positive multiple of 64", (long long)numel);
  if (((uintptr_t)codes & 3) || ((uintptr_t)w & 15)) return fail(QBLK_EINVAL, "nf4_dequantize: misaligned buffer");
  LevelArgs L;
  for (int i = 0; i < 16; ++i) L.level[i] = codebook().level[i];
  const int64_t n8 = numel / 8;
  hipLaunchKernelGGL(nf4_dequant_kernel, dim3((unsigned)ceil_div(n8, 256)), dim3(256), 0, st,
                     (const uint32_t*)codes, absmax, n8, (float4*)w, L);
  return check_launch("nf4_dequant_kernel");
}

}  // namespace qblk

extern "C" int32_t qblk_nf4_codebook(float* levels) {
  if (!levels) return qblk::fail(QBLK_EINVAL, "qblk_nf4_codebook: null");
  for (int i = 0; i < 16; ++i) levels[i] = qblk::codebook().level[i];
  return QBLK_OK;
}
