// 8-bit floating-point operands: per-tensor scaled quantization and the
// fp8 product's C-ABI.
//
// The pages keep 16-bit copies of the weights for their fp16 GEMM tier and
// name a BF16 mode; gfx950 also multiplies 8-bit operands (OCP E4M3 and
// E5M2) at twice the 16-bit MFMA rate. One scale per tensor:
// s = FMAX / max|x| (fp32 division; 1 for an all-zero tensor), each value
// x * s rounded once to fp32, clamped to [-FMAX, FMAX] (a NaN stays NaN),
// then converted with round to nearest even (v_cvt_pk_fp8_f32 /
// v_cvt_pk_bf8_f32). The product multiplies the accumulated sum by both
// operands' 1/s, which the quantizer leaves on the device.
//
// Two launches: per-workgroup maxima of |x| (fixed partition, so the
// maximum is the same on every run), then the conversion, whose workgroups
// each fold the partial maxima again before converting their share; the
// first workgroup stores 1/s.
#include "step.h"

#include "gemm.h"
#include "../../include/qblk.h"
#include "../../include/qblk_ops.h"

namespace qblk {
namespace {

constexpr int kAmaxParts = 1024;
constexpr float kE4m3Max = 448.f, kE5m2Max = 57344.f;

struct Fp8Job {
  int rows, cols;
  const float* x;
  int64_t ldx;
  uint8_t* q;
  int64_t ldq;
  float* parts;  // kAmaxParts partial maxima
  float* inv_scale;
  int e5m2;
  int vec;  // rows of 4-wide float / byte groups (cols, ldx, ldq multiples of 4, aligned)
};

__device__ __forceinline__ float load_x(const Fp8Job& j, int64_t e) {
  const int64_t r = e / j.cols, c = e - r * j.cols;
  return j.x[r * j.ldx + c];
}

__global__ __launch_bounds__(256) void fp8_amax_kernel(const Fp8Job j) {
  __shared__ float red[256];
  const int64_t n = (int64_t)j.rows * j.cols;
  float m = 0.f;
  if (j.vec) {
    const int64_t n4 = n / 4, c4 = j.cols / 4;
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < n4; e += (int64_t)gridDim.x * 256) {
      const int64_t r = e / c4, c = e - r * c4;
      const float4 v = *(const float4*)(j.x + r * j.ldx + 4 * c);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  } else {
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
      m = fmaxf(m, fabsf(load_x(j, e)));
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  if (threadIdx.x == 0) j.parts[blockIdx.x] = red[0];
}

__device__ __forceinline__ float clampf(float v, float lim) {
  // comparisons leave a NaN as it is (fminf / fmaxf would not)
  return v > lim ? lim : (v < -lim ? -lim : v);
}

// Two fp32 values -> two codes in the low 16 bits.
__device__ __forceinline__ uint32_t cvt2(float a, float b, int e5m2) {
  return e5m2 ? (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false)
              : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
}

__global__ __launch_bounds__(256) void fp8_convert_kernel(const Fp8Job j, int nparts) {
  __shared__ float red[256];
  __shared__ float s_scale;
  float m = 0.f;
  for (int i = threadIdx.x; i < nparts; i += 256) m = fmaxf(m, j.parts[i]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  const float fmax = j.e5m2 ? kE5m2Max : kE4m3Max;
  if (threadIdx.x == 0) {
    const float amax = red[0];
    const float s = amax > 0.f ? fmax / amax : 1.f;  // correctly rounded fp32 division
    s_scale = s;
    if (blockIdx.x == 0) j.inv_scale[0] = 1.f / s;
  }
  __syncthreads();
  const float s = s_scale;
  const int64_t n = (int64_t)j.rows * j.cols;
  if (j.vec) {
    const int64_t n4 = n / 4, c4 = j.cols / 4;
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < n4; e += (int64_t)gridDim.x * 256) {
      const int64_t r = e / c4, c = e - r * c4;
      const float4 v = *(const float4*)(j.x + r * j.ldx + 4 * c);
      const uint32_t lo = cvt2(clampf(v.x * s, fmax), clampf(v.y * s, fmax), j.e5m2);
      const uint32_t hi = cvt2(clampf(v.z * s, fmax), clampf(v.w * s, fmax), j.e5m2);
      *(uint32_t*)(j.q + r * j.ldq + 4 * c) = (lo & 0xffffu) | (hi << 16);
    }
  } else {
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
      const int64_t r = e / j.cols, c = e - r * j.cols;
      const float v = clampf(j.x[r * j.ldx + c] * s, fmax);
      j.q[r * j.ldq + c] = (uint8_t)(cvt2(v, 0.f, j.e5m2) & 0xffu);
    }
  }
}

int amax_parts(int rows, int cols) {
  const int64_t n = (int64_t)rows * cols;
  return (int)std::max<int64_t>(1, std::min<int64_t>(kAmaxParts, ceil_div(n, 256 * 16)));
}

}  // namespace
}  // namespace qblk

using namespace qblk;

extern "C" int32_t qblk_fp8_quantize_workspace_size(int32_t rows, int32_t cols, size_t* scratch_bytes) {
  if (rows <= 0 || cols <= 0) return fail(QBLK_EINVAL, "fp8_quantize: bad shape %d x %d", rows, cols);
  if (scratch_bytes) *scratch_bytes = (size_t)kAmaxParts * sizeof(float);
  return QBLK_OK;
}

extern "C" int32_t qblk_fp8_quantize(int32_t rows, int32_t cols, const float* x, int64_t ldx, int32_t e5m2,
                                     uint8_t* q, int64_t ldq, float* inv_scale_dev, void* scratch,
                                     size_t scratch_bytes, qblk_stream_t stream) {
  if (rows <= 0 || cols <= 0) return fail(QBLK_EINVAL, "fp8_quantize: bad shape %d x %d", rows, cols);
  if (!x || !q || !inv_scale_dev || !scratch) return fail(QBLK_EINVAL, "fp8_quantize: null pointer");
  if (ldx < cols || ldq < cols) return fail(QBLK_EINVAL, "fp8_quantize: ldx and ldq must be >= cols");
  if (e5m2 != 0 && e5m2 != 1) return fail(QBLK_EINVAL, "fp8_quantize: e5m2 must be 0 or 1");
  if (scratch_bytes < (size_t)kAmaxParts * sizeof(float) || (uintptr_t)scratch % 4)
    return fail(QBLK_EINVAL, "fp8_quantize: workspace too small or misaligned");
  Fp8Job j;
  j.rows = rows; j.cols = cols; j.x = x; j.ldx = ldx; j.q = q; j.ldq = ldq;
  j.parts = (float*)scratch; j.inv_scale = inv_scale_dev; j.e5m2 = e5m2;
  j.vec = cols % 4 == 0 && ldx % 4 == 0 && ldq % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)q % 4 == 0;
  const int parts = amax_parts(rows, cols);
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(fp8_amax_kernel, dim3(parts), dim3(256), 0, st, j);
  QBLK_TRY(check_launch("fp8_amax_kernel"));
  hipLaunchKernelGGL(fp8_convert_kernel, dim3(parts), dim3(256), 0, st, j, parts);
  return check_launch("fp8_convert_kernel");
}

namespace {
GemmDesc fp8_desc(int32_t M, int32_t N, int32_t K, const uint8_t* A, int64_t lda, int32_t a_e5m2, const uint8_t* B,
                  int64_t ldb, int32_t b_e5m2, const float* a_inv_scale, const float* b_inv_scale, float* C,
                  int64_t ldc, int32_t accumulate) {
  GemmDesc d;
  d.layout = Layout::NT;
  d.prec = Prec::FP8;
  d.M = M; d.N = N; d.K = K;
  d.a = A; d.lda = lda; d.a_src = Src::F8;
  d.b = seg1(B, N); d.ldb = ldb; d.b_src = Src::F8;
  d.c = seg1(C, M); d.ldc = ldc;
  d.accumulate = accumulate;
  d.f8_a_e5m2 = a_e5m2;
  d.f8_b_e5m2 = b_e5m2;
  d.scale_a_dev = a_inv_scale;
  d.scale_b_dev = b_inv_scale;
  return d;
}
}  // namespace

extern "C" int32_t qblk_gemm_fp8_workspace_size(int32_t M, int32_t N, int32_t K, size_t* scratch_bytes) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128) return fail(QBLK_EINVAL, "gemm_fp8: bad shape %d x %d x %d", M, N, K);
  const GemmDesc d = fp8_desc(M, N, K, nullptr, K, 0, nullptr, K, 0, nullptr, nullptr, nullptr, N, 0);
  if (scratch_bytes) *scratch_bytes = gemm_workspace(d);
  return QBLK_OK;
}

extern "C" int32_t qblk_gemm_fp8(int32_t M, int32_t N, int32_t K, const uint8_t* A, int64_t lda, int32_t a_e5m2,
                                 const uint8_t* B, int64_t ldb, int32_t b_e5m2, const float* a_inv_scale,
                                 const float* b_inv_scale, float* C, int64_t ldc, int32_t accumulate, void* scratch,
                                 size_t scratch_bytes, qblk_stream_t stream) {
  if (!A || !B || !C) return fail(QBLK_EINVAL, "gemm_fp8: null operand");
  if ((a_e5m2 != 0 && a_e5m2 != 1) || (b_e5m2 != 0 && b_e5m2 != 1))
    return fail(QBLK_EINVAL, "gemm_fp8: formats must be 0 (E4M3) or 1 (E5M2)");
  if (M <= 0 || N <= 0 || K <= 0 || K % 128) return fail(QBLK_EINVAL, "gemm_fp8: bad shape %d x %d x %d", M, N, K);
  if (lda < K || ldb < K || ldc < N || lda % 16 || ldb % 16 || (uintptr_t)A % 16 || (uintptr_t)B % 16)
    return fail(QBLK_EINVAL, "gemm_fp8: lda, ldb (>= K) must be multiples of 16 and A, B 16-byte aligned");
  GemmDesc d = fp8_desc(M, N, K, A, lda, a_e5m2, B, ldb, b_e5m2, a_inv_scale, b_inv_scale, C, ldc, accumulate);
  if (scratch && (uintptr_t)scratch % 16 == 0) {
    d.ws = (float*)scratch;
    d.ws_bytes = scratch_bytes;
  }
  return gemm(d, (hipStream_t)stream);
}
