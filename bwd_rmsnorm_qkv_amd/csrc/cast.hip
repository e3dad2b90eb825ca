// fp32 -> fp16 or bfloat16 (round to nearest even) copies of a row-major
// matrix, plain and/or transposed, for the 16-bit-operand contractions:
// every product of the block then reads both operands K-contiguous.
//
// One workgroup converts a 64 x 64 tile: 16-byte loads along the rows, the
// plain copy stored straight from registers, the transposed one through an
// LDS tile whose 65-float pitch keeps the column reads conflict-free.
#include "norms.h"

#include "../../include/qblk.h"

namespace qblk {
namespace {

__global__ __launch_bounds__(256) void cast_f16_kernel(int R, int C, const float* __restrict__ in, int64_t ldi,
                                                       f16* __restrict__ out, int64_t ldo,
                                                       f16* __restrict__ outT, int64_t ldt, int bf16) {
  __shared__ float tile[64][65];
  const int t = threadIdx.x;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int lc = (t & 15) * 4;
  const int col = c0 + lc;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int lr = p * 16 + (t >> 4);
    const int row = r0 + lr;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < R && col < C) v = *(const float4*)(in + (int64_t)row * ldi + col);
    if (out && row < R && col < C) {
      *(half4*)(out + (int64_t)row * ldo + col) = to_16x4(v, bf16);
    }
    tile[lr][lc] = v.x;
    tile[lr][lc + 1] = v.y;
    tile[lr][lc + 2] = v.z;
    tile[lr][lc + 3] = v.w;
  }
  if (!outT) return;
  __syncthreads();
  // outT row = input column; 16 threads cover 64 input rows, 4 each.
  const int lr = (t & 15) * 4;
  const int row = r0 + lr;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int lcc = p * 16 + (t >> 4);
    const int c = c0 + lcc;
    if (c >= C) continue;
    f16* dst = outT + (int64_t)c * ldt + row;
    if (row + 3 < R) {
      *(half4*)dst = to_16x4(make_float4(tile[lr][lcc], tile[lr + 1][lcc], tile[lr + 2][lcc], tile[lr + 3][lcc]),
                             bf16);
    } else {
      for (int j = 0; j < 4 && row + j < R; ++j) dst[j] = to_16(tile[lr + j][lcc], bf16);
    }
  }
}

// The copy alone (no transpose): float4 column j of row blockIdx.y (+
// k gridDim.y) per thread, no LDS.
__global__ __launch_bounds__(256) void cast_f16_rows_kernel(int R, int C, const float* __restrict__ in, int64_t ldi,
                                                            f16* __restrict__ out, int64_t ldo, int bf16) {
  const int j = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (j >= C) return;
  for (int r = blockIdx.y; r < R; r += gridDim.y)
    *(half4*)(out + (int64_t)r * ldo + j) = to_16x4(*(const float4*)(in + (int64_t)r * ldi + j), bf16);
}

}  // namespace


int cast_f16(int R, int C, const float* in, int64_t ldi, f16* out, int64_t ldo, f16* outT, int64_t ldt,
             hipStream_t st, bool bf16) {
  if (R <= 0 || C <= 0) return fail(QBLK_EINVAL, "cast_f16: bad shape %d x %d", R, C);
  if (C % 4 || ldi % 4 || (out && ldo % 4) || (outT && ldt % 4))
    return fail(QBLK_EINVAL, "cast_f16: columns and leading dimensions must be multiples of 4");
  if (!in || (!out && !outT)) return fail(QBLK_EINVAL, "cast_f16: null pointer");
  if (!outT) {
    const dim3 g((unsigned)ceil_div(C, 1024), (unsigned)std::min(R, 65535));
    hipLaunchKernelGGL(cast_f16_rows_kernel, g, dim3(256), 0, st, R, C, in, ldi, out, ldo, (int)bf16);
    return check_launch("cast_f16_rows_kernel");
  }
  const dim3 grid((unsigned)ceil_div(C, 64), (unsigned)ceil_div(R, 64));
  hipLaunchKernelGGL(cast_f16_kernel, grid, dim3(256), 0, st, R, C, in, ldi, out, ldo, outT, ldt, (int)bf16);
  return check_launch("cast_f16_kernel");
}

}  // namespace qblk
