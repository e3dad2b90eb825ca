// Internal interface of the MFMA GEMM engine.
//
// C[M,N] (+)= alpha * op(A) op(B) (+ R), fp32 accumulate, fp32 output.
// Three operand layouts cover every projection of the block with weights
// stored [out, in] row-major:
//   NT: A [M,K] K-contiguous, B [N,K] K-contiguous  (forward  y  = x W^T)
//   NN: A [M,K] K-contiguous, B [K,N] N-contiguous  (backward dx = dy W)
//   TN: A [K,M] M-contiguous, B [K,N] N-contiguous  (backward dW = dy^T x)
// Contractions run on v_mfma_f32_32x32x2_f32 (Prec::F32) or, with operands
// rounded to fp16 (nearest even) while they are staged into LDS,
// v_mfma_f32_32x32x16_f16 (Prec::F16).
#pragma once

#include "common.h"

namespace qblk {

// F16 / BF16: operands rounded to fp16 / bfloat16 (nearest even), fp32
// accumulate. With BF16, 16-bit operand storage (Src::F16) holds bfloat16
// bit patterns, and only the direct-to-LDS kernels run (16-bit storage of
// both operands, K a multiple of 64).
// FP8: 8-bit operands (OCP E4M3 or E5M2 per operand, see f8_a_e5m2 /
// f8_b_e5m2) in 8-bit storage (Src::F8), NT only, K a multiple of 128,
// on v_mfma_f32_32x32x64_f8f6f4; the product is multiplied by the device
// scalars scale_a_dev[0] * scale_b_dev[0] (the operands' inverse scales).
enum class Prec : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };
enum class Layout : int { NT = 0, NN = 1, TN = 2 };
enum class Src : int { F32 = 0, F16 = 1, NF4 = 2, F8 = 3 };

// Up to three row segments stored at different addresses that together act
// as one matrix: storage row r lives in segment s with start[s] <= r <
// start[s+1], at p[s] + (r - start[s]) * ld. Used to treat [Wq; Wk; Wv]
// (and [Wg; Wu]) as one operand and to split a dW output over its tensors.
struct Seg {
  const void* p[3] = {nullptr, nullptr, nullptr};
  int32_t start[4] = {0, 0, 0, 0};  // start[nseg] = total rows
  int32_t nseg = 1;
};

__host__ __device__ inline Seg seg1(const void* p, int rows) {
  Seg s;
  s.p[0] = p;
  s.start[0] = 0;
  s.start[1] = rows;
  s.nseg = 1;
  return s;
}

// NF4 operand: per segment packed codes (2 per byte, low nibble first) and
// one fp32 scale per 64 consecutive elements of the row-major storage.
struct Nf4Seg {
  const uint8_t* codes[3] = {nullptr, nullptr, nullptr};
  const float* scales[3] = {nullptr, nullptr, nullptr};
  float levels[16] = {};  // the NF4 codebook (filled by nf4_codebook_host)
};

// The 16 NormalFloat4 levels, ascending, as fp32 (computed once on the host).
const float* nf4_codebook_host();

// Optional extra K columns appended to the contraction (LoRA):
//   C += A_ext[M, kext] * B_ext^T.
// A_ext is fp32 [M, kext] K-contiguous, times a_scale. For NT, B_ext is
// fp32 [N, kext] K-contiguous; for NN it is fp32 [kext, N] N-contiguous.
// When blockdiag > 0, B_ext is block diagonal over the B segments: the
// rows (NT) or columns (NN) of B-segment s only see ext columns
// [s*blockdiag, (s+1)*blockdiag), and b_ext holds one pointer per segment.
struct KExt {
  int32_t kext = 0;
  const float* a = nullptr;
  int64_t lda = 0;
  float a_scale = 1.f;
  const float* b[3] = {nullptr, nullptr, nullptr};
  int64_t ldb = 0;
  int32_t blockdiag = 0;
};

struct GemmDesc {
  Layout layout = Layout::NT;
  Prec prec = Prec::F32;
  int32_t M = 0, N = 0, K = 0;
  const void* a = nullptr;
  int64_t lda = 0;
  Src a_src = Src::F32;
  Seg b;
  int64_t ldb = 0;
  Src b_src = Src::F32;
  Nf4Seg nf4;          // when b_src == Src::NF4
  Seg c;               // fp32 output rows (segments along M)
  int64_t ldc = 0;
  const float* r = nullptr;  // optional residual [M, N] added in the epilogue
  int64_t ldr = 0;
  int32_t accumulate = 0;    // 1: C += result
  float alpha = 1.f;
  KExt ext;
  // When c_cols_blockdiag > 0 the output keeps only columns
  // [s*c_cols_blockdiag, (s+1)*c_cols_blockdiag) of rows in C-segment s,
  // written at column 0 of that segment (the diagonal blocks of a product).
  int32_t c_cols_blockdiag = 0;
  // Optional workspace for split-K partial sums (deterministic: partials
  // are added in a fixed order by a second kernel). NULL: no split.
  float* ws = nullptr;
  size_t ws_bytes = 0;
  // Optional fp16 copy of the final output (single C segment, no
  // diagonal-block mode): c16[row * ldc16 + col] = (fp16) C[row, col].
  f16* c16 = nullptr;
  int64_t ldc16 = 0;
  // Fused-NF4 kernel (fp16 A, NF4 B) only: one more 64-wide K tile of fp16
  // operands contracted after the K columns of A and B (the LoRA branch):
  // C += ext16_a [M, 64] * ext16_b^T with ext16_b [N, 64] (NT) or
  // [64, N] (NN), row strides ext16_lda / ext16_ldb. NULL: none.
  const f16* ext16_a = nullptr;
  int64_t ext16_lda = 0;
  const f16* ext16_b = nullptr;
  int64_t ext16_ldb = 0;
  // FP8 only: operand formats (0 E4M3, 1 E5M2) and the device scalars
  // the accumulated product is multiplied by (NULL: 1).
  int32_t f8_a_e5m2 = 0, f8_b_e5m2 = 0;
  const float* scale_a_dev = nullptr;
  const float* scale_b_dev = nullptr;
};

int gemm(const GemmDesc& d, hipStream_t stream);
// Whether gemm() runs this NF4-B product on the fused decode kernel (fp16
// A, NT or NN, K and ldb multiples of 64, see gemm.hip); ext16_* need it.
bool gemm_nf4_fused(const GemmDesc& d);
// Split-K workspace bytes of the fused NF4 kernel for an M x N product over
// k_total K columns (the LoRA tile included).
size_t gemm_nf4_workspace(int M, int N, int k_total);
// Bytes of split-K workspace the GEMM would use for this shape (0 if none).
size_t gemm_workspace(const GemmDesc& d);

}  // namespace qblk
