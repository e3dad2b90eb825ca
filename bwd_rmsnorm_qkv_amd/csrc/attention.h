// Internal interface of the GQA causal attention kernels.
#pragma once

#include "common.h"
#include "gemm.h"

namespace qblk {

struct AttnArgs {
  int batch, seq, heads, kv_heads, head_dim;
  const float* q;  int64_t ldq;   // [T, heads*d] (row stride ldq)
  const float* k;  int64_t ldk;   // [T, kv_heads*d]
  const float* v;  int64_t ldv;
  float* o;        int64_t ldo;   // [T, heads*d]
  float* lse;                     // [batch, heads, seq], natural log
  // backward only
  const float* d_o; int64_t lddo;
  float* dq; int64_t lddq;
  float* dk; int64_t lddk;
  float* dv; int64_t lddv;
};

int attention_check(int batch, int seq, int heads, int kv_heads, int head_dim);
size_t attention_bwd_scratch(int batch, int seq, int heads, int head_dim);
int attention_kv_split(int batch, int seq, int heads);
// Whether the per-head kernels take one tile per 2-wave workgroup instead of
// causal tile pairs (16-bit operands, no key-range split, at least two
// (tile, head) units per CU).
bool attention_unpaired(int batch, int seq, int heads, bool sixteen_bit);
int attention_group_waves(int batch, int seq, int heads, int kv_heads);
int attention_forward(const AttnArgs& a, Prec p, hipStream_t st);
int attention_backward(const AttnArgs& a, Prec p, void* scratch, hipStream_t st);

}  // namespace qblk

namespace qblk {

// Attention on tiled copies (head_dim 64 or 128, seq a multiple of 8): the
// operands are 16-bit copies (fp32 = 0) or fp32 tensors (fp32 = 1, head_dim
// 64): q, k, v row-major [T, heads*d] / [T, kv_heads*d] and d_o
// [T, heads*d]. Every tile reaches LDS by direct global -> LDS copies; the
// transposed operands (V^T, K^T, Q^T, dO^T) are read out of the row tiles.
struct AttnDmaArgs {
  int batch, seq, heads, kv_heads, head_dim;
  int fp32;
  const void *q, *k, *v;    int64_t ldq, ldk, ldv;
  float* o; int64_t ldo;   // fp32 [T, heads*d]
  f16* o16;                // optional fp16 copy of o (same stride), may be NULL
  float* lse;              // [batch, heads, seq], natural log
  // backward only
  const void* d_o; int64_t lddo;
  const float* do32; int64_t lddo32;  // fp32 dO (for delta = rowsum(dO o))
  float* dq; int64_t lddq;
  float* dk; int64_t lddk;
  float* dv; int64_t lddv;
  f16* dv16 = nullptr; int64_t lddv16 = 0;  // optional fp16 copy of dv
  int bf16 = 0;  // 16-bit operands and copies are bfloat16 (else fp16)
  // set by the launches: key-range splits, the backward's partial dQ and
  // the forward's partial outputs with their (max, sum) pairs
  int split = 1;
  float* dq_part = nullptr;
  float* o_part = nullptr;
  float* ml_part = nullptr;
};

bool attention_dma_supported(int batch, int seq, int heads, int kv_heads, int head_dim);
// scratch: attention_bwd_scratch bytes (the forward's key-range splits
// keep their partial outputs there), or NULL for no split.
int attention_dma_forward(const AttnDmaArgs& a, void* scratch, hipStream_t st);
// scratch: attention_bwd_scratch bytes.
int attention_dma_backward(const AttnDmaArgs& a, void* scratch, hipStream_t st);

}  // namespace qblk
