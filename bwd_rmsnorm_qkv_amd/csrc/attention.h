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
int attention_forward(const AttnArgs& a, Prec p, hipStream_t st);
int attention_backward(const AttnArgs& a, Prec p, void* scratch, hipStream_t st);

}  // namespace qblk
