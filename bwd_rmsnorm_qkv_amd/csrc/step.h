// Internal interface of the step kernels: cross-entropy rows, the global
// gradient norm and clip, AdamW, and NF4 encode/decode.
#pragma once

#include "common.h"

namespace qblk {

// Per row t of z [T, V] (in place): loss[t] = logsumexp(z_t) - z_t[tgt_t];
// argmax[t] (optional); z_t <- scale * (softmax(z_t) - onehot(tgt_t)).
int ce_rows(int T, int V, float* z, const int32_t* tgt, float scale, float* loss, int32_t* argmax,
            hipStream_t st);

size_t clip_scratch(int n, const int64_t* numel);
int clip_grad_norm(int n, float* const* g, const int64_t* numel, float max_norm, int apply,
                   float* norm_dev, float* scale_dev, void* scratch, hipStream_t st);
// The per-device static partial-sum array of the no-workspace clip (looked
// up on the current device) and its size in bytes.
int static_clip_scratch(void** out);
size_t static_clip_scratch_bytes();
// w16 (optional host array, entries may be NULL): a 16-bit copy (fp16, or
// bfloat16 with bf16; round to nearest even) of each updated weight written
// in the same pass.
int adamw(int n, float* const* w, const float* const* g, float* const* m, float* const* v,
          const int64_t* numel, float lr, float b1, float b2, float eps, float wd, int step,
          const float* scale_dev, hipStream_t st, f16* const* w16 = nullptr, bool bf16 = false);

int nf4_quantize(const float* w, int64_t numel, uint8_t* codes, float* absmax, hipStream_t st);
// fp16 decode (L[c] * a in fp32, rounded to nearest even) for the GEMMs.
int nf4_dequantize_f16(const uint8_t* codes, const float* absmax, int64_t numel, f16* w, hipStream_t st);
int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t numel, float* w,
                   hipStream_t st);

}  // namespace qblk
