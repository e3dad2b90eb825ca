// Internal interface of the block composition.
#pragma once

#include <functional>

#include "common.h"
#include "../../include/qblk.h"

namespace qblk {

// Forward activations kept for the backward (caller-owned `saved`).
struct Saved {
  float2* tab;     // RoPE cos/sin [seq, d/2]
  float* rho1;     // [T]
  float* n1;       // [T, h]
  float* qkv;      // [T, (H + 2KV) d] projection outputs before QK-norm
  float* rho_q;    // [T, H]
  float* rho_k;    // [T, KV]
  float* qr;       // [T, H d] attention queries (after QK-norm + RoPE)
  float* kr;       // [T, KV d] attention keys
  float* o;        // [T, H d] attention output
  float* lse;      // [B, H, S]
  float* r1;       // [T, h]
  float* rho2;     // [T]
  float* n2;       // [T, h]
  float* gu;       // [T, 2I] gate | up
  float* s;        // [T, I] SwiGLU output
  // Attention on tiled copies (when use_attention_dma) with 16-bit
  // operands: 16-bit copies of the attention inputs; NULL otherwise (fp32
  // configs read the fp32 tensors themselves).
  f16 *q16, *k16, *v16;
  // fp16 copies of the projection inputs n1, o, n2, s (fp16-operand configs
  // with T a multiple of 8), written by their producers; NULL otherwise.
  f16 *n1_16, *o16, *n2_16, *s16;
};

// The attention kernels on tiled copies apply to this config.
bool use_attention_dma(const qblk_config& c);

// fp16 copies of the dense block's projection weights W [out, in], read
// K-major by the forward (x W^T) and out-major by dX = dY W; [Wq; Wk; Wv]
// and [Wg; Wu] are stored stacked.
struct Packed16 {
  f16 *qkv, *o, *gu, *d;  // [qkv, h], [h, qd], [2I, h], [h, I]
};
void carve_pack16(const qblk_config& c, void* base, Packed16& p, size_t& bytes);
// Casts (round to nearest even) the weights of p into `out`.
int pack16(const qblk_config& c, const qblk_block_params& p, const Packed16& out, hipStream_t st);

// Backward temporaries (caller-owned `scratch`).
struct Scratch {
  float *ds, *dgu, *dn2, *dr1, *d_o, *dqr, *dkr, *dqkv, *dn1;
  char* attn;
  // per-block gamma-gradient partial sums: the post-attention norm's, the
  // QK norms', the input norm's (all summed by one launch at the end)
  float *red, *red_qk, *red_in;
  float* gemm_ws;  // split-K partial sums of the block's GEMMs
  size_t gemm_ws_bytes;
  // fp16-operand dense block only: operand copies and, when the caller
  // passes no packed weights, the weights' fp16 copies.
  f16* a16;  // fp16 copy of the current output gradient
  Packed16 pack;
  f16* do16;          // attention on tiled copies: dO copy (fp16 configs)
  // Set by the fp16-copies backward: producers write each output gradient's
  // fp16 copy straight into a16 and the projection hooks are then passed a
  // null fp32 gradient (the copy is already in a16).
  bool prod16 = false;
};

void carve_saved(const qblk_config& c, void* base, Saved& s, size_t& bytes);
// lora_rank > 0 (the NF4 block) sizes the GEMM workspace for the NF4 +
// LoRA GEMMs and leaves out the dense fp16 buffers.
void carve_scratch(const qblk_config& c, void* base, Scratch& s, size_t& bytes, int lora_rank = 0);
int check_config(const qblk_config* c);

// The projections of a block, forward: qkv = n1 [Wq;Wk;Wv]^T;
// out = res + o Wo^T; gu = n2 [Wg;Wu]^T; out = res + s Wd^T.
struct ProjFwd {
  std::function<int(const float*, float*, hipStream_t)> qkv;
  std::function<int(const float*, const float*, float*, hipStream_t)> o;
  std::function<int(const float*, float*, hipStream_t)> gate_up;
  std::function<int(const float*, const float*, float*, hipStream_t)> down;
};

// Backward: (dY, X, dX) per projection; the implementation also produces
// whatever parameter gradients it owns.
struct ProjBwd {
  std::function<int(const float*, const float*, float*, hipStream_t)> qkv, o, gate_up, down;
};

// attn_ws: the scratch's attention region (the forward's key-range
// splits keep partial outputs there), or NULL.
int block_forward_impl(const qblk_config& c, const ProjFwd& proj, const float* g_in, const float* g_post,
                       const float* g_q, const float* g_k, const float* x, float* y, const Saved& s,
                       void* attn_ws, hipStream_t st);
int block_backward_impl(const qblk_config& c, const ProjBwd& proj, const float* g_in, const float* g_post,
                        const float* g_q, const float* g_k, const float* x, const float* dy, const Saved& s,
                        float* dx, float* dg_in, float* dg_post, float* dg_q, float* dg_k, const Scratch& w,
                        hipStream_t st, bool accumulate = false);

int dense_block_forward(const qblk_config& c, const qblk_block_params& p, const float* x, float* y,
                        const Saved& s, const Scratch& w, hipStream_t st);
// accumulate: the parameter gradients are added into gr (micro-batch
// accumulation) instead of overwritten; dx is written either way.
int dense_block_backward(const qblk_config& c, const qblk_block_params& p, const qblk_block_grads& gr,
                         const float* x, const float* dy, const Saved& s, float* dx, const Scratch& w,
                         hipStream_t st, bool accumulate = false);

}  // namespace qblk
