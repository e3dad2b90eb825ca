/*
 * qblk.h — C ABI of libqblk: the GPU-resident training step of a Qwen3-style
 * decoder block on AMD MI355X (gfx950).
 *
 * Sources of the operations (docs.rs source pages of the crate
 * aprender-train, module entrenar):
 *   [block]   cuda_block.rs page (0.32.0): CudaTransformerBlock::forward,
 *             compute_attention_cuda, CudaTransformerBlock::backward with
 *             backward_ffn / backward_post_attn_norm / backward_attention /
 *             backward_residual_and_input_norm, optimizer_step, and the
 *             CudaNf4TransformerBlock (quantize_nf4, LoRA, NF4 backward).
 *   [trainer] cuda_trainer.rs page (0.34.0): gpu_forward, train_step_inner
 *             (fused_cross_entropy_cuda), gpu_backward, the squared-sum
 *             global clip and the fused clip state.
 *   [wgpu]    wgpu_trainer.rs page (0.38.0): lora_forward, lora_backward,
 *             ffn_backward, the cross-entropy of train_step.
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or synchronises. Workspace sizes come
 *     from the *_workspace_size queries. Host arrays are marked "host".
 *   - Activations are row-major [T, C] fp32 with token t = b*seq + s; each
 *     batch element is an independent sequence (positions restart at 0 and
 *     the causal mask stays inside it). Weights are [out, in] row-major fp32
 *     and a projection computes y = x W^T.
 *   - Every launch goes on `stream` (a hipStream_t; NULL = legacy default).
 *   - Return 0 (QBLK_OK) or a negative code; qblk_last_error() then holds a
 *     message (thread-local). Invalid arguments are rejected before any
 *     device work. Non-finite values are data, not errors.
 *   - Inputs and outputs must not overlap unless an argument says so.
 *   - Calls are re-entrant: the only library state is the loaded code, the
 *     per-thread error string and the static partial-sum array of
 *     qblk_clip_grad_norm_noalloc (the one entry point that shares state).
 */
#ifndef QBLK_H
#define QBLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* qblk_stream_t; /* = hipStream_t */

enum {
  QBLK_OK = 0,
  QBLK_EINVAL = -1,      /* bad argument: null pointer, shape, workspace too small */
  QBLK_EHIP = -2,        /* HIP launch or runtime error */
  QBLK_EUNSUPPORTED = -3 /* valid request the library does not implement */
};

/* Shapes of one decoder block ([block] TransformerConfig fields used by
 * CudaTransformerBlock::new). Requirements: hidden, intermediate and
 * heads*head_dim multiples of 8; head_dim in {16, 32, 64, 128};
 * heads % kv_heads == 0; seq >= 1, batch >= 1. */
typedef struct {
  int32_t hidden, heads, kv_heads, head_dim, intermediate, seq, batch;
  float eps;            /* RMSNorm epsilon, inside the square root, every norm */
  float rope_theta;     /* NeoX RoPE base: angle = s * theta^(-2i/head_dim) */
  int32_t qk_norm;      /* 1: per-head RMSNorm on Q and K before RoPE */
  int32_t gemm_precision; /* 0: fp32 contractions; 1: fp16 operands (round to
                             nearest even), fp32 accumulate, for every
                             projection and the attention products;
                             2: the same with bfloat16 operands (needs
                             seq*batch, hidden, intermediate and the
                             projection widths multiples of 64, head_dim
                             64 or 128; else QBLK_EUNSUPPORTED) */
} qblk_config;

/* The 11 trainable tensors of a block: w_q [H*d, h], w_k [KV*d, h],
 * w_v [KV*d, h], w_o [h, H*d], w_gate [I, h], w_up [I, h], w_down [h, I],
 * g_in [h], g_post [h], g_q [d], g_k [d] (fp32, device).
 * w16 (optional, gemm_precision 1 only): the fp16 copies of the seven
 * projection weights written by qblk_block_pack_f16 from these same fp32
 * weights ([block] set_fp16_weights keeps such copies). NULL: each
 * forward/backward call casts the weights into its scratch instead, with
 * identical results. The caller re-packs after changing the fp32 weights;
 * the library never checks that the copies are current. */
typedef struct {
  const float *w_q, *w_k, *w_v, *w_o, *w_gate, *w_up, *w_down;
  const float *g_in, *g_post, *g_q, *g_k;
  const void* w16;
} qblk_block_params;

/* Gradient outputs, same shapes; every field is OVERWRITTEN (not added). */
typedef struct {
  float *w_q, *w_k, *w_v, *w_o, *w_gate, *w_up, *w_down;
  float *g_in, *g_post, *g_q, *g_k;
} qblk_block_grads;

/* Bytes of the two workspaces of qblk_block_forward/backward for cfg:
 * `saved` carries the forward activations to the backward (it must stay
 * untouched in between); `scratch` is temporary for either call. */
int32_t qblk_block_workspace_size(const qblk_config* cfg, size_t* saved_bytes,
                                  size_t* scratch_bytes);

/* Bytes of the packed fp16 weight set of a block (qblk_block_params.w16). */
int32_t qblk_block_pack_f16_size(const qblk_config* cfg, size_t* bytes);

/* Writes the packed fp16 weight set ([block] set_fp16_weights, cast_f32_to_f16
 * with round to nearest even; bfloat16 when cfg->gemm_precision is 2) of
 * p's fp32 projection weights into `packed`
 * (device, 16-byte aligned, at least qblk_block_pack_f16_size bytes): each
 * weight as stored and transposed, for the forward and the dX products. */
int32_t qblk_block_pack_f16(const qblk_config* cfg, const qblk_block_params* p, void* packed,
                            size_t packed_bytes, qblk_stream_t stream);

/* Block forward, [block] CudaTransformerBlock::forward and
 * compute_attention_cuda: n1 = RMSNorm(x; g_in); q, k, v = n1 W^T;
 * per-head RMSNorm of q and k (g_q, g_k); NeoX RoPE; GQA causal softmax
 * attention (query head h reads KV head h / (heads/kv_heads)); a = o W_o^T;
 * r1 = x + a; n2 = RMSNorm(r1; g_post); s = silu(n2 W_gate^T) * (n2 W_up^T);
 * y = r1 + s W_down^T.
 * x, y: [T, hidden] (T = seq*batch). saved/scratch: workspaces of at least
 * the sizes reported by qblk_block_workspace_size (16-byte aligned); scratch
 * is required (the GEMMs keep split-K partial sums there). */
int32_t qblk_block_forward(const qblk_config* cfg, const qblk_block_params* p, const float* x,
                           float* y, void* saved, size_t saved_bytes, void* scratch,
                           size_t scratch_bytes, qblk_stream_t stream);

/* Block backward, [block] CudaTransformerBlock::backward: given the x and
 * `saved` of the matching forward and the upstream gradient dy [T, hidden],
 * writes dx [T, hidden] and all 11 parameter gradients (overwritten). The
 * residual gradients are added after each norm backward; the QK-norm
 * backward (absent from the page) is the true derivative. */
int32_t qblk_block_backward(const qblk_config* cfg, const qblk_block_params* p, const float* x,
                            const float* dy, const void* saved, size_t saved_bytes, float* dx,
                            const qblk_block_grads* grads, void* scratch, size_t scratch_bytes,
                            qblk_stream_t stream);

/* The same backward for gradient accumulation over micro-batches ([trainer]
 * GPU-resident gradient accumulation over the accumulation steps: the
 * micro-batches' gradients summed on the device before one clip and one
 * AdamW step): the 11 parameter gradients are added
 * into `grads` (dW products with beta = 1, gamma column sums added), so
 * after k calls they hold the sum over the k micro-batches; a call adds
 * exactly the value qblk_block_backward would write (one fp32 addition per
 * element). dx is overwritten as in qblk_block_backward. Same arguments,
 * workspaces and errors. */
int32_t qblk_block_backward_accumulate(const qblk_config* cfg, const qblk_block_params* p, const float* x,
                                       const float* dy, const void* saved, size_t saved_bytes, float* dx,
                                       const qblk_block_grads* grads, void* scratch, size_t scratch_bytes,
                                       qblk_stream_t stream);

/* Scratch bytes of qblk_fused_cross_entropy (holds the normalised hidden
 * states and the [tokens, vocab] fp32 logits, overwritten by their
 * gradient). */
int32_t qblk_cross_entropy_workspace_size(int32_t tokens, int32_t hidden, int32_t vocab,
                                          size_t* scratch_bytes);

/* Final RMSNorm + LM head + cross-entropy, forward and backward
 * ([trainer] gpu_forward, fused_cross_entropy_cuda, gpu_backward):
 *   hf = RMSNorm(y_last; g_final) (skipped when g_final is NULL);
 *   z = hf W_lm^T with W_lm [vocab, hidden];
 *   loss_partials[t] = logsumexp(z_t) - z_t[targets[t]] (unscaled, fp32);
 *   argmax[t] = first index of the row maximum (NULL: not written);
 *   dz = loss_scale * (softmax(z) - onehot(targets));
 *   dw_lm = dz^T hf (overwritten); dy_last = d/dy_last (overwritten);
 *   dg_final = d/dg_final (overwritten; ignored when g_final is NULL).
 * targets: device int32 [tokens], each in [0, vocab). The loss is
 * loss_scale * sum(loss_partials), summed by the caller. */
int32_t qblk_fused_cross_entropy(int32_t tokens, int32_t hidden, int32_t vocab, float eps,
                                 const float* y_last, const float* g_final, const float* w_lm,
                                 const int32_t* targets, float loss_scale, float* loss_partials,
                                 int32_t* argmax, float* dy_last, float* dg_final, float* dw_lm,
                                 void* scratch, size_t scratch_bytes, qblk_stream_t stream);

/* The same for gradient accumulation over micro-batches: dw_lm and
 * dg_final are added into (dz^T hf and the gamma column sum added with one
 * fp32 addition per element); loss_partials, argmax and dy_last are written
 * as above. With loss_scale = 1 / (all micro-batches' tokens) the sums over
 * the micro-batches are the gradients of the whole batch's mean loss. */
int32_t qblk_fused_cross_entropy_accumulate(int32_t tokens, int32_t hidden, int32_t vocab, float eps,
                                            const float* y_last, const float* g_final, const float* w_lm,
                                            const int32_t* targets, float loss_scale, float* loss_partials,
                                            int32_t* argmax, float* dy_last, float* dg_final, float* dw_lm,
                                            void* scratch, size_t scratch_bytes, qblk_stream_t stream);

/* Scratch bytes of qblk_clip_grad_norm for n tensors (numel: host array). */
int32_t qblk_clip_workspace_size(int32_t n, const int64_t* numel, size_t* scratch_bytes);

/* Global L2 gradient clip ([trainer] squared-sum clip and fused clip state):
 * norm = sqrt(sum over all n tensors of sum g^2) (fp64 final reduction);
 * scale = max_norm / norm if norm > max_norm, else 1; a non-finite norm
 * (some gradient NaN or infinite) gives scale = NaN, which makes
 * qblk_adamw_step skip the update. Writes norm_dev[0]
 * and scale_dev[0] (device fp32). With apply = 1 every gradient is
 * multiplied by scale in place; with apply = 0 they are left untouched
 * (pass scale_dev to qblk_adamw_step instead).
 * grads, numel: host arrays of n device pointers / element counts. */
int32_t qblk_clip_grad_norm(int32_t n, float* const* grads, const int64_t* numel, float max_norm,
                            int32_t apply, float* norm_dev, float* scale_dev, void* scratch,
                            size_t scratch_bytes, qblk_stream_t stream);

/* The same clip without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight loops,
 * harnesses that forbid allocation). Same arguments, results (bitwise
 * those of qblk_clip_grad_norm) and errors, minus `scratch`. Its partial
 * sums live in a library-owned static device array, one per GPU (about
 * 256 KiB, held until the process ends), looked up on the first call on
 * each device; `stream` must belong to the current device. At most
 * QBLK_CLIP_NOALLOC_MAX_TENSORS tensors (QBLK_EINVAL above). Every call on a
 * GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must not be
 * issued; calls ordered on one stream are fine. No allocation, no host
 * synchronisation. */
#define QBLK_CLIP_NOALLOC_MAX_TENSORS 2048
int32_t qblk_clip_grad_norm_noalloc(int32_t n, float* const* grads, const int64_t* numel, float max_norm,
                                    int32_t apply, float* norm_dev, float* scale_dev, qblk_stream_t stream);

/* AdamW on n tensors ([block] optimizer_step, adamw_step_cuda; the formula
 * is not printed: decoupled weight decay with bias correction):
 *   g' = g * (grad_scale_dev ? grad_scale_dev[0] : 1)
 *   m = beta1 m + (1-beta1) g';  v = beta2 v + (1-beta2) g'^2
 *   w = w - lr * (m/(1-beta1^step) / (sqrt(v/(1-beta2^step)) + eps) + weight_decay * w)
 * step >= 1. w, m, v updated in place; g is read only. Pointer arrays and
 * numel are host arrays of device pointers. When grad_scale_dev[0] is not
 * finite (the clip's mark of non-finite gradients) nothing is written: the
 * device-side form of the trainer's guard that skips the optimizer step on
 * a non-finite loss or gradient ([trainer] train_step_inner NaN guard and
 * the accumulated-gradient check before the optimizer). */
int32_t qblk_adamw_step(int32_t n, float* const* w, const float* const* g, float* const* m,
                        float* const* v, const int64_t* numel, float lr, float beta1, float beta2,
                        float eps, float weight_decay, int32_t step, const float* grad_scale_dev,
                        qblk_stream_t stream);

/* AdamW that also writes the 16-bit copy of every updated weight in the same
 * pass (round to nearest even), so a training step with 16-bit GEMM
 * operands needs no separate cast of the fp32 masters ([block]
 * set_fp16_weights refreshes such copies after each update). Same arguments
 * and errors as qblk_adamw_step, plus w16: host array of n device pointers
 * to 16-bit buffers of numel[i] elements (2-byte aligned; an entry may be
 * NULL: no copy for that tensor), and w16_bf16: 0 fp16 copies, 1 bfloat16
 * (match the block's gemm_precision 1 or 2). For the packed set of
 * qblk_block_pack_f16 the pointers are packed + 2 * offset, offsets from
 * qblk_block_pack_f16_offsets. */
int32_t qblk_adamw_step_pack16(int32_t n, float* const* w, const float* const* g, float* const* m,
                               float* const* v, const int64_t* numel, void* const* w16, int32_t w16_bf16, float lr,
                               float beta1, float beta2, float eps, float weight_decay, int32_t step,
                               const float* grad_scale_dev, qblk_stream_t stream);

/* Element offsets (fp16 elements from the start of the packed set) of the
 * seven projection weights w_q, w_k, w_v, w_o, w_gate, w_up, w_down in the
 * packed fp16 weight set of qblk_block_pack_f16 (host array of 7). */
int32_t qblk_block_pack_f16_offsets(const qblk_config* cfg, int64_t* offsets);

/* ---------------------------------------------------------------- NF4 --- */

/* The 16 NormalFloat4 levels used by the NF4 kernels, ascending, written to
 * the HOST array levels[16]. */
int32_t qblk_nf4_codebook(float* levels);

/* NF4 encoding ([block] CudaNf4TransformerBlock, quantize_nf4 over blocks of
 * 64 elements of the flattened row-major tensor): per block a = max|w|
 * (fp32, written to absmax[numel/64]); code = nearest level of w/a computed
 * in fp32 (ties to the lower level; a zero block gets the zero level);
 * element 2i in the low nibble of codes[i] (numel/2 bytes).
 * numel must be a positive multiple of 64. */
int32_t qblk_nf4_quantize(const float* w, int64_t numel, uint8_t* codes, float* absmax,
                          qblk_stream_t stream);

/* w[i] = level[code_i] * absmax[i/64] (fp32). numel must be a positive
 * multiple of 64; codes must be 4-byte and w 16-byte aligned (EINVAL). */
int32_t qblk_nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t numel, float* w,
                            qblk_stream_t stream);

/* Frozen NF4 block with LoRA on all 7 projections ([block]
 * CudaNf4TransformerBlock; LoRA as [wgpu] lora_forward): projection p
 * computes y = x W~_p^T + (alpha/rank) (x A_p^T) B_p^T with
 * W~_p = dequant(codes_p, absmax_p) [out, in], A_p [rank, in], B_p
 * [out, rank] (fp32). Index p: 0 q, 1 k, 2 v, 3 o, 4 gate, 5 up, 6 down.
 * Norm gammas are frozen. */
typedef struct {
  const uint8_t* codes[7];
  const float* absmax[7];
  const float* lora_a[7];
  const float* lora_b[7];
  const float *g_in, *g_post, *g_q, *g_k;
  int32_t rank;
  float alpha;
} qblk_nf4_block_params;

/* LoRA gradients, overwritten: lora_a[p] [rank, in], lora_b[p] [out, rank]. */
typedef struct {
  float* lora_a[7];
  float* lora_b[7];
} qblk_lora_grads;

int32_t qblk_nf4_block_workspace_size(const qblk_config* cfg, int32_t rank, size_t* saved_bytes,
                                      size_t* scratch_bytes);

/* Forward of the NF4 + LoRA block (same chain as qblk_block_forward).
 * Requires cfg->gemm_precision == 1 and rank in {4, 8, 12, 16, 20} (the
 * LoRA columns of the fused Q/K/V product, 3 x rank, ride in one 64-wide
 * K tile). */
int32_t qblk_block_forward_nf4_lora(const qblk_config* cfg, const qblk_nf4_block_params* p,
                                    const float* x, float* y, void* saved, size_t saved_bytes,
                                    void* scratch, size_t scratch_bytes, qblk_stream_t stream);

/* Backward of the NF4 + LoRA block ([block] CudaNf4TransformerBlock::backward;
 * LoRA gradients as [wgpu] lora_backward): dx [T, hidden] and the 14 LoRA
 * gradients only; the base weights and the norm gammas get none. */
int32_t qblk_block_backward_nf4_lora(const qblk_config* cfg, const qblk_nf4_block_params* p,
                                     const float* x, const float* dy, const void* saved,
                                     size_t saved_bytes, float* dx, const qblk_lora_grads* grads,
                                     void* scratch, size_t scratch_bytes, qblk_stream_t stream);

/* Last error message of the calling thread ("" if none). */
const char* qblk_last_error(void);
void qblk_clear_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QBLK_H */
