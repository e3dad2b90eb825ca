// C-ABI entry points of libqblk: argument checks, workspace sizes, and the
// calls into the kernels. Declarations and documentation: include/qblk.h
// and include/qblk_ops.h.
#include "../../include/qblk.h"
#include "../../include/qblk_ops.h"
#include "attention.h"
#include "block.h"
#include "gemm.h"
#include "norms.h"
#include "step.h"

using namespace qblk;

namespace {

hipStream_t S(qblk_stream_t s) { return (hipStream_t)s; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" {

// ------------------------------------------------------------------ block

int32_t qblk_block_workspace_size(const qblk_config* cfg, size_t* saved_bytes, size_t* scratch_bytes) {
  QBLK_TRY(check_config(cfg));
  Saved s;
  Scratch w;
  size_t a = 0, b = 0;
  carve_saved(*cfg, nullptr, s, a);
  carve_scratch(*cfg, nullptr, w, b);
  if (saved_bytes) *saved_bytes = a;
  if (scratch_bytes) *scratch_bytes = b;
  return QBLK_OK;
}

static int check_params(const qblk_block_params* p) {
  if (!p) return fail(QBLK_EINVAL, "params is NULL");
  const void* ptrs[] = {p->w_q, p->w_k, p->w_v, p->w_o, p->w_gate, p->w_up, p->w_down,
                        p->g_in, p->g_post, p->g_q, p->g_k};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return fail(QBLK_EINVAL, "params: null or misaligned (16 B) pointer");
  if (p->w16 && !aligned16(p->w16)) return fail(QBLK_EINVAL, "params: misaligned (16 B) w16");
  return QBLK_OK;
}

int32_t qblk_block_pack_f16_size(const qblk_config* cfg, size_t* bytes) {
  QBLK_TRY(check_config(cfg));
  if (!bytes) return fail(QBLK_EINVAL, "block_pack_f16_size: bytes is NULL");
  Packed16 pk;
  carve_pack16(*cfg, nullptr, pk, *bytes);
  return QBLK_OK;
}

int32_t qblk_block_pack_f16(const qblk_config* cfg, const qblk_block_params* p, void* packed,
                            size_t packed_bytes, qblk_stream_t stream) {
  QBLK_TRY(check_config(cfg));
  QBLK_TRY(check_params(p));
  if (!packed || !aligned16(packed)) return fail(QBLK_EINVAL, "block_pack_f16: null or misaligned buffer");
  Packed16 pk;
  size_t need = 0;
  carve_pack16(*cfg, nullptr, pk, need);
  if (packed_bytes < need) return fail(QBLK_EINVAL, "block_pack_f16: buffer %zu < %zu", packed_bytes, need);
  carve_pack16(*cfg, packed, pk, need);
  return pack16(*cfg, *p, pk, S(stream));
}

int32_t qblk_block_forward(const qblk_config* cfg, const qblk_block_params* p, const float* x, float* y,
                           void* saved, size_t saved_bytes, void* scratch, size_t scratch_bytes,
                           qblk_stream_t stream) {
  QBLK_TRY(check_config(cfg));
  QBLK_TRY(check_params(p));
  if (!x || !y || !saved || !scratch || !aligned16(x) || !aligned16(y) || !aligned16(saved) ||
      !aligned16(scratch))
    return fail(QBLK_EINVAL, "block_forward: null or misaligned buffer");
  Saved s;
  Scratch w;
  size_t need = 0, need_w = 0;
  carve_saved(*cfg, nullptr, s, need);
  carve_scratch(*cfg, nullptr, w, need_w);
  if (saved_bytes < need) return fail(QBLK_EINVAL, "block_forward: saved workspace %zu < %zu", saved_bytes, need);
  if (scratch_bytes < need_w)
    return fail(QBLK_EINVAL, "block_forward: scratch workspace %zu < %zu", scratch_bytes, need_w);
  carve_saved(*cfg, saved, s, need);
  carve_scratch(*cfg, scratch, w, need_w);
  return dense_block_forward(*cfg, *p, x, y, s, w, S(stream));
}

static int32_t block_backward_common(const qblk_config* cfg, const qblk_block_params* p, const float* x,
                                     const float* dy, const void* saved, size_t saved_bytes, float* dx,
                                     const qblk_block_grads* grads, void* scratch, size_t scratch_bytes,
                                     qblk_stream_t stream, bool accumulate) {
  QBLK_TRY(check_config(cfg));
  QBLK_TRY(check_params(p));
  if (!grads) return fail(QBLK_EINVAL, "block_backward: grads is NULL");
  const void* gp[] = {grads->w_q, grads->w_k, grads->w_v, grads->w_o, grads->w_gate, grads->w_up,
                      grads->w_down, grads->g_in, grads->g_post, grads->g_q, grads->g_k};
  for (const void* q : gp)
    if (!q || !aligned16(q)) return fail(QBLK_EINVAL, "block_backward: null or misaligned gradient pointer");
  if (!x || !dy || !dx || !saved || !scratch || !aligned16(x) || !aligned16(dy) || !aligned16(dx) ||
      !aligned16(saved) || !aligned16(scratch))
    return fail(QBLK_EINVAL, "block_backward: null or misaligned buffer");
  Saved s;
  Scratch w;
  size_t need_s = 0, need_w = 0;
  carve_saved(*cfg, nullptr, s, need_s);
  carve_scratch(*cfg, nullptr, w, need_w);
  if (saved_bytes < need_s) return fail(QBLK_EINVAL, "block_backward: saved workspace %zu < %zu", saved_bytes, need_s);
  if (scratch_bytes < need_w)
    return fail(QBLK_EINVAL, "block_backward: scratch workspace %zu < %zu", scratch_bytes, need_w);
  carve_saved(*cfg, (void*)saved, s, need_s);
  carve_scratch(*cfg, scratch, w, need_w);
  return dense_block_backward(*cfg, *p, *grads, x, dy, s, dx, w, S(stream), accumulate);
}

int32_t qblk_block_backward(const qblk_config* cfg, const qblk_block_params* p, const float* x, const float* dy,
                            const void* saved, size_t saved_bytes, float* dx, const qblk_block_grads* grads,
                            void* scratch, size_t scratch_bytes, qblk_stream_t stream) {
  return block_backward_common(cfg, p, x, dy, saved, saved_bytes, dx, grads, scratch, scratch_bytes, stream,
                               false);
}

int32_t qblk_block_backward_accumulate(const qblk_config* cfg, const qblk_block_params* p, const float* x,
                                       const float* dy, const void* saved, size_t saved_bytes, float* dx,
                                       const qblk_block_grads* grads, void* scratch, size_t scratch_bytes,
                                       qblk_stream_t stream) {
  return block_backward_common(cfg, p, x, dy, saved, saved_bytes, dx, grads, scratch, scratch_bytes, stream,
                               true);
}

// ------------------------------------------------------- cross-entropy

static size_t ce_gemm_ws(int T, int h, int V) {
  GemmDesc a;
  a.layout = Layout::NN; a.prec = Prec::F32;
  a.M = T; a.N = h; a.K = V;
  GemmDesc f = a;
  f.layout = Layout::NT; f.N = V; f.K = h;
  GemmDesc b = a;
  b.layout = Layout::TN; b.M = V; b.N = h; b.K = T;
  return std::max(gemm_workspace(a), std::max(gemm_workspace(f), gemm_workspace(b)));
}

static void ce_layout(int T, int h, int V, float** hf, float** z, float** dhf, float** red, float** ws,
                      size_t* ws_bytes, size_t* bytes, void* base) {
  size_t off = 0;
  auto take = [&](size_t n) {
    off = (off + 255) & ~(size_t)255;
    float* p = base ? (float*)((char*)base + off) : nullptr;
    off += n * sizeof(float);
    return p;
  };
  *hf = take((size_t)T * h);
  *z = take((size_t)T * V);
  *dhf = take((size_t)T * h);
  *red = take(rmsnorm_bwd_scratch(T, h) / sizeof(float) + T);
  *ws_bytes = ce_gemm_ws(T, h, V);
  *ws = take(*ws_bytes / sizeof(float) + 1);
  *bytes = off;
}

int32_t qblk_cross_entropy_workspace_size(int32_t tokens, int32_t hidden, int32_t vocab, size_t* scratch_bytes) {
  if (tokens <= 0 || hidden <= 0 || vocab <= 0) return fail(QBLK_EINVAL, "cross_entropy: bad sizes");
  float *a, *b, *c, *d, *e;
  size_t n = 0, wsb = 0;
  ce_layout(tokens, hidden, vocab, &a, &b, &c, &d, &e, &wsb, &n, nullptr);
  if (scratch_bytes) *scratch_bytes = n;
  return QBLK_OK;
}

static int32_t fused_ce_common(int32_t tokens, int32_t hidden, int32_t vocab, float eps, const float* y_last,
                               const float* g_final, const float* w_lm, const int32_t* targets, float loss_scale,
                               float* loss_partials, int32_t* argmax, float* dy_last, float* dg_final, float* dw_lm,
                               void* scratch, size_t scratch_bytes, qblk_stream_t stream, bool accumulate) {
  if (tokens <= 0 || hidden <= 0 || vocab <= 0) return fail(QBLK_EINVAL, "cross_entropy: bad sizes");
  if (hidden % 4 || vocab % 4) return fail(QBLK_EINVAL, "cross_entropy: hidden and vocab must be multiples of 4");
  if (!y_last || !w_lm || !targets || !loss_partials || !dy_last || !dw_lm || !scratch)
    return fail(QBLK_EINVAL, "cross_entropy: null pointer");
  if (g_final && !dg_final) return fail(QBLK_EINVAL, "cross_entropy: dg_final is NULL");
  if (g_final) QBLK_TRY(rmsnorm_check(tokens, hidden));
  float *hf, *z, *dhf, *red, *ws;
  size_t need = 0, wsb = 0;
  ce_layout(tokens, hidden, vocab, &hf, &z, &dhf, &red, &ws, &wsb, &need, nullptr);
  if (scratch_bytes < need) return fail(QBLK_EINVAL, "cross_entropy: scratch %zu < %zu", scratch_bytes, need);
  ce_layout(tokens, hidden, vocab, &hf, &z, &dhf, &red, &ws, &wsb, &need, scratch);
  hipStream_t st = S(stream);
  const float* h_in = y_last;
  if (g_final) {
    QBLK_TRY(rmsnorm_forward(tokens, hidden, eps, y_last, nullptr, g_final, hf, nullptr, nullptr, red, st));
    h_in = hf;
  }
  GemmDesc f;  // z = hf W_lm^T
  f.ws = ws; f.ws_bytes = wsb;
  f.layout = Layout::NT; f.prec = Prec::F32;
  f.M = tokens; f.N = vocab; f.K = hidden;
  f.a = h_in; f.lda = hidden;
  f.b = seg1(w_lm, vocab); f.ldb = hidden;
  f.c = seg1(z, tokens); f.ldc = vocab;
  QBLK_TRY(gemm(f, st));
  QBLK_TRY(ce_rows(tokens, vocab, z, targets, loss_scale, loss_partials, argmax, st));
  GemmDesc a;  // dhf = dz W_lm
  a.ws = ws; a.ws_bytes = wsb;
  a.layout = Layout::NN; a.prec = Prec::F32;
  a.M = tokens; a.N = hidden; a.K = vocab;
  a.a = z; a.lda = vocab;
  a.b = seg1(w_lm, vocab); a.ldb = hidden;
  a.c = seg1(g_final ? dhf : dy_last, tokens); a.ldc = hidden;
  QBLK_TRY(gemm(a, st));
  GemmDesc b;  // dW_lm = dz^T hf
  b.ws = ws; b.ws_bytes = wsb;
  b.layout = Layout::TN; b.prec = Prec::F32;
  b.M = vocab; b.N = hidden; b.K = tokens;
  b.a = z; b.lda = vocab;
  b.b = seg1(h_in, tokens); b.ldb = hidden;
  b.c = seg1(dw_lm, vocab); b.ldc = hidden;
  b.accumulate = accumulate;
  QBLK_TRY(gemm(b, st));
  if (g_final) {
    QBLK_TRY(rmsnorm_backward_partials(tokens, hidden, eps, y_last, g_final, dhf, nullptr, dy_last, nullptr, red,
                                       st));
    const ColsumJob j{rmsnorm_bwd_parts(tokens, hidden), hidden, red, dg_final, accumulate};
    QBLK_TRY(colsum_jobs(1, &j, st));
  }
  return QBLK_OK;
}

int32_t qblk_fused_cross_entropy(int32_t tokens, int32_t hidden, int32_t vocab, float eps, const float* y_last,
                                 const float* g_final, const float* w_lm, const int32_t* targets,
                                 float loss_scale, float* loss_partials, int32_t* argmax, float* dy_last,
                                 float* dg_final, float* dw_lm, void* scratch, size_t scratch_bytes,
                                 qblk_stream_t stream) {
  return fused_ce_common(tokens, hidden, vocab, eps, y_last, g_final, w_lm, targets, loss_scale, loss_partials,
                         argmax, dy_last, dg_final, dw_lm, scratch, scratch_bytes, stream, false);
}

int32_t qblk_fused_cross_entropy_accumulate(int32_t tokens, int32_t hidden, int32_t vocab, float eps,
                                            const float* y_last, const float* g_final, const float* w_lm,
                                            const int32_t* targets, float loss_scale, float* loss_partials,
                                            int32_t* argmax, float* dy_last, float* dg_final, float* dw_lm,
                                            void* scratch, size_t scratch_bytes, qblk_stream_t stream) {
  return fused_ce_common(tokens, hidden, vocab, eps, y_last, g_final, w_lm, targets, loss_scale, loss_partials,
                         argmax, dy_last, dg_final, dw_lm, scratch, scratch_bytes, stream, true);
}

int32_t qblk_cross_entropy_rows(int32_t tokens, int32_t vocab, float* z, const int32_t* targets, float loss_scale,
                                float* loss_partials, int32_t* argmax, qblk_stream_t stream) {
  if (tokens <= 0 || vocab <= 0) return fail(QBLK_EINVAL, "cross_entropy_rows: bad sizes");
  if (!z || !targets || !loss_partials) return fail(QBLK_EINVAL, "cross_entropy_rows: null pointer");
  if (vocab % 4 == 0 && !aligned16(z)) return fail(QBLK_EINVAL, "cross_entropy_rows: z must be 16-byte aligned");
  return ce_rows(tokens, vocab, z, targets, loss_scale, loss_partials, argmax, S(stream));
}

// ------------------------------------------------------- clip and AdamW

int32_t qblk_clip_workspace_size(int32_t n, const int64_t* numel, size_t* scratch_bytes) {
  if (n <= 0 || !numel) return fail(QBLK_EINVAL, "clip: n=%d", n);
  if (scratch_bytes) *scratch_bytes = clip_scratch(n, numel);
  return QBLK_OK;
}

int32_t qblk_clip_grad_norm(int32_t n, float* const* grads, const int64_t* numel, float max_norm, int32_t apply,
                            float* norm_dev, float* scale_dev, void* scratch, size_t scratch_bytes,
                            qblk_stream_t stream) {
  if (n <= 0 || !grads || !numel || !norm_dev || !scale_dev || !scratch)
    return fail(QBLK_EINVAL, "clip: null argument or n <= 0");
  if (!(max_norm > 0.f)) return fail(QBLK_EINVAL, "clip: max_norm must be positive");
  for (int i = 0; i < n; ++i)
    if (!grads[i] || numel[i] < 0) return fail(QBLK_EINVAL, "clip: tensor %d", i);
  if (scratch_bytes < clip_scratch(n, numel)) return fail(QBLK_EINVAL, "clip: scratch too small");
  return clip_grad_norm(n, grads, numel, max_norm, apply, norm_dev, scale_dev, scratch, S(stream));
}

int32_t qblk_clip_grad_norm_noalloc(int32_t n, float* const* grads, const int64_t* numel, float max_norm,
                                    int32_t apply, float* norm_dev, float* scale_dev, qblk_stream_t stream) {
  if (n <= 0 || !grads || !numel || !norm_dev || !scale_dev)
    return fail(QBLK_EINVAL, "clip (no workspace): null argument or n <= 0");
  if (!(max_norm > 0.f)) return fail(QBLK_EINVAL, "clip (no workspace): max_norm must be positive");
  for (int i = 0; i < n; ++i)
    if (!grads[i] || numel[i] < 0) return fail(QBLK_EINVAL, "clip (no workspace): tensor %d", i);
  if (clip_scratch(n, numel) > static_clip_scratch_bytes())
    return fail(QBLK_EINVAL, "clip (no workspace): %d tensors exceed the limit of %d", n,
                QBLK_CLIP_NOALLOC_MAX_TENSORS);
  void* ws = nullptr;
  QBLK_TRY(static_clip_scratch(&ws));
  return clip_grad_norm(n, grads, numel, max_norm, apply, norm_dev, scale_dev, ws, S(stream));
}

int32_t qblk_adamw_step(int32_t n, float* const* w, const float* const* g, float* const* m, float* const* v,
                        const int64_t* numel, float lr, float beta1, float beta2, float eps, float weight_decay,
                        int32_t step, const float* grad_scale_dev, qblk_stream_t stream) {
  if (n <= 0 || !w || !g || !m || !v || !numel) return fail(QBLK_EINVAL, "adamw: null argument or n <= 0");
  if (step < 1) return fail(QBLK_EINVAL, "adamw: step must be >= 1");
  for (int i = 0; i < n; ++i)
    if (!w[i] || !g[i] || !m[i] || !v[i] || numel[i] < 0) return fail(QBLK_EINVAL, "adamw: tensor %d", i);
  return adamw(n, w, g, m, v, numel, lr, beta1, beta2, eps, weight_decay, step, grad_scale_dev, S(stream));
}

int32_t qblk_adamw_step_pack16(int32_t n, float* const* w, const float* const* g, float* const* m,
                               float* const* v, const int64_t* numel, void* const* w16, int32_t w16_bf16, float lr,
                               float beta1, float beta2, float eps, float weight_decay, int32_t step,
                               const float* grad_scale_dev, qblk_stream_t stream) {
  if (n <= 0 || !w || !g || !m || !v || !numel || !w16)
    return fail(QBLK_EINVAL, "adamw_pack16: null argument or n <= 0");
  if (w16_bf16 != 0 && w16_bf16 != 1) return fail(QBLK_EINVAL, "adamw_pack16: w16_bf16 must be 0 or 1");
  if (step < 1) return fail(QBLK_EINVAL, "adamw_pack16: step must be >= 1");
  for (int i = 0; i < n; ++i) {
    if (!w[i] || !g[i] || !m[i] || !v[i] || numel[i] < 0) return fail(QBLK_EINVAL, "adamw_pack16: tensor %d", i);
    if ((uintptr_t)w16[i] % 2) return fail(QBLK_EINVAL, "adamw_pack16: fp16 copy %d misaligned", i);
  }
  return adamw(n, w, g, m, v, numel, lr, beta1, beta2, eps, weight_decay, step, grad_scale_dev, S(stream),
               (f16* const*)w16, w16_bf16 == 1);
}

int32_t qblk_block_pack_f16_offsets(const qblk_config* cfg, int64_t* offsets) {
  QBLK_TRY(check_config(cfg));
  if (!offsets) return fail(QBLK_EINVAL, "block_pack_f16_offsets: offsets is NULL");
  Packed16 pk;
  size_t bytes = 0;
  char* const base = (char*)(uintptr_t)4096;  // any 256-aligned address: only differences are used
  carve_pack16(*cfg, base, pk, bytes);
  const int64_t h = cfg->hidden, qd = (int64_t)cfg->heads * cfg->head_dim, kvd = (int64_t)cfg->kv_heads * cfg->head_dim;
  const int64_t I = cfg->intermediate;
  const f16* b16 = (const f16*)base;
  offsets[0] = pk.qkv - b16;
  offsets[1] = offsets[0] + qd * h;
  offsets[2] = offsets[1] + kvd * h;
  offsets[3] = pk.o - b16;
  offsets[4] = pk.gu - b16;
  offsets[5] = offsets[4] + I * h;
  offsets[6] = pk.d - b16;
  return QBLK_OK;
}

// ---------------------------------------------------------------- NF4

int32_t qblk_nf4_quantize(const float* w, int64_t numel, uint8_t* codes, float* absmax, qblk_stream_t stream) {
  if (numel <= 0 || numel % 64) return fail(QBLK_EINVAL, "nf4_quantize: numel %lld not a positive multiple of 64", (long long)numel);
  if (!w || !codes || !absmax) return fail(QBLK_EINVAL, "nf4_quantize: null pointer");
  return nf4_quantize(w, numel, codes, absmax, S(stream));
}

int32_t qblk_nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t numel, float* w,
                            qblk_stream_t stream) {
  if (!w || !codes || !absmax) return fail(QBLK_EINVAL, "nf4_dequantize: null pointer");
  return nf4_dequantize(codes, absmax, numel, w, S(stream));
}

// ------------------------------------------------------- single steps

int32_t qblk_gemm_workspace_size(int32_t layout, int32_t precision, int32_t M, int32_t N, int32_t K,
                                 size_t* scratch_bytes) {
  if (layout < 0 || layout > 2 || precision < 0 || precision > 2) return fail(QBLK_EINVAL, "gemm: layout/precision");
  if (M <= 0 || N <= 0 || K <= 0) return fail(QBLK_EINVAL, "gemm: bad shape");
  // enough for either operand storage (fp16 storage plans its own splits)
  size_t need = 0;
  for (int f16src = 0; f16src < 2; ++f16src) {
    GemmDesc d;
    d.layout = (Layout)layout;
    d.prec = (Prec)precision;
    d.M = M; d.N = N; d.K = K;
    if (f16src) d.a_src = d.b_src = Src::F16;
    need = std::max(need, gemm_workspace(d));
  }
  if (scratch_bytes) *scratch_bytes = need;
  return QBLK_OK;
}

int32_t qblk_gemm(int32_t layout, int32_t precision, int32_t M, int32_t N, int32_t K, const float* A, int64_t lda,
                  const float* B, int64_t ldb, float* C, int64_t ldc, int32_t accumulate, void* scratch,
                  size_t scratch_bytes, qblk_stream_t stream) {
  return qblk_gemm_ex(layout, precision, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, accumulate, scratch, scratch_bytes,
                      stream);
}

int32_t qblk_gemm_ex(int32_t layout, int32_t precision, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda,
                     int32_t a_dtype, const void* B, int64_t ldb, int32_t b_dtype, float* C, int64_t ldc,
                     int32_t accumulate, void* scratch, size_t scratch_bytes, qblk_stream_t stream) {
  if (layout < 0 || layout > 2 || precision < 0 || precision > 2) return fail(QBLK_EINVAL, "gemm: layout/precision");
  if (a_dtype < 0 || a_dtype > 2 || b_dtype < 0 || b_dtype > 2) return fail(QBLK_EINVAL, "gemm: operand dtype");
  // bfloat16 storage goes with bfloat16 operands only, and back
  if ((precision == 2) != (a_dtype == 2) || (precision == 2) != (b_dtype == 2))
    return fail(QBLK_EINVAL, "gemm: bfloat16 operands (precision 2) need bfloat16 storage (dtype 2) of both");
  if (lda % 4 || ldb % 4) return fail(QBLK_EINVAL, "gemm: lda and ldb must be multiples of 4");
  if (!A || !B || !C || !aligned16(A) || !aligned16(B)) return fail(QBLK_EINVAL, "gemm: null or misaligned operand");
  GemmDesc d;
  d.layout = (Layout)layout;
  d.prec = (Prec)precision;
  d.M = M; d.N = N; d.K = K;
  d.a = A; d.lda = lda;
  d.a_src = a_dtype ? Src::F16 : Src::F32;  // Src::F16: 16-bit storage (fp16, or bfloat16 with precision 2)
  d.b_src = b_dtype ? Src::F16 : Src::F32;
  const int brows = d.layout == Layout::NT ? N : K;
  d.b = seg1(B, brows); d.ldb = ldb;
  d.c = seg1(C, M); d.ldc = ldc;
  d.accumulate = accumulate;
  if (scratch && aligned16(scratch)) {
    d.ws = (float*)scratch;
    d.ws_bytes = scratch_bytes;
  }
  return gemm(d, S(stream));
}

int32_t qblk_rmsnorm_workspace_size(int32_t rows, int32_t n, size_t* scratch_bytes) {
  QBLK_TRY(rmsnorm_check(rows, n));
  if (scratch_bytes) *scratch_bytes = rmsnorm_bwd_scratch(rows, n);
  return QBLK_OK;
}

int32_t qblk_rmsnorm_forward(int32_t rows, int32_t n, float eps, const float* x, const float* res, const float* gamma,
                             float* y, float* sum_out, float* rho, void* scratch, size_t scratch_bytes,
                             qblk_stream_t stream) {
  (void)scratch;
  (void)scratch_bytes;
  if (!x || !gamma || !y || !rho) return fail(QBLK_EINVAL, "rmsnorm_forward: null pointer");
  if (res && !sum_out) return fail(QBLK_EINVAL, "rmsnorm_forward: sum_out needed with res");
  return rmsnorm_forward(rows, n, eps, x, res, gamma, y, nullptr, sum_out, rho, S(stream));
}

int32_t qblk_rmsnorm_backward(int32_t rows, int32_t n, float eps, const float* x, const float* gamma,
                              const float* dy, const float* dres, float* dx, float* dgamma, void* scratch,
                              size_t scratch_bytes, qblk_stream_t stream) {
  if (!x || !gamma || !dy || !dx || !dgamma || !scratch) return fail(QBLK_EINVAL, "rmsnorm_backward: null pointer");
  QBLK_TRY(rmsnorm_check(rows, n));
  if (scratch_bytes < rmsnorm_bwd_scratch(rows, n)) return fail(QBLK_EINVAL, "rmsnorm_backward: scratch too small");
  return rmsnorm_backward(rows, n, eps, x, gamma, dy, dres, dx, nullptr, dgamma, (float*)scratch, S(stream));
}

int32_t qblk_swiglu_forward(int32_t tokens, int32_t inter, const float* gu, float* s, qblk_stream_t stream) {
  if (tokens <= 0 || inter <= 0 || inter % 4) return fail(QBLK_EINVAL, "swiglu_forward: bad sizes");
  if (!gu || !s || !aligned16(gu) || !aligned16(s)) return fail(QBLK_EINVAL, "swiglu_forward: null or misaligned");
  return swiglu_forward(tokens, inter, gu, s, nullptr, S(stream));
}

int32_t qblk_swiglu_backward(int32_t tokens, int32_t inter, const float* gu, const float* ds, float* dgu,
                             qblk_stream_t stream) {
  if (tokens <= 0 || inter <= 0 || inter % 4) return fail(QBLK_EINVAL, "swiglu_backward: bad sizes");
  if (!gu || !ds || !dgu || !aligned16(gu) || !aligned16(ds) || !aligned16(dgu))
    return fail(QBLK_EINVAL, "swiglu_backward: null or misaligned");
  return swiglu_backward(tokens, inter, gu, ds, dgu, nullptr, S(stream));
}

static size_t qk_tab_bytes(int32_t seq, int32_t head_dim) {
  return ((size_t)seq * (head_dim / 2) * sizeof(float2) + 255) & ~(size_t)255;
}

static int check_qk(int32_t tokens, int32_t seq, int32_t heads, int32_t kv_heads, int32_t head_dim, int64_t ld_qkv) {
  if (tokens <= 0 || seq <= 0 || tokens % seq || heads <= 0 || kv_heads <= 0 || heads % kv_heads)
    return fail(QBLK_EINVAL, "qk_norm_rope: bad sizes");
  if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(QBLK_EUNSUPPORTED, "qk_norm_rope: head_dim %d", head_dim);
  if (ld_qkv < (int64_t)(heads + 2 * kv_heads) * head_dim || ld_qkv % 4)
    return fail(QBLK_EINVAL, "qk_norm_rope: ld_qkv");
  return QBLK_OK;
}

int32_t qblk_qk_norm_rope_workspace_size(int32_t tokens, int32_t seq, int32_t heads, int32_t kv_heads,
                                         int32_t head_dim, size_t* scratch_bytes) {
  QBLK_TRY(check_qk(tokens, seq, heads, kv_heads, head_dim, (int64_t)(heads + 2 * kv_heads) * head_dim));
  if (!scratch_bytes) return fail(QBLK_EINVAL, "qk_norm_rope_workspace_size: null");
  *scratch_bytes = qk_tab_bytes(seq, head_dim) + qk_norm_rope_bwd_scratch(tokens, heads, kv_heads, head_dim) + 256;
  return QBLK_OK;
}

int32_t qblk_qk_norm_rope_forward(int32_t tokens, int32_t seq, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                  int32_t qk_norm, float eps, float rope_theta, const float* qkv, int64_t ld_qkv,
                                  const float* g_q, const float* g_k, float* qr, float* kr, float* rho_q,
                                  float* rho_k, void* scratch, size_t scratch_bytes, qblk_stream_t stream) {
  QBLK_TRY(check_qk(tokens, seq, heads, kv_heads, head_dim, ld_qkv));
  if (!qkv || !qr || !kr || !scratch || (qk_norm && (!g_q || !g_k || !rho_q || !rho_k)))
    return fail(QBLK_EINVAL, "qk_norm_rope_forward: null pointer");
  if (scratch_bytes < qk_tab_bytes(seq, head_dim) || !aligned16(scratch))
    return fail(QBLK_EINVAL, "qk_norm_rope_forward: scratch");
  float2* tab = (float2*)scratch;
  QBLK_TRY(rope_table(seq, head_dim, rope_theta, tab, S(stream)));
  QkRopeArgs a{tokens, seq, heads, kv_heads, head_dim, qk_norm, eps, qkv, ld_qkv, g_q, g_k, tab, qr, kr, rho_q, rho_k};
  return qk_norm_rope_forward(a, S(stream));
}

int32_t qblk_qk_norm_rope_backward(int32_t tokens, int32_t seq, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                   int32_t qk_norm, float eps, float rope_theta, const float* qkv, int64_t ld_qkv,
                                   const float* g_q, const float* g_k, const float* dqr, const float* dkr,
                                   float* dqkv, float* dg_q, float* dg_k, void* scratch, size_t scratch_bytes,
                                   qblk_stream_t stream) {
  QBLK_TRY(check_qk(tokens, seq, heads, kv_heads, head_dim, ld_qkv));
  if (!qkv || !dqr || !dkr || !dqkv || !dg_q || !dg_k || !scratch || (qk_norm && (!g_q || !g_k)))
    return fail(QBLK_EINVAL, "qk_norm_rope_backward: null pointer");
  size_t need = 0;
  QBLK_TRY(qblk_qk_norm_rope_workspace_size(tokens, seq, heads, kv_heads, head_dim, &need));
  if (scratch_bytes < need || !aligned16(scratch)) return fail(QBLK_EINVAL, "qk_norm_rope_backward: scratch");
  float2* tab = (float2*)scratch;
  QBLK_TRY(rope_table(seq, head_dim, rope_theta, tab, S(stream)));
  QkRopeBwdArgs b{tokens, seq, heads, kv_heads, head_dim, qk_norm, eps, qkv, ld_qkv, g_q, g_k, tab,
                  dqr, dkr, dqkv, dg_q, dg_k};
  return qk_norm_rope_backward(b, (float*)((char*)scratch + qk_tab_bytes(seq, head_dim)), S(stream));
}

static int check_attn_ld(int32_t heads_or_kv, int32_t d, int64_t ld) {
  if (ld < (int64_t)heads_or_kv * d || ld % 4) return fail(QBLK_EINVAL, "attention: leading dimension");
  return 0;
}

int32_t qblk_attention_forward(int32_t batch, int32_t seq, int32_t heads, int32_t kv_heads, int32_t head_dim,
                               int32_t precision, const float* q, int64_t ldq, const float* k, int64_t ldk,
                               const float* v, int64_t ldv, float* o, int64_t ldo, float* lse, qblk_stream_t stream) {
  QBLK_TRY(attention_check(batch, seq, heads, kv_heads, head_dim));
  if (!q || !k || !v || !o || !lse) return fail(QBLK_EINVAL, "attention_forward: null pointer");
  QBLK_TRY(check_attn_ld(heads, head_dim, ldq));
  QBLK_TRY(check_attn_ld(kv_heads, head_dim, ldk));
  QBLK_TRY(check_attn_ld(kv_heads, head_dim, ldv));
  QBLK_TRY(check_attn_ld(heads, head_dim, ldo));
  AttnArgs a{};
  a.batch = batch; a.seq = seq; a.heads = heads; a.kv_heads = kv_heads; a.head_dim = head_dim;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.v = v; a.ldv = ldv; a.o = o; a.ldo = ldo; a.lse = lse;
  return attention_forward(a, precision ? Prec::F16 : Prec::F32, S(stream));
}

static AttnDmaArgs attn16_dense(int32_t batch, int32_t seq, int32_t heads, int32_t kv_heads, int32_t head_dim) {
  AttnDmaArgs a{};
  a.batch = batch; a.seq = seq; a.heads = heads; a.kv_heads = kv_heads; a.head_dim = head_dim;
  a.ldq = (int64_t)heads * head_dim;
  a.ldk = a.ldv = (int64_t)kv_heads * head_dim;
  a.ldo = a.lddo = a.lddo32 = a.lddq = (int64_t)heads * head_dim;
  a.lddk = a.lddv = (int64_t)kv_heads * head_dim;
  return a;
}

int32_t qblk_attention_forward_f16(int32_t batch, int32_t seq, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                   const void* q16, const void* k16, const void* v16, float* o, float* lse,
                                   qblk_stream_t stream) {
  AttnDmaArgs a = attn16_dense(batch, seq, heads, kv_heads, head_dim);
  a.q = q16; a.k = k16; a.v = v16;
  a.o = o; a.lse = lse;
  return attention_dma_forward(a, nullptr, S(stream));
}

int32_t qblk_attention_backward_f16(int32_t batch, int32_t seq, int32_t heads, int32_t kv_heads,
                                    int32_t head_dim, const void* q16, const void* k16, const void* v16,
                                    const float* o, const float* lse, const void* do16, const float* do32,
                                    float* dq, float* dk, float* dv, void* scratch, size_t scratch_bytes,
                                    qblk_stream_t stream) {
  QBLK_TRY(attention_check(batch, seq, heads, kv_heads, head_dim));
  if (scratch_bytes < attention_bwd_scratch(batch, seq, heads, head_dim))
    return fail(QBLK_EINVAL, "attention_backward_f16: scratch too small");
  AttnDmaArgs a = attn16_dense(batch, seq, heads, kv_heads, head_dim);
  a.q = q16; a.k = k16; a.v = v16;
  a.o = (float*)o; a.lse = (float*)lse;
  a.d_o = do16; a.do32 = do32;
  a.dq = dq; a.dk = dk; a.dv = dv;
  return attention_dma_backward(a, scratch, S(stream));
}

int32_t qblk_attention_workspace_size(int32_t batch, int32_t seq, int32_t heads, size_t* scratch_bytes) {
  if (batch <= 0 || seq <= 0 || heads <= 0) return fail(QBLK_EINVAL, "attention: bad sizes");
  // head_dim 128 upper bound
  if (scratch_bytes) *scratch_bytes = attention_bwd_scratch(batch, seq, heads, 128);
  return QBLK_OK;
}

int32_t qblk_attention_backward(int32_t batch, int32_t seq, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                int32_t precision, const float* q, int64_t ldq, const float* k, int64_t ldk,
                                const float* v, int64_t ldv, const float* o, int64_t ldo, const float* lse,
                                const float* d_o, int64_t lddo, float* dq, int64_t lddq, float* dk, int64_t lddk,
                                float* dv, int64_t lddv, void* scratch, size_t scratch_bytes, qblk_stream_t stream) {
  QBLK_TRY(attention_check(batch, seq, heads, kv_heads, head_dim));
  if (precision == 0 && head_dim > 64) return fail(QBLK_EUNSUPPORTED, "attention_backward: fp32 needs head_dim <= 64");
  if (!q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv || !scratch)
    return fail(QBLK_EINVAL, "attention_backward: null pointer");
  if (scratch_bytes < attention_bwd_scratch(batch, seq, heads, head_dim))
    return fail(QBLK_EINVAL, "attention_backward: scratch too small");
  QBLK_TRY(check_attn_ld(heads, head_dim, ldq));
  QBLK_TRY(check_attn_ld(kv_heads, head_dim, ldk));
  QBLK_TRY(check_attn_ld(kv_heads, head_dim, ldv));
  QBLK_TRY(check_attn_ld(heads, head_dim, ldo));
  QBLK_TRY(check_attn_ld(heads, head_dim, lddo));
  QBLK_TRY(check_attn_ld(heads, head_dim, lddq));
  QBLK_TRY(check_attn_ld(kv_heads, head_dim, lddk));
  QBLK_TRY(check_attn_ld(kv_heads, head_dim, lddv));
  AttnArgs a{};
  a.batch = batch; a.seq = seq; a.heads = heads; a.kv_heads = kv_heads; a.head_dim = head_dim;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.v = v; a.ldv = ldv;
  a.o = const_cast<float*>(o); a.ldo = ldo; a.lse = const_cast<float*>(lse);
  a.d_o = d_o; a.lddo = lddo; a.dq = dq; a.lddq = lddq; a.dk = dk; a.lddk = lddk; a.dv = dv; a.lddv = lddv;
  return attention_backward(a, precision ? Prec::F16 : Prec::F32, scratch, S(stream));
}

}  // extern "C"
