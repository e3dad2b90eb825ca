// Frozen-NF4 decoder block with LoRA on all seven projections.
//
// cuda_block.rs page: CudaNf4TransformerBlock (NF4 codes + per-block scales
// for the 7 projections, the fused dequant + GEMM path, a backward that
// yields activation and LoRA gradients only). wgpu_trainer.rs page:
// lora_forward / lora_backward (A [rank, in], B [out, rank], scale
// alpha/rank, with h = x A^T kept from the forward).
//
// Design. Two paths share the launch sequence of the dense block:
// * fp16 copies (T a multiple of 8): each projection group's NF4 codes are
//   decoded once per call into an fp16 scratch copy of W~ (HBM-bound, a
//   fraction of the product's time), the product runs on the direct-to-LDS
//   GEMM kernel with the activations' fp16 copies, and the LoRA branch adds
//   s h B^T (forward) or dh A (backward) with small accumulating GEMMs.
// * otherwise: the codes are decoded while the GEMM stages its B operand and
//   the LoRA branch rides in the same GEMM as extra K columns:
//   y = [x | s*h] [W~ | B]^T with h = x A^T, s = alpha/rank, against a
//   block-diagonal B for the fused groups; dX = dY W~ + (s dY B) A likewise.
// dA and dB are small TN GEMMs either way.
#include "../../include/qblk.h"
#include "block.h"
#include "gemm.h"
#include "norms.h"
#include "step.h"

#include <algorithm>

namespace qblk {
namespace {

struct Nf4Saved {
  Saved base;
  float *h_qkv, *h_o, *h_gu, *h_d;  // x A^T of each projection group
};

struct Nf4Scratch {
  Scratch base;
  float *dh_qkv, *dh_o, *dh_gu, *dh_d;  // s dY B
  float *sink_h, *sink_d;               // gamma gradients are not outputs
  f16* w16;                             // fp16 W~ of the current group (fp16 copies path)
  f16* dy16;                            // fp16 dY of the current group
};

size_t carve_nf4(const qblk_config& c, int r, void* saved, void* scratch, Nf4Saved* s, Nf4Scratch* w,
                 size_t* scratch_bytes) {
  size_t sb = 0, wb = 0;
  carve_saved(c, saved, s->base, sb);
  carve_scratch(c, scratch, w->base, wb, r);
  const size_t T = (size_t)c.seq * c.batch;
  auto take = [](void* base, size_t& off, size_t n) -> float* {
    off = (off + 255) & ~(size_t)255;
    float* p = base ? (float*)((char*)base + off) : nullptr;
    off += n * sizeof(float);
    return p;
  };
  s->h_qkv = take(saved, sb, T * 3 * r);
  s->h_o = take(saved, sb, T * r);
  s->h_gu = take(saved, sb, T * 2 * r);
  s->h_d = take(saved, sb, T * r);
  w->dh_qkv = take(scratch, wb, T * 3 * r);
  w->dh_o = take(scratch, wb, T * r);
  w->dh_gu = take(scratch, wb, T * 2 * r);
  w->dh_d = take(scratch, wb, T * r);
  w->sink_h = take(scratch, wb, 2 * (size_t)c.hidden);
  w->sink_d = take(scratch, wb, 2 * (size_t)c.head_dim);
  w->w16 = w->dy16 = nullptr;
  if (s->base.n1_16 || !saved) {  // sizing call, or the fp16 copies exist
    const size_t h = c.hidden, qd = (size_t)c.heads * c.head_dim, kvd = (size_t)c.kv_heads * c.head_dim;
    const size_t I = c.intermediate, qkv = qd + 2 * kvd;
    const size_t wmax = std::max({qkv * h, h * qd, 2 * I * h, h * I});
    const size_t dmax = std::max({qkv, h, 2 * I});
    float* a = take(scratch, wb, wmax / 2 + 64);
    float* b = take(scratch, wb, T * dmax / 2 + 64);
    if (s->base.n1_16) {
      w->w16 = (f16*)a;
      w->dy16 = (f16*)b;
    }
  }
  *scratch_bytes = wb;
  return sb;
}

int check_nf4(const qblk_config* c, const qblk_nf4_block_params* p) {
  QBLK_TRY(check_config(c));
  if (c->gemm_precision != 1) return fail(QBLK_EUNSUPPORTED, "nf4 block: needs gemm_precision = 1");
  if (!p) return fail(QBLK_EINVAL, "nf4 block: params is NULL");
  if (p->rank <= 0 || p->rank > 20 || p->rank % 4) return fail(QBLK_EINVAL, "nf4 block: rank must be 4..20, multiple of 4");
  for (int i = 0; i < 7; ++i)
    if (!p->codes[i] || !p->absmax[i] || !p->lora_a[i] || !p->lora_b[i])
      return fail(QBLK_EINVAL, "nf4 block: null pointer for projection %d", i);
  if (!p->g_in || !p->g_post || !p->g_q || !p->g_k) return fail(QBLK_EINVAL, "nf4 block: null gamma");
  const int64_t h = c->hidden, q = (int64_t)c->heads * c->head_dim, kv = (int64_t)c->kv_heads * c->head_dim,
                I = c->intermediate;
  const int64_t numel[7] = {q * h, kv * h, kv * h, h * q, I * h, I * h, h * I};
  for (int i = 0; i < 7; ++i)
    if (numel[i] % 64) return fail(QBLK_EINVAL, "nf4 block: projection %d numel not a multiple of 64", i);
  return QBLK_OK;
}

enum { PQ = 0, PK, PV, PO, PG, PU, PD };

Seg rows3(int a, int b, int c) {
  Seg s;
  s.start[0] = 0; s.start[1] = a; s.start[2] = a + b; s.start[3] = a + b + c;
  s.nseg = c ? 3 : (b ? 2 : 1);
  return s;
}

Nf4Seg nf4seg(const qblk_nf4_block_params& p, int i0, int i1, int i2) {
  Nf4Seg n;
  const int idx[3] = {i0, i1, i2};
  for (int j = 0; j < 3; ++j)
    if (idx[j] >= 0) {
      n.codes[j] = p.codes[idx[j]];
      n.scales[j] = p.absmax[idx[j]];
    }
  const float* lv = nf4_codebook_host();
  for (int j = 0; j < 16; ++j) n.levels[j] = lv[j];
  return n;
}

// Split-K workspace of the current call (set by the entry points below;
// calls on one thread are sequential, and the pointer only travels into the
// GemmDesc of launches issued by that same call).
thread_local const Scratch* t_ws = nullptr;

GemmDesc base(Layout l, int M, int N, int K) {
  GemmDesc g;
  if (t_ws) {
    g.ws = t_ws->gemm_ws;
    g.ws_bytes = t_ws->gemm_ws_bytes;
  }
  g.layout = l;
  g.prec = Prec::F16;
  g.M = M; g.N = N; g.K = K;
  return g;
}

// h = x [A_i0; A_i1; A_i2]^T : [T, n*r]
int lora_down(const qblk_nf4_block_params& p, int T, int in, const float* x, std::initializer_list<int> ids,
              float* h, hipStream_t st) {
  const int r = p.rank, n = (int)ids.size();
  GemmDesc g = base(Layout::NT, T, n * r, in);
  g.a = x; g.lda = in;
  int j = 0;
  for (int id : ids) {
    g.b.p[j] = p.lora_a[id];
    g.b.start[j] = j * r;
    ++j;
  }
  g.b.start[n] = n * r;
  g.b.nseg = n;
  g.ldb = in;
  g.c = seg1(h, T); g.ldc = n * r;
  return gemm(g, st);
}

// out = x [W~]^T (+ res) + s [h] blockdiag(B)^T
int nf4_fwd(const qblk_nf4_block_params& p, int T, int in, const float* x, std::initializer_list<int> ids,
            std::initializer_list<int> outs, const float* h, const float* res, float* out, hipStream_t st) {
  const int r = p.rank, n = (int)ids.size();
  int outd[3] = {0, 0, 0}, id3[3] = {-1, -1, -1}, j = 0;
  for (int o : outs) outd[j++] = o;
  j = 0;
  for (int id : ids) id3[j++] = id;
  int N = 0;
  for (int k = 0; k < n; ++k) N += outd[k];
  GemmDesc g = base(Layout::NT, T, N, in);
  g.a = x; g.lda = in;
  g.b = rows3(outd[0], outd[1], outd[2]); g.ldb = in;
  g.b_src = Src::NF4;
  g.nf4 = nf4seg(p, id3[0], id3[1], id3[2]);
  g.c = seg1(out, T); g.ldc = N;
  g.r = res; g.ldr = N;
  g.ext.kext = n * r;
  g.ext.a = h; g.ext.lda = n * r; g.ext.a_scale = p.alpha / (float)r;
  for (int k = 0; k < n; ++k) g.ext.b[k] = p.lora_b[id3[k]];
  g.ext.ldb = r;
  g.ext.blockdiag = n > 1 ? r : 0;
  return gemm(g, st);
}

// Backward of one projection group with output widths outs (stacked) and
// input width `in`: dX, dA, dB (W~ frozen).
int nf4_bwd(const qblk_nf4_block_params& p, const qblk_lora_grads& gr, int T, int in, const float* dy,
            const float* x, const float* h, std::initializer_list<int> ids, std::initializer_list<int> outs,
            float* dh, float* dx, hipStream_t st) {
  const int r = p.rank, n = (int)ids.size();
  const float sc = p.alpha / (float)r;
  int outd[3] = {0, 0, 0}, id3[3] = {-1, -1, -1}, j = 0;
  for (int o : outs) outd[j++] = o;
  j = 0;
  for (int id : ids) id3[j++] = id;
  int Nout = 0;
  for (int k = 0; k < n; ++k) Nout += outd[k];
  // dh[:, k r:(k+1) r] = s * dY_k B_k
  int col = 0;
  for (int k = 0; k < n; ++k) {
    GemmDesc g = base(Layout::NN, T, r, outd[k]);
    g.a = dy + col; g.lda = Nout;
    g.b = seg1(p.lora_b[id3[k]], outd[k]); g.ldb = r;
    g.c = seg1(dh + k * r, T); g.ldc = n * r;
    g.alpha = sc;
    QBLK_TRY(gemm(g, st));
    col += outd[k];
  }
  // dX = dY [W~_k stacked] + dh [A_k stacked]
  {
    GemmDesc g = base(Layout::NN, T, in, Nout);
    g.a = dy; g.lda = Nout;
    g.b = rows3(outd[0], outd[1], outd[2]); g.ldb = in;
    g.b_src = Src::NF4;
    g.nf4 = nf4seg(p, id3[0], id3[1], id3[2]);
    g.c = seg1(dx, T); g.ldc = in;
    g.ext.kext = n * r;
    g.ext.a = dh; g.ext.lda = n * r; g.ext.a_scale = 1.f;
    for (int k = 0; k < n; ++k) g.ext.b[k] = p.lora_a[id3[k]];
    g.ext.ldb = in;
    g.ext.blockdiag = n > 1 ? r : 0;
    QBLK_TRY(gemm(g, st));
  }
  // dB_k = s dY_k^T h_k (diagonal blocks of dY^T [h_0 | h_1 | ...])
  {
    GemmDesc g = base(Layout::TN, Nout, n * r, T);
    g.a = dy; g.lda = Nout;
    g.b = seg1(h, T); g.ldb = n * r;
    g.c = rows3(outd[0], outd[1], outd[2]);
    for (int k = 0; k < n; ++k) g.c.p[k] = gr.lora_b[id3[k]];
    g.ldc = r;
    g.c_cols_blockdiag = r;
    g.alpha = sc;
    QBLK_TRY(gemm(g, st));
  }
  // dA_k = dh_k^T X
  {
    GemmDesc g = base(Layout::TN, n * r, in, T);
    g.a = dh; g.lda = n * r;
    g.b = seg1(x, T); g.ldb = in;
    g.c = rows3(r, n > 1 ? r : 0, n > 2 ? r : 0);
    for (int k = 0; k < n; ++k) g.c.p[k] = gr.lora_a[id3[k]];
    g.ldc = in;
    QBLK_TRY(gemm(g, st));
  }
  return QBLK_OK;
}

// fp16 W~ of a projection group, stacked along out, into w16.
int dequant_group(const qblk_nf4_block_params& p, const int* id3, const int* outd, int n, int in, f16* w16,
                  hipStream_t st) {
  size_t off = 0;
  for (int k = 0; k < n; ++k) {
    const int64_t numel = (int64_t)outd[k] * in;
    QBLK_TRY(nf4_dequantize_f16(p.codes[id3[k]], p.absmax[id3[k]], numel, w16 + off, st));
    off += (size_t)numel;
  }
  return QBLK_OK;
}

// out (+ res) = x16 W~^T + s h blockdiag(B)^T on the fp16 copies path.
int nf4_fwd16(const qblk_nf4_block_params& p, const Nf4Scratch& w, int T, int in, const f16* x16,
              std::initializer_list<int> ids, std::initializer_list<int> outs, const float* h, const float* res,
              float* out, hipStream_t st) {
  const int r = p.rank, n = (int)ids.size();
  int outd[3] = {0, 0, 0}, id3[3] = {-1, -1, -1}, j = 0;
  for (int o : outs) outd[j++] = o;
  j = 0;
  for (int id : ids) id3[j++] = id;
  int N = 0;
  for (int k = 0; k < n; ++k) N += outd[k];
  QBLK_TRY(dequant_group(p, id3, outd, n, in, w.w16, st));
  GemmDesc g = base(Layout::NT, T, N, in);
  g.a = x16; g.lda = in; g.a_src = Src::F16;
  g.b = seg1(w.w16, N); g.ldb = in; g.b_src = Src::F16;
  g.c = seg1(out, T); g.ldc = N;
  g.r = res; g.ldr = N;
  QBLK_TRY(gemm(g, st));
  int col = 0;
  for (int k = 0; k < n; ++k) {  // out[:, block k] += s h_k B_k^T
    GemmDesc u = base(Layout::NT, T, outd[k], r);
    u.a = h + k * r; u.lda = n * r;
    u.b = seg1(p.lora_b[id3[k]], outd[k]); u.ldb = r;
    u.c = seg1(out + col, T); u.ldc = N;
    u.alpha = p.alpha / (float)r;
    u.accumulate = 1;
    QBLK_TRY(gemm(u, st));
    col += outd[k];
  }
  return QBLK_OK;
}

// Backward on the fp16 copies path: dX = dY16 W~ + dh [A stacked]; dA, dB
// as in nf4_bwd.
int nf4_bwd16(const qblk_nf4_block_params& p, const qblk_lora_grads& gr, const Nf4Scratch& w, int T, int in,
              const float* dy, const f16* x16, const float* x, const float* h, std::initializer_list<int> ids,
              std::initializer_list<int> outs, float* dh, float* dx, hipStream_t st) {
  const int r = p.rank, n = (int)ids.size();
  const float sc = p.alpha / (float)r;
  int outd[3] = {0, 0, 0}, id3[3] = {-1, -1, -1}, j = 0;
  for (int o : outs) outd[j++] = o;
  j = 0;
  for (int id : ids) id3[j++] = id;
  int Nout = 0;
  for (int k = 0; k < n; ++k) Nout += outd[k];
  (void)x16;
  int col = 0;
  for (int k = 0; k < n; ++k) {  // dh[:, k r:(k+1) r] = s dY_k B_k
    GemmDesc g = base(Layout::NN, T, r, outd[k]);
    g.a = dy + col; g.lda = Nout;
    g.b = seg1(p.lora_b[id3[k]], outd[k]); g.ldb = r;
    g.c = seg1(dh + k * r, T); g.ldc = n * r;
    g.alpha = sc;
    QBLK_TRY(gemm(g, st));
    col += outd[k];
  }
  QBLK_TRY(cast_f16(T, Nout, dy, Nout, w.dy16, Nout, nullptr, 0, st));
  QBLK_TRY(dequant_group(p, id3, outd, n, in, w.w16, st));
  {  // dX = dY W~
    GemmDesc g = base(Layout::NN, T, in, Nout);
    g.a = w.dy16; g.lda = Nout; g.a_src = Src::F16;
    g.b = seg1(w.w16, Nout); g.ldb = in; g.b_src = Src::F16;
    g.c = seg1(dx, T); g.ldc = in;
    QBLK_TRY(gemm(g, st));
  }
  {  // dX += dh [A_0; A_1; A_2]
    GemmDesc g = base(Layout::NN, T, in, n * r);
    g.a = dh; g.lda = n * r;
    g.b = rows3(r, n > 1 ? r : 0, n > 2 ? r : 0);
    for (int k = 0; k < n; ++k) g.b.p[k] = p.lora_a[id3[k]];
    g.ldb = in;
    g.c = seg1(dx, T); g.ldc = in;
    g.accumulate = 1;
    QBLK_TRY(gemm(g, st));
  }
  {  // dB_k = s dY_k^T h_k
    GemmDesc g = base(Layout::TN, Nout, n * r, T);
    g.a = dy; g.lda = Nout;
    g.b = seg1(h, T); g.ldb = n * r;
    g.c = rows3(outd[0], outd[1], outd[2]);
    for (int k = 0; k < n; ++k) g.c.p[k] = gr.lora_b[id3[k]];
    g.ldc = r;
    g.c_cols_blockdiag = r;
    g.alpha = sc;
    QBLK_TRY(gemm(g, st));
  }
  {  // dA_k = dh_k^T X
    GemmDesc g = base(Layout::TN, n * r, in, T);
    g.a = dh; g.lda = n * r;
    g.b = seg1(x, T); g.ldb = in;
    g.c = rows3(r, n > 1 ? r : 0, n > 2 ? r : 0);
    for (int k = 0; k < n; ++k) g.c.p[k] = gr.lora_a[id3[k]];
    g.ldc = in;
    QBLK_TRY(gemm(g, st));
  }
  return QBLK_OK;
}

}  // namespace
}  // namespace qblk

using namespace qblk;

extern "C" int32_t qblk_nf4_block_workspace_size(const qblk_config* cfg, int32_t rank, size_t* saved_bytes,
                                                 size_t* scratch_bytes) {
  QBLK_TRY(check_config(cfg));
  if (rank <= 0 || rank > 20 || rank % 4) return fail(QBLK_EINVAL, "nf4 block: rank must be 4..20, multiple of 4");
  Nf4Saved s;
  Nf4Scratch w;
  size_t wb = 0;
  const size_t sb = carve_nf4(*cfg, rank, nullptr, nullptr, &s, &w, &wb);
  if (saved_bytes) *saved_bytes = sb;
  if (scratch_bytes) *scratch_bytes = wb;
  return QBLK_OK;
}

extern "C" int32_t qblk_block_forward_nf4_lora(const qblk_config* cfg, const qblk_nf4_block_params* p,
                                               const float* x, float* y, void* saved, size_t saved_bytes,
                                               void* scratch, size_t scratch_bytes, qblk_stream_t stream) {
  QBLK_TRY(check_nf4(cfg, p));
  if (!x || !y || !saved || !scratch) return fail(QBLK_EINVAL, "nf4 forward: null buffer");
  Nf4Saved s;
  Nf4Scratch w;
  size_t wb = 0;
  const size_t sb = carve_nf4(*cfg, p->rank, nullptr, nullptr, &s, &w, &wb);
  if (saved_bytes < sb || scratch_bytes < wb) return fail(QBLK_EINVAL, "nf4 forward: workspace too small");
  carve_nf4(*cfg, p->rank, saved, scratch, &s, &w, &wb);
  const qblk_config& c = *cfg;
  const qblk_nf4_block_params& P = *p;
  const int T = c.seq * c.batch, h = c.hidden, qd = c.heads * c.head_dim, kvd = c.kv_heads * c.head_dim,
            I = c.intermediate;
  hipStream_t st = (hipStream_t)stream;
  t_ws = &w.base;
  ProjFwd proj;
  const bool f16p = w.w16 != nullptr;
  proj.qkv = [&](const float* n1, float* qkv, hipStream_t s_) {
    QBLK_TRY(lora_down(P, T, h, n1, {PQ, PK, PV}, s.h_qkv, s_));
    if (f16p) return nf4_fwd16(P, w, T, h, s.base.n1_16, {PQ, PK, PV}, {qd, kvd, kvd}, s.h_qkv, nullptr, qkv, s_);
    return nf4_fwd(P, T, h, n1, {PQ, PK, PV}, {qd, kvd, kvd}, s.h_qkv, nullptr, qkv, s_);
  };
  proj.o = [&](const float* o, const float* res, float* out, hipStream_t s_) {
    QBLK_TRY(lora_down(P, T, qd, o, {PO}, s.h_o, s_));
    if (f16p) return nf4_fwd16(P, w, T, qd, s.base.o16, {PO}, {h}, s.h_o, res, out, s_);
    return nf4_fwd(P, T, qd, o, {PO}, {h}, s.h_o, res, out, s_);
  };
  proj.gate_up = [&](const float* n2, float* gu, hipStream_t s_) {
    QBLK_TRY(lora_down(P, T, h, n2, {PG, PU}, s.h_gu, s_));
    if (f16p) return nf4_fwd16(P, w, T, h, s.base.n2_16, {PG, PU}, {I, I}, s.h_gu, nullptr, gu, s_);
    return nf4_fwd(P, T, h, n2, {PG, PU}, {I, I}, s.h_gu, nullptr, gu, s_);
  };
  proj.down = [&](const float* sv, const float* res, float* out, hipStream_t s_) {
    QBLK_TRY(lora_down(P, T, I, sv, {PD}, s.h_d, s_));
    if (f16p) return nf4_fwd16(P, w, T, I, s.base.s16, {PD}, {h}, s.h_d, res, out, s_);
    return nf4_fwd(P, T, I, sv, {PD}, {h}, s.h_d, res, out, s_);
  };
  const int rc = block_forward_impl(c, proj, P.g_in, P.g_post, P.g_q, P.g_k, x, y, s.base, st);
  t_ws = nullptr;
  return rc;
}

extern "C" int32_t qblk_block_backward_nf4_lora(const qblk_config* cfg, const qblk_nf4_block_params* p,
                                                const float* x, const float* dy, const void* saved,
                                                size_t saved_bytes, float* dx, const qblk_lora_grads* grads,
                                                void* scratch, size_t scratch_bytes, qblk_stream_t stream) {
  QBLK_TRY(check_nf4(cfg, p));
  if (!x || !dy || !saved || !dx || !grads || !scratch) return fail(QBLK_EINVAL, "nf4 backward: null buffer");
  for (int i = 0; i < 7; ++i)
    if (!grads->lora_a[i] || !grads->lora_b[i]) return fail(QBLK_EINVAL, "nf4 backward: null LoRA gradient %d", i);
  Nf4Saved s;
  Nf4Scratch w;
  size_t wb = 0;
  const size_t sb = carve_nf4(*cfg, p->rank, nullptr, nullptr, &s, &w, &wb);
  if (saved_bytes < sb || scratch_bytes < wb) return fail(QBLK_EINVAL, "nf4 backward: workspace too small");
  carve_nf4(*cfg, p->rank, (void*)saved, scratch, &s, &w, &wb);
  const qblk_config& c = *cfg;
  const qblk_nf4_block_params& P = *p;
  const qblk_lora_grads& G = *grads;
  const int T = c.seq * c.batch, h = c.hidden, qd = c.heads * c.head_dim, kvd = c.kv_heads * c.head_dim,
            I = c.intermediate;
  hipStream_t st = (hipStream_t)stream;
  t_ws = &w.base;
  ProjBwd proj;
  const bool f16p = w.w16 != nullptr;
  proj.down = [&](const float* dyv, const float* sv, float* ds, hipStream_t s_) {
    if (f16p) return nf4_bwd16(P, G, w, T, I, dyv, s.base.s16, sv, s.h_d, {PD}, {h}, w.dh_d, ds, s_);
    return nf4_bwd(P, G, T, I, dyv, sv, s.h_d, {PD}, {h}, w.dh_d, ds, s_);
  };
  proj.gate_up = [&](const float* dgu, const float* n2, float* dn2, hipStream_t s_) {
    if (f16p) return nf4_bwd16(P, G, w, T, h, dgu, s.base.n2_16, n2, s.h_gu, {PG, PU}, {I, I}, w.dh_gu, dn2, s_);
    return nf4_bwd(P, G, T, h, dgu, n2, s.h_gu, {PG, PU}, {I, I}, w.dh_gu, dn2, s_);
  };
  proj.o = [&](const float* dr1, const float* o, float* d_o, hipStream_t s_) {
    if (f16p) return nf4_bwd16(P, G, w, T, qd, dr1, s.base.o16, o, s.h_o, {PO}, {h}, w.dh_o, d_o, s_);
    return nf4_bwd(P, G, T, qd, dr1, o, s.h_o, {PO}, {h}, w.dh_o, d_o, s_);
  };
  proj.qkv = [&](const float* dqkv, const float* n1, float* dn1, hipStream_t s_) {
    if (f16p)
      return nf4_bwd16(P, G, w, T, h, dqkv, s.base.n1_16, n1, s.h_qkv, {PQ, PK, PV}, {qd, kvd, kvd}, w.dh_qkv,
                       dn1, s_);
    return nf4_bwd(P, G, T, h, dqkv, n1, s.h_qkv, {PQ, PK, PV}, {qd, kvd, kvd}, w.dh_qkv, dn1, s_);
  };
  const int rc = block_backward_impl(c, proj, P.g_in, P.g_post, P.g_q, P.g_k, x, dy, s.base, dx, w.sink_h,
                                     w.sink_h + h, w.sink_d, w.sink_d + c.head_dim, w.base, st);
  t_ws = nullptr;
  return rc;
}
