// Decoder block forward and backward: the launch sequence over the kernels
// of this library, and the layout of the two caller-owned workspaces.
//
// cuda_block.rs page: CudaTransformerBlock::forward / compute_attention_cuda
// and CudaTransformerBlock::backward (backward_ffn, backward_post_attn_norm,
// the second-residual add, backward_attention, backward_residual_and_input_norm).
// Differences from the page's launch plan: Q, K and V come out of ONE GEMM
// over [Wq; Wk; Wv] (likewise gate and up), the residual adds ride in the
// O-projection and down GEMM epilogues, QK-norm and RoPE are one kernel over
// all heads, attention never materialises the [heads, seq, seq] scores, the
// GQA reduction of dK/dV happens on device without copies, and every gamma
// gradient is a deterministic two-stage sum instead of atomics.
#include "block.h"

#include "../../include/qblk.h"
#include "attention.h"
#include "gemm.h"
#include "norms.h"

#include <algorithm>
#include <vector>

namespace qblk {

// ------------------------------------------------------------- layouts

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t n) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

void carve_saved(const qblk_config& c, void* base, Saved& s, size_t& bytes) {
  const size_t T = (size_t)c.seq * c.batch, h = c.hidden, d = c.head_dim;
  const size_t qd = (size_t)c.heads * d, kvd = (size_t)c.kv_heads * d, I = c.intermediate;
  Carver cv(base);
  s.tab = cv.take<float2>((size_t)c.seq * (d / 2));
  s.rho1 = cv.take<float>(T);
  s.n1 = cv.take<float>(T * h);
  s.qkv = cv.take<float>(T * (qd + 2 * kvd));
  s.rho_q = cv.take<float>(T * c.heads);
  s.rho_k = cv.take<float>(T * c.kv_heads);
  s.qr = cv.take<float>(T * qd);
  s.kr = cv.take<float>(T * kvd);
  s.o = cv.take<float>(T * qd);
  s.lse = cv.take<float>(T * c.heads);
  s.r1 = cv.take<float>(T * h);
  s.rho2 = cv.take<float>(T);
  s.n2 = cv.take<float>(T * h);
  s.gu = cv.take<float>(T * 2 * I);
  s.s = cv.take<float>(T * I);
  s.n1_16 = s.o16 = s.n2_16 = s.s16 = nullptr;
  if (c.gemm_precision != 0 && T % 8 == 0) {
    s.n1_16 = cv.take<f16>(T * h);
    s.o16 = cv.take<f16>(T * qd);
    s.n2_16 = cv.take<f16>(T * h);
    s.s16 = cv.take<f16>(T * I);
  }
  s.q16 = s.k16 = s.v16 = nullptr;
  if (use_attention_dma(c) && c.gemm_precision != 0) {
    s.q16 = cv.take<f16>(T * qd);
    s.k16 = cv.take<f16>(T * kvd);
    s.v16 = cv.take<f16>(T * kvd);
  }
  bytes = cv.off;
}

bool use_attention_dma(const qblk_config& c) {
  return attention_dma_supported(c.batch, c.seq, c.heads, c.kv_heads, c.head_dim) &&
         (c.gemm_precision != 0 || c.head_dim == 64);
}

Prec prec_of(const qblk_config& c) {
  return c.gemm_precision == 2 ? Prec::BF16 : c.gemm_precision == 1 ? Prec::F16 : Prec::F32;
}

// The block's 16-bit operand copies hold bfloat16 (gemm_precision 2).
static bool bf(const qblk_config& c) { return c.gemm_precision == 2; }

// Largest split-K workspace any GEMM of the block asks for.
static size_t block_gemm_ws(const qblk_config& c, int r) {
  const int T = c.seq * c.batch, h = c.hidden, qd = c.heads * c.head_dim, kvd = c.kv_heads * c.head_dim;
  const int I = c.intermediate, qkv = qd + 2 * kvd;
  struct S { Layout l; int M, N, K; };
  std::vector<S> v = {
      {Layout::NT, T, qkv, h}, {Layout::NT, T, h, qd}, {Layout::NT, T, 2 * I, h}, {Layout::NT, T, h, I},
      {Layout::NN, T, I, h},   {Layout::TN, h, I, T},  {Layout::NN, T, h, 2 * I}, {Layout::TN, 2 * I, h, T},
      {Layout::NN, T, qd, h},  {Layout::TN, h, qd, T}, {Layout::NN, T, h, qkv},   {Layout::TN, qkv, h, T}};
  size_t m = 0;
  if (r > 0) {
    const int ins[4] = {h, qd, h, I}, outs[4] = {qkv, h, 2 * I, h}, ns[4] = {3, 1, 2, 1};
    const int outk[7] = {qd, kvd, kvd, h, I, I, h};
    for (int g = 0; g < 4; ++g) {
      // register-kernel path (fp32 LoRA operands)
      v.push_back({Layout::NT, T, ns[g] * r, ins[g]});
      v.push_back({Layout::TN, outs[g], ns[g] * r, T});
      v.push_back({Layout::TN, ns[g] * r, ins[g], T});
      // fp16 path: h and dh over 64 padded columns, dB, dA, the base
      // products (dense fallback) and the fused NF4 products with the LoRA tile
      v.push_back({Layout::NT, T, 64, ins[g]});
      v.push_back({Layout::NT, T, 64, outs[g]});
      v.push_back({Layout::TN, outs[g], 64, T});
      v.push_back({Layout::NT, T, outs[g], 64});
      v.push_back({Layout::NN, T, ins[g], 64});
      m = std::max(m, gemm_nf4_workspace(T, outs[g], ins[g] + 64));
      m = std::max(m, gemm_nf4_workspace(T, ins[g], outs[g] + 64));
    }
    for (int k = 0; k < 7; ++k) v.push_back({Layout::NN, T, r, outk[k]});
  }
  // the fp16-storage kernels plan their splits differently: size for both
  for (const S& x : v)
    for (int f16src = 0; f16src < 2; ++f16src) {
      GemmDesc d;
      d.layout = x.l;
      d.prec = prec_of(c);
      d.M = x.M; d.N = x.N; d.K = x.K;
      if (f16src) d.a_src = d.b_src = Src::F16;
      m = std::max(m, gemm_workspace(d));
    }
  return m;
}

void carve_scratch(const qblk_config& c, void* base, Scratch& s, size_t& bytes, int lora_rank) {
  const size_t T = (size_t)c.seq * c.batch, h = c.hidden, d = c.head_dim;
  const size_t qd = (size_t)c.heads * d, kvd = (size_t)c.kv_heads * d, I = c.intermediate;
  Carver cv(base);
  s.ds = cv.take<float>(T * I);
  s.dgu = cv.take<float>(T * 2 * I);
  s.dn2 = cv.take<float>(T * h);
  s.dr1 = cv.take<float>(T * h);
  s.d_o = cv.take<float>(T * qd);
  s.dqr = cv.take<float>(T * qd);
  s.dkr = cv.take<float>(T * kvd);
  s.dqkv = cv.take<float>(T * (qd + 2 * kvd));
  s.dn1 = cv.take<float>(T * h);
  s.attn = cv.take<char>(attention_bwd_scratch(c.batch, c.seq, c.heads, c.head_dim));
  s.red = cv.take<float>(rmsnorm_bwd_scratch((int)T, c.hidden) / sizeof(float) + 1);
  s.red_qk = cv.take<float>(qk_norm_rope_bwd_scratch((int)T, c.heads, c.kv_heads, c.head_dim) / sizeof(float) + 1);
  s.red_in = cv.take<float>(rmsnorm_bwd_scratch((int)T, c.hidden) / sizeof(float) + 1);
  s.gemm_ws_bytes = block_gemm_ws(c, lora_rank);
  s.gemm_ws = cv.take<float>(s.gemm_ws_bytes / sizeof(float) + 1);
  s.a16 = nullptr;
  s.pack = Packed16{};
  s.do16 = nullptr;
  if (use_attention_dma(c) && c.gemm_precision != 0) s.do16 = cv.take<f16>(T * qd);
  if (c.gemm_precision != 0 && (lora_rank == 0 || T % 8 == 0))
    s.a16 = cv.take<f16>(T * std::max({qd + 2 * kvd, 2 * I, h, qd}));
  if (c.gemm_precision != 0 && lora_rank == 0) {
    size_t pb = 0;
    carve_pack16(c, nullptr, s.pack, pb);
    char* pbase = cv.take<char>(pb);
    carve_pack16(c, pbase, s.pack, pb);
  }
  bytes = cv.off;
}

void carve_pack16(const qblk_config& c, void* base, Packed16& p, size_t& bytes) {
  const size_t h = c.hidden, d = c.head_dim;
  const size_t qd = (size_t)c.heads * d, kvd = (size_t)c.kv_heads * d, I = c.intermediate;
  const size_t qkv = qd + 2 * kvd;
  Carver cv(base);
  p.qkv = cv.take<f16>(qkv * h);
  p.o = cv.take<f16>(h * qd);
  p.gu = cv.take<f16>(2 * I * h);
  p.d = cv.take<f16>(h * I);
  bytes = cv.off;
}

int pack16(const qblk_config& c, const qblk_block_params& p, const Packed16& o, hipStream_t st) {
  const int h = c.hidden, d = c.head_dim;
  const int qd = c.heads * d, kvd = c.kv_heads * d, I = c.intermediate;
  auto one = [&](int rows, int cols, const float* w, f16* out) {
    return cast_f16(rows, cols, w, cols, out, cols, nullptr, 0, st, bf(c));
  };
  QBLK_TRY(one(qd, h, p.w_q, o.qkv));
  QBLK_TRY(one(kvd, h, p.w_k, o.qkv + (size_t)qd * h));
  QBLK_TRY(one(kvd, h, p.w_v, o.qkv + (size_t)(qd + kvd) * h));
  QBLK_TRY(one(h, qd, p.w_o, o.o));
  QBLK_TRY(one(I, h, p.w_gate, o.gu));
  QBLK_TRY(one(I, h, p.w_up, o.gu + (size_t)I * h));
  QBLK_TRY(one(h, I, p.w_down, o.d));
  return QBLK_OK;
}

int check_config(const qblk_config* c) {
  if (!c) return fail(QBLK_EINVAL, "config is NULL");
  if (c->hidden <= 0 || c->heads <= 0 || c->kv_heads <= 0 || c->head_dim <= 0 || c->intermediate <= 0 ||
      c->seq <= 0 || c->batch <= 0)
    return fail(QBLK_EINVAL, "config: non-positive dimension");
  if (c->heads % c->kv_heads) return fail(QBLK_EINVAL, "config: heads %% kv_heads != 0");
  if (c->hidden % 8 || c->intermediate % 8 || (c->heads * c->head_dim) % 8)
    return fail(QBLK_EINVAL, "config: hidden, intermediate and heads*head_dim must be multiples of 8");
  if (c->head_dim != 16 && c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(QBLK_EUNSUPPORTED, "config: head_dim %d not in {16, 32, 64, 128}", c->head_dim);
  if (c->gemm_precision < 0 || c->gemm_precision > 2)
    return fail(QBLK_EINVAL, "config: gemm_precision must be 0, 1 or 2");
  if (c->gemm_precision == 2) {
    const int64_t T = (int64_t)c->seq * c->batch;
    const int qkv = (c->heads + 2 * c->kv_heads) * c->head_dim;
    if (T % 64 || c->hidden % 64 || c->intermediate % 64 || (c->heads * c->head_dim) % 64 || qkv % 64 ||
        (c->head_dim != 64 && c->head_dim != 128) || c->seq % 8)
      return fail(QBLK_EUNSUPPORTED, "config: bfloat16 operands need seq*batch, hidden, intermediate and the "
                                     "projection widths multiples of 64, head_dim 64 or 128, seq a multiple of 8");
  }
  if (c->gemm_precision == 0 && c->head_dim == 128)
    return fail(QBLK_EUNSUPPORTED, "config: fp32 attention backward supports head_dim <= 64");
  if (!(c->eps >= 0.f) || !(c->rope_theta > 0.f)) return fail(QBLK_EINVAL, "config: eps/rope_theta");
  if (c->hidden > 4096) return fail(QBLK_EUNSUPPORTED, "config: hidden above 4096");
  return QBLK_OK;
}

// ---------------------------------------------------------------- forward

namespace {

AttnDmaArgs attn_dma_args(const qblk_config& c, const Saved& s) {
  const int T = c.seq * c.batch, d = c.head_dim;
  const int qd = c.heads * d, kvd = c.kv_heads * d;
  AttnDmaArgs a{};
  a.batch = c.batch; a.seq = c.seq; a.heads = c.heads; a.kv_heads = c.kv_heads; a.head_dim = d;
  if (s.q16) {  // fp16 copies
    a.fp32 = 0;
    a.q = s.q16; a.ldq = qd;
    a.k = s.k16; a.ldk = kvd;
    a.v = s.v16; a.ldv = kvd;
  } else {  // fp32: the tensors themselves
    a.fp32 = 1;
    a.q = s.qr; a.ldq = qd;
    a.k = s.kr; a.ldk = kvd;
    a.v = s.qkv + qd + kvd; a.ldv = qd + 2 * kvd;
  }
  a.bf16 = bf(c);
  a.o = s.o; a.ldo = qd;
  a.lse = s.lse;
  return a;
}

}  // namespace

// Projection hooks: the fp32/fp16 block uses the dense fp32 weights; the
// NF4 block substitutes dequant + LoRA GEMMs (nf4_block.hip).
int block_forward_impl(const qblk_config& c, const ProjFwd& proj, const float* g_in, const float* g_post,
                       const float* g_q, const float* g_k, const float* x, float* y, const Saved& s,
                       void* attn_ws, hipStream_t st) {
  const int T = c.seq * c.batch, h = c.hidden, d = c.head_dim;
  const int qd = c.heads * d, kvd = c.kv_heads * d, I = c.intermediate;
  const int ldqkv = qd + 2 * kvd;

  // the input norm's launch also writes the RoPE table (independent work)
  const RopeTabJob tj = rope_table_job(c.seq, d, c.rope_theta, s.tab);
  QBLK_TRY(rmsnorm_forward(T, h, c.eps, x, nullptr, g_in, s.n1, s.n1_16, nullptr, s.rho1, st, &tj, bf(c)));
  QBLK_TRY(proj.qkv(s.n1, s.qkv, st));
  QkRopeArgs qa{T, c.seq, c.heads, c.kv_heads, d, c.qk_norm, c.eps, s.qkv, ldqkv, g_q, g_k, s.tab,
                s.qr, s.kr, s.rho_q, s.rho_k};
  qa.bf16 = bf(c);
  if (s.q16) {  // attention reads only the fp16 operand copies, written here
    qa.q16 = s.q16;
    qa.k16 = s.k16;
    qa.v16 = s.v16;
    qa.qr = qa.kr = nullptr;
  }
  QBLK_TRY(qk_norm_rope_forward(qa, st));
  if (use_attention_dma(c)) {
    AttnDmaArgs af = attn_dma_args(c, s);
    af.o16 = s.o16;
    QBLK_TRY(attention_dma_forward(af, attn_ws, st));
  } else {
    AttnArgs aa{};
    aa.batch = c.batch; aa.seq = c.seq; aa.heads = c.heads; aa.kv_heads = c.kv_heads; aa.head_dim = d;
    aa.q = s.qr; aa.ldq = qd;
    aa.k = s.kr; aa.ldk = kvd;
    aa.v = s.qkv + qd + kvd; aa.ldv = ldqkv;
    aa.o = s.o; aa.ldo = qd;
    aa.lse = s.lse;
    QBLK_TRY(attention_forward(aa, prec_of(c), st));
    if (s.o16) QBLK_TRY(cast_f16(T, qd, s.o, qd, s.o16, qd, nullptr, 0, st, bf(c)));
  }
  QBLK_TRY(proj.o(s.o, x, s.r1, st));  // r1 = x + o Wo^T
  QBLK_TRY(rmsnorm_forward(T, h, c.eps, s.r1, nullptr, g_post, s.n2, s.n2_16, nullptr, s.rho2, st, nullptr, bf(c)));
  QBLK_TRY(proj.gate_up(s.n2, s.gu, st));
  QBLK_TRY(swiglu_forward(T, I, s.gu, s.s, s.s16, st, bf(c)));
  QBLK_TRY(proj.down(s.s, s.r1, y, st));  // y = r1 + s Wd^T
  return QBLK_OK;
}

int block_backward_impl(const qblk_config& c, const ProjBwd& proj, const float* g_in, const float* g_post,
                        const float* g_q, const float* g_k, const float* x, const float* dy, const Saved& s,
                        float* dx, float* dg_in, float* dg_post, float* dg_q, float* dg_k, const Scratch& w,
                        hipStream_t st, bool accumulate) {
  const int T = c.seq * c.batch, h = c.hidden, d = c.head_dim;
  const int qd = c.heads * d, kvd = c.kv_heads * d, I = c.intermediate;
  const int ldqkv = qd + 2 * kvd;

  // With prod16 each output gradient's fp16 copy comes from its producer
  // (SwiGLU backward, norm backward, the O projection's dX product, the
  // attention and QK-norm backward) and the hooks get a null fp32 pointer.
  const bool p16 = w.prod16, qkv16 = p16 && s.q16 != nullptr;
  // FFN: ds = dy Wd; dWd = dy^T s; SwiGLU backward; dn2 = dg Wg + du Wu; dWg, dWu.
  QBLK_TRY(proj.down(dy, s.s, w.ds, st));
  QBLK_TRY(swiglu_backward(T, I, s.gu, w.ds, p16 ? nullptr : w.dgu, p16 ? w.a16 : nullptr, st, bf(c)));
  QBLK_TRY(proj.gate_up(p16 ? nullptr : w.dgu, s.n2, w.dn2, st));
  // post-attention norm backward, plus the second residual's gradient dy
  // the gamma gradients are finished by one column-sum launch at the end
  ColsumJob jobs[kMaxColsumJobs];
  int nj = 0;
  QBLK_TRY(rmsnorm_backward_partials(T, h, c.eps, s.r1, g_post, w.dn2, dy, w.dr1, p16 ? w.a16 : nullptr, w.red,
                                     st, bf(c)));
  jobs[nj++] = ColsumJob{rmsnorm_bwd_parts(T, h), h, w.red, dg_post, accumulate};
  // O projection
  QBLK_TRY(proj.o(p16 ? nullptr : w.dr1, s.o, w.d_o, st));
  // attention backward: dq, dk at the attention inputs; dv straight into dqkv
  if (use_attention_dma(c)) {
    AttnDmaArgs ab = attn_dma_args(c, s);
    if (s.q16) {
      if (!p16) QBLK_TRY(cast_f16(T, qd, w.d_o, qd, w.do16, qd, nullptr, 0, st, bf(c)));
      ab.d_o = w.do16;
    } else {
      ab.d_o = w.d_o;
    }
    ab.lddo = qd;
    ab.do32 = w.d_o; ab.lddo32 = qd;
    ab.dq = w.dqr; ab.lddq = qd;
    ab.dk = w.dkr; ab.lddk = kvd;
    ab.dv = w.dqkv + qd + kvd; ab.lddv = ldqkv;
    if (qkv16) {
      ab.dv16 = w.a16 + qd + kvd;
      ab.lddv16 = ldqkv;
    }
    QBLK_TRY(attention_dma_backward(ab, w.attn, st));
  } else {
    AttnArgs aa{};
    aa.batch = c.batch; aa.seq = c.seq; aa.heads = c.heads; aa.kv_heads = c.kv_heads; aa.head_dim = d;
    aa.q = s.qr; aa.ldq = qd;
    aa.k = s.kr; aa.ldk = kvd;
    aa.v = s.qkv + qd + kvd; aa.ldv = ldqkv;
    aa.o = s.o; aa.ldo = qd;
    aa.lse = s.lse;
    aa.d_o = w.d_o; aa.lddo = qd;
    aa.dq = w.dqr; aa.lddq = qd;
    aa.dk = w.dkr; aa.lddk = kvd;
    aa.dv = w.dqkv + qd + kvd; aa.lddv = ldqkv;
    QBLK_TRY(attention_backward(aa, prec_of(c), w.attn, st));
  }
  QkRopeBwdArgs qb{T, c.seq, c.heads, c.kv_heads, d, c.qk_norm, c.eps, s.qkv, ldqkv, g_q, g_k, s.tab,
                   w.dqr, w.dkr, w.dqkv, dg_q, dg_k};
  if (qkv16) {
    qb.dqkv = nullptr;
    qb.dqkv16 = w.a16;
  }
  qb.accumulate_dg = accumulate;
  qb.bf16 = bf(c);
  QBLK_TRY(qk_norm_rope_backward_partials(qb, w.red_qk, jobs, nj, st));
  QBLK_TRY(proj.qkv(qkv16 ? nullptr : w.dqkv, s.n1, w.dn1, st));
  // input norm backward, plus the first residual's gradient dr1
  QBLK_TRY(rmsnorm_backward_partials(T, h, c.eps, x, g_in, w.dn1, w.dr1, dx, nullptr, w.red_in, st));
  jobs[nj++] = ColsumJob{rmsnorm_bwd_parts(T, h), h, w.red_in, dg_in, accumulate};
  return colsum_jobs(nj, jobs, st);
}

// ------------------------------------------------- dense (fp32 master) block

namespace {

GemmDesc nt(const qblk_config& c, const Scratch& w, int M, int N, int K, const float* a, int64_t lda, Seg b,
            int64_t ldb, float* out, int64_t ldc) {
  GemmDesc g;
  g.ws = w.gemm_ws;
  g.ws_bytes = w.gemm_ws_bytes;
  g.layout = Layout::NT;
  g.prec = prec_of(c);
  g.M = M; g.N = N; g.K = K;
  g.a = a; g.lda = lda;
  g.b = b; g.ldb = ldb;
  g.c = seg1(out, M); g.ldc = ldc;
  return g;
}

Seg seg3(const void* a, int na, const void* b, int nb, const void* cc, int nc) {
  Seg s;
  s.p[0] = a; s.p[1] = b; s.p[2] = cc;
  s.start[0] = 0; s.start[1] = na; s.start[2] = na + nb; s.start[3] = na + nb + nc;
  s.nseg = cc ? 3 : 2;
  return s;
}

// Both operands 16-bit (the direct-to-LDS GEMM kernel's operands), fp16 or
// bfloat16 as the block's precision says.
GemmDesc g16(const qblk_config& cfg, const Scratch& w, Layout l, int M, int N, int K, const f16* a, int64_t lda,
             const f16* b, int64_t ldb, Seg c, int64_t ldc) {
  GemmDesc g;
  g.ws = w.gemm_ws;
  g.ws_bytes = w.gemm_ws_bytes;
  g.layout = l;
  g.prec = prec_of(cfg);
  g.M = M; g.N = N; g.K = K;
  g.a = a; g.lda = lda; g.a_src = Src::F16;
  g.b = seg1(b, l == Layout::NT ? N : K); g.ldb = ldb; g.b_src = Src::F16;
  g.c = c; g.ldc = ldc;
  return g;
}

// The fp16 copies path needs fp16 row strides (T for the transposed
// attention copies) that are multiples of 8.
bool use_f16_copies(const qblk_config& c) {
  return c.gemm_precision != 0 && (c.seq * c.batch) % 8 == 0;
}

// The weights' fp16 copies: the caller's packed set, or cast into scratch.
int weights16(const qblk_config& c, const qblk_block_params& p, const Scratch& w, Packed16& W, hipStream_t st) {
  if (p.w16) {
    size_t b = 0;
    carve_pack16(c, (void*)p.w16, W, b);
    return QBLK_OK;
  }
  W = w.pack;
  return pack16(c, p, W, st);
}

// Forward products read the fp16 copies the producers wrote into `saved`
// (n1, o, n2, s) and the weights' fp16 copies: y (+ res) = act16 W16^T.
int dense16_forward(const qblk_config& c, const qblk_block_params& p, const float* x, float* y, const Saved& s,
                    const Scratch& w, hipStream_t st) {
  const int T = c.seq * c.batch, h = c.hidden, d = c.head_dim;
  const int qd = c.heads * d, kvd = c.kv_heads * d, I = c.intermediate, qkv = qd + 2 * kvd;
  Packed16 W;
  QBLK_TRY(weights16(c, p, w, W, st));
  auto proj = [&](const f16* act, int n_in, const f16* wt, int n_out, const float* res, float* out,
                  hipStream_t s_) -> int {
    GemmDesc g = g16(c, w, Layout::NT, T, n_out, n_in, act, n_in, wt, n_in, seg1(out, T), n_out);
    g.r = res; g.ldr = n_out;
    return gemm(g, s_);
  };
  ProjFwd pf;
  pf.qkv = [&](const float*, float* out, hipStream_t s_) { return proj(s.n1_16, h, W.qkv, qkv, nullptr, out, s_); };
  pf.o = [&](const float*, const float* res, float* out, hipStream_t s_) {
    return proj(s.o16, qd, W.o, h, res, out, s_);
  };
  pf.gate_up = [&](const float*, float* out, hipStream_t s_) {
    return proj(s.n2_16, h, W.gu, 2 * I, nullptr, out, s_);
  };
  pf.down = [&](const float*, const float* res, float* out, hipStream_t s_) {
    return proj(s.s16, I, W.d, h, res, out, s_);
  };
  // n1, n2 and s are read only through their fp16 copies on this path
  // (products and weight gradients; the norm backwards read x, r1 and the
  // saved rho): their fp32 forms are not written
  Saved s16 = s;
  s16.n1 = s16.n2 = s16.s = nullptr;
  return block_forward_impl(c, pf, p.g_in, p.g_post, p.g_q, p.g_k, x, y, s16, w.attn, st);
}

// dX = dY W (NN: dY16 [T, n_out] K-major, W16 [n_out, n_in] read out-major)
// and dW = dY^T X (TN: dY16 and the saved X16 [T, n_in], both read
// token-major); dY is cast to fp16 once for both.
int dense16_backward(const qblk_config& c, const qblk_block_params& p, const qblk_block_grads& gr,
                     const float* x, const float* dy, const Saved& s, float* dx, const Scratch& w,
                     hipStream_t st, bool accumulate) {
  const int T = c.seq * c.batch, h = c.hidden, d = c.head_dim;
  const int qd = c.heads * d, kvd = c.kv_heads * d, I = c.intermediate, qkv = qd + 2 * kvd;
  Packed16 W;
  QBLK_TRY(weights16(c, p, w, W, st));
  // dY's fp16 copy is in a16 already when the hook is passed no fp32 dY;
  // dx16 (optional) receives an fp16 copy of dX.
  auto dxdw = [&](const float* dyv, int n_out, const f16* x16, int n_in, const f16* wt, Seg cseg, float* dxo,
                  f16* dx16, hipStream_t s_) -> int {
    if (dyv) QBLK_TRY(cast_f16(T, n_out, dyv, n_out, w.a16, n_out, nullptr, 0, s_, bf(c)));
    GemmDesc gx = g16(c, w, Layout::NN, T, n_in, n_out, w.a16, n_out, wt, n_in, seg1(dxo, T), n_in);
    gx.c16 = dx16;
    gx.ldc16 = n_in;
    QBLK_TRY(gemm(gx, s_));
    GemmDesc gw = g16(c, w, Layout::TN, n_out, n_in, T, w.a16, n_out, x16, n_in, cseg, n_in);
    gw.accumulate = accumulate;
    return gemm(gw, s_);
  };
  ProjBwd pb;
  pb.down = [&](const float* dyv, const float*, float* ds, hipStream_t s_) {
    return dxdw(dyv, h, s.s16, I, W.d, seg1(gr.w_down, h), ds, nullptr, s_);
  };
  pb.gate_up = [&](const float* dgu, const float*, float* dn2, hipStream_t s_) {
    return dxdw(dgu, 2 * I, s.n2_16, h, W.gu, seg3(gr.w_gate, I, gr.w_up, I, nullptr, 0), dn2, nullptr, s_);
  };
  pb.o = [&](const float* dr1, const float*, float* d_o, hipStream_t s_) {
    // the attention backward reads dO's fp16 copy
    return dxdw(dr1, h, s.o16, qd, W.o, seg1(gr.w_o, h), d_o, s.q16 ? w.do16 : nullptr, s_);
  };
  pb.qkv = [&](const float* dqkv, const float*, float* dn1, hipStream_t s_) {
    return dxdw(dqkv, qkv, s.n1_16, h, W.qkv, seg3(gr.w_q, qd, gr.w_k, kvd, gr.w_v, kvd), dn1, nullptr, s_);
  };
  Scratch w16 = w;
  w16.prod16 = true;
  return block_backward_impl(c, pb, p.g_in, p.g_post, p.g_q, p.g_k, x, dy, s, dx, gr.g_in, gr.g_post,
                             gr.g_q, gr.g_k, w16, st, accumulate);
}

}  // namespace

int dense_block_forward(const qblk_config& c, const qblk_block_params& p, const float* x, float* y,
                        const Saved& s, const Scratch& w, hipStream_t st) {
  const int T = c.seq * c.batch, h = c.hidden, d = c.head_dim;
  const int qd = c.heads * d, kvd = c.kv_heads * d, I = c.intermediate;
  if (use_f16_copies(c)) return dense16_forward(c, p, x, y, s, w, st);
  ProjFwd proj;
  proj.qkv = [&](const float* n1, float* qkv, hipStream_t s_) {
    return gemm(nt(c, w, T, qd + 2 * kvd, h, n1, h, seg3(p.w_q, qd, p.w_k, kvd, p.w_v, kvd), h, qkv, qd + 2 * kvd),
                s_);
  };
  proj.o = [&](const float* o, const float* res, float* out, hipStream_t s_) {
    GemmDesc g = nt(c, w, T, h, qd, o, qd, seg1(p.w_o, h), qd, out, h);
    g.r = res; g.ldr = h;
    return gemm(g, s_);
  };
  proj.gate_up = [&](const float* n2, float* gu, hipStream_t s_) {
    Seg b = seg3(p.w_gate, I, p.w_up, I, nullptr, 0);
    return gemm(nt(c, w, T, 2 * I, h, n2, h, b, h, gu, 2 * I), s_);
  };
  proj.down = [&](const float* sv, const float* res, float* out, hipStream_t s_) {
    GemmDesc g = nt(c, w, T, h, I, sv, I, seg1(p.w_down, h), I, out, h);
    g.r = res; g.ldr = h;
    return gemm(g, s_);
  };
  return block_forward_impl(c, proj, p.g_in, p.g_post, p.g_q, p.g_k, x, y, s, w.attn, st);
}

int dense_block_backward(const qblk_config& c, const qblk_block_params& p, const qblk_block_grads& gr,
                         const float* x, const float* dy, const Saved& s, float* dx, const Scratch& w,
                         hipStream_t st, bool accumulate) {
  const int T = c.seq * c.batch, h = c.hidden, d = c.head_dim;
  const int qd = c.heads * d, kvd = c.kv_heads * d, I = c.intermediate;
  const Prec pr = prec_of(c);
  if (use_f16_copies(c)) return dense16_backward(c, p, gr, x, dy, s, dx, w, st, accumulate);
  // dX = dY W (NN, B = W [out, in] with out the contraction) and
  // dW = dY^T X (TN). `wseg` are the weights stacked along out; `cseg` the
  // gradient tensors split the same way.
  auto dxdw = [&](const float* dyv, int n_out, const float* xin, int n_in, Seg wseg, Seg cseg, float* dxo,
                  hipStream_t s_) -> int {
    GemmDesc a;
    a.ws = w.gemm_ws; a.ws_bytes = w.gemm_ws_bytes;
    a.layout = Layout::NN; a.prec = pr;
    a.M = T; a.N = n_in; a.K = n_out;
    a.a = dyv; a.lda = n_out;
    a.b = wseg; a.ldb = n_in;
    a.c = seg1(dxo, T); a.ldc = n_in;
    QBLK_TRY(gemm(a, s_));
    GemmDesc b;
    b.ws = w.gemm_ws; b.ws_bytes = w.gemm_ws_bytes;
    b.layout = Layout::TN; b.prec = pr;
    b.M = n_out; b.N = n_in; b.K = T;
    b.a = dyv; b.lda = n_out;
    b.b = seg1(xin, T); b.ldb = n_in;
    b.c = cseg; b.ldc = n_in;
    b.accumulate = accumulate;
    return gemm(b, s_);
  };
  ProjBwd proj;
  proj.down = [&](const float* dyv, const float* sv, float* ds, hipStream_t s_) {
    return dxdw(dyv, h, sv, I, seg1(p.w_down, h), seg1(gr.w_down, h), ds, s_);
  };
  proj.gate_up = [&](const float* dgu, const float* n2, float* dn2, hipStream_t s_) {
    return dxdw(dgu, 2 * I, n2, h, seg3(p.w_gate, I, p.w_up, I, nullptr, 0),
                seg3(gr.w_gate, I, gr.w_up, I, nullptr, 0), dn2, s_);
  };
  proj.o = [&](const float* dr1, const float* o, float* d_o, hipStream_t s_) {
    return dxdw(dr1, h, o, qd, seg1(p.w_o, h), seg1(gr.w_o, h), d_o, s_);
  };
  proj.qkv = [&](const float* dqkv, const float* n1, float* dn1, hipStream_t s_) {
    return dxdw(dqkv, qd + 2 * kvd, n1, h, seg3(p.w_q, qd, p.w_k, kvd, p.w_v, kvd),
                seg3(gr.w_q, qd, gr.w_k, kvd, gr.w_v, kvd), dn1, s_);
  };
  return block_backward_impl(c, proj, p.g_in, p.g_post, p.g_q, p.g_k, x, dy, s, dx, gr.g_in, gr.g_post,
                             gr.g_q, gr.g_k, w, st, accumulate);
}

}  // namespace qblk
