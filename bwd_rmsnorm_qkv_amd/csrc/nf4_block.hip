// Frozen-NF4 decoder block with LoRA on all seven projections.
//
// cuda_block.rs page: CudaNf4TransformerBlock (NF4 codes + per-block scales
// for the 7 projections, the fused dequant + GEMM path, a backward that
// yields activation and LoRA gradients only). wgpu_trainer.rs page:
// lora_forward / lora_backward (A [rank, in], B [out, rank], scale
// alpha/rank, with h = x A^T kept from the forward).
//
// Design. Two paths share the launch sequence of the dense block:
// * fp16 operands (T a multiple of 8): the activations' fp16 copies are
//   written by their producers. Each projection group runs ONE fused
//   dequant + GEMM (gemm_nf4_kernel: the NF4 codes are decoded into LDS
//   while the tile is staged, never written out) whose last K tile is the
//   LoRA branch: y = [x | s h] [W~ | B]^T with h = x A^T, s = alpha/rank,
//   B block-diagonal over the group's projections; backward dX = [dY | dh]
//   [W~ ; A] with dh = s dY B. The rank-r products (h, dh, dA, dB) run on
//   the fp16 DMA GEMM over 64 zero-padded LoRA columns. Shapes the fused
//   kernel does not take (K or the row length not a multiple of 64) decode
//   the group into an fp16 scratch copy and run the dense product instead.
// * otherwise (fp32 operand storage): the codes are decoded while the
//   register-staged GEMM stages its B operand and the LoRA branch rides in
//   the same GEMM as extra K columns; dA and dB are small TN GEMMs.
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
  // x A^T of each projection group: [T, n r] (fp32 operand path) or, on
  // the fp16 path, s x A^T over 64 zero-padded columns [T, 64] and its
  // fp16 copy (the LoRA K tile of the forward, the B side of dB).
  float *h_qkv, *h_o, *h_gu, *h_d;
  f16 *hs16_qkv, *hs16_o, *hs16_gu, *hs16_d;
};

struct Nf4Scratch {
  Scratch base;
  float *dh_qkv, *dh_o, *dh_gu, *dh_d;  // s dY B ([T, n r]; fp16 path: [T, 64])
  f16* dh16;                            // fp16 path: fp16 copy of the current group's dh [T, 64]
  // fp16 path, per projection group (q|k|v, o, gate|up, down), packed once
  // per call: [A_0; A_1; A_2; 0] [64, in], block-diagonal B [out, 64] and
  // its transpose [64, out]
  f16 *a16x[4], *bx16[4], *bt16[4];
  float *sink_h, *sink_d;               // gamma gradients are not outputs
  f16* w16;                             // fp16 W~ of the current group (dense fallback)
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
  const bool f16p = c.gemm_precision == 1 && T % 8 == 0;
  const size_t hw = f16p ? 64 : 3 * (size_t)r;
  s->h_qkv = take(saved, sb, T * hw);
  s->h_o = take(saved, sb, T * hw);
  s->h_gu = take(saved, sb, T * hw);
  s->h_d = take(saved, sb, T * hw);
  s->hs16_qkv = s->hs16_o = s->hs16_gu = s->hs16_d = nullptr;
  w->dh16 = w->w16 = nullptr;
  for (int g = 0; g < 4; ++g) w->a16x[g] = w->bx16[g] = w->bt16[g] = nullptr;
  if (f16p) {
    s->hs16_qkv = (f16*)take(saved, sb, T * 32);
    s->hs16_o = (f16*)take(saved, sb, T * 32);
    s->hs16_gu = (f16*)take(saved, sb, T * 32);
    s->hs16_d = (f16*)take(saved, sb, T * 32);
  }
  w->dh_qkv = take(scratch, wb, T * hw);
  w->dh_o = take(scratch, wb, T * hw);
  w->dh_gu = take(scratch, wb, T * hw);
  w->dh_d = take(scratch, wb, T * hw);
  w->sink_h = take(scratch, wb, 2 * (size_t)c.hidden);
  w->sink_d = take(scratch, wb, 2 * (size_t)c.head_dim);
  if (f16p) {
    const size_t h = c.hidden, qd = (size_t)c.heads * c.head_dim, kvd = (size_t)c.kv_heads * c.head_dim;
    const size_t I = c.intermediate, qkv = qd + 2 * kvd;
    const size_t wmax = std::max({qkv * h, h * qd, 2 * I * h, h * I});
    const size_t ins[4] = {h, qd, h, I}, outs[4] = {qkv, h, 2 * I, h};
    w->dh16 = (f16*)take(scratch, wb, T * 32);
    for (int g = 0; g < 4; ++g) {
      w->a16x[g] = (f16*)take(scratch, wb, 32 * ins[g]);
      w->bx16[g] = (f16*)take(scratch, wb, 32 * outs[g]);
      w->bt16[g] = (f16*)take(scratch, wb, 32 * outs[g]);
    }
    w->w16 = (f16*)take(scratch, wb, wmax / 2 + 64);
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

// fp16 W~ of a projection group, stacked along out, into w16 (the dense
// fallback of the fp16 path).
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

// The LoRA matrices of a group as fp16 operands over 64 padded columns:
//   mode 0: a16x [64, in],  row k r + j = A_k[j, :];
//   mode 1: bx16 [out, 64], row o of segment k holds B_k[o - start_k, :] at
//           columns k r .. k r + r - 1;
//   mode 2: bt16 [64, out], the transpose of mode 1.
// Every other element is zero.
struct LoraPack {
  const float* m[3];
  int start[4];  // segment starts along out (modes 1, 2)
  int n, r, in, out, mode;
};

// Several packs in one launch: job j fills dst[j] with its count[j]
// elements, taken by the workgroups from begin[j] / 256 on (every job
// starts on a workgroup boundary, so a workgroup's job is uniform and its
// fields are scalar loads).
constexpr int kMaxPackJobs = 8;
struct LoraPackJobs {
  LoraPack job[kMaxPackJobs];
  f16* dst[kMaxPackJobs];
  int begin[kMaxPackJobs + 1];  // in elements, multiples of 256
  int count[kMaxPackJobs];
  int njobs;
};

__global__ __launch_bounds__(256) void lora_pack16_kernel(const LoraPackJobs J) {
  // every index fits 32 bits (64 x the widest projection side per job)
  const int g0 = blockIdx.x * 256;
  int j = 0;
  while (j + 1 < J.njobs && g0 >= J.begin[j + 1]) ++j;
  j = __builtin_amdgcn_readfirstlane(j);
  const LoraPack& a = J.job[j];
  const int e = g0 - J.begin[j] + threadIdx.x;
  if (e >= J.count[j]) return;
  float v = 0.f;
  if (a.mode == 0) {
    const int row = e / a.in, col = e - row * a.in;
    if (row < a.n * a.r) {
      const int k = row / a.r;
      const float* m = k == 0 ? a.m[0] : k == 1 ? a.m[1] : a.m[2];
      v = m[(int64_t)(row - k * a.r) * a.in + col];
    }
  } else if (a.mode == 1) {
    const int o = e >> 6, c = e & 63;
    const int k = (a.n > 1 && o >= a.start[1]) + (a.n > 2 && o >= a.start[2]);
    const float* m = k == 0 ? a.m[0] : k == 1 ? a.m[1] : a.m[2];
    const int o0 = k == 0 ? a.start[0] : k == 1 ? a.start[1] : a.start[2];
    if (c >= k * a.r && c < (k + 1) * a.r) v = m[(int64_t)(o - o0) * a.r + (c - k * a.r)];
  } else {
    // the transpose: a thread takes columns 4 c4 .. 4 c4 + 3 of one row o
    // of B (one contiguous read; r is a multiple of 4, so they lie in one
    // block) and writes them down four rows of the [64, out] operand
    const int o = e % a.out, c4 = e / a.out;
    const int k = (a.n > 1 && o >= a.start[1]) + (a.n > 2 && o >= a.start[2]);
    const float* m = k == 0 ? a.m[0] : k == 1 ? a.m[1] : a.m[2];
    const int o0 = k == 0 ? a.start[0] : k == 1 ? a.start[1] : a.start[2];
    float q[4] = {0.f, 0.f, 0.f, 0.f};
    if (4 * c4 >= k * a.r && 4 * c4 < (k + 1) * a.r) {
      const float* src = m + (int64_t)(o - o0) * a.r + (4 * c4 - k * a.r);
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = src[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) J.dst[j][(int64_t)(4 * c4 + i) * a.out + o] = (f16)q[i];
    return;
  }
  J.dst[j][e] = (f16)v;
}

LoraPack lora_pack_job(const qblk_nf4_block_params& p, const int* id3, const int* outd, int n, int in, int mode) {
  LoraPack a{};
  a.n = n; a.r = p.rank; a.in = in; a.mode = mode;
  int o = 0;
  for (int k = 0; k < n; ++k) {
    a.m[k] = mode == 0 ? p.lora_a[id3[k]] : p.lora_b[id3[k]];
    a.start[k] = o;
    o += outd[k];
  }
  a.start[n] = o;
  a.out = o;
  return a;
}

struct Group {
  int id3[3] = {-1, -1, -1}, outd[3] = {0, 0, 0}, n = 0, N = 0;
  Group(std::initializer_list<int> ids, std::initializer_list<int> outs) {
    for (int id : ids) id3[n++] = id;
    int j = 0;
    for (int o : outs) outd[j++] = o;
    for (int k = 0; k < n; ++k) N += outd[k];
  }
};

// The 4 groups' packs of the given two modes into their buffers, one launch.
int lora_pack16_groups(const qblk_nf4_block_params& p, const Group* gs, const int* ins, int mode_a, f16* const* dst_a,
                       int mode_b, f16* const* dst_b, hipStream_t st) {
  LoraPackJobs J{};
  int64_t acc = 0;
  for (int gi = 0; gi < 4; ++gi)
    for (int t = 0; t < 2; ++t) {
      const int mode = t ? mode_b : mode_a;
      const LoraPack a = lora_pack_job(p, gs[gi].id3, gs[gi].outd, gs[gi].n, ins[gi], mode);
      J.job[J.njobs] = a;
      // mode 2 threads each write four elements
      const int64_t cnt = mode == 0 ? 64 * (int64_t)a.in : (mode == 1 ? 64 : 16) * (int64_t)a.out;
      J.dst[J.njobs] = (t ? dst_b : dst_a)[gi];
      J.begin[J.njobs] = (int)acc;
      J.count[J.njobs] = (int)cnt;
      acc += ceil_div(cnt, 256) * 256;
      ++J.njobs;
      if (acc >= (int64_t)1 << 31) return fail(QBLK_EUNSUPPORTED, "nf4 block: LoRA operands too large to pack");
    }
  J.begin[J.njobs] = (int)acc;
  hipLaunchKernelGGL(lora_pack16_kernel, dim3((unsigned)(acc / 256)), dim3(256), 0, st, J);
  return check_launch("lora_pack16_kernel");
}

// Forward of one group on the fp16 path:
//   hs = s x16 [A stacked]^T over 64 columns (fp32 `hs`, fp16 `hs16`);
//   out (+ res) = x16 W~^T + hs16 bx16^T, fused (NF4 decoded in the GEMM).
int nf4_fwd16(const qblk_nf4_block_params& p, const Nf4Scratch& w, int gi, int T, int in, const f16* x16,
              const Group& g, float* hs, f16* hs16, const float* res, float* out, hipStream_t st) {
  const float sc = p.alpha / (float)p.rank;
  const f16* a16x = w.a16x[gi];
  const f16* bx16 = w.bx16[gi];
  {
    GemmDesc d = base(Layout::NT, T, 64, in);
    d.a = x16; d.lda = in; d.a_src = Src::F16;
    d.b = seg1(a16x, 64); d.ldb = in; d.b_src = Src::F16;
    d.c = seg1(hs, T); d.ldc = 64;
    d.alpha = sc;
    d.c16 = hs16; d.ldc16 = 64;
    QBLK_TRY(gemm(d, st));
  }
  GemmDesc d = base(Layout::NT, T, g.N, in);
  d.a = x16; d.lda = in; d.a_src = Src::F16;
  d.b = rows3(g.outd[0], g.outd[1], g.outd[2]); d.ldb = in;
  d.b_src = Src::NF4;
  d.nf4 = nf4seg(p, g.id3[0], g.id3[1], g.id3[2]);
  d.c = seg1(out, T); d.ldc = g.N;
  d.r = res; d.ldr = g.N;
  d.ext16_a = hs16; d.ext16_lda = 64;
  d.ext16_b = bx16; d.ext16_ldb = 64;
  if (gemm_nf4_fused(d)) return gemm(d, st);
  // dense fallback: decoded copy, then the LoRA tile as an accumulating product
  QBLK_TRY(dequant_group(p, g.id3, g.outd, g.n, in, w.w16, st));
  GemmDesc e = base(Layout::NT, T, g.N, in);
  e.a = x16; e.lda = in; e.a_src = Src::F16;
  e.b = seg1(w.w16, g.N); e.ldb = in; e.b_src = Src::F16;
  e.c = seg1(out, T); e.ldc = g.N;
  e.r = res; e.ldr = g.N;
  QBLK_TRY(gemm(e, st));
  GemmDesc u = base(Layout::NT, T, g.N, 64);
  u.a = hs16; u.lda = 64; u.a_src = Src::F16;
  u.b = seg1(bx16, g.N); u.ldb = 64; u.b_src = Src::F16;
  u.c = seg1(out, T); u.ldc = g.N;
  u.accumulate = 1;
  return gemm(u, st);
}

// Backward of one group on the fp16 path, dY given as its fp16 copy dy16
// [T, N] (written by its producer):
//   dh = s dY16 B (over 64 columns; fp32 dh and its fp16 copy);
//   dX = dY16 W~ + dh16 [A stacked], fused (fp16 copy into dx16 if set);
//   dB_k = dY16_k^T hs16_k (diagonal blocks); dA_k = dh16_k^T X16.
int nf4_bwd16(const qblk_nf4_block_params& p, const qblk_lora_grads& gr, const Nf4Scratch& w, int gi, int T,
              int in, const f16* dy16, const f16* x16, const f16* hs16, const Group& g, float* dh, float* dx,
              f16* dx16, hipStream_t st) {
  const float sc = p.alpha / (float)p.rank;
  const int r = p.rank, n = g.n;
  const f16* a16x = w.a16x[gi];
  const f16* bt16 = w.bt16[gi];
  {
    GemmDesc d = base(Layout::NT, T, 64, g.N);
    d.a = dy16; d.lda = g.N; d.a_src = Src::F16;
    d.b = seg1(bt16, 64); d.ldb = g.N; d.b_src = Src::F16;
    d.c = seg1(dh, T); d.ldc = 64;
    d.alpha = sc;
    d.c16 = w.dh16; d.ldc16 = 64;
    QBLK_TRY(gemm(d, st));
  }
  {
    GemmDesc d = base(Layout::NN, T, in, g.N);
    d.a = dy16; d.lda = g.N; d.a_src = Src::F16;
    d.b = rows3(g.outd[0], g.outd[1], g.outd[2]); d.ldb = in;
    d.b_src = Src::NF4;
    d.nf4 = nf4seg(p, g.id3[0], g.id3[1], g.id3[2]);
    d.c = seg1(dx, T); d.ldc = in;
    d.c16 = dx16; d.ldc16 = in;
    d.ext16_a = w.dh16; d.ext16_lda = 64;
    d.ext16_b = a16x; d.ext16_ldb = in;
    if (gemm_nf4_fused(d)) {
      QBLK_TRY(gemm(d, st));
    } else {
      QBLK_TRY(dequant_group(p, g.id3, g.outd, n, in, w.w16, st));
      GemmDesc e = base(Layout::NN, T, in, g.N);
      e.a = dy16; e.lda = g.N; e.a_src = Src::F16;
      e.b = seg1(w.w16, g.N); e.ldb = in; e.b_src = Src::F16;
      e.c = seg1(dx, T); e.ldc = in;
      QBLK_TRY(gemm(e, st));
      GemmDesc u = base(Layout::NN, T, in, 64);
      u.a = w.dh16; u.lda = 64; u.a_src = Src::F16;
      u.b = seg1(a16x, 64); u.ldb = in; u.b_src = Src::F16;
      u.c = seg1(dx, T); u.ldc = in;
      u.c16 = dx16; u.ldc16 = in;
      u.accumulate = 1;
      QBLK_TRY(gemm(u, st));
    }
  }
  {  // dB_k = dY16_k^T hs16_k (s is in hs16)
    GemmDesc d = base(Layout::TN, g.N, 64, T);
    d.a = dy16; d.lda = g.N; d.a_src = Src::F16;
    d.b = seg1(hs16, T); d.ldb = 64; d.b_src = Src::F16;
    d.c = rows3(g.outd[0], g.outd[1], g.outd[2]);
    for (int k = 0; k < n; ++k) d.c.p[k] = gr.lora_b[g.id3[k]];
    d.ldc = r;
    d.c_cols_blockdiag = r;
    QBLK_TRY(gemm(d, st));
  }
  {  // dA_k = dh16_k^T X16
    GemmDesc d = base(Layout::TN, n * r, in, T);
    d.a = w.dh16; d.lda = 64; d.a_src = Src::F16;
    d.b = seg1(x16, T); d.ldb = in; d.b_src = Src::F16;
    d.c = rows3(r, n > 1 ? r : 0, n > 2 ? r : 0);
    for (int k = 0; k < n; ++k) d.c.p[k] = gr.lora_a[g.id3[k]];
    d.ldc = in;
    QBLK_TRY(gemm(d, st));
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
  const Group gq({PQ, PK, PV}, {qd, kvd, kvd}), go({PO}, {h}), ggu({PG, PU}, {I, I}), gd({PD}, {h});
  proj.qkv = [&](const float* n1, float* qkv, hipStream_t s_) {
    if (f16p) return nf4_fwd16(P, w, 0, T, h, s.base.n1_16, gq, s.h_qkv, s.hs16_qkv, nullptr, qkv, s_);
    QBLK_TRY(lora_down(P, T, h, n1, {PQ, PK, PV}, s.h_qkv, s_));
    return nf4_fwd(P, T, h, n1, {PQ, PK, PV}, {qd, kvd, kvd}, s.h_qkv, nullptr, qkv, s_);
  };
  proj.o = [&](const float* o, const float* res, float* out, hipStream_t s_) {
    if (f16p) return nf4_fwd16(P, w, 1, T, qd, s.base.o16, go, s.h_o, s.hs16_o, res, out, s_);
    QBLK_TRY(lora_down(P, T, qd, o, {PO}, s.h_o, s_));
    return nf4_fwd(P, T, qd, o, {PO}, {h}, s.h_o, res, out, s_);
  };
  proj.gate_up = [&](const float* n2, float* gu, hipStream_t s_) {
    if (f16p) return nf4_fwd16(P, w, 2, T, h, s.base.n2_16, ggu, s.h_gu, s.hs16_gu, nullptr, gu, s_);
    QBLK_TRY(lora_down(P, T, h, n2, {PG, PU}, s.h_gu, s_));
    return nf4_fwd(P, T, h, n2, {PG, PU}, {I, I}, s.h_gu, nullptr, gu, s_);
  };
  proj.down = [&](const float* sv, const float* res, float* out, hipStream_t s_) {
    if (f16p) return nf4_fwd16(P, w, 3, T, I, s.base.s16, gd, s.h_d, s.hs16_d, res, out, s_);
    QBLK_TRY(lora_down(P, T, I, sv, {PD}, s.h_d, s_));
    return nf4_fwd(P, T, I, sv, {PD}, {h}, s.h_d, res, out, s_);
  };
  // on the fp16 path every product reads the fp16 copies of n1, n2 and s:
  // their fp32 forms are not written
  Saved sv = s.base;
  if (f16p) {
    sv.n1 = sv.n2 = sv.s = nullptr;
    const Group gs[4] = {gq, go, ggu, gd};
    const int ins[4] = {h, qd, h, I};
    const int rc = lora_pack16_groups(P, gs, ins, 0, w.a16x, 1, w.bx16, st);
    if (rc) {
      t_ws = nullptr;
      return rc;
    }
  }
  const int rc = block_forward_impl(c, proj, P.g_in, P.g_post, P.g_q, P.g_k, x, y, sv, w.base.attn, st);
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
  const Group gq({PQ, PK, PV}, {qd, kvd, kvd}), go({PO}, {h}), ggu({PG, PU}, {I, I}), gd({PD}, {h});
  // fp16 path: each output gradient's fp16 copy comes from its producer
  // (into a16) and the hooks get a null fp32 pointer, as in the dense block
  f16* const dy16 = w.base.a16;
  // the upstream gradient of the block (and any output gradient that came
  // as fp32) is cast once into the fp16 slot
  auto as16 = [&](const float* g, int n, hipStream_t s_) -> int {
    return g ? cast_f16(T, n, g, n, dy16, n, nullptr, 0, s_) : QBLK_OK;
  };
  proj.down = [&](const float* dyv, const float* sv, float* ds, hipStream_t s_) {
    if (f16p) {
      QBLK_TRY(as16(dyv, h, s_));
      return nf4_bwd16(P, G, w, 3, T, I, dy16, s.base.s16, s.hs16_d, gd, w.dh_d, ds, nullptr, s_);
    }
    return nf4_bwd(P, G, T, I, dyv, sv, s.h_d, {PD}, {h}, w.dh_d, ds, s_);
  };
  proj.gate_up = [&](const float* dgu, const float* n2, float* dn2, hipStream_t s_) {
    if (f16p) {
      QBLK_TRY(as16(dgu, 2 * I, s_));
      return nf4_bwd16(P, G, w, 2, T, h, dy16, s.base.n2_16, s.hs16_gu, ggu, w.dh_gu, dn2, nullptr, s_);
    }
    return nf4_bwd(P, G, T, h, dgu, n2, s.h_gu, {PG, PU}, {I, I}, w.dh_gu, dn2, s_);
  };
  proj.o = [&](const float* dr1, const float* o, float* d_o, hipStream_t s_) {
    // the attention backward reads dO's fp16 copy
    if (f16p) {
      QBLK_TRY(as16(dr1, h, s_));
      return nf4_bwd16(P, G, w, 1, T, qd, dy16, s.base.o16, s.hs16_o, go, w.dh_o, d_o,
                       s.base.q16 ? w.base.do16 : nullptr, s_);
    }
    return nf4_bwd(P, G, T, qd, dr1, o, s.h_o, {PO}, {h}, w.dh_o, d_o, s_);
  };
  proj.qkv = [&](const float* dqkv, const float* n1, float* dn1, hipStream_t s_) {
    if (f16p) {
      QBLK_TRY(as16(dqkv, qd + 2 * kvd, s_));
      return nf4_bwd16(P, G, w, 0, T, h, dy16, s.base.n1_16, s.hs16_qkv, gq, w.dh_qkv, dn1, nullptr, s_);
    }
    return nf4_bwd(P, G, T, h, dqkv, n1, s.h_qkv, {PQ, PK, PV}, {qd, kvd, kvd}, w.dh_qkv, dn1, s_);
  };
  Scratch wb16 = w.base;
  wb16.prod16 = f16p;
  if (f16p) {
    const Group gs[4] = {gq, go, ggu, gd};
    const int ins[4] = {h, qd, h, I};
    const int rc = lora_pack16_groups(P, gs, ins, 2, w.bt16, 0, w.a16x, st);
    if (rc) {
      t_ws = nullptr;
      return rc;
    }
  }
  const int rc = block_backward_impl(c, proj, P.g_in, P.g_post, P.g_q, P.g_k, x, dy, s.base, dx, w.sink_h,
                                     w.sink_h + h, w.sink_d, w.sink_d + c.head_dim, wb16, st);
  t_ws = nullptr;
  return rc;
}
