// GQA causal softmax attention, forward and backward, on MFMA (gfx950).
//
// cuda_block.rs page: compute_attention_cuda (QK^T, 1/sqrt(d), causal mask
// keeping key j <= query i, row softmax, times V; query head h reads KV head
// h / (heads/kv_heads)) and backward_attention (softmax backward, the
// matmul backward and the GQA reduction of dK and dV over the query heads of
// a group). Here the [heads, seq, seq] score matrix is never stored: the
// forward keeps a running max and sum per query (log-sum-exp saved for the
// backward), and the backward recomputes the probabilities tile by tile.
//
// Orientation. Tiles are 32 queries x 32 keys. The forward computes
// S^T = K Q^T so that in each 32 x 32 accumulator a lane owns ONE query
// (column l % 32) and 16 keys (rows 8g + 4(l/32) + r): the running max, the
// sum and the rescale of the output are per-lane scalars, and P^T, still in
// the accumulator, is directly the B operand of O^T += V^T P^T (the key
// order of that product is chosen to match the accumulator rows; V is staged
// transposed in LDS so the matching A operand is two short LDS reads).
// The dQ kernel uses the same orientation; the dK/dV kernel swaps it
// (S = Q K^T, a lane owns one key) so that dV^T += dO^T P and dK^T += Q^T dS
// take the accumulator directly.
//
// Operands are rounded to fp16 while staged (Prec::F16, v_mfma_f32_32x32x16_f16)
// or kept fp32 (Prec::F32, v_mfma_f32_32x32x2_f32); softmax math is fp32.
// Head dims below 32 are zero-padded to 32.
#include "attention.h"

#include "../../include/qblk.h"

#include <type_traits>

namespace qblk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <Prec P, int DP>
struct AT;

template <int DP>
struct AT<Prec::F16, DP> {
  using T = f16;
  using Chunk = half8;
  static constexpr int NC = DP / 16;  // contraction chunks over head_dim
  static constexpr int PR = DP + 8;   // pitch of [32][DP] tiles
  static constexpr int PT = 32 + 8;   // pitch of [DP][32] tiles
  // Chunk c of a row: elements [16c + 8kh, 16c + 8kh + 8).
  static __device__ __forceinline__ Chunk lds_chunk(const T* row, int c, int kh) {
    return *(const half8*)(row + 16 * c + 8 * kh);
  }
  static __device__ __forceinline__ Chunk glb_chunk(const float* row, int c, int kh, int D) {
    Chunk r;
    const int d0 = 16 * c + 8 * kh;
    if (d0 < D) {
      const float4 a = *(const float4*)(row + d0), b = *(const float4*)(row + d0 + 4);
      r[0] = (f16)a.x; r[1] = (f16)a.y; r[2] = (f16)a.z; r[3] = (f16)a.w;
      r[4] = (f16)b.x; r[5] = (f16)b.y; r[6] = (f16)b.z; r[7] = (f16)b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = (f16)0.f;
    }
    return r;
  }
  static __device__ __forceinline__ floatx16 mma(Chunk a, Chunk b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  // out[db] += Xt^T-block times the 32x32 accumulator p (keys/queries in
  // accumulator row order). Xt is [DP][PT] with the contraction index
  // contiguous.
  static __device__ __forceinline__ void acc_product(const T* Xt, const floatx16& p, int lane,
                                                     floatx16 (&out)[DP / 32]) {
    const int i = lane & 31, kh = lane >> 5;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      half8 b;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = (f16)p[8 * s + j];
#pragma unroll
      for (int db = 0; db < DP / 32; ++db) {
        const T* row = Xt + (db * 32 + i) * PT;
        const half4 lo = *(const half4*)(row + 16 * s + 4 * kh);
        const half4 hi = *(const half4*)(row + 16 * s + 8 + 4 * kh);
        half8 a;
        a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
        a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
        out[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, out[db], 0, 0, 0);
      }
    }
  }
};

template <int DP>
struct AT<Prec::F32, DP> {
  using T = float;
  using Chunk = float4;
  static constexpr int NC = DP / 8;  // chunk c: elements [8c + 4kh, 8c + 4kh + 4)
  static constexpr int PR = DP + 4;
  static constexpr int PT = 32 + 4;
  static __device__ __forceinline__ Chunk lds_chunk(const T* row, int c, int kh) {
    return *(const float4*)(row + 8 * c + 4 * kh);
  }
  static __device__ __forceinline__ Chunk glb_chunk(const float* row, int c, int kh, int D) {
    const int d0 = 8 * c + 4 * kh;
    return d0 < D ? *(const float4*)(row + d0) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  static __device__ __forceinline__ floatx16 mma(Chunk a, Chunk b, floatx16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ void acc_product(const T* Xt, const floatx16& p, int lane,
                                                     floatx16 (&out)[DP / 32]) {
    const int i = lane & 31, kh = lane >> 5;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int db = 0; db < DP / 32; ++db) {
        const float4 a = *(const float4*)(Xt + (db * 32 + i) * PT + 8 * g + 4 * kh);
        out[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, p[4 * g + 0], out[db], 0, 0, 0);
        out[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, p[4 * g + 1], out[db], 0, 0, 0);
        out[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, p[4 * g + 2], out[db], 0, 0, 0);
        out[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, p[4 * g + 3], out[db], 0, 0, 0);
      }
    }
  }
};

template <typename T>
__device__ __forceinline__ void put4(T* p, float4 v);
template <>
__device__ __forceinline__ void put4<float>(float* p, float4 v) {
  *(float4*)p = v;
}
template <>
__device__ __forceinline__ void put4<f16>(f16* p, float4 v) {
  *(half4*)p = to_half4(v);
}

// 32 rows x DP columns (columns >= D and rows >= nvalid are zero) into
// [32][PR]; optionally also transposed into [DP][PT].
// Each thread takes 4 x 4 micro-blocks (4 rows, 4 columns): four 16-byte
// global loads, four row writes, and — for the transposed copy — the 4 x 4
// transpose in registers written as four 4-element column writes.
template <typename T, int DP, int PR, int PT, bool ROWS, bool TRANS>
__device__ __forceinline__ void stage_tile(T* s, T* st, const float* g, int64_t ld, int nvalid,
                                           int D, int tid, int nthr) {
  constexpr int C4 = DP / 4;
  for (int c = tid; c < 8 * C4; c += nthr) {
    const int r0 = (c / C4) * 4, d4 = (c % C4) * 4;
    float4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r0 + j < nvalid && d4 < D) v[j] = *(const float4*)(g + (int64_t)(r0 + j) * ld + d4);
    }
    if (ROWS) {
#pragma unroll
      for (int j = 0; j < 4; ++j) put4<T>(s + (r0 + j) * PR + d4, v[j]);
    }
    if (TRANS) {
      put4<T>(st + (d4 + 0) * PT + r0, make_float4(v[0].x, v[1].x, v[2].x, v[3].x));
      put4<T>(st + (d4 + 1) * PT + r0, make_float4(v[0].y, v[1].y, v[2].y, v[3].y));
      put4<T>(st + (d4 + 2) * PT + r0, make_float4(v[0].z, v[1].z, v[2].z, v[3].z));
      put4<T>(st + (d4 + 3) * PT + r0, make_float4(v[0].w, v[1].w, v[2].w, v[3].w));
    }
  }
}

__device__ __forceinline__ float half_max(float v) { return cross_half_max(v); }
__device__ __forceinline__ float half_sum(float v) { return cross_half_sum(v); }

// ------------------------------------------------------------ forward
// grid (q tiles, kv groups, batch); one wave per query head of the group.
template <Prec P, int DP>
__global__ __launch_bounds__(512) void attn_fwd_kernel(const AttnArgs a) {
  using A = AT<P, DP>;
  using T = typename A::T;
  __shared__ __attribute__((aligned(16))) T sK[32 * A::PR];
  __shared__ __attribute__((aligned(16))) T sVt[DP * A::PT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nthr = blockDim.x;
  const int G = a.heads / a.kv_heads, grp = blockIdx.y, b = blockIdx.z;
  const int h = grp * G + w;
  const int D = a.head_dim, S = a.seq;
  const int qt = blockIdx.x, q0 = qt * 32;
  const int64_t tok0 = (int64_t)b * S;
  const int i = lane & 31, kh = lane >> 5;
  const float sc = kLog2e / sqrtf((float)D);

  typename A::Chunk qc[A::NC];
  {
    const int qi = min(q0 + i, S - 1);
    const float* row = a.q + (tok0 + qi) * a.ldq + (int64_t)h * D;
#pragma unroll
    for (int c = 0; c < A::NC; ++c) qc[c] = A::glb_chunk(row, c, kh, D);
  }
  floatx16 o[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int qi = q0 + i;

  for (int kt = 0; kt <= qt; ++kt) {
    const int kv0 = kt * 32;
    __syncthreads();
    stage_tile<T, DP, A::PR, A::PT, true, false>(sK, nullptr, a.k + (tok0 + kv0) * a.ldk + (int64_t)grp * D,
                                                 a.ldk, min(32, S - kv0), D, tid, nthr);
    stage_tile<T, DP, A::PR, A::PT, false, true>(nullptr, sVt, a.v + (tok0 + kv0) * a.ldv + (int64_t)grp * D,
                                                 a.ldv, min(32, S - kv0), D, tid, nthr);
    __syncthreads();
    floatx16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int c = 0; c < A::NC; ++c) s = A::mma(A::lds_chunk(sK + i * A::PR, c, kh), qc[c], s);
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kj = kv0 + 8 * g + 4 * kh + r;
        float v = s[4 * g + r] * sc;
        if (kj > qi || kj >= S) v = -INFINITY;
        s[4 * g + r] = v;
        mx = fmaxf(mx, v);
      }
    mx = half_max(mx);
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = exp2f(s[e] - mn);
      s[e] = p;
      ps += p;
    }
    l = l * alpha + half_sum(ps);
    m = mn;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    A::acc_product(sVt, s, lane, o);
  }
  if (qi < S) {
    const float inv = 1.0f / l;
    float* orow = a.o + (tok0 + qi) * a.ldo + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = db * 32 + 8 * g + 4 * kh + r;
          if (d < D) orow[d] = o[db][4 * g + r] * inv;
        }
    if (kh == 0) a.lse[((int64_t)b * a.heads + h) * S + qi] = (m + log2f(l)) * kLn2;
  }
}

// ---------------------------------------------------------- backward
// delta[b, h, s] = sum_d dO * O  (the softmax-backward row term).
__global__ __launch_bounds__(256) void attn_delta_kernel(const AttnArgs a, float* delta) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t T = (int64_t)a.batch * a.seq;
  if (item >= T * a.heads) return;
  const int64_t t = item / a.heads;
  const int h = (int)(item % a.heads);
  const int D = a.head_dim;
  const float* o = a.o + t * a.ldo + (int64_t)h * D;
  const float* d = a.d_o + t * a.lddo + (int64_t)h * D;
  float s = 0.f;
  for (int j = lane; j < D; j += 64) s += o[j] * d[j];
  s = wave_sum(s);
  if (lane == 0) {
    const int b = (int)(t / a.seq), sq = (int)(t % a.seq);
    delta[((int64_t)b * a.heads + h) * a.seq + sq] = s;
  }
}

// dQ: grid (q tiles, kv groups, batch); one wave per query head.
template <Prec P, int DP>
__global__ __launch_bounds__(512) void attn_dq_kernel(const AttnArgs a, const float* delta) {
  using A = AT<P, DP>;
  using T = typename A::T;
  __shared__ __attribute__((aligned(16))) T sK[32 * A::PR];
  __shared__ __attribute__((aligned(16))) T sV[32 * A::PR];
  __shared__ __attribute__((aligned(16))) T sKt[DP * A::PT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nthr = blockDim.x;
  const int G = a.heads / a.kv_heads, grp = blockIdx.y, b = blockIdx.z;
  const int h = grp * G + w;
  const int D = a.head_dim, S = a.seq;
  const int qt = blockIdx.x, q0 = qt * 32;
  const int64_t tok0 = (int64_t)b * S;
  const int i = lane & 31, kh = lane >> 5;
  const float sc = kLog2e / sqrtf((float)D);
  const int qi = q0 + i, qc_i = min(qi, S - 1);

  typename A::Chunk qc[A::NC], dc[A::NC];
  {
    const float* qrow = a.q + (tok0 + qc_i) * a.ldq + (int64_t)h * D;
    const float* drow = a.d_o + (tok0 + qc_i) * a.lddo + (int64_t)h * D;
#pragma unroll
    for (int c = 0; c < A::NC; ++c) {
      qc[c] = A::glb_chunk(qrow, c, kh, D);
      dc[c] = A::glb_chunk(drow, c, kh, D);
    }
  }
  const int64_t rowi = ((int64_t)b * a.heads + h) * S + qc_i;
  const float lse2 = a.lse[rowi] * kLog2e;
  const float dl = delta[rowi];
  floatx16 dq[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;

  for (int kt = 0; kt <= qt; ++kt) {
    const int kv0 = kt * 32, nv = min(32, S - kv0);
    __syncthreads();
    stage_tile<T, DP, A::PR, A::PT, true, true>(sK, sKt, a.k + (tok0 + kv0) * a.ldk + (int64_t)grp * D,
                                                a.ldk, nv, D, tid, nthr);
    stage_tile<T, DP, A::PR, A::PT, true, false>(sV, nullptr, a.v + (tok0 + kv0) * a.ldv + (int64_t)grp * D,
                                                 a.ldv, nv, D, tid, nthr);
    __syncthreads();
    floatx16 s, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s[e] = 0.f;
      dp[e] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < A::NC; ++c) {
      s = A::mma(A::lds_chunk(sK + i * A::PR, c, kh), qc[c], s);
      dp = A::mma(A::lds_chunk(sV + i * A::PR, c, kh), dc[c], dp);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * g + r;
        const int kj = kv0 + 8 * g + 4 * kh + r;
        const float p = (kj > qi || kj >= S) ? 0.f : exp2f(s[e] * sc - lse2);
        s[e] = p * (dp[e] - dl);  // dS^T, unscaled
      }
    A::acc_product(sKt, s, lane, dq);
  }
  if (qi < S) {
    const float inv = 1.0f / sqrtf((float)D);
    float* row = a.dq + (tok0 + qi) * a.lddq + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = db * 32 + 8 * g + 4 * kh + r;
          if (d < D) row[d] = dq[db][4 * g + r] * inv;
        }
  }
}

// dK, dV per query head: grid (kv tiles, heads, batch); one wave. Results
// go to per-head partial buffers [T, heads, D], summed over each group by
// attn_gqa_reduce_kernel in a fixed order.
template <Prec P, int DP>
__global__ __launch_bounds__(64) void attn_dkv_kernel(const AttnArgs a, const float* delta,
                                                      float* dk_part, float* dv_part) {
  using A = AT<P, DP>;
  using T = typename A::T;
  __shared__ __attribute__((aligned(16))) T sQ[32 * A::PR];
  __shared__ __attribute__((aligned(16))) T sQt[DP * A::PT];
  __shared__ __attribute__((aligned(16))) T sO[32 * A::PR];   // dO rows
  __shared__ __attribute__((aligned(16))) T sOt[DP * A::PT];  // dO transposed
  __shared__ float sL[32], sDl[32];
  const int lane = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.heads / a.kv_heads, grp = h / G;
  const int D = a.head_dim, S = a.seq;
  const int kt = blockIdx.x, kv0 = kt * 32;
  const int64_t tok0 = (int64_t)b * S;
  const int i = lane & 31, kh = lane >> 5;
  const float sc = kLog2e / sqrtf((float)D);
  const int kj = kv0 + i;  // this lane's key (column of every accumulator)

  typename A::Chunk kc[A::NC], vc[A::NC];
  {
    const int kr = min(kj, S - 1);
    const float* krow = a.k + (tok0 + kr) * a.ldk + (int64_t)grp * D;
    const float* vrow = a.v + (tok0 + kr) * a.ldv + (int64_t)grp * D;
#pragma unroll
    for (int c = 0; c < A::NC; ++c) {
      kc[c] = A::glb_chunk(krow, c, kh, D);
      vc[c] = A::glb_chunk(vrow, c, kh, D);
    }
  }
  floatx16 dk[DP / 32], dv[DP / 32];
#pragma unroll
  for (int db = 0; db < DP / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[db][e] = 0.f;
      dv[db][e] = 0.f;
    }
  const int nqt = (S + 31) / 32;
  for (int qt = kt; qt < nqt; ++qt) {
    const int q0 = qt * 32, nv = min(32, S - q0);
    __syncthreads();
    stage_tile<T, DP, A::PR, A::PT, true, true>(sQ, sQt, a.q + (tok0 + q0) * a.ldq + (int64_t)h * D, a.ldq,
                                                nv, D, lane, 64);
    stage_tile<T, DP, A::PR, A::PT, true, true>(sO, sOt, a.d_o + (tok0 + q0) * a.lddo + (int64_t)h * D,
                                                a.lddo, nv, D, lane, 64);
    if (lane < 32) {
      const int64_t ri = ((int64_t)b * a.heads + h) * S + min(q0 + lane, S - 1);
      sL[lane] = a.lse[ri] * kLog2e;
      sDl[lane] = delta[ri];
    }
    __syncthreads();
    floatx16 s, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s[e] = 0.f;
      dp[e] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < A::NC; ++c) {
      s = A::mma(A::lds_chunk(sQ + i * A::PR, c, kh), kc[c], s);
      dp = A::mma(A::lds_chunk(sO + i * A::PR, c, kh), vc[c], dp);
    }
    // accumulator rows are queries q0 + 8g + 4kh + r, column is key kj
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * g + r, ql = 8 * g + 4 * kh + r;
        const int qq = q0 + ql;
        const float p = (kj > qq || qq >= S || kj >= S) ? 0.f : exp2f(s[e] * sc - sL[ql]);
        s[e] = p;
        dp[e] = p * (dp[e] - sDl[ql]);
      }
    A::acc_product(sOt, s, lane, dv);   // dV^T += dO^T P
    A::acc_product(sQt, dp, lane, dk);  // dK^T += Q^T dS
  }
  if (kj < S) {
    const float inv = 1.0f / sqrtf((float)D);
    float* krow = dk_part + ((tok0 + kj) * a.heads + h) * (int64_t)D;
    float* vrow = dv_part + ((tok0 + kj) * a.heads + h) * (int64_t)D;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = db * 32 + 8 * g + 4 * kh + r;
          if (d < D) {
            krow[d] = dk[db][4 * g + r] * inv;
            vrow[d] = dv[db][4 * g + r];
          }
        }
  }
}

// Index space: T kv_heads D sums of dK and dV over the group's heads and
// the Z key-range splits (split-major, then head, in that fixed order);
// with Z > 1 also T heads D sums of dQ over its Z splits (dq_part [Z, T,
// heads, D]) written to dq.
__global__ void attn_gqa_reduce_kernel(int64_t T, int heads, int kv_heads, int D, int bf16,
                                       const float* dk_part, const float* dv_part, float* dk,
                                       int64_t lddk, float* dv, int64_t lddv, f16* dv16, int64_t lddv16, int Z,
                                       const float* dq_part, float* dq, int64_t lddq) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t n = T * kv_heads * D;
  const int64_t part = T * heads * D;  // elements of one split's partial buffer
  if (idx >= n) {
    const int64_t e = idx - n;
    if (Z <= 1 || e >= part) return;
    const int64_t t = e / ((int64_t)heads * D);
    const int c = (int)(e % ((int64_t)heads * D));
    float s = 0.f;
    for (int z = 0; z < Z; ++z) s += dq_part[z * part + e];
    dq[t * lddq + c] = s;
    return;
  }
  const int64_t t = idx / ((int64_t)kv_heads * D);
  const int rem = (int)(idx % ((int64_t)kv_heads * D));
  const int g = rem / D, j = rem % D;
  const int G = heads / kv_heads;
  float sk = 0.f, sv = 0.f;
  for (int z = 0; z < Z; ++z)
    for (int w = 0; w < G; ++w) {
      const int64_t o = z * part + (t * heads + g * G + w) * (int64_t)D + j;
      sk += dk_part[o];
      sv += dv_part[o];
    }
  dk[t * lddk + g * D + j] = sk;
  dv[t * lddv + g * D + j] = sv;
  if (dv16) dv16[t * lddv16 + g * D + j] = to_16(sv, bf16);
}

template <Prec P, int DP>
int fwd_launch(const AttnArgs& a, hipStream_t st) {
  const int G = a.heads / a.kv_heads;
  dim3 grid((unsigned)ceil_div(a.seq, 32), (unsigned)a.kv_heads, (unsigned)a.batch);
  hipLaunchKernelGGL((attn_fwd_kernel<P, DP>), grid, dim3(64 * G), 0, st, a);
  return check_launch("attn_fwd_kernel");
}

template <Prec P, int DP>
int bwd_launch(const AttnArgs& a, float* delta, float* dk_part, float* dv_part, hipStream_t st) {
  const int G = a.heads / a.kv_heads;
  const int64_t T = (int64_t)a.batch * a.seq;
  hipLaunchKernelGGL(attn_delta_kernel, dim3((unsigned)ceil_div(T * a.heads, 4)), dim3(256), 0, st, a,
                     delta);
  QBLK_TRY(check_launch("attn_delta_kernel"));
  dim3 gq((unsigned)ceil_div(a.seq, 32), (unsigned)a.kv_heads, (unsigned)a.batch);
  hipLaunchKernelGGL((attn_dq_kernel<P, DP>), gq, dim3(64 * G), 0, st, a, (const float*)delta);
  QBLK_TRY(check_launch("attn_dq_kernel"));
  dim3 gk((unsigned)ceil_div(a.seq, 32), (unsigned)a.heads, (unsigned)a.batch);
  hipLaunchKernelGGL((attn_dkv_kernel<P, DP>), gk, dim3(64), 0, st, a, (const float*)delta, dk_part,
                     dv_part);
  QBLK_TRY(check_launch("attn_dkv_kernel"));
  const int64_t n = T * a.kv_heads * a.head_dim;
  hipLaunchKernelGGL(attn_gqa_reduce_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, T,
                     a.heads, a.kv_heads, a.head_dim, 0, (const float*)dk_part, (const float*)dv_part, a.dk,
                     a.lddk, a.dv, a.lddv, (f16*)nullptr, (int64_t)0, 1, (const float*)nullptr, (float*)nullptr,
                     (int64_t)0);
  return check_launch("attn_gqa_reduce_kernel");
}

// ====================================================================
// Direct global -> LDS tiles (head_dim 64 / 128; fp16 or fp32 elements)
//
// Same orientations as above; what changes is how tiles reach LDS and how
// P (or dS) becomes an MFMA operand. Every tile is a plain copy of a 32-row
// slab of a matrix: row tiles [32][D] from the row-major inputs and
// transposed tiles [D][32] from transposed copies, so no thread converts or
// transposes anything and the copies run as global_load_lds_dwordx4 (1 KB
// per wave instruction) into two LDS stages.
//
// A lane reads the 16-byte logical chunk 2c + (lane / 32) of its row for
// contraction step c, both for LDS tiles and for the operands it keeps in
// registers, so A and B agree on which K each MFMA lane carries:
// * fp16 (v_mfma_f32_32x32x16_f16): one chunk = 8 halves = one MFMA;
// * fp32 (v_mfma_f32_32x32x2f32): one chunk = 4 floats = four MFMAs.
// For the products contracting over the 32 keys (or queries) held in an
// accumulator (rows 8g + 4(lane/32) + r): in fp32 the accumulator value
// 4g + r is directly the B operand of the MFMA pairing key 8g + r (lanes
// 0-31) with key 8g + 4 + r (lanes 32-63), and the A operand is the float4
// at chunk 2g + kh of the transposed tile. In fp16 the lane halves trade
// four packed values with v_permlane32_swap so that each lane holds 8
// consecutive keys, the natural order of the transposed tile.

template <typename T>
struct AttnElem;
template <>
struct AttnElem<f16> {
  using Chunk = half8;
  static constexpr int EPC = 8;  // elements per 16-byte chunk
  static __device__ __forceinline__ floatx16 mma(Chunk a, Chunk b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct AttnElem<bf16> {  // bfloat16 bit patterns in the same 16-byte chunks
  using Chunk = half8;
  static constexpr int EPC = 8;
  static __device__ __forceinline__ floatx16 mma(Chunk a, Chunk b, floatx16 c) { return mfma16<true>(a, b, c); }
};
template <>
struct AttnElem<float> {
  using Chunk = float4;
  static constexpr int EPC = 4;
  static __device__ __forceinline__ floatx16 mma(Chunk a, Chunk b, floatx16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, c, 0, 0, 0);
    return c;
  }
};

// Row tile: 32 rows x D elements, rows unpadded, 16-byte chunks permuted
// within each row by an XOR with a function of the row. The function is
// chosen so that (a) 16 consecutive rows read at one logical chunk hit 16
// distinct 16-byte bank groups of the 256-byte LDS cycle, and (b) the
// transposed fp16 reads, which take 4 consecutive rows x 4 consecutive
// chunks per half-wave, hit 16 distinct groups as well:
// * 256-byte rows (16 chunks): row bits 0-1 -> chunk bits 2-3, row bits
//   2-3 -> chunk bits 0-1;
// * 128-byte rows (8 chunks, two rows per bank cycle): row bit 1 -> chunk
//   bit 2, row bits 2-3 -> chunk bits 0-1.
template <typename T, int D>
struct RowTile {
  static constexpr int NCH = D * (int)sizeof(T) / 16;  // chunks per row
  static_assert(NCH == 8 || NCH == 16, "row tile width");
  static constexpr int RPI = 64 / NCH;  // rows per 1 KB wave copy
  static constexpr int NI = 32 / RPI;   // wave copies per tile
  static constexpr int STEPS = NCH / 2; // contraction steps over D
  static constexpr int ELEMS = 32 * D;
  static __device__ __forceinline__ int sw(int row) {
    return NCH == 16 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  }
};

template <typename C>
__device__ __forceinline__ C lds_at(const void* base, uint32_t off) {
  return *(const C*)((const char*)base + off);
}

// Per-lane byte offsets, inside one stage, of the row reads of a row tile:
// contraction step c reads the chunk 2c + kh of row i of the wave's slot.
template <typename T, int D>
struct RowReads {
  using RT = RowTile<T, D>;
  uint32_t v[RT::STEPS];
  __device__ __forceinline__ RowReads(int i, int kh, int slot) {
#pragma unroll
    for (int c = 0; c < RT::STEPS; ++c)
      v[c] = (uint32_t)((slot + i * D + (((2 * c + kh) ^ RT::sw(i)) * AttnElem<T>::EPC)) * (int)sizeof(T));
  }
};

// Per-lane byte offsets of the fp16 transposed reads (ds_read_b64_tr_b16)
// of a row tile X [32][D]: fragment (db, s2) holds, for head_dim column
// db*32 + (lane % 32), the 8 keys 16 s2 + 8 kh .. +7 as two reads rr = 0, 1.
// Within each 16-lane group, output lane j takes element k from source lane
// 4k + j/4, so source lane s reads columns 4(s % 4) .. +3 of row s / 4 + base
// and lane j ends up with 4 consecutive rows of column j. s2 adds 16 rows,
// which leaves the swizzle unchanged.
template <int D>
struct TrReads {
  using RT = RowTile<f16, D>;
  uint32_t v[D / 32][2];
  __device__ __forceinline__ TrReads(int lane, int slot) {
    const int sl = lane & 15, q1 = (lane >> 4) & 1, kh = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = 8 * kh + 4 * rr + (sl >> 2);
        const int col = db * 32 + 16 * q1 + 4 * (sl & 3);
        v[db][rr] = (uint32_t)((slot + row * D + (((col >> 3) ^ RT::sw(row)) << 3) + (col & 7)) * 2);
      }
  }
  __device__ __forceinline__ half8 frag(const void* X, int db, int s2) const {
    typedef short short4v __attribute__((ext_vector_type(4)));
    half8 out;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const char* addr = (const char*)X + v[db][rr] + s2 * 16 * D * 2;
      const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)addr);
      const half4 h = __builtin_bit_cast(half4, r);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * rr + e] = h[e];
    }
    return out;
  }
};

// fp32 transposed reads straight out of a row tile X [32][D] (D = 64): the
// A operand of the r-th MFMA of group g (32x32x2) is X[key][d] with
// key = 8g + 4kh + r and d = 32 db + i, one float per lane. With the row
// tile's swizzle (16 chunks of 4 floats; row bits 0-1 -> chunk bits 2-3,
// row bits 2-3 -> chunk bits 0-1) that float sits in chunk
// ((db ^ (r >> 1)) << 3) | ((i >> 2) ^ kh ^ 4 (r & 1) ^ (2g & 3)) of row
// key. Holds the lane's parts of that address (slot: the wave's tile
// within the stage, in floats).
struct Rt32Reads {
  int lx, lb;  // (i >> 2) ^ kh; slot + 4 kh rows + the float within the chunk
  __device__ __forceinline__ Rt32Reads(int lane, int slot) {
    const int i = lane & 31, kh = lane >> 5;
    lx = (i >> 2) ^ kh;
    lb = slot + kh * 4 * 64 + (i & 3);
  }
};

// Source offsets (bytes) of the wave copies of a tile: copy j moves rows
// j*RPI .. j*RPI + RPI-1, one 16-byte chunk per lane into the lane's slot,
// fetched from the logical chunk that the swizzle stores there. Rows are
// ld elements apart in the source.
template <typename T, int NCH, int NI, typename Tile>
struct CopyOffsets {
  uint32_t v[NI];
  __device__ __forceinline__ CopyOffsets(int lane, int64_t ld) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = j * (64 / NCH) + lane / NCH;
      const int lc = (lane % NCH) ^ Tile::sw(row);
      v[j] = (uint32_t)((row * ld + lc * (16 / (int)sizeof(T))) * (int64_t)sizeof(T));
    }
  }
};
template <typename T, int D>
using RowCopy = CopyOffsets<T, RowTile<T, D>::NCH, RowTile<T, D>::NI, RowTile<T, D>>;

// Row tile: rows r0 .. r0+31 of a [T, *] matrix, columns col0 .. col0+D-1.
// Whole tiles use the precomputed offsets; a tile running past the end of
// the sequence clamps its rows to S-1 (those rows are masked).
template <typename T, int D>
__device__ __forceinline__ void copy_row_tile(T* tile, const T* base, int64_t ld, int64_t tok0, int r0, int S,
                                              int col0, const RowCopy<T, D>& off, int lane) {
  using RT = RowTile<T, D>;
  if (r0 + 32 <= S) {
    const char* slab = (const char*)(base + (tok0 + r0) * ld + col0);
#pragma unroll
    for (int j = 0; j < RT::NI; ++j) dma16_asm(slab + off.v[j], tile + j * (1024 / sizeof(T)));
  } else {
#pragma unroll
    for (int j = 0; j < RT::NI; ++j) {
      const int row = j * RT::RPI + lane / RT::NCH;
      const int lc = (lane % RT::NCH) ^ RT::sw(row);
      dma16_asm(base + (tok0 + min(r0 + row, S - 1)) * ld + col0 + lc * AttnElem<T>::EPC,
            tile + j * (1024 / sizeof(T)));
    }
  }
}

// Register operand: chunk 2c + kh of a row.
template <typename T, int D>
__device__ __forceinline__ void load_row_frags(const T* row, int kh, typename AttnElem<T>::Chunk (&f)[RowTile<T, D>::STEPS]) {
#pragma unroll
  for (int c = 0; c < RowTile<T, D>::STEPS; ++c)
    f[c] = *(const typename AttnElem<T>::Chunk*)(row + (2 * c + kh) * AttnElem<T>::EPC);
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));

template <bool BF>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  half2v h;
  h[0] = to_16(a, BF);
  h[1] = to_16(b, BF);
  return __builtin_bit_cast(unsigned, h);
}

// fp16: accumulator values 8 s2 .. 8 s2 + 7 as the B operand of a product
// contracting over rows 16 s2 .. 16 s2 + 15: after the swap, lane half kh
// holds rows 16 s2 + 8 kh + j, j = 0..7, in order.
template <bool BF>
__device__ __forceinline__ half8 acc_rows_operand(const floatx16& p, int s2) {
  unsigned r0a = pack2<BF>(p[8 * s2 + 0], p[8 * s2 + 1]), r0b = pack2<BF>(p[8 * s2 + 2], p[8 * s2 + 3]);
  unsigned r1a = pack2<BF>(p[8 * s2 + 4], p[8 * s2 + 5]), r1b = pack2<BF>(p[8 * s2 + 6], p[8 * s2 + 7]);
  const auto x = __builtin_amdgcn_permlane32_swap(r0a, r1a, false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(r0b, r1b, false, false);
  uint4v u;
  u[0] = x[0];
  u[1] = y[0];
  u[2] = x[1];
  u[3] = y[1];
  return __builtin_bit_cast(half8, u);
}

// fp16: out[db] += X^T-block times the 32 x 32 accumulator p, contracting
// over the accumulator's rows; X is a row tile [32][D] read transposed.
template <int D, bool BF>
__device__ __forceinline__ void acc_rows_product_tr(const void* X, const TrReads<D>& rd, const floatx16& p,
                                                    floatx16 (&out)[D / 32]) {
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const half8 bp = acc_rows_operand<BF>(p, s2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) out[db] = mfma16<BF>(rd.frag(X, db, s2), bp, out[db]);
  }
}

// fp32: the same product with X^T read out of the row tile X (Rt32Reads):
// group g's accumulator value 4g + r is the B operand pairing key 8g + r
// (lanes 0-31) with key 8g + 4 + r (lanes 32-63).
template <int D>
__device__ __forceinline__ void acc_rows_product_rt32(const float* X, const Rt32Reads& rd, const floatx16& p,
                                                      floatx16 (&out)[D / 32]) {
  static_assert(D == 64, "fp32 row tiles of 64 columns");
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lc = rd.lx ^ (((r & 1) << 2) ^ ((2 * g) & 3));
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const float a = X[(8 * g + r) * D + rd.lb + ((((db ^ (r >> 1)) << 3) | lc) << 2)];
        out[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[4 * g + r], out[db], 0, 0, 0);
      }
    }
}

// Transposed-operand reads of the kernels, out of the row tiles: fp16
// through the transposing LDS instruction, fp32 one float per lane.
template <typename T, int D>
using XtReads = std::conditional_t<sizeof(T) == 2, TrReads<D>, Rt32Reads>;

template <typename T, int D>
__device__ __forceinline__ XtReads<T, D> make_xt_reads(int lane, int slot_rows) {
  if constexpr (sizeof(T) == 2) return TrReads<D>(lane, slot_rows);
  else return Rt32Reads(lane, slot_rows);
}

template <typename T, int D>
__device__ __forceinline__ void acc_rows_product_any(const T* X, const XtReads<T, D>& rd, const floatx16& p,
                                                     floatx16 (&out)[D / 32]) {
  if constexpr (sizeof(T) == 2) acc_rows_product_tr<D, std::is_same_v<T, bf16>>(X, rd, p, out);
  else acc_rows_product_rt32<D>(X, rd, p, out);
}

using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;
template <int N>
using IC = std::integral_constant<int, N>;

// One LDS stage as its own __shared__ object (distinct objects: the
// compiler adds no waits between a copy into one and reads of another).
template <typename T, int TAG, int ELEMS>
__device__ __forceinline__ T* att_lds() {
  __shared__ __attribute__((aligned(16))) T buf[ELEMS];
  return buf;
}

// s_waitcnt vmcnt with a runtime bound, rounded down to a power of two
// (a smaller count only waits longer).
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if (n >= 32) wait_vmcnt<32>();
  else if (n >= 16) wait_vmcnt<16>();
  else if (n >= 8) wait_vmcnt<8>();
  else if (n >= 4) wait_vmcnt<4>();
  else if (n >= 2) wait_vmcnt<2>();
  else if (n >= 1) wait_vmcnt<1>();
  else wait_vmcnt<0>();
}

// Ring of NS LDS stages private to one wave over its n tiles: issue(t,
// IC<s>) starts the copies of tile t into stage s (per_tile vector-memory
// instructions), pre(t) runs before the refill of step t, body(t, IC<s>)
// consumes tile t from stage s. Step t waits for the wave's own copies of
// tile t (tiles t+1 .. t+NS-2 may stay in flight); no barrier is needed, as
// no other wave touches these stages, and the stage refilled at step t was
// last read in step t-1, whose reads have all returned. Whole rounds of NS
// steps run without branches around the bodies; the last n % NS follow.
template <int NS, typename Issue, typename Pre, typename Body>
__device__ __forceinline__ void wave_ring(int n, int per_tile, Issue&& issue, Pre&& pre, Body&& body) {
  static_assert(NS >= 2 && NS <= 4, "stages");
  if (0 < n) issue(0, IC<0>{});
  if constexpr (NS > 2) if (1 < n) issue(1, IC<1>{});
  if constexpr (NS > 3) if (2 < n) issue(2, IC<2>{});
  auto one = [&](auto S, int t) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value;
    pre(t);
    const int ahead = min(NS - 2, n - 1 - t);
    wait_vmcnt_le(ahead > 0 ? ahead * per_tile : 0);
    if (t + NS - 1 < n) issue(t + NS - 1, IC<(st + NS - 1) % NS>{});
    body(t, S);
  };
  const int nfull = n / NS * NS;
  for (int t = 0; t < nfull; t += NS) {
    one(IC<0>{}, t);
    one(IC<1>{}, t + 1);
    if constexpr (NS > 2) one(IC<2>{}, t + 2);
    if constexpr (NS > 3) one(IC<3>{}, t + 3);
  }
  const int left = n - nfull;
  if (left > 0) one(IC<0>{}, nfull);
  if constexpr (NS > 2) if (left > 1) one(IC<1>{}, nfull + 1);
  if constexpr (NS > 3) if (left > 2) one(IC<2>{}, nfull + 2);
}

// Waves per workgroup and LDS stages per wave of the three kernels: the W
// waves of a workgroup split one (tile, head) unit's key (or query) range
// between them, each with private stages, and combine at the end. Paired
// workgroups (PAIR) take causal tiles t and ntl-1-t one after the other
// with FWD_W, DQ_W or DKV_W waves; unpaired ones take one tile with
// UNPAIRED_W waves (half the stages: two workgroups per CU), see
// attention_unpaired.
template <typename T>
struct AttnSplit {
  static constexpr int FWD_W = 4, DQ_W = 4, DKV_W = 4, UNPAIRED_W = 2;
  static constexpr int FWD_NS = 2, DQ_NS = 2, DKV_NS = 2;
};

// Combine of the W waves' accumulator blocks (NB blocks of 16 floats per
// lane) in one exchange: block db belongs to wave db % W; every wave parks
// the blocks it does not own in LDS, and each owner adds the W values of its
// blocks in wave order (its own from registers), each times scale(ww). The
// slots are 4 KiB regions (16 x 64 floats, float4 per lane) laid over the
// kernel's four stage buffers, CAP per buffer; slot(db * W + ww) holds wave
// ww's block db. The caller puts a barrier between its last reads of those
// stages and park_blocks, and one between park_blocks and sum_owned.
template <int CAP>
__device__ __forceinline__ float* stage_slot(int i, void* b0, void* b1, void* b2, void* b3) {
  const int b = i / CAP;
  char* p = (char*)(b == 0 ? b0 : b == 1 ? b1 : b == 2 ? b2 : b3);
  return (float*)(p + (i % CAP) * 4096);
}
template <int W, int NB, class Slot>
__device__ __forceinline__ void park_blocks(const floatx16 (&v)[NB], int w, int lane, Slot&& slot) {
#pragma unroll
  for (int db = 0; db < NB; ++db)
    if (db % W != w) {
      float4* p = (float4*)slot(db * W + w);
#pragma unroll
      for (int g = 0; g < 4; ++g) p[g * 64 + lane] = make_float4(v[db][4 * g], v[db][4 * g + 1], v[db][4 * g + 2], v[db][4 * g + 3]);
    }
}
template <int W, int NB, bool SCALED, class Slot, class Scale>
__device__ __forceinline__ void sum_owned(floatx16 (&v)[NB], int w, int lane, Slot&& slot, Scale&& scale) {
#pragma unroll
  for (int db = 0; db < NB; ++db)
    if (db % W == w) {
      floatx16 acc;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        floatx16 x;
        if (ww == w) {
          x = v[db];
        } else {
          const float4* p = (const float4*)slot(db * W + ww);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 q = p[g * 64 + lane];
            x[4 * g] = q.x;
            x[4 * g + 1] = q.y;
            x[4 * g + 2] = q.z;
            x[4 * g + 3] = q.w;
          }
        }
        if constexpr (SCALED) {
          const float f = scale(ww);
#pragma unroll
          for (int e = 0; e < 16; ++e) x[e] *= f;
        }
        if (ww == 0) acc = x;
        else
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] += x[e];
      }
      v[db] = acc;
    }
}
struct NoScale {
  __device__ __forceinline__ float operator()(int) const { return 1.f; }
};

// 2^x on the hardware unit: no denormal rescaling; inputs are <= 0 except
// under the bounded stale maximum of the forward pass (<= kRescaleSlack).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// The forward pass keeps each row's reference maximum m stale until a tile
// raises the row maximum more than this many powers of two above it, so the
// output rescale runs on few tiles; probabilities relative to m stay below
// 2^kRescaleSlack, far inside fp16 range.
constexpr float kRescaleSlack = 8.f;

// Forward: grid (pairs of q tiles, heads, batch), the later tile first, or
// (q tiles, heads, batch) when not PAIR. The W
// waves take key tiles w, w+W, ...; each keeps its own reference max, sum
// and output; they are merged with a log-sum-exp combine and wave 0 writes
// o and lse. Only the diagonal tile needs the causal mask: every earlier
// key tile lies wholly below the diagonal and inside the sequence.
template <typename T, int D, int W, bool PAIR>
__global__ __launch_bounds__(W * 64) void attn_dma_fwd_kernel(const AttnDmaArgs a) {
  using RT = RowTile<T, D>;
  using E = AttnElem<T>;
  constexpr int NS = AttnSplit<T>::FWD_NS;
  // V is staged as a row tile and V^T read out of it
  constexpr int VE = RT::ELEMS, VNI = RT::NI;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto sK = [](auto S) { return att_lds<T, 2 * decltype(S)::value, W * RT::ELEMS>(); };
  auto sV = [](auto S) { return att_lds<T, 2 * decltype(S)::value + 1, W * VE>(); };
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const int G = a.heads / a.kv_heads, h = blockIdx.y, grp = h / G, b = blockIdx.z;
  const int S = a.seq;
  // Z workgroups share a tile pair, split z taking the key tiles
  // z W + w + t Z W; with Z > 1 each writes its partial output (relative to
  // its own maximum) with that maximum and sum, merged by
  // attn_fwd_combine_kernel
  const int Z = a.split, z = blockIdx.x % Z;
  // PAIR: tiles t and ntl-1-t share a workgroup (pass 0 the later tile):
  // every workgroup then has the same causal work, and half as many fit one
  // wave; otherwise workgroup pr takes tile pr
  const int ntl = (S + 31) / 32, pr = blockIdx.x / Z;
  const int npass = !PAIR || 2 * pr + 1 == ntl ? 1 : 2;
  for (int pass = 0; pass < npass; ++pass) {
    if (pass) __syncthreads();  // the previous tile's combine is done with the stages
    const int qt = !PAIR ? pr : pass == 0 ? ntl - 1 - pr : pr, q0 = qt * 32;
    const int64_t tok0 = (int64_t)b * S;
    const int i = lane & 31, kh = lane >> 5;
    const float sc = kLog2e / sqrtf((float)D);
    const int qi = q0 + i;

    const RowReads<T, D> rk(i, kh, w * RT::ELEMS);
    const XtReads<T, D> rv = make_xt_reads<T, D>(lane, w * VE);
    const RowCopy<T, D> ck(lane, a.ldk), cv(lane, a.ldv);

    typename E::Chunk qc[RT::STEPS];
    load_row_frags<T, D>(q + (tok0 + min(qi, S - 1)) * a.ldq + (int64_t)h * D, kh, qc);
    floatx16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
    float m = -INFINITY, l = 0.f;
    const int w0 = z * W + w, WZ = W * Z;
    const int n = w0 <= qt ? (qt - w0) / WZ + 1 : 0;  // key tiles w0, w0+WZ, .. <= qt

    auto issue = [&](int t, T* sk, T* sv) __attribute__((always_inline)) {
      const int kv0 = (w0 + WZ * t) * 32;
      copy_row_tile<T, D>(sk + w * RT::ELEMS, k, a.ldk, tok0, kv0, S, grp * D, ck, lane);
      copy_row_tile<T, D>(sv + w * VE, v, a.ldv, tok0, kv0, S, grp * D, cv, lane);
    };
    auto compute = [&](const T* sk, const T* sv, int t) __attribute__((always_inline)) {
      const int kv0 = (w0 + WZ * t) * 32;
      floatx16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int c = 0; c < RT::STEPS; ++c) s = E::mma(lds_at<typename E::Chunk>(sk, rk.v[c]), qc[c], s);
      if (kv0 == q0) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kv0 + 8 * g + 4 * kh + r > qi) s[4 * g + r] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
      mx = half_max(mx) * sc;
      if (__any(mx > m + kRescaleSlack)) {
        const float mn = fmaxf(m, mx);
        const float alpha = exp2_hw(m - mn);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
        m = mn;
      }
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2_hw(fmaf(s[e], sc, -m));
        s[e] = p;
        ps += p;
      }
      l += half_sum(ps);
      acc_rows_product_any<T, D>(sv, rv, s, o);
    };
    wave_ring<NS>(
        n, RT::NI + VNI, [&](int t, auto St) __attribute__((always_inline)) { issue(t, sK(St), sV(St)); },
        [](int) {}, [&](int t, auto St) __attribute__((always_inline)) { compute(sK(St), sV(St), t); });

    // Log-sum-exp combine in one exchange: every wave parks its reference
    // max and sum (slot NB W) and the output blocks it does not own; after
    // the barrier each wave derives the common max, every wave's rescale
    // factor and the total sum, adds its blocks in wave order and writes
    // them (wave 0 also the lse).
    constexpr int NB = D / 32, CAP = W * RT::ELEMS * (int)sizeof(T) / 4096;
    static_assert(VE == RT::ELEMS && NB * W + 1 <= 4 * CAP, "combine space");
    auto slot = [&](int i) __attribute__((always_inline)) {
      return stage_slot<CAP>(i, sK(I0{}), sV(I0{}), sK(I1{}), sV(I1{}));
    };
    float* ml = slot(NB * W);
    __syncthreads();
    ml[(2 * w) * 64 + lane] = m;
    ml[(2 * w + 1) * 64 + lane] = l;
    park_blocks<W, NB>(o, w, lane, slot);
    __syncthreads();
    float M = ml[lane];
#pragma unroll
    for (int ww = 1; ww < W; ++ww) M = fmaxf(M, ml[(2 * ww) * 64 + lane]);
    float fw[W], L = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const float mw = ml[(2 * ww) * 64 + lane];
      fw[ww] = mw == -INFINITY ? 0.f : exp2f(mw - M);
      const float lw = ml[(2 * ww + 1) * 64 + lane] * fw[ww];
      L = ww == 0 ? lw : L + lw;
    }
    sum_owned<W, NB, true>(o, w, lane, slot, [&](int ww) __attribute__((always_inline)) { return fw[ww]; });
    if (Z > 1) {
      // this split's output relative to its maximum M, and M, L
      if (qi < S) {
        const int64_t row = (z * (int64_t)a.batch * S + tok0 + qi) * a.heads + h;
        float* op = a.o_part + row * D + 4 * kh;
#pragma unroll
        for (int db = 0; db < NB; ++db)
          if (db % W == w) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *(float4*)(op + db * 32 + 8 * g) =
                  make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
          }
        if (w == 0 && kh == 0) *(float2*)(a.ml_part + 2 * row) = make_float2(M, L);
      }
      continue;
    }
    if (qi < S) {
      const float inv = 1.0f / L;
      const int64_t ooff = (tok0 + qi) * a.ldo + (int64_t)h * D + 4 * kh;
#pragma unroll
      for (int db = 0; db < NB; ++db)
        if (db % W == w) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 vv =
                make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
            *(float4*)(a.o + ooff + db * 32 + 8 * g) = vv;
            if (a.o16) *(half4*)(a.o16 + ooff + db * 32 + 8 * g) = to_16x4(vv, std::is_same_v<T, bf16>);
          }
        }
      if (w == 0 && kh == 0) a.lse[((int64_t)b * a.heads + h) * S + qi] = (M + log2f(L)) * kLn2;
    }
  }
}

// dQ: grid (pairs of q tiles, heads, batch), or (q tiles, heads, batch) when
// not PAIR; the W waves take key tiles w, w+W, ...
// (K and V through private LDS stages, K^T read out of the K row tile); the
// waves' partial dQ blocks are summed in wave order and written. Only the
// diagonal tile is masked.
template <typename T, int D, int W, bool PAIR>
__global__ __launch_bounds__(W * 64) void attn_dma_dq_kernel(const AttnDmaArgs a, float* delta) {
  using RT = RowTile<T, D>;
  using E = AttnElem<T>;
  constexpr int NS = AttnSplit<T>::DQ_NS;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto sK = [](auto S) { return att_lds<T, 3 * decltype(S)::value, W * RT::ELEMS>(); };
  auto sV = [](auto S) { return att_lds<T, 3 * decltype(S)::value + 1, W * RT::ELEMS>(); };
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const T* d_o = (const T*)a.d_o;
  const int G = a.heads / a.kv_heads, h = blockIdx.y, grp = h / G, b = blockIdx.z;
  const int S = a.seq;
  // Z workgroups share a tile pair, split z taking the key tiles
  // z W + w + t Z W (all W Z waves interleaved); with Z > 1 each writes its
  // partial dQ to dq_part[z], summed in split order afterwards
  const int Z = a.split, z = blockIdx.x % Z;
  // PAIR: tiles t and ntl-1-t share a workgroup (pass 0 the later tile):
  // every workgroup then has the same causal work, and half as many fit one
  // wave; otherwise workgroup pr takes tile pr
  const int ntl = (S + 31) / 32, pr = blockIdx.x / Z;
  const int npass = !PAIR || 2 * pr + 1 == ntl ? 1 : 2;
  for (int pass = 0; pass < npass; ++pass) {
    if (pass) __syncthreads();  // the previous tile's combine is done with the stages
    const int qt = !PAIR ? pr : pass == 0 ? ntl - 1 - pr : pr, q0 = qt * 32;
    const int64_t tok0 = (int64_t)b * S;
    const int i = lane & 31, kh = lane >> 5;
    const float sc = kLog2e / sqrtf((float)D);
    const int qi = q0 + i, qc_i = min(qi, S - 1);

    const RowReads<T, D> rr(i, kh, w * RT::ELEMS);
    const XtReads<T, D> rkt = make_xt_reads<T, D>(lane, w * RT::ELEMS);
    const RowCopy<T, D> ck(lane, a.ldk), cv(lane, a.ldv);

    typename E::Chunk qc[RT::STEPS], dc[RT::STEPS];
    load_row_frags<T, D>(q + (tok0 + qc_i) * a.ldq + (int64_t)h * D, kh, qc);
    load_row_frags<T, D>(d_o + (tok0 + qc_i) * a.lddo + (int64_t)h * D, kh, dc);
    const int64_t rowi = ((int64_t)b * a.heads + h) * S + qc_i;
    const float lse2 = a.lse[rowi] * kLog2e;
    // delta = rowsum(dO o) of the tile's rows (fp32 operands): wave w sums
    // columns w D/W .. (w+1) D/W - 1, the lane halves (kh) half of them each;
    // the waves' parts are added in wave order through the first K stage
    // before any copy lands there, and wave 0 stores delta for the dK/dV
    // kernel.
    float dl;
    {
      constexpr int CW = D / W / 2;  // columns per lane
      const int64_t c0 = (int64_t)h * D + w * (D / W) + kh * CW;
      const float* orow = a.o + (tok0 + qc_i) * a.ldo + c0;
      const float* drow = a.do32 + (tok0 + qc_i) * a.lddo32 + c0;
      float4 o4[CW / 4], d4[CW / 4];
#pragma unroll
      for (int j = 0; j < CW / 4; ++j) {
        o4[j] = *(const float4*)(orow + 4 * j);
        d4[j] = *(const float4*)(drow + 4 * j);
      }
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < CW / 4; ++j)
        part += o4[j].x * d4[j].x + o4[j].y * d4[j].y + o4[j].z * d4[j].z + o4[j].w * d4[j].w;
      part = cross_half_sum(part);
      float* x = (float*)att_lds<T, 0, W * RT::ELEMS>();
      x[w * 64 + lane] = part;
      __syncthreads();
      dl = x[lane];
#pragma unroll
      for (int ww = 1; ww < W; ++ww) dl += x[ww * 64 + lane];
      __syncthreads();  // the stage is refilled from here on
      if (z == 0 && w == 0 && kh == 0 && qi < S) delta[rowi] = dl;
    }
    floatx16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;
    const int w0 = z * W + w, WZ = W * Z;  // first key tile and stride of this wave
    const int n = w0 <= qt ? (qt - w0) / WZ + 1 : 0;

    auto issue = [&](int t, T* sk, T* sv) __attribute__((always_inline)) {
      const int kv0 = (w0 + WZ * t) * 32;
      copy_row_tile<T, D>(sk + w * RT::ELEMS, k, a.ldk, tok0, kv0, S, grp * D, ck, lane);
      copy_row_tile<T, D>(sv + w * RT::ELEMS, v, a.ldv, tok0, kv0, S, grp * D, cv, lane);
    };
    auto compute = [&](const T* sk, const T* sv, int t) __attribute__((always_inline)) {
      const int kv0 = (w0 + WZ * t) * 32;
      floatx16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = 0.f;
        dp[e] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < RT::STEPS; ++c) {
        s = E::mma(lds_at<typename E::Chunk>(sk, rr.v[c]), qc[c], s);
        dp = E::mma(lds_at<typename E::Chunk>(sv, rr.v[c]), dc[c], dp);
      }
      if (kv0 == q0) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * g + r;
            const int kj = kv0 + 8 * g + 4 * kh + r;
            const float p = (kj > qi || kj >= S) ? 0.f : exp2_hw(fmaf(s[e], sc, -lse2));
            s[e] = p * (dp[e] - dl);  // dS^T, unscaled
          }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = exp2_hw(fmaf(s[e], sc, -lse2)) * (dp[e] - dl);
      }
      acc_rows_product_any<T, D>(sk, rkt, s, dq);
    };
    wave_ring<NS>(
        n, 2 * RT::NI, [&](int t, auto St) __attribute__((always_inline)) { issue(t, sK(St), sV(St)); },
        [](int) {}, [&](int t, auto St) __attribute__((always_inline)) { compute(sK(St), sV(St), t); });

    // one exchange: each wave adds the blocks it owns in wave order and
    // writes them
    constexpr int NB = D / 32, CAP = W * RT::ELEMS * (int)sizeof(T) / 4096;
    static_assert(NB * W <= 4 * CAP, "combine space");
    auto slot = [&](int i) __attribute__((always_inline)) {
      return stage_slot<CAP>(i, sK(I0{}), sV(I0{}), sK(I1{}), sV(I1{}));
    };
    __syncthreads();
    park_blocks<W, NB>(dq, w, lane, slot);
    __syncthreads();
    sum_owned<W, NB, false>(dq, w, lane, slot, NoScale{});
    if (qi < S) {
      const float inv = 1.0f / sqrtf((float)D);
      float* row = Z == 1 ? a.dq + (tok0 + qi) * a.lddq + (int64_t)h * D + 4 * kh
                          : a.dq_part + ((z * (int64_t)a.batch * S + tok0 + qi) * a.heads + h) * D + 4 * kh;
#pragma unroll
      for (int db = 0; db < NB; ++db)
        if (db % W == w) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(float4*)(row + db * 32 + 8 * g) = make_float4(dq[db][4 * g] * inv, dq[db][4 * g + 1] * inv,
                                                            dq[db][4 * g + 2] * inv, dq[db][4 * g + 3] * inv);
        }
    }
  }
}

// dK, dV per query head: grid (pairs of kv tiles, heads, batch), or (kv
// tiles, heads, batch) when not PAIR; the W waves take
// query tiles kt+w, kt+w+W, ... (Q and dO through private LDS stages, Q^T
// and dO^T read out of those row tiles); the partials are summed in wave order into
// per-head buffers [T, heads, D], summed over each group afterwards. Masks
// apply only on the diagonal tile and on a query tile that runs past the
// end of the sequence.
template <typename T, int D, int W, bool PAIR>
__global__ __launch_bounds__(W * 64) void attn_dma_dkv_kernel(const AttnDmaArgs a, const float* delta,
                                                             float* dk_part, float* dv_part) {
  using RT = RowTile<T, D>;
  using E = AttnElem<T>;
  constexpr int NS = AttnSplit<T>::DKV_NS;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto sQ = [](auto S) { return att_lds<T, 4 * decltype(S)::value, W * RT::ELEMS>(); };
  auto sO = [](auto S) { return att_lds<T, 4 * decltype(S)::value + 1, W * RT::ELEMS>(); };
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const T* d_o = (const T*)a.d_o;
  const int h = blockIdx.y, b = blockIdx.z;
  const int G = a.heads / a.kv_heads, grp = h / G;
  const int S = a.seq;
  // Z workgroups share a tile pair, split z taking the query tiles
  // kt + z W + w + t Z W; each writes its partials to dk_part[z], dv_part[z]
  const int Z = a.split, z = blockIdx.x % Z;
  // PAIR: tiles t and ntl-1-t share a workgroup (pass 0 the later tile):
  // every workgroup then has the same causal work, and half as many fit one
  // wave; otherwise workgroup pr takes tile pr
  const int ntl = (S + 31) / 32, pr = blockIdx.x / Z;
  const int npass = !PAIR || 2 * pr + 1 == ntl ? 1 : 2;
  dk_part += z * (int64_t)a.batch * S * a.heads * D;
  dv_part += z * (int64_t)a.batch * S * a.heads * D;
  for (int pass = 0; pass < npass; ++pass) {
    if (pass) __syncthreads();  // the previous tile's combine is done with the stages
    const int kt = !PAIR ? pr : pass == 0 ? ntl - 1 - pr : pr, kv0 = kt * 32;
    const int64_t tok0 = (int64_t)b * S;
    const int i = lane & 31, kh = lane >> 5;
    const float sc = kLog2e / sqrtf((float)D);
    const int kj = kv0 + i;  // this lane's key (column of every accumulator)

    const RowReads<T, D> rr(i, kh, w * RT::ELEMS);
    const XtReads<T, D> rxt = make_xt_reads<T, D>(lane, w * RT::ELEMS);
    const RowCopy<T, D> cq(lane, a.ldq), co(lane, a.lddo);

    typename E::Chunk kc[RT::STEPS], vc[RT::STEPS];
    {
      const int kr = min(kj, S - 1);
      load_row_frags<T, D>(k + (tok0 + kr) * a.ldk + (int64_t)grp * D, kh, kc);
      load_row_frags<T, D>(v + (tok0 + kr) * a.ldv + (int64_t)grp * D, kh, vc);
    }
    floatx16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dk[db][e] = 0.f;
        dv[db][e] = 0.f;
      }
    const int nqt = (S + 31) / 32;
    const float* lse_h = a.lse + ((int64_t)b * a.heads + h) * S;
    const float* dl_h = delta + ((int64_t)b * a.heads + h) * S;
    const int w0 = z * W + w, WZ = W * Z;
    const int n = kt + w0 < nqt ? (nqt - 1 - kt - w0) / WZ + 1 : 0;  // query tiles kt+w0, kt+w0+WZ, ..
    auto qtile = [&](int t) { return kt + w0 + WZ * t; };

    auto issue = [&](int t, T* sq, T* so) __attribute__((always_inline)) {
      const int q0 = qtile(t) * 32;
      copy_row_tile<T, D>(sq + w * RT::ELEMS, q, a.ldq, tok0, q0, S, h * D, cq, lane);
      copy_row_tile<T, D>(so + w * RT::ELEMS, d_o, a.lddo, tok0, q0, S, h * D, co, lane);
    };
    // log-sum-exp (in powers of two) and delta of this lane's 16 query rows
    // q0 + 8g + 4kh + r of the next query tile, loaded one step ahead and
    // before that step's tile copies are issued, so waiting for them never
    // waits for the copies.
    float4 lq[4], dq4[4], lq_n[4], dq4_n[4];
    auto load_ld = [&](int t, float4 (&L)[4], float4 (&Dl)[4]) __attribute__((always_inline)) {
      const int q0 = qtile(t) * 32;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr = q0 + 8 * g + 4 * kh;
        L[g] = qr < S ? *(const float4*)(lse_h + qr) : make_float4(0.f, 0.f, 0.f, 0.f);
        Dl[g] = qr < S ? *(const float4*)(dl_h + qr) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    auto compute = [&](const T* sq, const T* so, int t) __attribute__((always_inline)) {
      const int q0 = qtile(t) * 32;
      floatx16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = 0.f;
        dp[e] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < RT::STEPS; ++c) {
        s = E::mma(lds_at<typename E::Chunk>(sq, rr.v[c]), kc[c], s);
        dp = E::mma(lds_at<typename E::Chunk>(so, rr.v[c]), vc[c], dp);
      }
      auto sm = [&](auto Masked) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * g + r;
            const float L = r == 0 ? lq[g].x : r == 1 ? lq[g].y : r == 2 ? lq[g].z : lq[g].w;
            const float Dl = r == 0 ? dq4[g].x : r == 1 ? dq4[g].y : r == 2 ? dq4[g].z : dq4[g].w;
            float p = exp2_hw(fmaf(s[e], sc, -L * kLog2e));
            if constexpr (decltype(Masked)::value) {
              const int qq = q0 + 8 * g + 4 * kh + r;
              if (kj > qq || qq >= S || kj >= S) p = 0.f;
            }
            s[e] = p;
            dp[e] = p * (dp[e] - Dl);
          }
      };
      if (q0 == kv0 || q0 + 32 > S) sm(std::true_type{});
      else sm(std::false_type{});
      acc_rows_product_any<T, D>(so, rxt, s, dv);   // dV^T += dO^T P
      acc_rows_product_any<T, D>(sq, rxt, dp, dk);  // dK^T += Q^T dS
    };
    if (n > 0) load_ld(0, lq_n, dq4_n);
    wave_ring<NS>(
        n, 2 * RT::NI, [&](int t, auto St) __attribute__((always_inline)) { issue(t, sQ(St), sO(St)); },
        [&](int t) __attribute__((always_inline)) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            lq[g] = lq_n[g];
            dq4[g] = dq4_n[g];
          }
          if (t + 1 < n) load_ld(t + 1, lq_n, dq4_n);
        },
        [&](int t, auto St) __attribute__((always_inline)) { compute(sQ(St), sO(St), t); });

    // one exchange over the 2 NB blocks (dK's, then dV's): each wave adds
    // the blocks it owns in wave order and writes them
    constexpr int NB = D / 32, CAP = W * RT::ELEMS * (int)sizeof(T) / 4096;
    static_assert(2 * NB * W <= 4 * CAP, "combine space");
    auto slot = [&](int i) __attribute__((always_inline)) {
      return stage_slot<CAP>(i, sQ(I0{}), sO(I0{}), sQ(I1{}), sO(I1{}));
    };
    floatx16 kv[2 * NB];
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      kv[db] = dk[db];
      kv[NB + db] = dv[db];
    }
    __syncthreads();
    park_blocks<W, 2 * NB>(kv, w, lane, slot);
    __syncthreads();
    sum_owned<W, 2 * NB, false>(kv, w, lane, slot, NoScale{});
    if (kj < S) {
      const float inv = 1.0f / sqrtf((float)D);
      float* krow = dk_part + ((tok0 + kj) * a.heads + h) * (int64_t)D + 4 * kh;
      float* vrow = dv_part + ((tok0 + kj) * a.heads + h) * (int64_t)D + 4 * kh;
#pragma unroll
      for (int j = 0; j < 2 * NB; ++j)
        if (j % W == w) {
          const int db = j % NB;
          const float sc = j < NB ? inv : 1.f;
          float* row = (j < NB ? krow : vrow) + db * 32;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(float4*)(row + 8 * g) = make_float4(kv[j][4 * g] * sc, kv[j][4 * g + 1] * sc, kv[j][4 * g + 2] * sc,
                                                  kv[j][4 * g + 3] * sc);
        }
    }
  }
}

// Copies of one row tile split over the G waves of a KV group: wave w
// issues the 1 KB copies j = w, w + G, ... (its n of them), with the
// source offsets of those copies precomputed.
template <typename T, int D, int G>
struct GrpCopy {
  using RT = RowTile<T, D>;
  static constexpr int CPW = (RT::NI + G - 1) / G;
  uint32_t v[CPW];
  int n;
  __device__ __forceinline__ GrpCopy(int lane, int w, int64_t ld) {
    n = 0;
#pragma unroll
    for (int jj = 0; jj < CPW; ++jj) {
      const int j = jj * G + w;
      if (j < RT::NI) n = jj + 1;
      const int row = j * RT::RPI + lane / RT::NCH;
      const int lc = (lane % RT::NCH) ^ RT::sw(row);
      v[jj] = (uint32_t)((row * ld + lc * AttnElem<T>::EPC) * (int64_t)sizeof(T));
    }
  }
  // rows r0 .. r0+31 of a [T, *] matrix, columns col0 .. col0+D-1; a tile
  // running past the sequence clamps its rows to S-1 (they are masked)
  __device__ __forceinline__ void copy(T* tile, const T* base, int64_t ld, int64_t tok0, int r0, int S, int col0,
                                       int lane, int w) const {
    if (r0 + 32 <= S) {
      const char* slab = (const char*)(base + (tok0 + r0) * ld + col0);
#pragma unroll
      for (int jj = 0; jj < CPW; ++jj)
        if (jj < n) dma16_asm(slab + v[jj], tile + (jj * G + w) * (1024 / sizeof(T)));
    } else {
#pragma unroll
      for (int jj = 0; jj < CPW; ++jj)
        if (jj < n) {
          const int j = jj * G + w;
          const int row = j * RT::RPI + lane / RT::NCH;
          const int lc = (lane % RT::NCH) ^ RT::sw(row);
          dma16_asm(base + (tok0 + min(r0 + row, S - 1)) * ld + col0 + lc * AttnElem<T>::EPC,
                    tile + j * (1024 / sizeof(T)));
        }
    }
  }
};

// Forward with the key and value tiles shared by a KV group (16-bit
// operands): grid (pairs of q tiles, KV heads, batch); wave w = hw + G hf
// computes query head grp G + hw (lane owns a query, as in
// attn_dma_fwd_kernel) over the key tiles hf, hf + NH, ... of its q tile.
// Each half hf streams its key and value tiles through a ring of NS stages
// shared by its G waves (each wave issues its share of the copies), so the
// LDS fill per tile is one K and one V tile for G heads instead of one per
// head; with NH = 2 halves two waves share each SIMD, one's softmax beside
// the other's MFMAs. Step j: each wave waits for its own copies of its
// half's tile j, a barrier (every copy of step j landed, every wave is done
// with step j-1), the copies of step j+2 into the stages of step j-1, then
// the tile. The two halves of a head then merge their (max, sum, output)
// through LDS, each wave writing half of the head's columns. Tiles t and
// ntl-1-t share a workgroup as in the other kernels.
template <typename T, int D, int G, int NH>
__global__ __launch_bounds__(G* NH * 64) void attn_grp_fwd_kernel(const AttnDmaArgs a) {
  using RT = RowTile<T, D>;
  using E = AttnElem<T>;
  static_assert(sizeof(T) == 2, "16-bit operands");
  static_assert(NH == 1 || NH == 2, "key halves");
  // merge space: a wave parks NB/2 blocks of 4 KB in one stage buffer, and
  // the 8 waves' (max, sum) pairs fill 4 KB of another
  static_assert(NH == 1 || (G * NH <= 8 && (D / 64) * 4096 <= RT::ELEMS * (int)sizeof(T) &&
                            4096 <= RT::ELEMS * (int)sizeof(T)), "merge space");
  constexpr int NS = 3, NB = D / 32;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hw = w % G, hf = w / G;
  // stage buffers: index 2 (NS hf' + s) + (0 K, 1 V)
  auto buf = [](int idx) __attribute__((always_inline)) -> T* {
    switch (idx) {
      case 0: return att_lds<T, 60, RT::ELEMS>();
      case 1: return att_lds<T, 61, RT::ELEMS>();
      case 2: return att_lds<T, 62, RT::ELEMS>();
      case 3: return att_lds<T, 63, RT::ELEMS>();
      case 4: return att_lds<T, 64, RT::ELEMS>();
      case 5: return att_lds<T, 65, RT::ELEMS>();
    }
    if constexpr (NH == 2) {
      switch (idx) {
        case 6: return att_lds<T, 66, RT::ELEMS>();
        case 7: return att_lds<T, 67, RT::ELEMS>();
        case 8: return att_lds<T, 68, RT::ELEMS>();
        case 9: return att_lds<T, 69, RT::ELEMS>();
        case 10: return att_lds<T, 70, RT::ELEMS>();
      }
      return att_lds<T, 71, RT::ELEMS>();
    }
    return nullptr;
  };
  T* const sK0 = buf(2 * NS * hf), *const sV0 = buf(2 * NS * hf + 1);
  T* const sK1 = buf(2 * NS * hf + 2), *const sV1 = buf(2 * NS * hf + 3);
  T* const sK2 = buf(2 * NS * hf + 4), *const sV2 = buf(2 * NS * hf + 5);
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const int grp = blockIdx.y, h = grp * G + hw, b = blockIdx.z;
  const int S = a.seq;
  const int ntl = (S + 31) / 32, pr = blockIdx.x;
  const int npass = 2 * pr + 1 == ntl ? 1 : 2;
  const int i = lane & 31, kh = lane >> 5;
  const float sc = kLog2e / sqrtf((float)D);
  const int64_t tok0 = (int64_t)b * S;
  const RowReads<T, D> rk(i, kh, 0);
  const TrReads<D> rv(lane, 0);
  const GrpCopy<T, D, G> ck(lane, hw, a.ldk), cv(lane, hw, a.ldv);
  const int per_tile = ck.n + cv.n;  // this wave's copies per tile
  for (int pass = 0; pass < npass; ++pass) {
    if (pass) __syncthreads();  // every wave is done with the previous pass's stages
    const int qt = pass == 0 ? ntl - 1 - pr : pr, q0 = qt * 32;
    const int qi = q0 + i;
    typename E::Chunk qc[RT::STEPS];
    load_row_frags<T, D>(q + (tok0 + min(qi, S - 1)) * a.ldq + (int64_t)h * D, kh, qc);
    floatx16 o[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
    float m = -INFINITY, l = 0.f;
    const int nt = qt + 1;                 // key tiles 0 .. qt
    const int nh = (nt - hf + NH - 1) / NH;  // this half's: hf, hf + NH, ...
    const int nsteps = (nt + NH - 1) / NH;

    auto issue = [&](int j, T* sk, T* sv) __attribute__((always_inline)) {
      const int kv0 = (j * NH + hf) * 32;
      ck.copy(sk, k, a.ldk, tok0, kv0, S, grp * D, lane, hw);
      cv.copy(sv, v, a.ldv, tok0, kv0, S, grp * D, lane, hw);
    };
    auto compute = [&](const T* sk, const T* sv, int j) __attribute__((always_inline)) {
      const int kv0 = (j * NH + hf) * 32;
      floatx16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int c = 0; c < RT::STEPS; ++c) s = E::mma(lds_at<typename E::Chunk>(sk, rk.v[c]), qc[c], s);
      if (kv0 == q0) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kv0 + 8 * g + 4 * kh + r > qi) s[4 * g + r] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
      mx = half_max(mx) * sc;
      if (__any(mx > m + kRescaleSlack)) {
        const float mn = fmaxf(m, mx);
        const float alpha = exp2_hw(m - mn);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
        m = mn;
      }
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2_hw(fmaf(s[e], sc, -m));
        s[e] = p;
        ps += p;
      }
      l += half_sum(ps);
      acc_rows_product_tr<D, std::is_same_v<T, bf16>>(sv, rv, s, o);
    };
    if (0 < nh) issue(0, sK0, sV0);
    if (1 < nh) issue(1, sK1, sV1);
    auto step = [&](T* sk, T* sv, T* rk2, T* rv2, int j) __attribute__((always_inline)) {
      if (j + 1 < nh) wait_vmcnt_le(per_tile);
      else wait_vmcnt<0>();
      __syncthreads();
      if (j + 2 < nh) issue(j + 2, rk2, rv2);
      if (j < nh) compute(sk, sv, j);
    };
    const int nfull = nsteps / NS * NS;
    for (int j = 0; j < nfull; j += NS) {
      step(sK0, sV0, sK2, sV2, j);
      step(sK1, sV1, sK0, sV0, j + 1);
      step(sK2, sV2, sK1, sV1, j + 2);
    }
    if (nsteps - nfull > 0) step(sK0, sV0, sK2, sV2, nfull);
    if (nsteps - nfull > 1) step(sK1, sV1, sK0, sV0, nfull + 1);

    float M = m, L = l;
    if constexpr (NH == 2) {
      // the two halves of head hw merge: wave (hw, hf) parks its max, sum
      // and the blocks its partner writes (db / (NB/2) != hf), reads the
      // partner's and adds them, half 0's term first
      constexpr int OWN = NB / 2;
      __syncthreads();  // every wave is done with the stages
      float* park = (float*)buf(w);
      float* ml = (float*)buf(2 * NS * NH - 1) + 128 * w;  // [m, l] x 64 lanes per wave, last buffer's tail
#pragma unroll
      for (int db = 0; db < NB; ++db)
        if (db / OWN != hf) {
          float4* p = (float4*)(park + (db % OWN) * 1024);
#pragma unroll
          for (int g = 0; g < 4; ++g) p[g * 64 + lane] = make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
        }
      ml[lane] = m;
      ml[64 + lane] = l;
      __syncthreads();
      const int pw = hw + G * (1 - hf);  // partner wave
      const float* pml = (const float*)buf(2 * NS * NH - 1) + 128 * pw;
      const float mp = pml[lane], lp = pml[64 + lane];
      M = fmaxf(m, mp);
      const float f = m == -INFINITY ? 0.f : exp2f(m - M), fp = mp == -INFINITY ? 0.f : exp2f(mp - M);
      L = hf == 0 ? l * f + lp * fp : lp * fp + l * f;
      const float* ppark = (const float*)buf(pw);
#pragma unroll
      for (int db = 0; db < NB; ++db)
        if (db / OWN == hf) {
          const float4* p = (const float4*)(ppark + (db % OWN) * 1024);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 x = p[g * 64 + lane];
            const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float own = o[db][4 * g + r] * f, oth = xv[r] * fp;
              o[db][4 * g + r] = hf == 0 ? own + oth : oth + own;
            }
          }
        }
    }
    if (qi < S) {
      const float inv = 1.0f / L;
      const int64_t ooff = (tok0 + qi) * a.ldo + (int64_t)h * D + 4 * kh;
#pragma unroll
      for (int db = 0; db < NB; ++db)
        if (NH == 1 || db / (NB / 2) == hf) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 vv = make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                                          o[db][4 * g + 3] * inv);
            *(float4*)(a.o + ooff + db * 32 + 8 * g) = vv;
            if (a.o16) *(half4*)(a.o16 + ooff + db * 32 + 8 * g) = to_16x4(vv, std::is_same_v<T, bf16>);
          }
        }
      if (kh == 0 && hf == 0) a.lse[((int64_t)b * a.heads + h) * S + qi] = (M + log2f(L)) * kLn2;
    }
  }
}

// dQ with the key and value tiles shared by a KV group (16-bit operands),
// the layout of attn_grp_fwd_kernel: wave w = hw + G hf takes query head
// grp G + hw over the key tiles hf, hf + NH, ... of its q tile (K and V
// through the half's shared ring), recomputes P from the LSE, forms dS and
// accumulates dQ = dS K; delta = rowsum(dO o) is summed by the two halves
// over half the columns each and stored for the dK/dV kernel. The halves'
// dQ blocks are added in LDS (half 0 first), each wave writing half of the
// head's columns.
template <typename T, int D, int G, int NH>
__global__ __launch_bounds__(G* NH * 64) void attn_grp_dq_kernel(const AttnDmaArgs a, float* delta) {
  using RT = RowTile<T, D>;
  using E = AttnElem<T>;
  static_assert(sizeof(T) == 2, "16-bit operands");
  static_assert(NH == 1 || NH == 2, "key halves");
  static_assert(NH == 1 || (G * NH <= 8 && (D / 64) * 4096 <= RT::ELEMS * (int)sizeof(T) &&
                            4096 <= RT::ELEMS * (int)sizeof(T)), "merge space");
  constexpr int NS = 3, NB = D / 32;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hw = w % G, hf = w / G;
  auto buf = [](int idx) __attribute__((always_inline)) -> T* {
    switch (idx) {
      case 0: return att_lds<T, 72, RT::ELEMS>();
      case 1: return att_lds<T, 73, RT::ELEMS>();
      case 2: return att_lds<T, 74, RT::ELEMS>();
      case 3: return att_lds<T, 75, RT::ELEMS>();
      case 4: return att_lds<T, 76, RT::ELEMS>();
      case 5: return att_lds<T, 77, RT::ELEMS>();
    }
    if constexpr (NH == 2) {
      switch (idx) {
        case 6: return att_lds<T, 78, RT::ELEMS>();
        case 7: return att_lds<T, 79, RT::ELEMS>();
        case 8: return att_lds<T, 80, RT::ELEMS>();
        case 9: return att_lds<T, 81, RT::ELEMS>();
        case 10: return att_lds<T, 82, RT::ELEMS>();
      }
      return att_lds<T, 83, RT::ELEMS>();
    }
    return nullptr;
  };
  T* const sK0 = buf(2 * NS * hf), *const sV0 = buf(2 * NS * hf + 1);
  T* const sK1 = buf(2 * NS * hf + 2), *const sV1 = buf(2 * NS * hf + 3);
  T* const sK2 = buf(2 * NS * hf + 4), *const sV2 = buf(2 * NS * hf + 5);
  // the last stage buffer (stage 2 of the last half) is free until step 0
  // refills it: the delta exchange and, after the loop, the merge's sums
  float* const xchg = (float*)buf(2 * NS * NH - 1);
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const T* d_o = (const T*)a.d_o;
  const int grp = blockIdx.y, h = grp * G + hw, b = blockIdx.z;
  const int S = a.seq;
  const int ntl = (S + 31) / 32, pr = blockIdx.x;
  const int npass = 2 * pr + 1 == ntl ? 1 : 2;
  const int i = lane & 31, kh = lane >> 5;
  const float sc = kLog2e / sqrtf((float)D);
  const int64_t tok0 = (int64_t)b * S;
  const RowReads<T, D> rr(i, kh, 0);
  const TrReads<D> rkt(lane, 0);
  const GrpCopy<T, D, G> ck(lane, hw, a.ldk), cv(lane, hw, a.ldv);
  const int per_tile = ck.n + cv.n;
  for (int pass = 0; pass < npass; ++pass) {
    if (pass) __syncthreads();  // every wave is done with the previous pass's stages
    const int qt = pass == 0 ? ntl - 1 - pr : pr, q0 = qt * 32;
    const int qi = q0 + i, qc_i = min(qi, S - 1);
    const int64_t rowi = ((int64_t)b * a.heads + h) * S + qc_i;
    const float lse2 = a.lse[rowi] * kLog2e;
    float dl;
    {
      // delta over columns hf D/NH .. (hf+1) D/NH - 1 of the head, the lane
      // halves (kh) half of those each
      constexpr int CW = D / NH / 2;
      const int64_t c0 = (int64_t)h * D + hf * (D / NH) + kh * CW;
      const float* orow = a.o + (tok0 + qc_i) * a.ldo + c0;
      const float* drow = a.do32 + (tok0 + qc_i) * a.lddo32 + c0;
      float4 o4[CW / 4], d4[CW / 4];
#pragma unroll
      for (int j = 0; j < CW / 4; ++j) {
        o4[j] = *(const float4*)(orow + 4 * j);
        d4[j] = *(const float4*)(drow + 4 * j);
      }
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < CW / 4; ++j)
        part += o4[j].x * d4[j].x + o4[j].y * d4[j].y + o4[j].z * d4[j].z + o4[j].w * d4[j].w;
      part = cross_half_sum(part);
      if constexpr (NH == 2) {
        xchg[w * 64 + lane] = part;
        __syncthreads();
        const float p0 = xchg[hw * 64 + lane], p1 = xchg[(hw + G) * 64 + lane];
        dl = p0 + p1;
      } else {
        dl = part;
      }
      if (hf == 0 && kh == 0 && qi < S) delta[rowi] = dl;
    }
    // the operand fragments after the delta sums (fewer live registers)
    typename E::Chunk qc[RT::STEPS], dc[RT::STEPS];
    load_row_frags<T, D>(q + (tok0 + qc_i) * a.ldq + (int64_t)h * D, kh, qc);
    load_row_frags<T, D>(d_o + (tok0 + qc_i) * a.lddo + (int64_t)h * D, kh, dc);
    floatx16 dq[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;
    const int nt = qt + 1;
    const int nh = (nt - hf + NH - 1) / NH;
    const int nsteps = (nt + NH - 1) / NH;

    auto issue = [&](int j, T* sk, T* sv) __attribute__((always_inline)) {
      const int kv0 = (j * NH + hf) * 32;
      ck.copy(sk, k, a.ldk, tok0, kv0, S, grp * D, lane, hw);
      cv.copy(sv, v, a.ldv, tok0, kv0, S, grp * D, lane, hw);
    };
    auto compute = [&](const T* sk, const T* sv, int j) __attribute__((always_inline)) {
      const int kv0 = (j * NH + hf) * 32;
      floatx16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = 0.f;
        dp[e] = 0.f;
      }
      // S^T, then dP^T: a scheduling fence between them keeps the V
      // fragments' reads from being hoisted beside the K ones (registers)
#pragma unroll
      for (int c = 0; c < RT::STEPS; ++c) s = E::mma(lds_at<typename E::Chunk>(sk, rr.v[c]), qc[c], s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < RT::STEPS; ++c) dp = E::mma(lds_at<typename E::Chunk>(sv, rr.v[c]), dc[c], dp);
      if (kv0 == q0) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * g + r;
            const int kj = kv0 + 8 * g + 4 * kh + r;
            const float p = (kj > qi || kj >= S) ? 0.f : exp2_hw(fmaf(s[e], sc, -lse2));
            s[e] = p * (dp[e] - dl);  // dS^T, unscaled
          }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = exp2_hw(fmaf(s[e], sc, -lse2)) * (dp[e] - dl);
      }
      acc_rows_product_tr<D, std::is_same_v<T, bf16>>(sk, rkt, s, dq);
    };
    if (0 < nh) issue(0, sK0, sV0);
    if (1 < nh) issue(1, sK1, sV1);
    auto step = [&](T* sk, T* sv, T* rk2, T* rv2, int j) __attribute__((always_inline)) {
      if (j + 1 < nh) wait_vmcnt_le(per_tile);
      else wait_vmcnt<0>();
      __syncthreads();
      if (j + 2 < nh) issue(j + 2, rk2, rv2);
      if (j < nh) compute(sk, sv, j);
    };
    const int nfull = nsteps / NS * NS;
    for (int j = 0; j < nfull; j += NS) {
      step(sK0, sV0, sK2, sV2, j);
      step(sK1, sV1, sK0, sV0, j + 1);
      step(sK2, sV2, sK1, sV1, j + 2);
    }
    if (nsteps - nfull > 0) step(sK0, sV0, sK2, sV2, nfull);
    if (nsteps - nfull > 1) step(sK1, sV1, sK0, sV0, nfull + 1);

    if constexpr (NH == 2) {
      // wave (hw, hf) parks the blocks its partner writes and adds the
      // partner's parked ones to its own, half 0's term first
      constexpr int OWN = NB / 2;
      __syncthreads();  // every wave is done with the stages
      float* park = (float*)buf(w);
#pragma unroll
      for (int db = 0; db < NB; ++db)
        if (db / OWN != hf) {
          float4* p = (float4*)(park + (db % OWN) * 1024);
#pragma unroll
          for (int g = 0; g < 4; ++g)
            p[g * 64 + lane] = make_float4(dq[db][4 * g], dq[db][4 * g + 1], dq[db][4 * g + 2], dq[db][4 * g + 3]);
        }
      __syncthreads();
      const float* ppark = (const float*)buf(hw + G * (1 - hf));
#pragma unroll
      for (int db = 0; db < NB; ++db)
        if (db / OWN == hf) {
          const float4* p = (const float4*)(ppark + (db % OWN) * 1024);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 x = p[g * 64 + lane];
            const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
              dq[db][4 * g + r] = hf == 0 ? dq[db][4 * g + r] + xv[r] : xv[r] + dq[db][4 * g + r];
          }
        }
    }
    if (qi < S) {
      const float inv = 1.0f / sqrtf((float)D);
      float* row = a.dq + (tok0 + qi) * a.lddq + (int64_t)h * D + 4 * kh;
#pragma unroll
      for (int db = 0; db < NB; ++db)
        if (NH == 1 || db / (NB / 2) == hf) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(float4*)(row + db * 32 + 8 * g) = make_float4(dq[db][4 * g] * inv, dq[db][4 * g + 1] * inv,
                                                            dq[db][4 * g + 2] * inv, dq[db][4 * g + 3] * inv);
        }
    }
  }
}

// dK, dV per query head with the query-side tiles shared by KB key tiles
// (16-bit operands): grid (pairs of blocks of KB key tiles, heads, batch);
// wave w owns key tile KB b + w of block b (lane owns a key, as in
// attn_dma_dkv_kernel) and the workgroup streams the block's query tiles
// (Q and dO, each copied once for the KB key tiles, the waves issuing
// their shares) through a ring of NS stages; a wave skips the query tiles
// below its key tile. Step t: the wave waits for its own copies of tile t,
// a barrier, the copies of tile t+2 into the stage of tile t-1, then the
// tile. The per-head partials go to dk_part / dv_part as in the per-tile
// kernel. Blocks b and nkb-1-b share a workgroup (the first has the most
// query tiles).
template <typename T, int D, int KB>
__global__ __launch_bounds__(KB * 64) void attn_grp_dkv_kernel(const AttnDmaArgs a, const float* delta,
                                                               float* dk_part, float* dv_part) {
  using RT = RowTile<T, D>;
  using E = AttnElem<T>;
  static_assert(sizeof(T) == 2, "16-bit operands");
  constexpr int NS = 3, NB = D / 32;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto sQ = [](auto S) { return att_lds<T, 84 + 2 * decltype(S)::value, RT::ELEMS>(); };
  auto sO = [](auto S) { return att_lds<T, 85 + 2 * decltype(S)::value, RT::ELEMS>(); };
  // per stage: the tile's 32 log-sum-exps then its 32 deltas
  auto sL = [](auto S) { return att_lds<float, 90 + decltype(S)::value, 64>(); };
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const T* d_o = (const T*)a.d_o;
  const int h = blockIdx.y, b = blockIdx.z;
  const int G = a.heads / a.kv_heads, grp = h / G;
  const int S = a.seq;
  const int ntl = (S + 31) / 32, nkb = (ntl + KB - 1) / KB, pr = blockIdx.x;
  const int npass = 2 * pr + 1 == nkb ? 1 : 2;
  const int i = lane & 31, kh = lane >> 5;
  const float sc = kLog2e / sqrtf((float)D);
  const int64_t tok0 = (int64_t)b * S;
  const RowReads<T, D> rr(i, kh, 0);
  const TrReads<D> rxt(lane, 0);
  const GrpCopy<T, D, KB> cq(lane, w, a.ldq), co(lane, w, a.lddo);
  // wave 0 also copies the tile's log-sum-exps and deltas (16 lanes)
  const int per_tile = cq.n + co.n + (w == 0 ? 1 : 0);
  const float* lse_h = a.lse + ((int64_t)b * a.heads + h) * S;
  const float* dl_h = delta + ((int64_t)b * a.heads + h) * S;
  for (int pass = 0; pass < npass; ++pass) {
    if (pass) __syncthreads();  // every wave is done with the previous pass's stages
    const int bi = pass == 0 ? pr : nkb - 1 - pr;
    const int qs = bi * KB;           // first query tile of the stream
    const int kt = qs + w, kv0 = kt * 32;
    const int kj = kv0 + i;           // this lane's key (column of every accumulator)
    typename E::Chunk kc[RT::STEPS], vc[RT::STEPS];
    {
      const int kr = min(kj, S - 1);
      load_row_frags<T, D>(k + (tok0 + kr) * a.ldk + (int64_t)grp * D, kh, kc);
      load_row_frags<T, D>(v + (tok0 + kr) * a.ldv + (int64_t)grp * D, kh, vc);
    }
    floatx16 dk[NB], dv[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dk[db][e] = 0.f;
        dv[db][e] = 0.f;
      }
    const int n = ntl - qs;  // query tiles qs .. ntl-1

    // Q and dO tiles, and in wave 0 the tile's log-sum-exps and deltas
    // (lanes 0-7 and 8-15, 16 bytes each; rows past S are not read: S is a
    // multiple of 8)
    auto issue = [&](int t, T* sq, T* so, float* sl) __attribute__((always_inline)) {
      const int q0 = (qs + t) * 32;
      cq.copy(sq, q, a.ldq, tok0, q0, S, h * D, lane, w);
      co.copy(so, d_o, a.lddo, tok0, q0, S, h * D, lane, w);
      if (w == 0) {
        const int r = q0 + 4 * (lane & 7);
        if (lane < 16 && r < S) dma16_asm((lane < 8 ? lse_h : dl_h) + r, sl);
      }
    };
    auto compute = [&](const T* sq, const T* so, const float* sl, int t) __attribute__((always_inline)) {
      const int q0 = (qs + t) * 32;
      float4 lq[4], dq4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lq[g] = *(const float4*)(sl + 8 * g + 4 * kh);
        dq4[g] = *(const float4*)(sl + 32 + 8 * g + 4 * kh);
      }
      floatx16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = 0.f;
        dp[e] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < RT::STEPS; ++c) {
        s = E::mma(lds_at<typename E::Chunk>(sq, rr.v[c]), kc[c], s);
        dp = E::mma(lds_at<typename E::Chunk>(so, rr.v[c]), vc[c], dp);
      }
      auto sm = [&](auto Masked) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * g + r;
            float L = r == 0 ? lq[g].x : r == 1 ? lq[g].y : r == 2 ? lq[g].z : lq[g].w;
            float Dl = r == 0 ? dq4[g].x : r == 1 ? dq4[g].y : r == 2 ? dq4[g].z : dq4[g].w;
            bool off = false;
            if constexpr (decltype(Masked)::value) {
              const int qq = q0 + 8 * g + 4 * kh + r;
              off = kj > qq || qq >= S || kj >= S;
              if (qq >= S) L = Dl = 0.f;  // rows past S were not copied
            }
            float p = exp2_hw(fmaf(s[e], sc, -L * kLog2e));
            if (off) p = 0.f;
            s[e] = p;
            dp[e] = p * (dp[e] - Dl);
          }
      };
      if (q0 == kv0 || q0 + 32 > S) sm(std::true_type{});
      else sm(std::false_type{});
      acc_rows_product_tr<D, std::is_same_v<T, bf16>>(so, rxt, s, dv);   // dV^T += dO^T P
      acc_rows_product_tr<D, std::is_same_v<T, bf16>>(sq, rxt, dp, dk);  // dK^T += Q^T dS
    };
    issue(0, sQ(I0{}), sO(I0{}), sL(I0{}));
    if (1 < n) issue(1, sQ(I1{}), sO(I1{}), sL(I1{}));
    auto step = [&](auto St, int t) __attribute__((always_inline)) {
      constexpr int st = decltype(St)::value;
      if (t + 1 < n) wait_vmcnt_le(per_tile);
      else wait_vmcnt<0>();
      __syncthreads();
      if (t + 2 < n) issue(t + 2, sQ(IC<(st + 2) % NS>{}), sO(IC<(st + 2) % NS>{}), sL(IC<(st + 2) % NS>{}));
      if (qs + t >= kt && kt < ntl) compute(sQ(St), sO(St), sL(St), t);
    };
    const int nfull = n / NS * NS;
    for (int t = 0; t < nfull; t += NS) {
      step(IC<0>{}, t);
      step(IC<1>{}, t + 1);
      step(IC<2>{}, t + 2);
    }
    if (n - nfull > 0) step(IC<0>{}, nfull);
    if (n - nfull > 1) step(IC<1>{}, nfull + 1);
    if (kt < ntl && kj < S) {
      const float inv = 1.0f / sqrtf((float)D);
      float* krow = dk_part + ((tok0 + kj) * a.heads + h) * (int64_t)D + 4 * kh;
      float* vrow = dv_part + ((tok0 + kj) * a.heads + h) * (int64_t)D + 4 * kh;
#pragma unroll
      for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          *(float4*)(krow + db * 32 + 8 * g) =
              make_float4(dk[db][4 * g] * inv, dk[db][4 * g + 1] * inv, dk[db][4 * g + 2] * inv, dk[db][4 * g + 3] * inv);
          *(float4*)(vrow + db * 32 + 8 * g) =
              make_float4(dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]);
        }
    }
  }
}

// Merge of the forward's Z key-range splits per (token, head): with
// M = max M_z and f_z = 2^(M_z - M), o = sum f_z O_z / sum f_z L_z (split
// order), lse = (M + log2 sum f_z L_z) ln 2. One thread per 4 columns.
__global__ __launch_bounds__(256) void attn_fwd_combine_kernel(const AttnDmaArgs a, int D) {
  const int64_t T = (int64_t)a.batch * a.seq;
  const int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x;
  const int c4 = D / 4;
  if (e >= T * a.heads * c4) return;
  const int64_t row = e / c4;  // token * heads + head
  const int col = 4 * (int)(e % c4);
  const int Z = a.split;
  float M = -INFINITY;
  for (int z = 0; z < Z; ++z) M = fmaxf(M, a.ml_part[2 * (z * T * a.heads + row)]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int z = 0; z < Z; ++z) {
    const float2 ml = *(const float2*)(a.ml_part + 2 * (z * T * a.heads + row));
    const float f = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
    L += ml.y * f;
    const float4 v = *(const float4*)(a.o_part + (z * T * a.heads + row) * D + col);
    acc.x += f * v.x;
    acc.y += f * v.y;
    acc.z += f * v.z;
    acc.w += f * v.w;
  }
  const float inv = 1.0f / L;
  const int64_t tok = row / a.heads;
  const int h = (int)(row % a.heads);
  const float4 o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  const int64_t off = tok * a.ldo + (int64_t)h * D + col;
  *(float4*)(a.o + off) = o;
  if (a.o16) *(half4*)(a.o16 + off) = to_16x4(o, a.bf16 != 0);
  if (col == 0) {
    const int b = (int)(tok / a.seq), sq = (int)(tok % a.seq);
    a.lse[((int64_t)b * a.heads + h) * a.seq + sq] = (M + log2f(L)) * kLn2;
  }
}

template <typename T, int D>
int fwd_dma_launch(const AttnDmaArgs& a0, void* scratch, hipStream_t st) {
  AttnDmaArgs a = a0;
  if constexpr (sizeof(T) == 2) {
    const int G = attention_group_waves(a.batch, a.seq, a.heads, a.kv_heads);
    if (G) {
      dim3 grid((unsigned)ceil_div(ceil_div(a.seq, 32), 2), (unsigned)a.kv_heads, (unsigned)a.batch);
      if (G == 2) hipLaunchKernelGGL((attn_grp_fwd_kernel<T, D, 2, 2>), grid, dim3(256), 0, st, a);
      else if (G == 4) hipLaunchKernelGGL((attn_grp_fwd_kernel<T, D, 4, 2>), grid, dim3(512), 0, st, a);
      else hipLaunchKernelGGL((attn_grp_fwd_kernel<T, D, 8, 1>), grid, dim3(512), 0, st, a);
      return check_launch("attn_grp_fwd_kernel");
    }
  }
  a.split = scratch ? attention_kv_split(a.batch, a.seq, a.heads) : 1;
  const int64_t ntok = (int64_t)a.batch * a.seq;
  if (a.split > 1) {
    a.o_part = (float*)scratch;
    a.ml_part = a.o_part + a.split * ntok * a.heads * D;
  }
  if (attention_unpaired(a.batch, a.seq, a.heads, sizeof(T) == 2)) {
    constexpr int UW = AttnSplit<T>::UNPAIRED_W;
    dim3 grid((unsigned)ceil_div(a.seq, 32), (unsigned)a.heads, (unsigned)a.batch);
    hipLaunchKernelGGL((attn_dma_fwd_kernel<T, D, UW, false>), grid, dim3(64 * UW), 0, st, a);
    return check_launch("attn_dma_fwd_kernel");
  }
  // tiles are processed in pairs (Z workgroups per pair)
  dim3 grid((unsigned)(ceil_div(ceil_div(a.seq, 32), 2) * a.split), (unsigned)a.heads, (unsigned)a.batch);
  hipLaunchKernelGGL((attn_dma_fwd_kernel<T, D, AttnSplit<T>::FWD_W, true>), grid, dim3(64 * AttnSplit<T>::FWD_W), 0,
                     st, a);
  QBLK_TRY(check_launch("attn_dma_fwd_kernel"));
  if (a.split == 1) return 0;
  const int64_t n = ntok * a.heads * (D / 4);
  hipLaunchKernelGGL(attn_fwd_combine_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, a, D);
  return check_launch("attn_fwd_combine_kernel");
}

template <typename T, int D>
int bwd_dma_launch(const AttnDmaArgs& a0, float* delta, float* dk_part, float* dv_part, float* dq_part,
                   hipStream_t st) {
  AttnDmaArgs a = a0;
  a.split = attention_kv_split(a.batch, a.seq, a.heads);
  a.dq_part = dq_part;
  const int64_t T_ = (int64_t)a.batch * a.seq;
  // tiles are processed in pairs (Z workgroups per pair)
  dim3 grid((unsigned)(ceil_div(ceil_div(a.seq, 32), 2) * a.split), (unsigned)a.heads, (unsigned)a.batch);
  int G = 0;
  if constexpr (sizeof(T) == 2) G = attention_group_waves(a.batch, a.seq, a.heads, a.kv_heads);
  constexpr int UW = AttnSplit<T>::UNPAIRED_W;
  const bool unpaired = !G && attention_unpaired(a.batch, a.seq, a.heads, sizeof(T) == 2);
  const dim3 ugrid((unsigned)ceil_div(a.seq, 32), (unsigned)a.heads, (unsigned)a.batch);
  if (G) {
    // (the group kernels run only where the key-range split is 1)
    dim3 ggrid((unsigned)ceil_div(ceil_div(a.seq, 32), 2), (unsigned)a.kv_heads, (unsigned)a.batch);
    if constexpr (sizeof(T) == 2) {
      if (G == 2) hipLaunchKernelGGL((attn_grp_dq_kernel<T, D, 2, 2>), ggrid, dim3(256), 0, st, a, delta);
      else if (G == 4) hipLaunchKernelGGL((attn_grp_dq_kernel<T, D, 4, 2>), ggrid, dim3(512), 0, st, a, delta);
      else hipLaunchKernelGGL((attn_grp_dq_kernel<T, D, 8, 1>), ggrid, dim3(512), 0, st, a, delta);
    }
    QBLK_TRY(check_launch("attn_grp_dq_kernel"));
  } else if (unpaired) {
    hipLaunchKernelGGL((attn_dma_dq_kernel<T, D, UW, false>), ugrid, dim3(64 * UW), 0, st, a, delta);
    QBLK_TRY(check_launch("attn_dma_dq_kernel"));
  } else {
    hipLaunchKernelGGL((attn_dma_dq_kernel<T, D, AttnSplit<T>::DQ_W, true>), grid, dim3(64 * AttnSplit<T>::DQ_W), 0,
                       st, a, delta);
    QBLK_TRY(check_launch("attn_dma_dq_kernel"));
  }
  if (G) {
    // blocks of 4 key tiles share the query-side stream; pairs of blocks
    const int64_t nkb = ceil_div(ceil_div(a.seq, 32), 4);
    dim3 kgrid((unsigned)ceil_div(nkb, 2), (unsigned)a.heads, (unsigned)a.batch);
    if constexpr (sizeof(T) == 2)
      hipLaunchKernelGGL((attn_grp_dkv_kernel<T, D, 4>), kgrid, dim3(256), 0, st, a, (const float*)delta, dk_part,
                         dv_part);
    QBLK_TRY(check_launch("attn_grp_dkv_kernel"));
  } else if (unpaired) {
    hipLaunchKernelGGL((attn_dma_dkv_kernel<T, D, UW, false>), ugrid, dim3(64 * UW), 0, st, a, (const float*)delta,
                       dk_part, dv_part);
    QBLK_TRY(check_launch("attn_dma_dkv_kernel"));
  } else {
    hipLaunchKernelGGL((attn_dma_dkv_kernel<T, D, AttnSplit<T>::DKV_W, true>), grid, dim3(64 * AttnSplit<T>::DKV_W),
                       0, st, a, (const float*)delta, dk_part, dv_part);
    QBLK_TRY(check_launch("attn_dma_dkv_kernel"));
  }
  const int64_t n = T_ * a.kv_heads * D + (a.split > 1 ? T_ * a.heads * D : 0);
  hipLaunchKernelGGL(attn_gqa_reduce_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, T_, a.heads,
                     a.kv_heads, D, a.bf16, (const float*)dk_part, (const float*)dv_part, a.dk, a.lddk, a.dv, a.lddv,
                     a.dv16, a.lddv16, a.split, (const float*)dq_part, a.dq, a.lddq);
  return check_launch("attn_gqa_reduce_kernel");
}

}  // namespace

int attention_check(int batch, int seq, int heads, int kv_heads, int head_dim) {
  if (batch <= 0 || seq <= 0 || heads <= 0 || kv_heads <= 0)
    return fail(QBLK_EINVAL, "attention: batch=%d seq=%d heads=%d kv_heads=%d", batch, seq, heads, kv_heads);
  if (heads % kv_heads) return fail(QBLK_EINVAL, "attention: heads %% kv_heads != 0");
  if (heads / kv_heads > 8) return fail(QBLK_EUNSUPPORTED, "attention: more than 8 query heads per KV head");
  if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(QBLK_EUNSUPPORTED, "attention: head_dim %d not in {16, 32, 64, 128}", head_dim);
  return 0;
}

// Key-range splits of the tiled backward: a pair of 32-row tiles per
// workgroup and one workgroup per CU (their LDS) leave CUs idle when
// pairs x heads x batch is at most half the 256 CUs; two workgroups then
// share each pair (each half the key or query tiles), their partial sums
// added in split order by the GQA reduction.
int attention_kv_split(int batch, int seq, int heads) {
  const int64_t wgs = ceil_div(ceil_div(seq, 32), 2) * (int64_t)heads * batch;
  return 2 * wgs <= 256 ? 2 : 1;
}

// Unpaired 2-wave workgroups (AttnSplit::UNPAIRED_W) for the per-head
// kernels with 16-bit operands when the (tile, head) units number at least
// two per CU and no key-range split applies: two workgroups per CU then
// overlap one's first copies and final combine with the other's tiles
// instead of running a pair's two passes back to back (the Qwen3-4B block
// at seq 512: the step ≈ 1 % faster, forward, dQ and dK/dV alike). The
// fp32 kernels of the 36-layer stack's layers (seq 1024, 8 heads) measured
// slower that way and stay paired.
bool attention_unpaired(int batch, int seq, int heads, bool sixteen_bit) {
  return sixteen_bit && attention_kv_split(batch, seq, heads) == 1 &&
         ceil_div(seq, 32) * (int64_t)heads * batch >= 2 * 256;
}

// The group-shared forward (16-bit operands): G = heads / kv_heads waves
// per workgroup, one per query head of a KV group, when G is 2, 4 or 8 and
// its grid (tile pairs x KV heads x batch) gives at least half the 256 CUs
// a workgroup; 0 otherwise (the per-head kernel with its key-range split
// then fills the CUs better).
int attention_group_waves(int batch, int seq, int heads, int kv_heads) {
  const int G = heads / kv_heads;
  if (G != 2 && G != 4 && G != 8) return 0;
  const int64_t wgs = ceil_div(ceil_div(seq, 32), 2) * (int64_t)kv_heads * batch;
  return wgs >= 128 ? G : 0;
}

size_t attention_bwd_scratch(int batch, int seq, int heads, int head_dim) {
  const size_t T = (size_t)batch * seq;
  const size_t Z = (size_t)attention_kv_split(batch, seq, heads);
  // delta, Z dK and Z dV partial buffers, and with Z > 1 Z dQ partials
  return (T * heads + (2 * Z + (Z > 1 ? Z : 0)) * T * heads * head_dim) * sizeof(float);
}

int attention_forward(const AttnArgs& a, Prec p, hipStream_t st) {
  QBLK_TRY(attention_check(a.batch, a.seq, a.heads, a.kv_heads, a.head_dim));
  const int dp = a.head_dim < 32 ? 32 : a.head_dim;
  if (p == Prec::F16) {
    if (dp == 32) return fwd_launch<Prec::F16, 32>(a, st);
    if (dp == 64) return fwd_launch<Prec::F16, 64>(a, st);
    return fwd_launch<Prec::F16, 128>(a, st);
  }
  if (dp == 32) return fwd_launch<Prec::F32, 32>(a, st);
  if (dp == 64) return fwd_launch<Prec::F32, 64>(a, st);
  return fwd_launch<Prec::F32, 128>(a, st);
}

int attention_backward(const AttnArgs& a, Prec p, void* scratch, hipStream_t st) {
  QBLK_TRY(attention_check(a.batch, a.seq, a.heads, a.kv_heads, a.head_dim));
  const int64_t T = (int64_t)a.batch * a.seq;
  float* delta = (float*)scratch;
  float* dk_part = delta + T * a.heads;
  float* dv_part = dk_part + T * a.heads * a.head_dim;
  const int dp = a.head_dim < 32 ? 32 : a.head_dim;
  if (p == Prec::F16) {
    if (dp == 32) return bwd_launch<Prec::F16, 32>(a, delta, dk_part, dv_part, st);
    if (dp == 64) return bwd_launch<Prec::F16, 64>(a, delta, dk_part, dv_part, st);
    return bwd_launch<Prec::F16, 128>(a, delta, dk_part, dv_part, st);
  }
  if (dp == 32) return bwd_launch<Prec::F32, 32>(a, delta, dk_part, dv_part, st);
  if (dp == 64) return bwd_launch<Prec::F32, 64>(a, delta, dk_part, dv_part, st);
  return fail(QBLK_EUNSUPPORTED, "attention backward: fp32 needs head_dim <= 64");
}

bool attention_dma_supported(int batch, int seq, int heads, int kv_heads, int head_dim) {
  return attention_check(batch, seq, heads, kv_heads, head_dim) == 0 && (head_dim == 64 || head_dim == 128) &&
         seq % 8 == 0;
}

static int check_dma(const AttnDmaArgs& a) {
  QBLK_TRY(attention_check(a.batch, a.seq, a.heads, a.kv_heads, a.head_dim));
  if (!attention_dma_supported(a.batch, a.seq, a.heads, a.kv_heads, a.head_dim))
    return fail(QBLK_EUNSUPPORTED, "attention (tiled copies): head_dim must be 64 or 128 and seq a multiple of 8");
  if (a.ldq % 8 || a.ldk % 8 || a.ldv % 8 || a.ldo % 4)
    return fail(QBLK_EINVAL, "attention (tiled copies): row strides must be multiples of 8 (o: 4)");
  const void* ptrs[] = {a.q, a.k, a.v, a.o, a.lse};
  for (const void* p : ptrs)
    if (!p || ((uintptr_t)p & 15)) return fail(QBLK_EINVAL, "attention (tiled copies): null or misaligned pointer");
  return 0;
}

int attention_dma_forward(const AttnDmaArgs& a, void* scratch, hipStream_t st) {
  QBLK_TRY(check_dma(a));
  if (scratch && ((uintptr_t)scratch & 15))
    return fail(QBLK_EINVAL, "attention (tiled copies): misaligned scratch");
  if (a.fp32) {
    if (a.head_dim != 64) return fail(QBLK_EUNSUPPORTED, "attention (tiled copies): fp32 needs head_dim 64");
    return fwd_dma_launch<float, 64>(a, scratch, st);
  }
  if (a.bf16)
    return a.head_dim == 64 ? fwd_dma_launch<bf16, 64>(a, scratch, st) : fwd_dma_launch<bf16, 128>(a, scratch, st);
  return a.head_dim == 64 ? fwd_dma_launch<f16, 64>(a, scratch, st) : fwd_dma_launch<f16, 128>(a, scratch, st);
}

int attention_dma_backward(const AttnDmaArgs& a, void* scratch, hipStream_t st) {
  QBLK_TRY(check_dma(a));
  const void* ptrs[] = {a.v, a.d_o, a.do32, a.dq, a.dk, a.dv, scratch};
  for (const void* p : ptrs)
    if (!p || ((uintptr_t)p & 15)) return fail(QBLK_EINVAL, "attention backward (tiled copies): null or misaligned pointer");
  if (a.lddo % 8 || a.lddo32 % 4 || a.lddq % 4 || a.lddk % 4 || a.lddv % 4)
    return fail(QBLK_EINVAL, "attention backward (tiled copies): row strides");
  const int64_t T = (int64_t)a.batch * a.seq;
  const int64_t part = T * a.heads * a.head_dim;
  const int Z = attention_kv_split(a.batch, a.seq, a.heads);
  float* delta = (float*)scratch;
  float* dk_part = delta + T * a.heads;
  float* dv_part = dk_part + Z * part;
  float* dq_part = dv_part + Z * part;  // used when Z > 1
  if (a.fp32) {
    if (a.head_dim != 64) return fail(QBLK_EUNSUPPORTED, "attention backward (tiled copies): fp32 needs head_dim 64");
    return bwd_dma_launch<float, 64>(a, delta, dk_part, dv_part, dq_part, st);
  }
  if (a.bf16)
    return a.head_dim == 64 ? bwd_dma_launch<bf16, 64>(a, delta, dk_part, dv_part, dq_part, st)
                            : bwd_dma_launch<bf16, 128>(a, delta, dk_part, dv_part, dq_part, st);
  return a.head_dim == 64 ? bwd_dma_launch<f16, 64>(a, delta, dk_part, dv_part, dq_part, st)
                          : bwd_dma_launch<f16, 128>(a, delta, dk_part, dv_part, dq_part, st);
}

}  // namespace qblk
