// MFMA GEMM engine for gfx950: every projection of the decoder block, its
// backward (dX and dW), the LM head, and the NF4-dequant + LoRA variants.
//
// Tiling. A workgroup of WM x WN waves computes a BM x BN tile of C; each
// wave owns TM x TN blocks of 32 x 32, accumulated by v_mfma_f32_32x32x2_f32
// (fp32) or v_mfma_f32_32x32x16_f16 (fp16 operands). K advances in steps of
// BK elements (64 bytes of operand per row). Operand tiles are staged through
// LDS as [row][k] with k contiguous, double buffered: the global loads of
// tile t+1 are issued before the MFMAs of tile t and written to the other
// LDS buffer afterwards, so one barrier per K step suffices.
//
// Lane/K mapping. For a 32-row block, lane l works on row l % 32 and on the
// K half (l / 32); it reads that half of the row (BK/2 contiguous elements)
// with two 16-byte LDS reads and feeds the MFMA steps from it. A and B use
// the same K assignment, so the contraction is exact whatever order the
// hardware sums its K lanes in. The accumulator of a 32 x 32 block holds, in
// lane l, column l % 32 and rows 8g + 4(l/32) + r for register 4g + r.
//
// Operand layouts are handled by the staging code: K-contiguous rows are
// loaded as 16-byte chunks; M/N-contiguous operands are loaded as 4 (rows)
// by KM (k) micro-blocks and transposed in registers before the LDS write.
#include "gemm.h"

#include "../../include/qblk.h"

namespace qblk {
namespace {

template <Prec P>
struct PT;
template <>
struct PT<Prec::F32> {
  using T = float;
  static constexpr int BK = 16;
  static constexpr int PAD = 4;
};
template <>
struct PT<Prec::F16> {
  using T = f16;
  static constexpr int BK = 32;
  static constexpr int PAD = 8;
};

__device__ __forceinline__ int seg_of(const Seg& s, int r) {
  int sg = 0;
  if (s.nseg > 1 && r >= s.start[1]) sg = 1;
  if (s.nseg > 2 && r >= s.start[2]) sg = 2;
  return sg;
}

__device__ __forceinline__ const float* seg_row_f32(const Seg& s, int64_t ld, int r) {
  const int sg = seg_of(s, r);
  return (const float*)s.p[sg] + (int64_t)(r - s.start[sg]) * ld;
}

__device__ __forceinline__ const f16* seg_row_f16(const Seg& s, int64_t ld, int r) {
  const int sg = seg_of(s, r);
  return (const f16*)s.p[sg] + (int64_t)(r - s.start[sg]) * ld;
}

__device__ __forceinline__ float4 ld4_f16(const f16* p) {
  const half4 h = *(const half4*)p;
  return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
}

// Four NF4 elements at flat index e (a multiple of 4) of one segment.
__device__ __forceinline__ float4 ld4_nf4(const uint8_t* codes, const float* scales, int64_t e,
                                          const float* lv) {
  const uint16_t c = *(const uint16_t*)(codes + (e >> 1));
  const float a = scales[e >> 6];
  return make_float4(lv[c & 15] * a, lv[(c >> 4) & 15] * a, lv[(c >> 8) & 15] * a,
                     lv[(c >> 12) & 15] * a);
}

template <typename T>
__device__ __forceinline__ void st4(T* p, float4 v);
template <>
__device__ __forceinline__ void st4<float>(float* p, float4 v) {
  *(float4*)p = v;
}
template <>
__device__ __forceinline__ void st4<f16>(f16* p, float4 v) {
  *(half4*)p = to_half4(v);
}

// ------------------------------------------------------------- staging

// R x BK tile from K-contiguous storage rows.
template <int R, int BK, int NT>
struct KRows {
  static constexpr int CPR = BK / 4;
  static constexpr int CPT = (R * CPR) / NT;
  static_assert(CPT >= 1 && (R * CPR) % NT == 0, "tile/threads mismatch");
  float4 v[CPT];

  template <class Fetch>
  __device__ __forceinline__ void load(Fetch f, int row0, int nrows, int k0, int K, int tid) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + j * NT, r = c / CPR, kc = c % CPR;
      const int gr = row0 + r, gk = k0 + kc * 4;
      v[j] = (gr < nrows && gk < K) ? f(gr, gk) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  template <typename T, int PITCH>
  __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + j * NT, r = c / CPR, kc = c % CPR;
      st4<T>(s + r * PITCH + kc * 4, v[j]);
    }
  }
};

// BK x R tile from storage whose rows are k and whose columns are the R
// tile rows (M- or N-contiguous); written to LDS transposed as [R][BK].
template <int R, int BK, int NT>
struct KCols {
  static constexpr int QUADS = R / 4;
  static constexpr int KM = (BK * R) / (4 * NT);
  static_assert(KM >= 1 && NT % QUADS == 0 && (NT / QUADS) * KM == BK, "tile/threads mismatch");
  float4 v[KM];

  template <class Fetch>
  __device__ __forceinline__ void load(Fetch f, int row0, int nrows, int k0, int K, int tid) {
    const int rq = tid % QUADS, kb = tid / QUADS;
    const int gr = row0 + rq * 4;
#pragma unroll
    for (int kk = 0; kk < KM; ++kk) {
      const int gk = k0 + kb * KM + kk;
      v[kk] = (gr < nrows && gk < K) ? f(gk, gr) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  template <typename T, int PITCH>
  __device__ __forceinline__ void store(T* s, int tid) const {
    const int rq = tid % QUADS, kb = tid / QUADS;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      T* dst = s + (rq * 4 + q) * PITCH + kb * KM;
#pragma unroll
      for (int kk = 0; kk < KM; ++kk) {
        const float x = q == 0 ? v[kk].x : q == 1 ? v[kk].y : q == 2 ? v[kk].z : v[kk].w;
        dst[kk] = (T)x;
      }
    }
  }
};

// ----------------------------------------------------------- MFMA core

template <Prec P, int TM, int TN>
struct Core;

template <int TM, int TN>
struct Core<Prec::F32, TM, TN> {
  template <int PITCH>
  static __device__ __forceinline__ void run(const float* sA, const float* sB, int lane,
                                             floatx16 (&acc)[TM][TN]) {
    const int i = lane & 31, kh = lane >> 5;
    float a[TM][8], b[TN][8];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const float* p = sA + (t * 32 + i) * PITCH + kh * 8;
      const float4 x0 = *(const float4*)p, x1 = *(const float4*)(p + 4);
      a[t][0] = x0.x; a[t][1] = x0.y; a[t][2] = x0.z; a[t][3] = x0.w;
      a[t][4] = x1.x; a[t][5] = x1.y; a[t][6] = x1.z; a[t][7] = x1.w;
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const float* p = sB + (t * 32 + i) * PITCH + kh * 8;
      const float4 x0 = *(const float4*)p, x1 = *(const float4*)(p + 4);
      b[t][0] = x0.x; b[t][1] = x0.y; b[t][2] = x0.z; b[t][3] = x0.w;
      b[t][4] = x1.x; b[t][5] = x1.y; b[t][6] = x1.z; b[t][7] = x1.w;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[tm][s], b[tn][s], acc[tm][tn], 0, 0, 0);
  }
};

template <int TM, int TN>
struct Core<Prec::F16, TM, TN> {
  template <int PITCH>
  static __device__ __forceinline__ void run(const f16* sA, const f16* sB, int lane,
                                             floatx16 (&acc)[TM][TN]) {
    const int i = lane & 31, kh = lane >> 5;
    half8 a[TM][2], b[TN][2];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const f16* p = sA + (t * 32 + i) * PITCH + kh * 16;
      a[t][0] = *(const half8*)p;
      a[t][1] = *(const half8*)(p + 8);
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const f16* p = sB + (t * 32 + i) * PITCH + kh * 16;
      b[t][0] = *(const half8*)p;
      b[t][1] = *(const half8*)(p + 8);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[tm][s], b[tn][s], acc[tm][tn], 0, 0, 0);
  }
};

// ------------------------------------------------------------- kernel

template <Prec P, Layout L, Src AS, Src BS, bool EXT, int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(const GemmDesc d) {
  using T = typename PT<P>::T;
  constexpr int BK = PT<P>::BK, PITCH = BK + PT<P>::PAD;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32, NT = WM * WN * 64;
  constexpr bool A_KROWS = (L != Layout::TN);
  constexpr bool B_KROWS = (L == Layout::NT);

  __shared__ __attribute__((aligned(16))) T sA[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) T sB[2][BN * PITCH];
  __shared__ float s_lv[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  if constexpr (BS == Src::NF4) {
    if (tid < 16) s_lv[tid] = d.nf4.levels[tid];
    __syncthreads();
  }

  using ATile = typename std::conditional<A_KROWS, KRows<BM, BK, NT>, KCols<BM, BK, NT>>::type;
  using BTile = typename std::conditional<B_KROWS, KRows<BN, BK, NT>, KCols<BN, BK, NT>>::type;
  ATile ta;
  BTile tb;

  const int nkt_base = (d.K + BK - 1) / BK;
  const int nkt = nkt_base + (EXT ? (d.ext.kext + BK - 1) / BK : 0);

  // Loads of K tile kt into registers.
  auto fetch = [&](int kt) {
    if (!EXT || kt < nkt_base) {
      const int k0 = kt * BK;
      // A operand
      if constexpr (A_KROWS) {
        ta.load([&](int r, int k) -> float4 {
                  if constexpr (AS == Src::F16)
                    return ld4_f16((const f16*)d.a + (int64_t)r * d.lda + k);
                  else
                    return *(const float4*)((const float*)d.a + (int64_t)r * d.lda + k);
                },
                m0, d.M, k0, d.K, tid);
      } else {
        ta.load([&](int k, int r) -> float4 {
                  if constexpr (AS == Src::F16)
                    return ld4_f16((const f16*)d.a + (int64_t)k * d.lda + r);
                  else
                    return *(const float4*)((const float*)d.a + (int64_t)k * d.lda + r);
                },
                m0, d.M, k0, d.K, tid);
      }
      // B operand
      if constexpr (B_KROWS) {
        tb.load([&](int n, int k) -> float4 {
                  if constexpr (BS == Src::NF4) {
                    const int sg = seg_of(d.b, n);
                    const int64_t e = (int64_t)(n - d.b.start[sg]) * d.ldb + k;
                    return ld4_nf4(d.nf4.codes[sg], d.nf4.scales[sg], e, s_lv);
                  } else if constexpr (BS == Src::F16) {
                    return ld4_f16(seg_row_f16(d.b, d.ldb, n) + k);
                  } else {
                    return *(const float4*)(seg_row_f32(d.b, d.ldb, n) + k);
                  }
                },
                n0, d.N, k0, d.K, tid);
      } else {
        tb.load([&](int k, int n) -> float4 {
                  if constexpr (BS == Src::NF4) {
                    const int sg = seg_of(d.b, k);
                    const int64_t e = (int64_t)(k - d.b.start[sg]) * d.ldb + n;
                    return ld4_nf4(d.nf4.codes[sg], d.nf4.scales[sg], e, s_lv);
                  } else if constexpr (BS == Src::F16) {
                    return ld4_f16(seg_row_f16(d.b, d.ldb, k) + n);
                  } else {
                    return *(const float4*)(seg_row_f32(d.b, d.ldb, k) + n);
                  }
                },
                n0, d.N, k0, d.K, tid);
      }
    } else if constexpr (EXT) {
      const int k0 = (kt - nkt_base) * BK;
      const KExt& x = d.ext;
      if constexpr (A_KROWS) {
        ta.load([&](int r, int k) -> float4 {
                  float4 v = *(const float4*)(x.a + (int64_t)r * x.lda + k);
                  v.x *= x.a_scale; v.y *= x.a_scale; v.z *= x.a_scale; v.w *= x.a_scale;
                  return v;
                },
                m0, d.M, k0, x.kext, tid);
      }
      if constexpr (B_KROWS) {
        // NT: B_ext row n, ext columns k..k+3, block diagonal over B segments
        tb.load([&](int n, int k) -> float4 {
                  if (x.blockdiag > 0) {
                    const int sg = seg_of(d.b, n);
                    const int lo = sg * x.blockdiag;
                    if (k < lo || k >= lo + x.blockdiag) return make_float4(0.f, 0.f, 0.f, 0.f);
                    return *(const float4*)(x.b[sg] + (int64_t)(n - d.b.start[sg]) * x.ldb + (k - lo));
                  }
                  return *(const float4*)(x.b[0] + (int64_t)n * x.ldb + k);
                },
                n0, d.N, k0, x.kext, tid);
      } else {
        // NN: B_ext rows are ext columns k, stacked in groups of blockdiag
        tb.load([&](int k, int n) -> float4 {
                  if (x.blockdiag > 0) {
                    const int sg = k / x.blockdiag;
                    return *(const float4*)(x.b[sg] + (int64_t)(k - sg * x.blockdiag) * x.ldb + n);
                  }
                  return *(const float4*)(x.b[0] + (int64_t)k * x.ldb + n);
                },
                n0, d.N, k0, x.kext, tid);
      }
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  fetch(0);
  ta.template store<T, PITCH>(sA[0], tid);
  tb.template store<T, PITCH>(sB[0], tid);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) fetch(kt + 1);
    Core<P, TM, TN>::template run<PITCH>(sA[cur] + wm * TM * 32 * PITCH,
                                         sB[cur] + wn * TN * 32 * PITCH, lane, acc);
    if (kt + 1 < nkt) {
      ta.template store<T, PITCH>(sA[cur ^ 1], tid);
      tb.template store<T, PITCH>(sB[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue: lane holds column n0 + wn*TN*32 + tn*32 + (lane % 32) and rows
  // m0 + wm*TM*32 + tm*32 + 8g + 4(lane/32) + r.
  const int i = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int col = n0 + wn * TN * 32 + tn * 32 + i;
      if (col >= d.N) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * TM * 32 + tm * 32 + 8 * g + 4 * kh + r;
          if (row >= d.M) continue;
          const int sg = seg_of(d.c, row);
          int ccol = col;
          if (d.c_cols_blockdiag > 0) {
            const int lo = sg * d.c_cols_blockdiag;
            if (col < lo || col >= lo + d.c_cols_blockdiag) continue;
            ccol = col - lo;
          }
          float* cp = (float*)d.c.p[sg] + (int64_t)(row - d.c.start[sg]) * d.ldc + ccol;
          float v = d.alpha * acc[tm][tn][4 * g + r];
          if (d.r) v += d.r[(int64_t)row * d.ldr + col];
          if (d.accumulate) v += *cp;
          *cp = v;
        }
      }
    }
  }
}

template <Prec P, Layout L, Src AS, Src BS, bool EXT>
int launch(const GemmDesc& d, hipStream_t st) {
  constexpr int WM = 2, WN = 2, TM = 2, TN = 2;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  dim3 grid((unsigned)ceil_div(d.N, BN), (unsigned)ceil_div(d.M, BM));
  hipLaunchKernelGGL((gemm_kernel<P, L, AS, BS, EXT, WM, WN, TM, TN>), grid, dim3(WM * WN * 64), 0,
                     st, d);
  return check_launch("gemm_kernel");
}

template <Prec P, Layout L>
int dispatch_src(const GemmDesc& d, hipStream_t st) {
  const bool ext = d.ext.kext > 0;
  if (d.b_src == Src::NF4) {
    if constexpr (L == Layout::TN) {
      return fail(QBLK_EUNSUPPORTED, "gemm: NF4 operand not supported for TN");
    } else {
      if (d.a_src != Src::F32) return fail(QBLK_EUNSUPPORTED, "gemm: NF4 B needs fp32 A");
      return ext ? launch<P, L, Src::F32, Src::NF4, true>(d, st)
                 : launch<P, L, Src::F32, Src::NF4, false>(d, st);
    }
  }
  if (ext) {
    if constexpr (L == Layout::TN) {
      return fail(QBLK_EUNSUPPORTED, "gemm: K extension not supported for TN");
    } else {
      if (d.a_src != Src::F32 || d.b_src != Src::F32)
        return fail(QBLK_EUNSUPPORTED, "gemm: K extension needs fp32 operands");
      return launch<P, L, Src::F32, Src::F32, true>(d, st);
    }
  }
  if (d.a_src == Src::F32 && d.b_src == Src::F32) return launch<P, L, Src::F32, Src::F32, false>(d, st);
  if (d.a_src == Src::F16 && d.b_src == Src::F32) return launch<P, L, Src::F16, Src::F32, false>(d, st);
  if (d.a_src == Src::F32 && d.b_src == Src::F16) return launch<P, L, Src::F32, Src::F16, false>(d, st);
  if (d.a_src == Src::F16 && d.b_src == Src::F16) return launch<P, L, Src::F16, Src::F16, false>(d, st);
  return fail(QBLK_EUNSUPPORTED, "gemm: operand source combination");
}

}  // namespace

int gemm(const GemmDesc& d, hipStream_t st) {
  if (d.M <= 0 || d.N <= 0 || d.K < 0) return fail(QBLK_EINVAL, "gemm: bad shape %d x %d x %d", d.M, d.N, d.K);
  if (d.K == 0 && d.ext.kext == 0) return fail(QBLK_EINVAL, "gemm: empty contraction");
  // Contiguous dimensions are read 4 elements at a time.
  const bool a_k = d.layout != Layout::TN;
  if ((a_k ? d.K : d.M) % 4 != 0) return fail(QBLK_EINVAL, "gemm: A contiguous dim must be a multiple of 4");
  if ((d.layout == Layout::NT ? d.K : d.N) % 4 != 0)
    return fail(QBLK_EINVAL, "gemm: B contiguous dim must be a multiple of 4");
  if (d.ext.kext % 4 != 0) return fail(QBLK_EINVAL, "gemm: K extension must be a multiple of 4");
  if (d.prec == Prec::F32) {
    if (d.b_src == Src::NF4) return fail(QBLK_EUNSUPPORTED, "gemm: NF4 needs fp16 operands");
    switch (d.layout) {
      case Layout::NT: return dispatch_src<Prec::F32, Layout::NT>(d, st);
      case Layout::NN: return dispatch_src<Prec::F32, Layout::NN>(d, st);
      case Layout::TN: return dispatch_src<Prec::F32, Layout::TN>(d, st);
    }
  } else {
    switch (d.layout) {
      case Layout::NT: return dispatch_src<Prec::F16, Layout::NT>(d, st);
      case Layout::NN: return dispatch_src<Prec::F16, Layout::NN>(d, st);
      case Layout::TN: return dispatch_src<Prec::F16, Layout::TN>(d, st);
    }
  }
  return fail(QBLK_EINVAL, "gemm: bad layout");
}

}  // namespace qblk
