// MFMA GEMM engine for gfx950: every projection of the decoder block, its
// backward (dX and dW), the LM head, and the NF4-dequant + LoRA variants.
//
// Tiling. A workgroup of 2 x 2 waves computes a BM x BN tile of C; each wave
// owns TM x TN blocks of 32 x 32 accumulated by v_mfma_f32_32x32x2_f32 (fp32)
// or v_mfma_f32_32x32x16_f16 (fp16 operands). K advances in tiles of BK
// elements. Operand tiles are staged through LDS as [row][k], k contiguous,
// with 16 bytes of padding per row (conflict-free 16-byte reads), double
// buffered: the global loads of tile t+1 are issued before the MFMAs of tile
// t and written to the other buffer afterwards (one barrier per tile).
//
// Staging. Every thread's share of a tile is fixed for the whole launch, so
// its row pointers (K-contiguous operands) or its column offset
// (M/N-contiguous operands) are computed once; a K step is then one 16-byte
// load per chunk. fp16 operands are copied to LDS as they are; fp32 operands
// are rounded to fp16 (nearest even) on the way when the contraction is
// fp16; NF4 codes are decoded (level * block scale) and rounded to fp16. An
// M/N-contiguous operand is transposed in registers: a thread loads KM
// consecutive k rows of one 16-byte column group and writes each column as
// one contiguous run of KM values.
//
// Lane/K mapping. For a 32-row block, lane l works on row l % 32 and on the
// K half (l / 32) of the tile, read as contiguous 16-byte chunks. A and B
// use the same K assignment, so the contraction is exact whatever order the
// hardware sums its K lanes in. The accumulator of a 32 x 32 block holds, in
// lane l, column l % 32 and rows 8g + 4(l/32) + r for register 4g + r.
//
// Skinny problems (few output tiles, long K) are split along K over more
// workgroups; the partial tiles go to a caller-provided workspace and a
// second kernel adds them in a fixed order (deterministic) and applies the
// epilogue. Workgroup ids are remapped so that tiles sharing a B tile run on
// the same XCD at the same time (one L2 per XCD).
#include "gemm.h"

#include <type_traits>

#include "../../include/qblk.h"

namespace qblk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <Prec P>
struct PT;
template <>
struct PT<Prec::F32> {
  using T = float;
  static constexpr int BK = 32;
};
template <>
struct PT<Prec::F16> {
  using T = f16;
  static constexpr int BK = 64;
};

template <Src S>
struct SrcT {
  using type = float;
};
template <>
struct SrcT<Src::F16> {
  using type = f16;
};

__device__ __forceinline__ int seg_of(const Seg& s, int r) {
  int sg = 0;
  if (s.nseg > 1 && r >= s.start[1]) sg = 1;
  if (s.nseg > 2 && r >= s.start[2]) sg = 2;
  return sg;
}

__device__ __forceinline__ float4 as_f4(u32x4 v) { return __builtin_bit_cast(float4, v); }
__device__ __forceinline__ half8 as_h8(u32x4 v) { return __builtin_bit_cast(half8, v); }

template <typename T, int N>
__device__ __forceinline__ void store_run(T* dst, const T (&x)[N]) {
  constexpr int BYTES = N * (int)sizeof(T);
  if constexpr (BYTES % 16 == 0) {
#pragma unroll
    for (int c = 0; c < BYTES / 16; ++c) {
      u32x4 w;
      __builtin_memcpy(&w, &x[c * 16 / sizeof(T)], 16);
      *(u32x4*)((char*)dst + 16 * c) = w;
    }
  } else if constexpr (BYTES == 8) {
    uint2 w;
    __builtin_memcpy(&w, &x[0], 8);
    *(uint2*)dst = w;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = x[i];
  }
}

// ------------------------------------------------------------- loaders

// R x BK tile from K-contiguous storage rows of fp32 or fp16 elements.
// Thread t owns chunks c = t + j NT (j < CPT): all at the same K offset kc,
// on rows spaced RSTEP apart.
template <int R, int BK, int NT, typename S>
struct RowLoader {
  static constexpr int EPC = 16 / sizeof(S);
  static constexpr int CPR = BK / EPC;
  static_assert(BK % EPC == 0 && NT % CPR == 0, "tile/threads mismatch");
  static constexpr int RSTEP = NT / CPR;
  static_assert(R % RSTEP == 0, "tile/threads mismatch");
  static constexpr int CPT = R / RSTEP;
  const S* p[CPT];
  int kc;
  struct Buf {
    u32x4 v[CPT];
  };

  template <class RowPtr>
  __device__ __forceinline__ void init(RowPtr rp, int row0, int nrows, int tid) {
    kc = (tid % CPR) * EPC;
    const int r0 = row0 + tid / CPR;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int r = r0 + j * RSTEP;
      p[j] = r < nrows ? rp(r) + kc : nullptr;
    }
  }
  __device__ __forceinline__ void load(Buf& b, int k0, int kend) const {
    const bool kin = k0 + kc < kend;
#pragma unroll
    for (int j = 0; j < CPT; ++j) b.v[j] = (kin && p[j]) ? *(const u32x4*)(p[j] + k0) : u32x4{0u, 0u, 0u, 0u};
  }
  template <typename T, int PITCH>
  __device__ __forceinline__ void store(const Buf& b, T* s, int tid, float scale = 1.f) const {
    const int r0 = tid / CPR;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      T* dst = s + (r0 + j * RSTEP) * PITCH + kc;
      if constexpr (sizeof(S) == sizeof(T)) {
        if constexpr (sizeof(S) == 4) {
          float4 f = as_f4(b.v[j]);
          f.x *= scale; f.y *= scale; f.z *= scale; f.w *= scale;
          *(float4*)dst = f;
        } else {
          *(u32x4*)dst = b.v[j];
        }
      } else {  // fp32 storage, fp16 contraction
        float4 f = as_f4(b.v[j]);
        f.x *= scale; f.y *= scale; f.z *= scale; f.w *= scale;
        *(half4*)dst = to_half4(f);
      }
    }
  }
};

// BK x R tile from storage whose rows are k and whose columns are the tile
// rows (M- or N-contiguous), written to LDS as [R][BK]. Thread t owns the
// column group cl = (t % GROUPS) CW (one 16-byte load per k row) and the k
// rows kb .. kb + KM - 1.
template <int R, int BK, int NT, typename S>
struct ColLoader {
  static constexpr int CW = 16 / sizeof(S);
  static constexpr int GROUPS = R / CW;
  static_assert(R % CW == 0 && NT % GROUPS == 0, "tile/threads mismatch");
  static constexpr int KG = NT / GROUPS;
  static_assert(BK % KG == 0, "tile/threads mismatch");
  static constexpr int KM = BK / KG;
  int cl, kb, col;
  bool cvalid;
  struct Buf {
    u32x4 v[KM];
  };

  __device__ __forceinline__ void init(int row0, int nrows, int tid) {
    cl = (tid % GROUPS) * CW;
    kb = (tid / GROUPS) * KM;
    col = row0 + cl;
    cvalid = col < nrows;
  }
  // Storage row k of segmented storage sg (k rows stacked over the segments).
  __device__ __forceinline__ void load(Buf& b, const Seg& sg, int64_t ld, int k0, int kend) const {
    const int kf = k0 + kb;
    const S* base = nullptr;
    {
      const int s = seg_of(sg, kf);
      const int send = (s + 1 < sg.nseg) ? sg.start[s + 1] : 0x7fffffff;
      if (kf + KM <= send) base = (const S*)sg.p[s] + (int64_t)(kf - sg.start[s]) * ld + col;
    }
#pragma unroll
    for (int kk = 0; kk < KM; ++kk) {
      const int k = kf + kk;
      const bool ok = cvalid && k < kend;
      if (!ok) {
        b.v[kk] = u32x4{0u, 0u, 0u, 0u};
      } else if (base) {
        b.v[kk] = *(const u32x4*)(base + (int64_t)kk * ld);
      } else {
        const int s = seg_of(sg, k);
        b.v[kk] = *(const u32x4*)((const S*)sg.p[s] + (int64_t)(k - sg.start[s]) * ld + col);
      }
    }
  }
  template <typename T, int PITCH>
  __device__ __forceinline__ void store(const Buf& b, T* s, int tid) const {
    (void)tid;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      T run[KM];
#pragma unroll
      for (int kk = 0; kk < KM; ++kk) {
        if constexpr (sizeof(S) == 4) {
          const float4 f = as_f4(b.v[kk]);
          run[kk] = (T)(c == 0 ? f.x : c == 1 ? f.y : c == 2 ? f.z : f.w);
        } else {
          run[kk] = (T)as_h8(b.v[kk])[c];
        }
      }
      store_run<T, KM>(s + (cl + c) * PITCH + kb, run);
    }
  }
};

// NF4 B operand, K-contiguous rows (forward y = x W~^T): chunks of 8
// elements (4 bytes of codes) and the scale of their 64-element block.
template <int R, int BK, int NT>
struct Nf4RowLoader {
  static constexpr int EPC = 8, CPR = BK / EPC;
  static_assert(BK % EPC == 0 && NT % CPR == 0, "tile/threads mismatch");
  static constexpr int RSTEP = NT / CPR;
  static constexpr int CPT = R / RSTEP;
  const uint8_t* cp[CPT];
  const float* sp[CPT];
  int64_t e0[CPT];
  int kc;
  struct Buf {
    uint32_t code[CPT];
    float sc[CPT];
  };

  __device__ __forceinline__ void init(const GemmDesc& d, int row0, int tid) {
    kc = (tid % CPR) * EPC;
    const int r0 = row0 + tid / CPR;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int n = r0 + j * RSTEP;
      if (n < d.N) {
        const int sg = seg_of(d.b, n);
        e0[j] = (int64_t)(n - d.b.start[sg]) * d.ldb + kc;
        cp[j] = d.nf4.codes[sg];
        sp[j] = d.nf4.scales[sg];
      } else {
        cp[j] = nullptr;
        sp[j] = nullptr;
        e0[j] = 0;
      }
    }
  }
  __device__ __forceinline__ void load(Buf& b, int k0, int kend) const {
    const bool kin = k0 + kc < kend;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      if (kin && cp[j]) {
        const int64_t e = e0[j] + k0;
        b.code[j] = *(const uint32_t*)(cp[j] + (e >> 1));
        b.sc[j] = sp[j][e >> 6];
      } else {
        b.code[j] = 0;
        b.sc[j] = 0.f;
      }
    }
  }
  template <typename T, int PITCH>
  __device__ __forceinline__ void store(const Buf& b, T* s, int tid, const float* lv) const {
    const int r0 = tid / CPR;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      half8 h;
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = (f16)(lv[(b.code[j] >> (4 * i)) & 15] * b.sc[j]);
      *(half8*)(s + (r0 + j * RSTEP) * PITCH + kc) = h;
    }
  }
};

// NF4 B operand stored [K, N] with N contiguous (backward dX = dY W~):
// column groups of 8 (4 bytes of codes per k row).
template <int R, int BK, int NT>
struct Nf4ColLoader {
  static constexpr int CW = 8, GROUPS = R / CW;
  static_assert(R % CW == 0 && NT % GROUPS == 0, "tile/threads mismatch");
  static constexpr int KG = NT / GROUPS;
  static constexpr int KM = BK / KG;
  int cl, kb, col;
  bool cvalid;
  struct Buf {
    uint32_t code[KM];
    float sc[KM];
  };

  __device__ __forceinline__ void init(int row0, int nrows, int tid) {
    cl = (tid % GROUPS) * CW;
    kb = (tid / GROUPS) * KM;
    col = row0 + cl;
    cvalid = col < nrows;
  }
  __device__ __forceinline__ void load(Buf& b, const GemmDesc& d, int k0, int kend) const {
#pragma unroll
    for (int kk = 0; kk < KM; ++kk) {
      const int k = k0 + kb + kk;
      if (cvalid && k < kend) {
        const int s = seg_of(d.b, k);
        const int64_t e = (int64_t)(k - d.b.start[s]) * d.ldb + col;
        b.code[kk] = *(const uint32_t*)(d.nf4.codes[s] + (e >> 1));
        b.sc[kk] = d.nf4.scales[s][e >> 6];
      } else {
        b.code[kk] = 0;
        b.sc[kk] = 0.f;
      }
    }
  }
  template <typename T, int PITCH>
  __device__ __forceinline__ void store(const Buf& b, T* s, int tid, const float* lv) const {
    (void)tid;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      T run[KM];
#pragma unroll
      for (int kk = 0; kk < KM; ++kk) run[kk] = (T)(lv[(b.code[kk] >> (4 * c)) & 15] * b.sc[kk]);
      store_run<T, KM>(s + (cl + c) * PITCH + kb, run);
    }
  }
};

// LoRA K-extension B operand for NT: row n of B-segment s sees ext columns
// [s*bd, (s+1)*bd) of B_ext[s] (bd = blockdiag; bd = 0: one plain matrix).
template <int R, int BK, int NT>
struct ExtRowLoaderNT {
  static constexpr int EPC = 4, CPR = BK / EPC, RSTEP = NT / CPR, CPT = R / RSTEP;
  const float* p[CPT];
  int lo[CPT], hi[CPT];
  int kc;
  struct Buf {
    float4 v[CPT];
  };
  __device__ __forceinline__ void init(const GemmDesc& d, int row0, int tid) {
    const KExt& x = d.ext;
    kc = (tid % CPR) * EPC;
    const int r0 = row0 + tid / CPR;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int n = r0 + j * RSTEP;
      p[j] = nullptr;
      lo[j] = hi[j] = 0;
      if (n < d.N) {
        if (x.blockdiag > 0) {
          const int sg = seg_of(d.b, n);
          lo[j] = sg * x.blockdiag;
          hi[j] = lo[j] + x.blockdiag;
          p[j] = x.b[sg] + (int64_t)(n - d.b.start[sg]) * x.ldb - lo[j];
        } else {
          lo[j] = 0;
          hi[j] = x.kext;
          p[j] = x.b[0] + (int64_t)n * x.ldb;
        }
      }
    }
  }
  __device__ __forceinline__ void load(Buf& b, int k0) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int k = k0 + kc;
      b.v[j] = (p[j] && k >= lo[j] && k < hi[j]) ? *(const float4*)(p[j] + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  template <typename T, int PITCH>
  __device__ __forceinline__ void store(const Buf& b, T* s, int tid) const {
    const int r0 = tid / CPR;
#pragma unroll
    for (int j = 0; j < CPT; ++j) *(half4*)(s + (r0 + j * RSTEP) * PITCH + kc) = to_half4(b.v[j]);
  }
};

// LoRA K-extension B operand for NN: ext row k is row (k % bd) of B_ext[k / bd]
// (bd = 0: row k of one matrix), columns contiguous.
template <int R, int BK, int NT>
struct ExtColLoaderNN {
  using CL = ColLoader<R, BK, NT, float>;
  using Buf = typename CL::Buf;
  CL c;
  __device__ __forceinline__ void init(int row0, int nrows, int tid) { c.init(row0, nrows, tid); }
  __device__ __forceinline__ void load(Buf& b, const GemmDesc& d, int k0) const {
    const KExt& x = d.ext;
#pragma unroll
    for (int kk = 0; kk < CL::KM; ++kk) {
      const int k = k0 + c.kb + kk;
      if (c.cvalid && k < x.kext) {
        const float* row = x.blockdiag > 0 ? x.b[k / x.blockdiag] + (int64_t)(k % x.blockdiag) * x.ldb
                                           : x.b[0] + (int64_t)k * x.ldb;
        b.v[kk] = *(const u32x4*)(row + c.col);
      } else {
        b.v[kk] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  template <typename T, int PITCH>
  __device__ __forceinline__ void store(const Buf& b, T* s, int tid) const {
    c.template store<T, PITCH>(b, s, tid);
  }
};

// ----------------------------------------------------------- MFMA core
// One K tile of BK elements from LDS into the wave's TM x TN accumulators.
// Lane l reads, for each of its blocks, row (l % 32) and the K half (l / 32)
// of the tile: KH = BK/2 contiguous elements.

template <Prec P, int TM, int TN, int BK>
struct Core;

template <int TM, int TN, int BK>
struct Core<Prec::F32, TM, TN, BK> {
  static constexpr int KH = BK / 2;
  template <int PITCH>
  static __device__ __forceinline__ void run(const float* sA, const float* sB, int lane,
                                             floatx16 (&acc)[TM][TN]) {
    const int i = lane & 31, kh = lane >> 5;
#pragma unroll
    for (int q = 0; q < KH / 4; ++q) {
      float4 a[TM], b[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) a[t] = *(const float4*)(sA + (t * 32 + i) * PITCH + kh * KH + 4 * q);
#pragma unroll
      for (int t = 0; t < TN; ++t) b[t] = *(const float4*)(sB + (t * 32 + i) * PITCH + kh * KH + 4 * q);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[tm].x, b[tn].x, acc[tm][tn], 0, 0, 0);
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[tm].y, b[tn].y, acc[tm][tn], 0, 0, 0);
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[tm].z, b[tn].z, acc[tm][tn], 0, 0, 0);
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[tm].w, b[tn].w, acc[tm][tn], 0, 0, 0);
        }
    }
  }
};

template <int TM, int TN, int BK>
struct Core<Prec::F16, TM, TN, BK> {
  static constexpr int KH = BK / 2;
  template <int PITCH>
  static __device__ __forceinline__ void run(const f16* sA, const f16* sB, int lane,
                                             floatx16 (&acc)[TM][TN]) {
    const int i = lane & 31, kh = lane >> 5;
#pragma unroll
    for (int s = 0; s < KH / 8; ++s) {
      half8 a[TM], b[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) a[t] = *(const half8*)(sA + (t * 32 + i) * PITCH + kh * KH + 8 * s);
#pragma unroll
      for (int t = 0; t < TN; ++t) b[t] = *(const half8*)(sB + (t * 32 + i) * PITCH + kh * KH + 8 * s);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[tm], b[tn], acc[tm][tn], 0, 0, 0);
    }
  }
};

// ------------------------------------------------------------- kernel

struct Grid {
  int tiles_m, tiles_n, splits, kchunk;
  int vec = 0;    // 1: output rows (and partials, residual) take 16-byte stores
  int bn = 0;     // tile width (ping-pong kernel: 256 or 192)
  int nfast = 0;  // ping-pong kernel: N tiles fastest (consecutive workgroups share an A tile)
  int deep = 0;   // 128 x 128 tiles, one workgroup per CU: three A and three B stages
};

// Final value of C[row, col]: the row pointer `cp` already routed through
// the output segments; plus the residual and/or the old C.
__device__ __forceinline__ void put_out(const GemmDesc& d, float* cp, int row, int col, float acc) {
  float v = d.alpha * acc;
  if (d.r) v += d.r[(int64_t)row * d.ldr + col];
  if (d.accumulate) v += *cp;
  *cp = v;
}

// 16 bytes of the final output, with the nontemporal hint: the outputs are
// written once and read back, if at all, by a later kernel (measured faster
// for every product of the block, the weight gradients most).
__device__ __forceinline__ void store_c4(float4* cp, const float4 o) {
  __builtin_nontemporal_store(floatx4{o.x, o.y, o.z, o.w}, (floatx4*)cp);
}

// Output row pointer (segment routing), or nullptr when the row is out of
// range; `lo` is the first column this row keeps (diagonal-block mode).
// The segment is picked by arithmetic on the scalar kernel arguments (its
// base as an offset from segment 0's, its first row as a sum), not by
// d.c.p[sg]: with a per-lane sg that is a vector load from the argument
// segment, and its wait (vmcnt counts stores too) would stall every
// epilogue iteration until all of the tile's earlier stores had completed.
// The offsets keep the pointer derived from a global one, so the stores
// stay global stores.
__device__ __forceinline__ float* out_row(const GemmDesc& d, int row, int& lo) {
  if (row >= d.M) return nullptr;
  const int in1 = d.c.nseg > 1 && row >= d.c.start[1];
  const int in2 = d.c.nseg > 2 && row >= d.c.start[2];
  const uintptr_t b0 = (uintptr_t)d.c.p[0];
  const int64_t o1 = (int64_t)((uintptr_t)d.c.p[1] - b0), o2 = (int64_t)((uintptr_t)d.c.p[2] - b0);
  const int64_t off = in2 * o2 + (in1 - in2) * o1;
  const int start = in1 * d.c.start[1] + in2 * (d.c.start[2] - d.c.start[1]);
  lo = d.c_cols_blockdiag > 0 ? (in1 + in2) * d.c_cols_blockdiag : 0;
  return (float*)((char*)d.c.p[0] + off) + (int64_t)(row - start) * d.ldc;
}

// Fast path of one epilogue pass over rows rowb .. rowb + R - 1 and the
// wave's 4 CPR columns from col0, when they all lie inside C (and inside one
// output segment), rows are 16-byte aligned and no diagonal-block mode is
// set. Lane (lr, lc) = (lane / CPR, lane % CPR) takes column col0 + 4 lc of
// rows lr, lr + RS, ... (RS = 64 / CPR rows per step; when CPR does not
// divide 64 the last 64 - RS CPR lanes idle): its pointers are formed once
// per pass and then advance by a constant stride, the staged values sit at
// fixed LDS offsets, so each store costs a handful of instructions. `part`
// (split-K partial of this tile's split) receives the raw sums instead.
// Returns false when the pass needs the general path.
template <int R, int CPR, class Slot>
__device__ __forceinline__ bool epi_pass_fast(const GemmDesc& d, bool vec, float* part, int rowb, int col0,
                                              const float* ep, Slot eslot, int lane) {
  constexpr int RS = 64 / CPR;  // rows per step
  static_assert(RS >= 1 && R % RS == 0, "rows per pass");
  if (!vec || d.c_cols_blockdiag > 0 || rowb + R > d.M || col0 + 4 * CPR > d.N) return false;
  const int last = rowb + R - 1;
  if (!part && d.c.nseg > 1 && (rowb >= d.c.start[1]) != (last >= d.c.start[1])) return false;
  if (!part && d.c.nseg > 2 && (rowb >= d.c.start[2]) != (last >= d.c.start[2])) return false;
  // every test above is uniform over the wave: from here on the pass is done
  if (lane >= RS * CPR) return true;  // idle lanes
  const int lr = lane / CPR, lc = lane % CPR;
  const int64_t col = col0 + 4 * lc;
  if (part) {
    float* pp = part + (int64_t)(rowb + lr) * d.N + col;
    const int64_t ps = (int64_t)RS * d.N;
#pragma unroll
    for (int q = 0; q < R / RS; ++q) *(float4*)(pp + q * ps) = *(const float4*)(ep + eslot(lr + q * RS, lc));
    return true;
  }
  int lo = 0;
  float* const cp = out_row(d, rowb + lr, lo) + col;
  const int64_t cs = (int64_t)RS * d.ldc;
  const float* const rp = d.r ? d.r + (int64_t)(rowb + lr) * d.ldr + col : nullptr;
  const int64_t rs = (int64_t)RS * d.ldr;
  f16* const hp = d.c16 ? d.c16 + (int64_t)(rowb + lr) * d.ldc16 + col : nullptr;
  const int64_t hs = (int64_t)RS * d.ldc16;
#pragma unroll
  for (int q = 0; q < R / RS; ++q) {
    const float4 v = *(const float4*)(ep + eslot(lr + q * RS, lc));
    float4 o = make_float4(d.alpha * v.x, d.alpha * v.y, d.alpha * v.z, d.alpha * v.w);
    if (rp) {
      const float4 rv = *(const float4*)(rp + q * rs);
      o.x += rv.x;
      o.y += rv.y;
      o.z += rv.z;
      o.w += rv.w;
    }
    if (d.accumulate) {
      const float4 cv = *(const float4*)(cp + q * cs);
      o.x += cv.x;
      o.y += cv.y;
      o.z += cv.z;
      o.w += cv.w;
    }
    store_c4((float4*)(cp + q * cs), o);
    if (hp) *(half4*)(hp + q * hs) = to_16x4(o, d.prec == Prec::BF16);
  }
  return true;
}

__device__ __forceinline__ void store_out(const GemmDesc& d, int row, int col, float acc) {
  int lo = 0;
  float* rp = out_row(d, row, lo);
  if (!rp) return;
  if (d.c_cols_blockdiag > 0 && (col < lo || col >= lo + d.c_cols_blockdiag)) return;
  put_out(d, rp + (col - lo), row, col, acc);
}

// C (or, with split-K, one partial of it) for one BM x BN tile and one K
// range. The linear workgroup id is remapped so that consecutive logical
// tiles (the M tiles that share a B tile) land on the same XCD (ids are
// dealt to the 8 XCDs round-robin) and are dispatched together.
template <Prec P, Layout L, Src AS, Src BS, bool EXT, int WM, int WN, int TM, int TN, int BK>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(const GemmDesc d, const Grid gd) {
  using T = typename PT<P>::T;
  using SA = typename SrcT<AS>::type;
  using SB = typename SrcT<BS>::type;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int PITCH = BK + PAD;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32, NT = WM * WN * 64;
  constexpr bool A_ROWS = (L != Layout::TN);
  constexpr bool B_ROWS = (L == Layout::NT);
  constexpr bool B_NF4 = (BS == Src::NF4);

  __shared__ __attribute__((aligned(16))) T sA[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) T sB[2][BN * PITCH];
  __shared__ float s_lv[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  const int total = gd.tiles_m * gd.tiles_n * gd.splits;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = total / 8, rem = total % 8;
  const int lt = xcd * per + min(xcd, rem) + slot;
  const int mt = lt % gd.tiles_m;
  const int nt = (lt / gd.tiles_m) % gd.tiles_n;
  const int sp = lt / (gd.tiles_m * gd.tiles_n);
  const int m0 = mt * BM, n0 = nt * BN;
  const int kb = sp * gd.kchunk;
  const int ke = min(d.K, kb + gd.kchunk);

  if constexpr (B_NF4) {
    if (tid < 16) s_lv[tid] = d.nf4.levels[tid];
    __syncthreads();
  }

  // ---- loaders (thread shares fixed for the launch)
  using ALoader = typename std::conditional<A_ROWS, RowLoader<BM, BK, NT, SA>, ColLoader<BM, BK, NT, SA>>::type;
  using BLoader = typename std::conditional<
      B_NF4, typename std::conditional<B_ROWS, Nf4RowLoader<BN, BK, NT>, Nf4ColLoader<BN, BK, NT>>::type,
      typename std::conditional<B_ROWS, RowLoader<BN, BK, NT, SB>, ColLoader<BN, BK, NT, SB>>::type>::type;
  ALoader la;
  BLoader lb;
  Seg aseg;
  if constexpr (A_ROWS) {
    la.init([&](int r) { return (const SA*)d.a + (int64_t)r * d.lda; }, m0, d.M, tid);
  } else {
    aseg = seg1(d.a, d.K);
    la.init(m0, d.M, tid);
  }
  if constexpr (B_NF4) {
    if constexpr (B_ROWS)
      lb.init(d, n0, tid);
    else
      lb.init(n0, d.N, tid);
  } else if constexpr (B_ROWS) {
    lb.init(
        [&](int n) {
          const int sg = seg_of(d.b, n);
          return (const SB*)d.b.p[sg] + (int64_t)(n - d.b.start[sg]) * d.ldb;
        },
        n0, d.N, tid);
  } else {
    lb.init(n0, d.N, tid);
  }

  // LoRA extension columns (fp32 sources), processed by split 0 after its
  // base K tiles.
  using EALoader = RowLoader<BM, BK, NT, float>;
  using EBLoader = typename std::conditional<B_ROWS, ExtRowLoaderNT<BN, BK, NT>, ExtColLoaderNN<BN, BK, NT>>::type;
  EALoader ea;
  EBLoader eb;
  if constexpr (EXT) {
    ea.init([&](int r) { return d.ext.a + (int64_t)r * d.ext.lda; }, m0, d.M, tid);
    if constexpr (B_ROWS)
      eb.init(d, n0, tid);
    else
      eb.init(n0, d.N, tid);
  }

  const int nkt_base = ke > kb ? (ke - kb + BK - 1) / BK : 0;
  const int nkt = nkt_base + ((EXT && sp == 0) ? (d.ext.kext + BK - 1) / BK : 0);

  // Register payload of one K tile.
  struct Regs {
    typename ALoader::Buf a;
    typename BLoader::Buf b;
  };
  Regs rg[1];
  // The LoRA extension is at most one K tile (checked on the host), so one
  // register set serves it.
  struct ExtRegs {
    typename EALoader::Buf a;
    typename EBLoader::Buf b;
  };
  ExtRegs er;

  auto fetch = [&](int kt, Regs& r) {
    if (!EXT || kt < nkt_base) {
      const int k0 = kb + kt * BK;
      if constexpr (A_ROWS)
        la.load(r.a, k0, ke);
      else
        la.load(r.a, aseg, d.lda, k0, ke);
      if constexpr (B_NF4) {
        if constexpr (B_ROWS)
          lb.load(r.b, k0, ke);
        else
          lb.load(r.b, d, k0, ke);
      } else if constexpr (B_ROWS) {
        lb.load(r.b, k0, ke);
      } else {
        lb.load(r.b, d.b, d.ldb, k0, ke);
      }
    } else if constexpr (EXT) {
      const int k0 = (kt - nkt_base) * BK;
      ea.load(er.a, k0, d.ext.kext);
      if constexpr (B_ROWS)
        eb.load(er.b, k0);
      else
        eb.load(er.b, d, k0);
    }
  };
  auto put = [&](int kt, int buf, const Regs& r) {
    if (!EXT || kt < nkt_base) {
      la.template store<T, PITCH>(r.a, sA[buf], tid);
      if constexpr (B_NF4)
        lb.template store<T, PITCH>(r.b, sB[buf], tid, s_lv);
      else
        lb.template store<T, PITCH>(r.b, sB[buf], tid);
    } else if constexpr (EXT) {
      ea.template store<T, PITCH>(er.a, sA[buf], tid, d.ext.a_scale);
      eb.template store<T, PITCH>(er.b, sB[buf], tid);
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  // Pipeline: the global loads of tile kt+1 are in flight while the MFMAs
  // of tile kt run; then they go to the other LDS buffer. (One register set
  // keeps two workgroups per CU resident, which hides more latency than a
  // second register set would.)
  if (nkt > 0) {
    fetch(0, rg[0]);
    put(0, 0, rg[0]);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) fetch(kt + 1, rg[0]);
    Core<P, TM, TN, BK>::template run<PITCH>(sA[cur] + wm * TM * 32 * PITCH, sB[cur] + wn * TN * 32 * PITCH,
                                             lane, acc);
    if (kt + 1 < nkt) put(kt + 1, cur ^ 1, rg[0]);
    __syncthreads();
  }

  // Epilogue: lane holds column n0 + wn*TN*32 + tn*32 + (lane % 32) and rows
  // m0 + wm*TM*32 + tm*32 + 8g + 4(lane/32) + r.
  const int i = lane & 31, kh = lane >> 5;
  if (gd.splits > 1) {
    float* part = d.ws + (int64_t)sp * d.M * d.N;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * TM * 32 + tm * 32 + 8 * g + 4 * kh + r;
          if (row >= d.M) continue;
          float* prow = part + (int64_t)row * d.N;
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            const int col = n0 + wn * TN * 32 + tn * 32 + i;
            if (col < d.N) prow[col] = acc[tm][tn][4 * g + r];
          }
        }
    return;
  }
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * TM * 32 + tm * 32 + 8 * g + 4 * kh + r;
        int lo = 0;
        float* rp = out_row(d, row, lo);
        if (!rp) continue;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int col = n0 + wn * TN * 32 + tn * 32 + i;
          if (col >= d.N) continue;
          if (d.c_cols_blockdiag > 0 && (col < lo || col >= lo + d.c_cols_blockdiag)) continue;
          put_out(d, rp + (col - lo), row, col, acc[tm][tn][4 * g + r]);
        }
      }
}

// --------------------------------------- fp16 fast path (direct LDS DMA)
//
// Both operands fp16 in storage, K a multiple of 64, any of the three
// layouts. Tiles move global -> LDS with global_load_lds_dwordx4 (16 bytes
// per lane straight into LDS: no registers, no conversion) into a ring of
// NS LDS stages, so the copies of the next NS-1 K tiles overlap the MFMAs
// of the current one. Each operand tile is a plain copy of its storage:
//
// * K-major (A of NT/NN, B of NT): BM rows x 64 halves, 128-byte rows;
//   16-byte chunks XOR-swizzled by (row >> 1) & 7, so the ds_read_b128 of
//   16 consecutive rows at one chunk hit 16 different bank groups.
// * MN-major (A of TN, B of NN/TN): 64 K-rows x BM halves; chunks swizzled
//   by (row & 3) << 2. The MFMA operand (8 consecutive K of one row m) is
//   gathered by two ds_read_b64_tr_b16: within each 16-lane group, output
//   lane j takes element k from the lane 4k + j/4 that read 4 consecutive
//   m at K-row k, so lane j ends up with 4 consecutive K of column j.
//
// Rows (or columns) past M or N read a clamped, valid address; their
// results are never stored.

// One LDS stage as its own __shared__ object: stages are distinct objects,
// so the compiler knows a copy into one cannot alias reads of another and
// adds no wait of its own between them.
template <int TAG, int ELEMS>
__device__ __forceinline__ f16* lds_stage() {
  __shared__ __attribute__((aligned(16))) f16 buf[ELEMS];
  return buf;
}

typedef short short4v __attribute__((ext_vector_type(4)));

// f(integral_constant<int, I>) for I in [B, E), unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// One operand of the DMA kernel: R rows of the tile (BM or BN), K-major or
// MN-major, BK = 64 or 32 K per stage, copied by NW waves.
template <int R, bool KMAJ, int NW, int BK_ = 64>
struct DmaOperand {
  static constexpr int BK = BK_;
  static_assert(BK == 64 || BK == 32, "K tile");
  static constexpr int J = R * BK / 512 / NW;  // 1 KB wave copies per stage per wave
  static_assert(J * 512 * NW == R * BK, "DMA split");
  // K-major rows: BK / 8 chunks of 16 bytes; the chunk swizzle puts 16
  // consecutive rows read at one chunk on 16 different bank groups.
  static constexpr int KCH = BK / 8;
  static __device__ __forceinline__ int ksw(int row) { return BK == 64 ? (row >> 1) & 7 : (row >> 2) & 3; }
  const f16* p[J];

  // Wave w's copy j fills the 1 KB at tile + 512 (NW j + w) halves.
  // K-major: 512 / BK rows of 2 BK bytes; MN-major: 1024 / (2R) K-rows x 2R bytes.
  __device__ __forceinline__ void init(const f16* base, int64_t ld, int r0, int rmax, int64_t kb, int lane, int w,
                                       const Seg* seg) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int blk = NW * j + w;
      if constexpr (KMAJ) {
        const int rsub = lane / KCH;
        const int row = (512 / BK) * blk + rsub;
        const int lc = (lane % KCH) ^ ksw(row);
        const int r = min(r0 + row, rmax - 1);
        if (seg) {
          const int sg = seg_of(*seg, r);
          p[j] = (const f16*)seg->p[sg] + (int64_t)(r - seg->start[sg]) * ld + kb + lc * 8;
        } else {
          p[j] = base + (int64_t)r * ld + kb + lc * 8;
        }
      } else {
        constexpr int CPR = R / 8;         // 16-byte chunks per K-row
        constexpr int RPI = 64 / CPR;      // K-rows per wave copy
        const int krow = blk * RPI + lane / CPR;
        const int lc = (lane % CPR) ^ ((krow & 3) << 2);
        const int col = min(r0 + lc * 8, rmax - 8);
        p[j] = base + (kb + krow) * ld + col;
      }
    }
  }
  // Copy j of this wave's share of K tile kt (j a compile-time index).
  __device__ __forceinline__ void issue_one(int kt, f16* tile, int64_t ld, int w, int j) const {
    const int64_t adv = KMAJ ? (int64_t)kt * BK : (int64_t)kt * BK * ld;
    dma16_asm(p[j] + adv, tile + 512 * (NW * j + w));
  }
  __device__ __forceinline__ void issue(int kt, f16* tile, int64_t ld, int w) const {
#pragma unroll
    for (int j = 0; j < J; ++j) issue_one(kt, tile, ld, w, j);
  }
  // Per-lane element offset of the K-major fragment of K step s within a
  // 32-row block (the swizzle of row rb + i equals that of i, rb being a
  // multiple of 32): computed once so each read is one base + immediate.
  static __device__ __forceinline__ int koff(int s, int lane) {
    const int i = lane & 31, kh = lane >> 5;
    return i * BK + (((2 * s + kh) ^ ksw(i)) << 3);
  }
  // MFMA operand for K step s (16 K) of the 32-row block starting at tile
  // row (K-major) or column (MN-major) rb: lane (i, kh) gets rows rb + i,
  // K = 16 s + 8 kh + 0..7. `ko` is koff(s, lane) (K-major only).
  static __device__ __forceinline__ half8 frag(const f16* tile, int rb, int s, int lane, int ko) {
    if constexpr (KMAJ) {
      return *(const half8*)(tile + rb * BK + ko);
    } else {
      const int sl = lane & 15, q1 = (lane >> 4) & 1, kh = lane >> 5;
      const int col = rb + 16 * q1 + 4 * (sl & 3);
      const int cpart = col & 7;
      half8 out;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int krow = 16 * s + 8 * kh + 4 * rr + (sl >> 2);
        const int ch = (col >> 3) ^ ((krow & 3) << 2);
        const f16* addr = tile + krow * R + ch * 8 + cpart;
        const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)addr);
        const half4 h = __builtin_bit_cast(half4, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[4 * rr + e] = h[e];
      }
      return out;
    }
  }
};

// An M/N-contiguous fp32 operand of the fp32 direct-to-LDS path: R fp32
// columns (2R 16-bit units) by 32 K-rows per stage, copied like a 16-bit
// MN-major tile of 2R columns (chunks swizzled by (krow & 3) << 2). The
// fragment of K step s (8 K) for lane (i, kh) is the 4 values at K-rows
// 8s + 4kh + j, column rb + i, read one float each (K-row 8s + 4kh + j has
// swizzle j): the arrangement of the K-major fp32 fragments, so the two
// kinds pair in one MFMA. The kernel hands over units (ld doubled, K and
// its split offsets doubled); columns and rows convert here. Storage rows
// may lie in up to three segments whose boundaries fall on 32-row K tiles:
// each copy then takes its tile's segment (the same for every lane).
template <int R, int NW>
struct DmaOperandF32MN {
  static constexpr int RU = 2 * R;      // 16-bit units per K-row
  static constexpr int CPR = RU / 8;    // 16-byte chunks per K-row
  static constexpr int RPI = 64 / CPR;  // K-rows per 1 KB wave copy
  static constexpr int J = RU * 32 / 512 / NW;
  static_assert(J * 512 * NW == RU * 32 && RPI >= 1, "DMA split");
  int64_t off[J];  // this lane's offset (units) of copy j inside a K tile
  const f16* p0;    // segment 0's base (the operand's without segments)
  int64_t d1, d2;   // segments 1 and 2: their bases' offsets from p0 (units)
  int s1, s2, kb_rows;  // segment starts (past the end when absent)
  __device__ __forceinline__ void init(const f16* base_, int64_t ld, int r0, int rmax, int64_t kb, int lane, int w,
                                       const Seg* seg_) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int blk = NW * j + w;
      const int krow = blk * RPI + lane / CPR;
      const int lc = (lane % CPR) ^ ((krow & 3) << 2);
      const int col = min(2 * r0 + lc * 8, 2 * rmax - 8);
      off[j] = (int64_t)krow * ld + col;
    }
    // the segment table is copied into scalars: indexing the kernel
    // argument's table at run time would put the whole descriptor in
    // private memory
    // (arithmetic on the offsets, as in out_row: a selected pointer was
    // compiled to an indexed load from a private copy of the operand)
    const int ns = seg_ ? seg_->nseg : 1;
    p0 = ns > 1 ? (const f16*)seg_->p[0] : base_;
    d1 = ns > 1 ? (const f16*)seg_->p[1] - p0 : 0;
    d2 = ns > 2 ? (const f16*)seg_->p[2] - p0 : 0;
    s1 = ns > 1 ? seg_->start[1] : 0x7fffffff;
    s2 = ns > 2 ? seg_->start[2] : 0x7fffffff;
    kb_rows = (int)(kb / 2);
  }
  __device__ __forceinline__ void issue_one(int kt, f16* tile, int64_t ld, int w, int j) const {
    const int r = kb_rows + kt * 32;  // the tile's first storage row
    const int in1 = r >= s1, in2 = r >= s2;
    const int64_t so = in2 * d2 + (in1 - in2) * d1;
    const int st = in1 * s1 + in2 * (s2 - s1);
    dma16_asm(p0 + so + (int64_t)(r - st) * ld + off[j], tile + 512 * (NW * j + w));
  }
  __device__ __forceinline__ void issue(int kt, f16* tile, int64_t ld, int w) const {
#pragma unroll
    for (int j = 0; j < J; ++j) issue_one(kt, tile, ld, w, j);
  }
  static __device__ __forceinline__ int koff(int, int) { return 0; }
  static __device__ __forceinline__ half8 frag(const f16* tile, int rb, int s, int lane, int) {
    const int i = lane & 31, kh = lane >> 5, m = rb + i;
    const f16* col = tile + (8 * s + 4 * kh) * RU + (m & 3) * 2;
    float4 v;
    v.x = *(const float*)(col + (((m >> 2) ^ 0) << 3));
    v.y = *(const float*)(col + 1 * RU + (((m >> 2) ^ 4) << 3));
    v.z = *(const float*)(col + 2 * RU + (((m >> 2) ^ 8) << 3));
    v.w = *(const float*)(col + 3 * RU + (((m >> 2) ^ 12) << 3));
    return __builtin_bit_cast(half8, v);
  }
};

// fp8 MFMA over 64 K: a and b are 32 bytes of 8-bit operands per lane.
// FA / FB pick each operand's format (0 E4M3, 1 E5M2). The lane's 32 bytes
// hold K values in the same arrangement for A and B, so the block product
// is the dot product over those 64 K whatever order the unit takes them in.
typedef int int8v __attribute__((ext_vector_type(8)));
template <int FA, int FB>
__device__ __forceinline__ floatx16 mfma8(half8 a0, half8 a1, half8 b0, half8 b1, floatx16 c) {
  const int4 x0 = __builtin_bit_cast(int4, a0), x1 = __builtin_bit_cast(int4, a1);
  const int4 y0 = __builtin_bit_cast(int4, b0), y1 = __builtin_bit_cast(int4, b1);
  const int8v a = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  const int8v b = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
  // scale operands 0: the unscaled v_mfma_f32_32x32x64_f8f6f4
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// fp32 operands over 8 K (in the 16-bit staging: one K step of 16 units):
// the lane's 16 bytes of A and of B hold 4 fp32 K values each, in the same
// arrangement for both (lane half kh: K 4 kh .. 4 kh + 3 of the step), so
// four v_mfma_f32_32x32x2_f32 with the j-th value of each lane (K pairs
// (j, 4 + j) across the two halves) give the block product over those 8 K.
__device__ __forceinline__ floatx16 mfma32x4(half8 a, half8 b, floatx16 c) {
  const float4 x = __builtin_bit_cast(float4, a), y = __builtin_bit_cast(float4, b);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y.z, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y.w, c, 0, 0, 0);
}

// EK: operand kind. 0 fp16, 1 bfloat16 (16-bit elements, K tiles of 64);
// 2 + fa + 2 fb: fp8 with A format fa and B format fb (0 E4M3, 1 E5M2);
// 6: fp32 (NT; the descriptor in 16-bit units like fp8's: K, lda, ldb and
// the split-K chunk doubled, a K tile then 32 fp32 values).
// The fp8 kernels take the descriptor in 16-bit units (K, lda, ldb and
// the split-K chunk halved: two fp8 values per unit), so staging, copies
// and fragment reads are those of the 16-bit kernel; a K tile then holds
// 128 fp8 values and feeds two fp8 MFMAs per 32 x 32 block, each taking
// the fragments of two 16-bit K steps.
template <int BM, int BN, int WM, int WN, int NS, int NB, bool AK, bool BK_, int EK>
__global__ __launch_bounds__(WM* WN * 64) void gemm_dma_kernel(const GemmDesc d, const Grid gd) {
  constexpr bool BF = EK == 1, F8 = EK >= 2 && EK <= 5, F32 = EK == 6;
  constexpr int FA = F8 ? (EK - 2) & 1 : 0, FB = F8 ? (EK - 2) >> 1 : 0;
  static_assert(!F8 || (AK && BK_), "fp8 operands: both K-major (NT)");

  constexpr int BK = 64;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "tile");
  using OA = std::conditional_t<F32 && !AK, DmaOperandF32MN<BM, NW>, DmaOperand<BM, AK, NW>>;
  using OB = std::conditional_t<F32 && !BK_, DmaOperandF32MN<BN, NW>, DmaOperand<BN, BK_, NW>>;
  constexpr int JS = OA::J + OB::J;

  // the wave index as a scalar: the copies' LDS addresses (M0) then need
  // no per-copy move from a vector register
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w % WM, wn = w / WM;

  const int total = gd.tiles_m * gd.tiles_n * gd.splits;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = total / 8, rem = total % 8;
  const int lt = xcd * per + min(xcd, rem) + slot;
  const int mt = lt % gd.tiles_m;
  const int nt = (lt / gd.tiles_m) % gd.tiles_n;
  const int sp = lt / (gd.tiles_m * gd.tiles_n);
  const int m0 = mt * BM, n0 = nt * BN;
  const int kb = sp * gd.kchunk;
  const int ke = min(d.K, kb + gd.kchunk);
  const int nkt = ke > kb ? (ke - kb) / BK : 0;

  OA oa;
  OB ob;
  oa.init((const f16*)d.a, d.lda, m0, d.M, kb, lane, w, nullptr);
  ob.init((const f16*)d.b.p[0], d.ldb, n0, d.N, kb, lane, w, (BK_ || F32) ? &d.b : nullptr);

  floatx16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  int ko[BK / 16];
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) ko[s] = OA::koff(s, lane);
  // The fragments of K step s+1 are read from LDS (into the other register
  // set) before the MFMAs of step s; scheduling fences keep the two phases
  // apart, so every MFMA's operands were requested a whole phase earlier
  // (left to itself the scheduler pairs each read with the MFMA that
  // consumes it and waits on the LDS latency every time).
  // The refill copies of this tile (A of tile ka into da if ca, B of tile
  // kb2 into db if cb) are interleaved with the MFMAs: copy c goes after
  // MFMA floor(c NM / NC), so its issue overlaps the MFMA before it instead
  // of holding up the whole tile.
  auto compute8 = [&](const f16* sa, const f16* sb, bool ca, int ka, f16* da, bool cb, int kb2, f16* db)
      __attribute__((always_inline)) {
    // fp8: MFMA p (of 2) takes the fragments of 16-bit steps 2p and 2p + 1;
    // the second pair's fragments are read before the first pair's MFMAs
    half8 av[2][2][TM], bv[2][2][TN];
    auto frag = [&](int s, half8* a, half8* b) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < TM; ++t) a[t] = OA::frag(sa, wm * TM * 32 + t * 32, s, lane, ko[s]);
#pragma unroll
      for (int t = 0; t < TN; ++t) b[t] = OB::frag(sb, wn * TN * 32 + t * 32, s, lane, ko[s]);
    };
    constexpr int NM = 2 * TM * TN, NC = OA::J + OB::J;
    frag(0, av[0][0], bv[0][0]);
    frag(1, av[0][1], bv[0][1]);
    static_for<0, 2>([&](auto Px) __attribute__((always_inline)) {
      constexpr int p = decltype(Px)::value;
      if constexpr (p == 0) {
        frag(2, av[1][0], bv[1][0]);
        frag(3, av[1][1], bv[1][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, TM * TN>([&](auto Jx) __attribute__((always_inline)) {
        constexpr int j = decltype(Jx)::value, tm = j / TN, tn = j % TN, i = p * TM * TN + j;
        acc[tm][tn] = mfma8<FA, FB>(av[p][0][tm], av[p][1][tm], bv[p][0][tn], bv[p][1][tn], acc[tm][tn]);
        static_for<(i * NC) / NM, ((i + 1) * NC) / NM>([&](auto Cx) __attribute__((always_inline)) {
          constexpr int c = decltype(Cx)::value;
          if constexpr (c < OA::J) {
            if (ca) oa.issue_one(ka, da, d.lda, w, c);
          } else {
            if (cb) ob.issue_one(kb2, db, d.ldb, w, c - OA::J);
          }
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto compute = [&](const f16* sa, const f16* sb, bool ca, int ka, f16* da, bool cb, int kb2, f16* db)
      __attribute__((always_inline)) {
    if constexpr (F8) {
      compute8(sa, sb, ca, ka, da, cb, kb2, db);
      return;
    }
    half8 av[2][TM], bv[2][TN];
    auto frag = [&](int s, half8* a, half8* b) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < TM; ++t) a[t] = OA::frag(sa, wm * TM * 32 + t * 32, s, lane, ko[s]);
#pragma unroll
      for (int t = 0; t < TN; ++t) b[t] = OB::frag(sb, wn * TN * 32 + t * 32, s, lane, ko[s]);
    };
    constexpr int NM = (BK / 16) * TM * TN, NC = OA::J + OB::J;
    frag(0, av[0], bv[0]);
    static_for<0, BK / 16>([&](auto Sx) __attribute__((always_inline)) {
      constexpr int s = decltype(Sx)::value;
      if constexpr (s + 1 < BK / 16) frag(s + 1, av[(s + 1) & 1], bv[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, TM * TN>([&](auto Jx) __attribute__((always_inline)) {
        constexpr int j = decltype(Jx)::value, tm = j / TN, tn = j % TN, i = s * TM * TN + j;
        if constexpr (F32)
          acc[tm][tn] = mfma32x4(av[s & 1][tm], bv[s & 1][tn], acc[tm][tn]);
        else
          acc[tm][tn] = mfma16<BF>(av[s & 1][tm], bv[s & 1][tn], acc[tm][tn]);
        static_for<(i * NC) / NM, ((i + 1) * NC) / NM>([&](auto Cx) __attribute__((always_inline)) {
          constexpr int c = decltype(Cx)::value;
          if constexpr (c < OA::J) {
            if (ca) oa.issue_one(ka, da, d.lda, w, c);
          } else {
            if (cb) ob.issue_one(kb2, db, d.ldb, w, c - OA::J);
          }
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  auto stA = [](auto S) { return lds_stage<2 * decltype(S)::value, BM * BK>(); };
  // the B stages back to back; B's stage is tracked at run time (NB may
  // differ from NS)
  f16* const sB0 = lds_stage<1, NB * BN * BK>();
  auto stB = [&](int i) { return sB0 + i * (BN * BK); };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // Prologue: tiles 0 .. NS-2 in flight (A then B per tile); with a deeper
  // B ring (NB = NS + 1) also B of tile NS-1.
  if (0 < nkt) {
    oa.issue(0, stA(I0{}), d.lda, w);
    ob.issue(0, stB(0), d.ldb, w);
  }
  if constexpr (NS > 2) if (1 < nkt) {
    oa.issue(1, stA(I1{}), d.lda, w);
    ob.issue(1, stB(1), d.ldb, w);
  }
  if constexpr (NS > 3) if (2 < nkt) {
    oa.issue(2, stA(I2{}), d.lda, w);
    ob.issue(2, stB(2), d.ldb, w);
  }
  if constexpr (NB > NS) if (NS - 1 < nkt) ob.issue(NS - 1, stB(NS - 1), d.ldb, w);

  // Step kt: wait for this wave's copies of tile kt (later copies may stay
  // in flight), barrier (every wave's copies of tile kt landed and every
  // wave is done with tile kt-1), then the MFMAs of tile kt, with the
  // refill of the stages of tile kt-1 (A of tile kt+NS-1, B of tile
  // kt+NB-1) interleaved.
  int bs = 0;  // B stage of tile kt
  auto step = [&](auto S, int kt) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    if constexpr (NB > NS) {
      // issued after tile kt: A and B of tiles kt+1 .. kt+NS-2, then B of
      // tile kt+NS-1 (NS = 2: only that B)
      static_assert(NS == 2 && NB == 3, "deeper B ring: two A stages, three B stages");
      if (kt + 1 < nkt) wait_vmcnt<OB::J>();
      else wait_vmcnt<0>();
    } else {
      if (kt + NS - 2 < nkt) wait_vmcnt<JS * (NS - 2)>();
      else wait_vmcnt<0>();
    }
    __syncthreads();
    const int bfree = bs == 0 ? NB - 1 : bs - 1;  // B stage of tile kt-1
    compute(stA(S), stB(bs), kt + NS - 1 < nkt, kt + NS - 1, stA(std::integral_constant<int, (s + NS - 1) % NS>{}),
            kt + NB - 1 < nkt, kt + NB - 1, stB(bfree));
    bs = bs + 1 == NB ? 0 : bs + 1;
  };
  // Whole rounds of NS tiles run without branches around the MFMAs (a
  // conditional step inside the loop makes the compiler copy every
  // accumulator out of and back into AGPRs each iteration); the last
  // nkt % NS tiles follow.
  const int nfull = nkt / NS * NS;
  for (int kt = 0; kt < nfull; kt += NS) {
    step(I0{}, kt);
    step(I1{}, kt + 1);
    if constexpr (NS > 2) step(I2{}, kt + 2);
    if constexpr (NS > 3) step(I3{}, kt + 3);
  }
  const int left = nkt - nfull;
  if (left > 0) step(I0{}, nfull);
  if constexpr (NS > 2) if (left > 1) step(I1{}, nfull + 1);
  if constexpr (NS > 3) if (left > 2) step(I2{}, nfull + 2);
  if constexpr (F8) {
    // the operands' inverse scales (split-K partials carry them too)
    const float sc = (d.scale_a_dev ? d.scale_a_dev[0] : 1.f) * (d.scale_b_dev ? d.scale_b_dev[0] : 1.f);
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[a][b][e] *= sc;
  }

  constexpr int WC = TN * 32;  // wave tile width
  if constexpr (WC < 64) {
    // Narrow wave tiles (64 x 64 workgroup tiles of 32 x 32 per wave): each
    // lane stores its accumulators directly, one column per lane and 32
    // consecutive columns per row (128-byte row pieces per wave store).
    const int ii = lane & 31, kh = lane >> 5;
    float* part = gd.splits > 1 ? d.ws + (int64_t)sp * d.M * d.N : nullptr;
    const int bd = d.c_cols_blockdiag;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * TM * 32 + tm * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
        if (row >= d.M) continue;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int col = n0 + wn * WC + tn * 32 + ii;
          if (col >= d.N) continue;
          if (part) {
            part[(int64_t)row * d.N + col] = acc[tm][tn][e];
            continue;
          }
          int lo = 0;
          float* rp = out_row(d, row, lo);
          if (bd > 0 && (col < lo || col >= lo + bd)) continue;
          put_out(d, rp + (col - lo), row, col, acc[tm][tn][e]);
          if (d.c16) d.c16[(int64_t)row * d.ldc16 + col] = to_16(rp[col - lo], BF);
        }
      }
    return;
  }
  // Epilogue through LDS: the wave parks one 32-row block (tm) of its tile
  // at a time in its own slice of the (now idle) stage buffers and reads it
  // back so that every lane writes 16 contiguous bytes and each wave
  // instruction whole rows of the output: a quarter of the store
  // instructions of element-wise stores. The float4 slots of a row are
  // XOR-swizzled by row bit 2, so the two half-waves, which park rows r and
  // r + 4, write different banks.
  constexpr int CPR = WC / 4;  // float4 slots per row
  static_assert(WC < 64 || (CPR >= 16 && (32 * CPR) % 64 == 0), "epilogue row width");
  static_assert(WC < 64 || (BM == BN && 2 * 32 * WC * 4 <= BM * BK * 2 && NW <= 8), "epilogue staging space");
  const int ii = lane & 31, kh = lane >> 5;
  __syncthreads();  // every wave is done reading the stages
  float* ep;
  switch (w >> 1) {  // two wave slices per stage buffer
    case 0: ep = (float*)stA(I0{}); break;
    case 1: ep = (float*)stB(0); break;
    case 2: ep = (float*)stA(I1{}); break;
    default: ep = (float*)stB(1); break;
  }
  ep += (w & 1) * 32 * WC;
  auto eslot = [](int r, int c) { return r * WC + ((c ^ (((r >> 2) & 1) << 3)) << 2); };
  const int col0 = n0 + wn * WC;
  float* part = gd.splits > 1 ? d.ws + (int64_t)sp * d.M * d.N : nullptr;
  const int bd = d.c_cols_blockdiag;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int c = tn * 32 + ii;
          ep[eslot(8 * g + 4 * kh + r, c >> 2) + (c & 3)] = acc[tm][tn][4 * g + r];
        }
    const int rowb = m0 + wm * TM * 32 + tm * 32;
    if (epi_pass_fast<32, CPR>(d, gd.vec, part, rowb, col0, ep, eslot, lane)) continue;
#pragma unroll 1
    for (int q = 0; q < 32 * CPR / 64; ++q) {
      const int L = q * 64 + lane, rr = L / CPR, c = L % CPR;
      const float4 v = *(const float4*)(ep + eslot(rr, c));
      const int row = rowb + rr, col = col0 + 4 * c;
      if (row >= d.M || col >= d.N) continue;
      const float vv[4] = {v.x, v.y, v.z, v.w};
      if (part) {
        float* pp = part + (int64_t)row * d.N + col;
        if (gd.vec && col + 4 <= d.N) *(float4*)pp = v;
        else
          for (int j = 0; j < 4 && col + j < d.N; ++j) pp[j] = vv[j];
        continue;
      }
      int lo = 0;
      float* rp = out_row(d, row, lo);
      if (!rp) continue;
      if (gd.vec && col + 4 <= d.N && (bd == 0 || (col >= lo && col + 4 <= lo + bd))) {
        float4 o = make_float4(d.alpha * v.x, d.alpha * v.y, d.alpha * v.z, d.alpha * v.w);
        if (d.r) {
          const float4 rv = *(const float4*)(d.r + (int64_t)row * d.ldr + col);
          o.x += rv.x;
          o.y += rv.y;
          o.z += rv.z;
          o.w += rv.w;
        }
        float4* cp = (float4*)(rp + (col - lo));
        if (d.accumulate) {
          const float4 cv = *cp;
          o.x += cv.x;
          o.y += cv.y;
          o.z += cv.z;
          o.w += cv.w;
        }
        store_c4(cp, o);
        if (d.c16) *(half4*)(d.c16 + (int64_t)row * d.ldc16 + col) = to_16x4(o, BF);
      } else {
        for (int j = 0; j < 4 && col + j < d.N; ++j) {
          if (bd > 0 && (col + j < lo || col + j >= lo + bd)) continue;
          put_out(d, rp + (col + j - lo), row, col + j, vv[j]);
          if (d.c16) d.c16[(int64_t)row * d.ldc16 + col + j] = to_16(rp[col + j - lo], BF);
        }
      }
    }
  }
}

// ------------------------------------------ NF4 B operand, decoded in LDS
//
// The fused dequant + GEMM of the frozen NF4 weights (y = x W~^T forward,
// NT; dX = dY W~ backward, NN). A (fp16 activations, K-major) is copied
// global -> LDS by DMA exactly as in gemm_dma_kernel. B arrives as NF4
// codes (half a byte per weight, one fp32 scale per 64 consecutive
// elements of the row-major [out, in] storage): every thread loads 16 bytes
// of codes (32 weights of one storage row, inside one 64-element block) and
// their scale one step ahead, and at the start of the next step decodes
// them into the B stage in the layout the DMA kernel's fragment reads
// expect (K-major rows with the (row >> 1) & 7 chunk swizzle for NT,
// K-rows with the (krow & 3) << 2 swizzle for NN). Decode: a 256-entry LDS
// table maps a code byte to its two levels as an fp16 pair, which one
// packed fp16 multiply scales by the block's scale (rounded to fp16): one
// table read and one multiply per two weights. The codes are 4x smaller
// than an fp16 copy, so B's traffic drops by 4x; A and the MFMA loop follow
// gemm_dma_kernel's (here 128 x 128 tiles of 4 waves, two workgroups per
// CU, two stages per operand, or the 256 x 256 tiles below).
//
// LoRA rides as one more K tile after the NF4 ones: A from ext16_a
// ([M, 64] fp16, DMA), B from ext16_b (fp16, copied to LDS as it is).

struct Nf4Lut {
  uint32_t v[256];  // byte b -> (fp16 L[b & 15]) | (fp16 L[b >> 4]) << 16
};

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_scale(uint32_t pair, half2v s) {
  const half2v v = __builtin_bit_cast(half2v, pair) * s;
  return __builtin_bit_cast(uint32_t, v);
}

// Tiles: 128 x 128 with 4 waves of 64 x 64, two workgroups per CU, or
// 256 x 256 with 8 waves of 64 x 128, one workgroup per CU (two waves per
// SIMD): each decoded B tile then serves 256 rows of A, half the decode
// work per product, and each A tile 256 columns. Two workgroups per CU need
// at most 256 registers per lane (the second launch-bounds argument):
// without it the 128 x 128 kernel's accumulators went to AGPRs beside 212
// VGPRs and only one workgroup fit.
template <bool NN, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64, WM * WN == 4 ? 2 : 1) void gemm_nf4_kernel(const GemmDesc d,
                                                                                     const Grid gd) {
  constexpr int BK = 64, NW = WM * WN, TM = BM / WM / 32, TN = BN / WN / 32;
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "tile");
  // B's decode shares: NT two threads per tile row, NN NW threads per K-row
  static_assert(BN == 32 * NW, "B tile width");
  using OA = DmaOperand<BM, true, NW>;
  using OB = DmaOperand<BN, !NN, NW>;  // fragment reads of the decoded stage

  __shared__ Nf4Lut lut;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w % WM, wn = w / WM;
  if (tid < 256) {
    const f16 lo = (f16)d.nf4.levels[tid & 15], hi = (f16)d.nf4.levels[tid >> 4];
    lut.v[tid] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }

  const int total = gd.tiles_m * gd.tiles_n * gd.splits;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = total / 8, rem = total % 8;
  const int lt = xcd * per + min(xcd, rem) + slot;
  const int mt = lt % gd.tiles_m;
  const int nt = (lt / gd.tiles_m) % gd.tiles_n;
  const int sp = lt / (gd.tiles_m * gd.tiles_n);
  const int m0 = mt * BM, n0 = nt * BN;
  const int nkt_main = d.K / BK;
  const int nkt_all = nkt_main + (d.ext16_a ? 1 : 0);
  const int kt0 = sp * (gd.kchunk / BK);
  const int kt1 = min(nkt_all, kt0 + gd.kchunk / BK);

  OA oa, oax;
  oa.init((const f16*)d.a, d.lda, m0, d.M, 0, lane, w, nullptr);
  if (d.ext16_a) oax.init(d.ext16_a, d.ext16_lda, m0, d.M, 0, lane, w, nullptr);
  auto issueA = [&](int kt, f16* st, int j) __attribute__((always_inline)) {
    if (kt < nkt_main) oa.issue_one(kt, st, d.lda, w, j);
    else oax.issue_one(0, st, d.ext16_lda, w, j);
  };

  // This thread's share of a B tile: NT, storage row n0 + (tid >> 1),
  // K elements 32 (tid & 1) .. + 31 of the tile; NN, K-row tid / NW of the
  // tile, columns n0 + 32 (tid % NW) .. + 31.
  const int brow = NN ? tid / NW : tid >> 1;
  const int bpart = NN ? tid % NW : tid & 1;
  const uint8_t* ncodes = nullptr;  // NT: codes of this row at K = 32 bpart
  const float* nscale = nullptr;    // NT: scales of this row
  int bcol = 0;                     // NN: first column
  if constexpr (!NN) {
    const int n = min(n0 + brow, d.N - 1);
    const int sg = seg_of(d.b, n);
    const int64_t e = (int64_t)(n - d.b.start[sg]) * d.ldb;
    ncodes = d.nf4.codes[sg] + (e + 32 * bpart) / 2;
    nscale = d.nf4.scales[sg] + e / 64;
  } else {
    bcol = min(n0 + 32 * bpart, d.N - 32);
  }
  // codes (16 bytes: 32 weights) and scale of an NF4 tile, loaded a tile
  // ahead; the LoRA tile's fp16 share is read chunk by chunk at decode time
  struct BReg {
    u32x4 q;
    float sc;
  };
  auto loadB = [&](int kt, BReg& r) __attribute__((always_inline)) {
    if (kt < nkt_main) {
      if constexpr (!NN) {
        r.q = *(const u32x4*)(ncodes + (int64_t)kt * (BK / 2));
        r.sc = nscale[kt];
      } else {
        const int k0 = kt * BK;  // the tile's K-rows lie in one segment
        const int sg = seg_of(d.b, k0);
        const int64_t e = (int64_t)(k0 + brow - d.b.start[sg]) * d.ldb + bcol;
        r.q = *(const u32x4*)(d.nf4.codes[sg] + e / 2);
        r.sc = d.nf4.scales[sg][e / 64];
      }
    }
  };
  // Decode (or copy, for the LoRA tile) 8-element chunk i of the thread's
  // share into stage sb at the position the fragment reads expect. The
  // table reads (lut_read; the LoRA chunk's global read) and the scaling +
  // store (lut_store) are split so that the MFMAs of a K step run while
  // the reads are in flight.
  auto lut_read = [&](int kt, const BReg& r, int i, uint32_t (&lv)[4]) __attribute__((always_inline)) {
    if (kt < nkt_main) {
      const uint32_t c = r.q[i];
#pragma unroll
      for (int b = 0; b < 4; ++b) lv[b] = lut.v[(c >> (8 * b)) & 255];
    } else {
      const f16* src = NN ? d.ext16_b + (int64_t)brow * d.ext16_ldb + bcol
                          : d.ext16_b + (int64_t)min(n0 + brow, d.N - 1) * d.ext16_ldb + 32 * bpart;
      const u32x4 x = *(const u32x4*)(src + 8 * i);
#pragma unroll
      for (int b = 0; b < 4; ++b) lv[b] = x[b];
    }
  };
  auto lut_store = [&](int kt, const BReg& r, int i, const uint32_t (&lv)[4], f16* sb) __attribute__((always_inline)) {
    u32x4 out;
    if (kt < nkt_main) {
      const f16 s16 = (f16)r.sc;
      const half2v s2 = {s16, s16};
#pragma unroll
      for (int b = 0; b < 4; ++b) out[b] = pk_scale(lv[b], s2);
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) out[b] = lv[b];
    }
    const int c = 4 * bpart + i;  // 8-element chunk within the tile row
    int pos;
    if constexpr (!NN) pos = brow * BK + ((c ^ ((brow >> 1) & 7)) << 3);
    else pos = brow * BN + ((c ^ ((brow & 3) << 2)) << 3);
    *(u32x4*)(sb + pos) = out;
  };
  auto storeB = [&](int kt, const BReg& r, f16* sb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lv[4] = {0u, 0u, 0u, 0u};
      lut_read(kt, r, i, lv);
      lut_store(kt, r, i, lv, sb);
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  int ko[BK / 16];
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) ko[s] = OA::koff(s, lane);

  f16* const sA0 = lds_stage<20, BM * BK>();
  f16* const sA1 = lds_stage<21, BM * BK>();
  f16* const sB0 = lds_stage<22, BN * BK>();
  f16* const sB1 = lds_stage<23, BN * BK>();

  // MFMAs of one tile; the A copies of tile kn (into da) are spread over
  // them as in gemm_dma_kernel, and the decode of B tile kd (codes in rd,
  // into db) is cut into the four K steps: chunk s's table reads are issued
  // before step s's MFMAs, its scaling and store after them.
  auto compute = [&](const f16* sa, const f16* sb, bool ca, int kn, f16* da, bool cd, int kd, const BReg& rd,
                     f16* db) __attribute__((always_inline)) {
    half8 av[2][TM], bv[2][TN];
    auto frag = [&](int s, half8* a, half8* b) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < TM; ++t) a[t] = OA::frag(sa, wm * TM * 32 + t * 32, s, lane, ko[s]);
#pragma unroll
      for (int t = 0; t < TN; ++t) b[t] = OB::frag(sb, wn * TN * 32 + t * 32, s, lane, ko[s]);
    };
    constexpr int NM = (BK / 16) * TM * TN, NC = OA::J;
    frag(0, av[0], bv[0]);
    static_for<0, BK / 16>([&](auto Sx) __attribute__((always_inline)) {
      constexpr int s = decltype(Sx)::value;
      if constexpr (s + 1 < BK / 16) frag(s + 1, av[(s + 1) & 1], bv[(s + 1) & 1]);
      uint32_t lv[4] = {0u, 0u, 0u, 0u};
      if (cd) lut_read(kd, rd, s, lv);
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, TM * TN>([&](auto Jx) __attribute__((always_inline)) {
        constexpr int j = decltype(Jx)::value, tm = j / TN, tn = j % TN, i = s * TM * TN + j;
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[s & 1][tm], bv[s & 1][tn], acc[tm][tn], 0, 0, 0);
        static_for<(i * NC) / NM, ((i + 1) * NC) / NM>([&](auto Cx) __attribute__((always_inline)) {
          constexpr int c = decltype(Cx)::value;
          if (ca) issueA(kn, da, c);
        });
      });
      __builtin_amdgcn_sched_barrier(0);
      if (cd) lut_store(kd, rd, s, lv, db);
    });
  };

  // Prologue: A of the first tile in flight, its B decoded (the table
  // written above is complete after the barrier), the codes of the second
  // tile in flight.
  BReg rb0, rb1;
  if (kt0 < kt1) {
    loadB(kt0, rb0);
#pragma unroll
    for (int j = 0; j < OA::J; ++j) issueA(kt0, sA0, j);
  }
  __syncthreads();
  if (kt0 < kt1) storeB(kt0, rb0, sB0);
  if (kt0 + 1 < kt1) loadB(kt0 + 1, rb1);

  // Step kt (stage p = (kt - kt0) & 1): wait for A of tile kt and the codes
  // of tile kt+1 (both issued in the previous step), barrier (the decoded B
  // of tile kt is visible, every wave is done with tile kt-1's stages), then
  // load the codes of tile kt+2 and run tile kt's MFMAs with A of tile kt+1
  // copied and B of tile kt+1 decoded into the other stages alongside.
  auto step = [&](auto P, int kt) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    f16* const sa = p ? sA1 : sA0;
    f16* const sb = p ? sB1 : sB0;
    f16* const na = p ? sA0 : sA1;
    f16* const nb = p ? sB0 : sB1;
    BReg& cur = p ? rb0 : rb1;  // codes of tile kt+1
    BReg& nxt = p ? rb1 : rb0;  // receives the codes of tile kt+2
    wait_vmcnt<0>();
    __syncthreads();
    if (kt + 2 < kt1) loadB(kt + 2, nxt);
    compute(sa, sb, kt + 1 < kt1, kt + 1, na, kt + 1 < kt1, kt + 1, cur, nb);
  };
  int kt = kt0;
  for (; kt + 1 < kt1; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
  }
  if (kt < kt1) step(std::integral_constant<int, 0>{}, kt);

  // Epilogue: as gemm_dma_kernel's (staged through the idle stages, two
  // waves' 32-row slices per stage buffer).
  constexpr int WC = TN * 32;
  constexpr int CPR = WC / 4;
  static_assert(2 * 32 * WC * 4 <= BM * BK * 2 && 2 * 32 * WC * 4 <= BN * BK * 2 && NW <= 8, "epilogue staging");
  const int ii = lane & 31, kh = lane >> 5;
  __syncthreads();
  float* ep;
  switch (w >> 1) {
    case 0: ep = (float*)sA0; break;
    case 1: ep = (float*)sB0; break;
    case 2: ep = (float*)sA1; break;
    default: ep = (float*)sB1; break;
  }
  ep += (w & 1) * 32 * WC;
  auto eslot = [](int r, int c) { return r * WC + ((c ^ (((r >> 2) & 1) << 3)) << 2); };
  const int col0 = n0 + wn * WC;
  float* part = gd.splits > 1 ? d.ws + (int64_t)sp * d.M * d.N : nullptr;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int c = tn * 32 + ii;
          ep[eslot(8 * g + 4 * kh + r, c >> 2) + (c & 3)] = acc[tm][tn][4 * g + r];
        }
    const int rowb = m0 + wm * TM * 32 + tm * 32;
    if (epi_pass_fast<32, CPR>(d, gd.vec, part, rowb, col0, ep, eslot, lane)) continue;
#pragma unroll 1
    for (int q = 0; q < 32 * CPR / 64; ++q) {
      const int L = q * 64 + lane, rr = L / CPR, c = L % CPR;
      const float4 v = *(const float4*)(ep + eslot(rr, c));
      const int row = rowb + rr, col = col0 + 4 * c;
      if (row >= d.M || col >= d.N) continue;
      const float vv[4] = {v.x, v.y, v.z, v.w};
      if (part) {
        float* pp = part + (int64_t)row * d.N + col;
        for (int j = 0; j < 4 && col + j < d.N; ++j) pp[j] = vv[j];
        continue;
      }
      int lo = 0;
      float* rp = out_row(d, row, lo);
      if (!rp) continue;
      for (int j = 0; j < 4 && col + j < d.N; ++j) {
        put_out(d, rp + (col + j - lo), row, col + j, vv[j]);
        if (d.c16) d.c16[(int64_t)row * d.ldc16 + col + j] = (f16)rp[col + j - lo];
      }
    }
  }
}

// Ping-pong variant of the 256 x 256 tile: the two halves of the workgroup
// (waves 0-3 and 4-7; each SIMD holds one of each) alternate between an
// MFMA phase (16 MFMAs: two K steps of the wave's 64 x 128 block) and an
// operand phase (the LDS reads of the next two K steps), with a workgroup
// barrier between phases and raised priority for the MFMA phase, so every
// SIMD has one wave issuing MFMAs while the other gathers operands. Per K
// tile (stage S): the leading half runs MFMA(h0) read(h1) MFMA(h1)
// read(next tile h0), the trailing half read(h0) MFMA(h0) read(h1)
// MFMA(h1). Stage S is free from the fourth phase on (its last reads, the
// trailing half's h1, returned before the third barrier) and is refilled
// there with tile kt+2, which must have landed (wait + barrier) by the
// fourth phase of the next tile, when the leading half reads it: copies
// run a whole K tile ahead of their first read. With NB = 3 the B operand
// (the weights of a forward product, streamed from HBM while A stays in L2)
// has a third stage and its copies run two K tiles ahead: B(kt+3) goes into
// the stage tile kt just freed.
template <int BN, bool AK, bool BK_, int NB, bool BF>
__global__ __launch_bounds__(512) void gemm_pp_kernel(const GemmDesc d, const Grid gd) {
  constexpr int BM = 256, WM = 4, WN = 2, BK = 64;
  static_assert(BN == 256 || (BN == 192 && BK_), "192-wide tiles need a K-major B");
  static_assert(NB == 2 || NB == 3, "B stages");
  static_assert(2 * BM * BK * 2 + NB * BN * BK * 2 <= 160 * 1024, "LDS");
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  using OA = DmaOperand<BM, AK, NW>;
  using OB = DmaOperand<BN, BK_, NW>;
  constexpr int JS = OA::J + OB::J;

  // the wave index as a scalar: the copies' LDS addresses (M0) then need
  // no per-copy move from a vector register
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w % WM, wn = w / WM;

  const int total = gd.tiles_m * gd.tiles_n * gd.splits;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = total / 8, rem = total % 8;
  const int lt = xcd * per + min(xcd, rem) + slot;
  const int mt = gd.nfast ? (lt / gd.tiles_n) % gd.tiles_m : lt % gd.tiles_m;
  const int nt = gd.nfast ? lt % gd.tiles_n : (lt / gd.tiles_m) % gd.tiles_n;
  const int sp = lt / (gd.tiles_m * gd.tiles_n);
  const int m0 = mt * BM, n0 = nt * BN;
  const int kb = sp * gd.kchunk;
  const int ke = min(d.K, kb + gd.kchunk);
  const int nkt = ke > kb ? (ke - kb) / BK : 0;

  OA oa;
  OB ob;
  oa.init((const f16*)d.a, d.lda, m0, d.M, kb, lane, w, nullptr);
  ob.init((const f16*)d.b.p[0], d.ldb, n0, d.N, kb, lane, w, BK_ ? &d.b : nullptr);

  floatx16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  int ko[BK / 16];
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) ko[s] = OA::koff(s, lane);
  half8 av[2][TM], bv[2][TN];  // two K steps of operands
  auto read = [&](const f16* sa, const f16* sb, auto H) __attribute__((always_inline)) {
    constexpr int h = decltype(H)::value;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int t = 0; t < TM; ++t) av[ks][t] = OA::frag(sa, wm * TM * 32 + t * 32, 2 * h + ks, lane, ko[2 * h + ks]);
#pragma unroll
      for (int t = 0; t < TN; ++t) bv[ks][t] = OB::frag(sb, wn * TN * 32 + t * 32, 2 * h + ks, lane, ko[2 * h + ks]);
    }
  };
  auto mfma = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = mfma16<BF>(av[ks][tm], bv[ks][tn], acc[tm][tn]);
    __builtin_amdgcn_s_setprio(0);
  };
  // The wave's copies of a refill (Mode bit 0: A of tile ka into sa if ca;
  // bit 1: B of tile kb2 into sb if cb), spread over the slots of an
  // instruction stream of ns steps: copy c goes after step floor(c ns / NC).
  // Interleaved, a copy's issue overlaps the MFMA (or LDS read) before it
  // instead of delaying the whole phase.
  auto copies_after = [&](auto Step, auto Steps, auto Mode, bool ca, int ka, f16* sa, bool cb, int kb2, f16* sb)
      __attribute__((always_inline)) {
    constexpr int i = decltype(Step)::value, ns = decltype(Steps)::value, mode = decltype(Mode)::value;
    constexpr int JA = (mode & 1) ? OA::J : 0, NC = JA + ((mode & 2) ? OB::J : 0);
    static_for<(i * NC) / ns, ((i + 1) * NC) / ns>([&](auto C) __attribute__((always_inline)) {
      constexpr int c = decltype(C)::value;
      if constexpr (c < JA) {
        if (ca) oa.issue_one(ka, sa, d.lda, w, c);
      } else {
        if (cb) ob.issue_one(kb2, sb, d.ldb, w, c - JA);
      }
    });
  };
  auto mfma_copy = [&](auto Mode, bool ca, int ka, f16* sa, bool cb, int kb2, f16* sb) __attribute__((always_inline)) {
    constexpr int NM = 2 * TM * TN;
    __builtin_amdgcn_s_setprio(1);
    static_for<0, NM>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value, ks = i / (TM * TN), tm = (i / TN) % TM, tn = i % TN;
      acc[tm][tn] = mfma16<BF>(av[ks][tm], bv[ks][tn], acc[tm][tn]);
      copies_after(I, std::integral_constant<int, NM>{}, Mode, ca, ka, sa, cb, kb2, sb);
    });
    __builtin_amdgcn_s_setprio(0);
  };
  auto read_copy = [&](const f16* ra, const f16* rb, auto H, auto Mode, bool ca, int ka, f16* sa, bool cb, int kb2,
                       f16* sb) __attribute__((always_inline)) {
    constexpr int h = decltype(H)::value, NR = 2 * (TM + TN);
    static_for<0, NR>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value, ks = i / (TM + TN), t = i % (TM + TN);
      if constexpr (t < TM) av[ks][t] = OA::frag(ra, wm * TM * 32 + t * 32, 2 * h + ks, lane, ko[2 * h + ks]);
      else bv[ks][t - TM] = OB::frag(rb, wn * TN * 32 + (t - TM) * 32, 2 * h + ks, lane, ko[2 * h + ks]);
      copies_after(I, std::integral_constant<int, NR>{}, Mode, ca, ka, sa, cb, kb2, sb);
    });
  };
  using MA = std::integral_constant<int, 1>;
  using MB = std::integral_constant<int, 2>;
  using MAB = std::integral_constant<int, 3>;
  auto phase_end = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  auto stA = [](auto S) { return lds_stage<2 * decltype(S)::value, BM * BK>(); };
  f16* const sB0 = lds_stage<1, NB * BN * BK>();  // the B stages, back to back
  auto stB = [&](int i) { return sB0 + i * (BN * BK); };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // The two halves run the same barriers; each is its own instantiation,
  // so no branch sits between a wave's MFMAs.
  auto run = [&](auto Lead) __attribute__((always_inline)) {
    constexpr bool lead = decltype(Lead)::value;
    if (0 < nkt) {
      oa.issue(0, stA(I0{}), d.lda, w);
      ob.issue(0, stB(0), d.ldb, w);
    }
    if (1 < nkt) {
      oa.issue(1, stA(I1{}), d.lda, w);
      ob.issue(1, stB(1), d.ldb, w);
    }
    if (NB == 3 && 2 < nkt) ob.issue(2, stB(2), d.ldb, w);
    // tile 0 landed; the copies issued after it may still be in flight
    if (NB == 3 && 2 < nkt) wait_vmcnt<OA::J + 2 * OB::J>();
    else if (1 < nkt) wait_vmcnt<JS>();
    else wait_vmcnt<0>();
    phase_end();
    if constexpr (lead) read(stA(I0{}), stB(0), I0{});
    phase_end();
    int bs = 0;  // B stage of tile kt
    auto step = [&](auto S, int kt) __attribute__((always_inline)) {
      using SN = std::integral_constant<int, 1 - decltype(S)::value>;
      const int bn1 = bs + 1 == NB ? 0 : bs + 1;
      f16* const sb = stB(bs);
      // with two B stages the A copies of tile kt+1 (into the stage of tile
      // kt-1) go in each half's operand phase of this tile, apart from the
      // fourth phase's B copies
      const bool ca1 = NB == 2 && kt >= 1 && kt + 1 < nkt;
      if constexpr (lead) mfma();
      else if constexpr (NB == 2) read_copy(stA(S), sb, I0{}, MA{}, ca1, kt + 1, stA(SN{}), false, 0, nullptr);
      else read(stA(S), sb, I0{});
      phase_end();
      if constexpr (!lead) mfma();
      else if constexpr (NB == 2) read_copy(stA(S), sb, I1{}, MA{}, ca1, kt + 1, stA(SN{}), false, 0, nullptr);
      else read(stA(S), sb, I1{});
      phase_end();
      if constexpr (lead) mfma();
      else read(stA(S), sb, I1{});
      // this wave's copies of tile kt+1; with three B stages the B copy of
      // tile kt+2, issued after them, may stay in flight
      if (NB == 3 && kt + 2 < nkt) wait_vmcnt<OB::J>();
      else wait_vmcnt<0>();
      phase_end();
      // the stages of tile kt are free now (their last reads returned
      // before the barrier): refill B with tile kt+NB and, with three B
      // stages, A with tile kt+2 (with two, A follows in the next tile's
      // operand phases), ahead of their first reads, the copies interleaved
      // with the phase's LDS reads (leading half) or MFMAs (trailing half)
      const bool ca = NB != 2 && kt + 2 < nkt, cb = kt + NB < nkt;
      using M4 = std::conditional_t<NB == 2, MB, MAB>;
      if constexpr (lead) {
        if (kt + 1 < nkt) read_copy(stA(SN{}), stB(bn1), I0{}, M4{}, ca, kt + 2, stA(S), cb, kt + NB, sb);
        else {
          if (ca) oa.issue(kt + 2, stA(S), d.lda, w);
          if (cb) ob.issue(kt + NB, sb, d.ldb, w);
        }
      } else {
        mfma_copy(M4{}, ca, kt + 2, stA(S), cb, kt + NB, sb);
      }
      phase_end();
      bs = bn1;
    };
    for (int kt = 0; kt + 1 < nkt; kt += 2) {
      step(I0{}, kt);
      step(I1{}, kt + 1);
    }
    if (nkt & 1) step(I0{}, nkt - 1);
  };
  if (w < NW / 2) run(std::true_type{});
  else run(std::false_type{});

  // Epilogue through LDS: the wave parks RP rows (a 32-row block tm, or
  // half of it when two such slices would not fit a stage buffer) of its
  // tile at a time in its own slice of the (now idle) stage buffers
  // and reads them back so that every lane writes 16 contiguous bytes and
  // each wave instruction whole rows of the output: a quarter of the store
  // instructions of element-wise stores. The two half-waves park rows r and
  // r + 4 at once: with power-of-two rows the float4 slots are XOR-swizzled
  // by row bit 2, otherwise rows are padded by 8 floats, so the two land on
  // different banks.
  constexpr int WC = TN * 32;  // wave tile width
  constexpr int CPR = WC / 4;  // float4 slots per row
  constexpr bool POW2 = (CPR & (CPR - 1)) == 0;
  constexpr int PITCH = POW2 ? WC : WC + 8;
  constexpr int RP = 2 * 32 * PITCH * 4 <= BN * BK * 2 ? 32 : 16;  // rows per pass
  static_assert(CPR >= 16 && (RP * CPR) % 64 == 0, "epilogue row width");
  static_assert(2 * RP * PITCH * 4 <= BN * BK * 2 && NW <= 8, "epilogue staging space");
  const int ii = lane & 31, kh = lane >> 5;
  __syncthreads();  // every wave is done reading the stages
  float* ep;
  switch (w >> 1) {  // two wave slices per stage buffer
    case 0: ep = (float*)stA(I0{}); break;
    case 1: ep = (float*)stB(0); break;
    case 2: ep = (float*)stA(I1{}); break;
    default: ep = (float*)stB(1); break;
  }
  ep += (w & 1) * RP * PITCH;
  auto eslot = [](int r, int c) { return r * PITCH + ((POW2 ? (c ^ (((r >> 2) & 1) << 3)) : c) << 2); };
  const int col0 = n0 + wn * WC;
  float* part = gd.splits > 1 ? d.ws + (int64_t)sp * d.M * d.N : nullptr;
  const int bd = d.c_cols_blockdiag;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int hh = 0; hh < 32 / RP; ++hh) {
#pragma unroll
      for (int g2 = 0; g2 < RP / 8; ++g2)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            const int c = tn * 32 + ii;
            ep[eslot(8 * g2 + 4 * kh + r, c >> 2) + (c & 3)] = acc[tm][tn][4 * (hh * (RP / 8) + g2) + r];
          }
      const int rowb = m0 + wm * TM * 32 + tm * 32 + RP * hh;
      if (epi_pass_fast<RP, CPR>(d, gd.vec, part, rowb, col0, ep, eslot, lane)) continue;
#pragma unroll 1
      for (int q = 0; q < RP * CPR / 64; ++q) {
        const int L = q * 64 + lane, rr = L / CPR, c = L % CPR;
        const float4 v = *(const float4*)(ep + eslot(rr, c));
        const int row = rowb + rr, col = col0 + 4 * c;
        if (row >= d.M || col >= d.N) continue;
        const float vv[4] = {v.x, v.y, v.z, v.w};
        if (part) {
          float* pp = part + (int64_t)row * d.N + col;
          if (gd.vec && col + 4 <= d.N) *(float4*)pp = v;
          else
            for (int j = 0; j < 4 && col + j < d.N; ++j) pp[j] = vv[j];
          continue;
        }
        int lo = 0;
        float* rp = out_row(d, row, lo);
        if (!rp) continue;
        if (gd.vec && col + 4 <= d.N && (bd == 0 || (col >= lo && col + 4 <= lo + bd))) {
          float4 o = make_float4(d.alpha * v.x, d.alpha * v.y, d.alpha * v.z, d.alpha * v.w);
          if (d.r) {
            const float4 rv = *(const float4*)(d.r + (int64_t)row * d.ldr + col);
            o.x += rv.x;
            o.y += rv.y;
            o.z += rv.z;
            o.w += rv.w;
          }
          float4* cp = (float4*)(rp + (col - lo));
          if (d.accumulate) {
            const float4 cv = *cp;
            o.x += cv.x;
            o.y += cv.y;
            o.z += cv.z;
            o.w += cv.w;
          }
          store_c4(cp, o);
          if (d.c16) *(half4*)(d.c16 + (int64_t)row * d.ldc16 + col) = to_16x4(o, BF);
        } else {
          for (int j = 0; j < 4 && col + j < d.N; ++j) {
            if (bd > 0 && (col + j < lo || col + j >= lo + bd)) continue;
            put_out(d, rp + (col + j - lo), row, col + j, vv[j]);
            if (d.c16) d.c16[(int64_t)row * d.ldc16 + col + j] = to_16(rp[col + j - lo], BF);
          }
        }
      }
    }
}

// out = alpha * sum over splits (fixed order) [+ R] [+ C], routed like the
// direct epilogue.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmDesc d, int splits, int vec) {
  const int64_t mn = (int64_t)d.M * d.N;
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c0 >= d.N) return;
  const int bd = d.c_cols_blockdiag;
  for (int row = blockIdx.y; row < d.M; row += gridDim.y) {
    int lo = 0;
    float* rp = out_row(d, row, lo);
    if (!rp) return;
    const float* src = d.ws + (int64_t)row * d.N + c0;
    if (vec && c0 + 4 <= d.N) {
      float4 v = *(const float4*)src;
      for (int p = 1; p < splits; ++p) {
        const float4 u = *(const float4*)(src + p * mn);
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
      }
      if (bd == 0 || (c0 >= lo && c0 + 4 <= lo + bd)) {
        float4 o = make_float4(d.alpha * v.x, d.alpha * v.y, d.alpha * v.z, d.alpha * v.w);
        if (d.r) {
          const float4 rv = *(const float4*)(d.r + (int64_t)row * d.ldr + c0);
          o.x += rv.x;
          o.y += rv.y;
          o.z += rv.z;
          o.w += rv.w;
        }
        float4* cp = (float4*)(rp + (c0 - lo));
        if (d.accumulate) {
          const float4 cv = *cp;
          o.x += cv.x;
          o.y += cv.y;
          o.z += cv.z;
          o.w += cv.w;
        }
        store_c4(cp, o);
        if (d.c16) *(half4*)(d.c16 + (int64_t)row * d.ldc16 + c0) = to_16x4(o, d.prec == Prec::BF16);
      } else {
        const float vv[4] = {v.x, v.y, v.z, v.w};
        for (int j = 0; j < 4; ++j)
          if (c0 + j >= lo && c0 + j < lo + bd) put_out(d, rp + (c0 + j - lo), row, c0 + j, vv[j]);
      }
    } else {
      for (int j = 0; j < 4 && c0 + j < d.N; ++j) {
        float sj = 0.f;
        for (int p = 0; p < splits; ++p) sj += src[p * mn + j];
        const int col = c0 + j;
        if (bd > 0 && (col < lo || col >= lo + bd)) continue;
        put_out(d, rp + (col - lo), row, col, sj);
        if (d.c16) d.c16[(int64_t)row * d.ldc16 + col] = to_16(rp[col - lo], d.prec == Prec::BF16);
      }
    }
  }
}

// Split-K finish for 16-byte rows without diagonal blocks: each thread takes
// 4 columns of R consecutive rows and issues every partial load of those
// rows before any epilogue; a workgroup spans up to 1024 columns (fewer
// threads for narrow outputs). One row per workgroup (R = 1) runs wherever
// the grid allows it: the most workgroups, each thread with its splits'
// loads in flight, measured faster than 2, 4 or 8 rows per thread at every
// split product of the blocks (e.g. ≈ 3 µs of the Qwen3-4B-shaped block
// step at seq 512, ≈ 5 µs of a seq-1024 fp32 layer of the 36-layer stack).
// The partials are added in split order, as in
// splitk_reduce_kernel.
template <int R>
__global__ __launch_bounds__(256) void splitk_reduce_rows_kernel(const GemmDesc d, int splits) {
  const int64_t mn = (int64_t)d.M * d.N;
  const int c0 = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (c0 >= d.N) return;
  const int r0 = blockIdx.y * R;
  float4 v[R];
#pragma unroll
  for (int j = 0; j < R; ++j) v[j] = *(const float4*)(d.ws + (int64_t)min(r0 + j, d.M - 1) * d.N + c0);
  for (int p = 1; p < splits; ++p) {
    float4 u[R];
#pragma unroll
    for (int j = 0; j < R; ++j) u[j] = *(const float4*)(d.ws + p * mn + (int64_t)min(r0 + j, d.M - 1) * d.N + c0);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      v[j].x += u[j].x;
      v[j].y += u[j].y;
      v[j].z += u[j].z;
      v[j].w += u[j].w;
    }
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int row = r0 + j;
    if (row >= d.M) break;
    int lo = 0;
    float* rp = out_row(d, row, lo);
    float4 o = make_float4(d.alpha * v[j].x, d.alpha * v[j].y, d.alpha * v[j].z, d.alpha * v[j].w);
    if (d.r) {
      const float4 rv = *(const float4*)(d.r + (int64_t)row * d.ldr + c0);
      o.x += rv.x;
      o.y += rv.y;
      o.z += rv.z;
      o.w += rv.w;
    }
    float4* cp = (float4*)(rp + c0);
    if (d.accumulate) {
      const float4 cv = *cp;
      o.x += cv.x;
      o.y += cv.y;
      o.z += cv.z;
      o.w += cv.w;
    }
    store_c4(cp, o);
    if (d.c16) *(half4*)(d.c16 + (int64_t)row * d.ldc16 + c0) = to_16x4(o, d.prec == Prec::BF16);
  }
}

constexpr int kTargetWgs = 256;  // one 4-wave workgroup per CU (LDS-limited)
constexpr int kMinKtPerSplit = 8;
constexpr int kMaxSplits = 32;

// Register-staged kernel tiles: 128 x 128 (2 x 2 waves of 2 x 2 blocks of
// 32 x 32) or 64 x 64 (2 x 2 waves of one 32 x 32 block each), the K tile
// 64 fp16 / 32 fp32 elements. Products with short K (<= 1408) whose
// 128-wide tiles number fewer than 256 take the 64-wide ones: 4x the
// tiles fill the CUs without splitting K as far, which measured faster on
// every such product of the 36-layer stack's block (fp32: e.g. 1024 x 512
// x 512 in 15 instead of 29 us); long-K products keep the 128-wide tiles,
// whose operand reuse wins there (1024 x 512 x 2816: 50 against 70 us).
constexpr int kRegSmallK = 1408;
constexpr int kRegTargetBig = 512, kRegTargetSmall = 512;

bool reg_small_tiles(const GemmDesc& d) {
  return d.K <= kRegSmallK && ceil_div(d.M, 128) * ceil_div(d.N, 128) < 256;
}

// target_wgs > 0: split K so that tiles x splits reaches it (rounding up);
// target_wgs < 0: so that it stays within -target_wgs (rounding down, one
// wave of workgroups).
Grid plan_tiles(const GemmDesc& d, size_t ws_bytes, int bm, int bn, int bk, int target_wgs = kTargetWgs) {
  Grid g;
  g.tiles_m = (int)ceil_div(d.M, bm);
  g.tiles_n = (int)ceil_div(d.N, bn);
  const int tiles = g.tiles_m * g.tiles_n;
  const int nkt = (int)ceil_div(d.K, bk);
  int splits = target_wgs > 0 ? (int)ceil_div(target_wgs, tiles) : -target_wgs / tiles;
  splits = std::min(splits, std::max(1, nkt / kMinKtPerSplit));
  splits = std::min(splits, kMaxSplits);
  if (splits > 1 && (size_t)splits * d.M * d.N * sizeof(float) > ws_bytes) splits = 1;
  if (splits < 1) splits = 1;
  const int kt_per = (int)ceil_div(nkt, splits);
  splits = std::max(1, (int)ceil_div(nkt, kt_per));  // no empty split
  g.splits = splits;
  g.kchunk = kt_per * bk;
  return g;
}

// Ping-pong configurations: 256 x 256 for every layout, 256 x 192 for NT
// (with a third B stage where the LDS allows it).
constexpr int kPpNb192 = 3;
struct PpCfg {
  static constexpr int bm = 256, bn = 256, threads = 512;
  static constexpr bool narrow = true;  // also runs 256 x 192 tiles (NT)
  template <int BN, bool AK, bool BKM, int NB>
  static void launch(const GemmDesc& d, const Grid& g, hipStream_t st) {
    const unsigned nwg = (unsigned)(g.tiles_m * g.tiles_n * g.splits);
    if (d.prec == Prec::BF16)
      hipLaunchKernelGGL((gemm_pp_kernel<BN, AK, BKM, NB, true>), dim3(nwg), dim3(threads), 0, st, d, g);
    else
      hipLaunchKernelGGL((gemm_pp_kernel<BN, AK, BKM, NB, false>), dim3(nwg), dim3(threads), 0, st, d, g);
  }
  static void launch(const GemmDesc& d, const Grid& g, hipStream_t st) {
    switch (d.layout) {
      case Layout::NT:
        if (g.bn == 192) launch<192, true, true, kPpNb192>(d, g, st);
        else launch<256, true, true, 2>(d, g, st);
        break;
      case Layout::NN: launch<256, true, false, 2>(d, g, st); break;
      case Layout::TN: launch<256, false, false, 2>(d, g, st); break;
    }
  }
};

template <int BM, int BN, int WM, int WN, int NS, int NB = NS>
struct DmaCfg {
  static constexpr int bm = BM, bn = BN, threads = WM * WN * 64;
  static constexpr bool narrow = false;
  template <bool AK, bool BKM>
  static void launch(const GemmDesc& d, const Grid& g, hipStream_t st) {
    const unsigned nwg = (unsigned)(g.tiles_m * g.tiles_n * g.splits);
    if (d.prec == Prec::BF16)
      hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, WM, WN, NS, NB, AK, BKM, 1>), dim3(nwg), dim3(threads), 0, st, d,
                         g);
    else
      hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, WM, WN, NS, NB, AK, BKM, 0>), dim3(nwg), dim3(threads), 0, st, d,
                         g);
  }
  // fp8 operands (NT), the descriptor in 16-bit units
  template <int EK>
  static void launch8(const GemmDesc& d, const Grid& g, hipStream_t st) {
    const unsigned nwg = (unsigned)(g.tiles_m * g.tiles_n * g.splits);
    hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, WM, WN, NS, NB, true, true, EK>), dim3(nwg), dim3(threads), 0, st, d,
                       g);
  }
  // fp32 operands, the descriptor in 16-bit units
  template <bool AK, bool BKM>
  static void launch32(const GemmDesc& d, const Grid& g, hipStream_t st) {
    const unsigned nwg = (unsigned)(g.tiles_m * g.tiles_n * g.splits);
    hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, WM, WN, NS, NB, AK, BKM, 6>), dim3(nwg), dim3(threads), 0, st, d,
                       g);
  }
  static void launch32(const GemmDesc& d, const Grid& g, hipStream_t st) {
    switch (d.layout) {
      case Layout::NT: launch32<true, true>(d, g, st); break;
      case Layout::NN: launch32<true, false>(d, g, st); break;
      case Layout::TN: launch32<false, false>(d, g, st); break;
    }
  }
  static void launch8(const GemmDesc& d, const Grid& g, hipStream_t st) {
    switch (d.f8_a_e5m2 + 2 * d.f8_b_e5m2) {
      case 0: launch8<2>(d, g, st); break;
      case 1: launch8<3>(d, g, st); break;
      case 2: launch8<4>(d, g, st); break;
      default: launch8<5>(d, g, st); break;
    }
  }
  static void launch(const GemmDesc& d, const Grid& g, hipStream_t st) {
    switch (d.layout) {
      case Layout::NT: launch<true, true>(d, g, st); break;
      case Layout::NN: launch<true, false>(d, g, st); break;
      case Layout::TN: launch<false, false>(d, g, st); break;
    }
  }
};
// 128 x 128 tiles, 8 waves of 32 x 64, two workgroups per CU (80 KB LDS
// each: two A stages, three B stages), or, when the grid leaves one
// workgroup per CU, three stages of each (96 KB: the copies run a tile
// further ahead); and 256 x 256 tiles, 8 waves of 64 x 128, one workgroup
// per CU (the ping-pong kernel). A wave streams its share of a tile's
// copies at a bounded rate (global->LDS probes: about 10 B/clk per CU with
// 4 copying waves, 21 B/clk with 8 or more), so 8 waves of 32 x 64 fill
// the 128 x 128 tiles faster than 4 of 64 x 64, which their twice as many
// fragment reads per MFMA do not cost back (the Qwen3-4B block step at seq
// 512 ≈ 1 % faster, the NF4 block ≈ 1.7 %). The fp8 products keep 4 waves
// of 64 x 64 (F8Cfg), as measured.
using Nt16Small = DmaCfg<128, 128, 4, 2, 2, 3>;
using Nt16Deep = DmaCfg<128, 128, 4, 2, 3, 3>;
using F8Cfg = DmaCfg<128, 128, 2, 2, 2, 3>;
using F32Small = DmaCfg<64, 64, 2, 2, 3, 3>;
using Nt16Big = PpCfg;

// Big tiles pay off once they alone give at least half the CUs a tile.
// Weight-gradient products (TN) take the small tiles instead when the big
// ones would leave much of their last round of CUs idle and the small ones
// fill theirs better (fraction of workgroup slots used over the rounds).
bool nt16_big(const GemmDesc& d) {
  const int64_t big = ceil_div(d.M, Nt16Big::bm) * ceil_div(d.N, Nt16Big::bn);
  if (big < 128) return false;
  if (d.layout == Layout::TN) {
    const int64_t small = ceil_div(d.M, Nt16Small::bm) * ceil_div(d.N, Nt16Small::bn);
    const double ub = (double)big / (ceil_div(big, kTargetWgs) * kTargetWgs);
    const double us = (double)small / (ceil_div(small, 2 * kTargetWgs) * 2 * kTargetWgs);
    if (ub < 0.8 && us > ub + 0.1) return false;
  }
  return true;
}

// The DMA kernel applies when both operands are fp16 in storage with
// 16-byte aligned rows, K is a whole number of 64-wide tiles, nothing
// extends the contraction, an MN-major operand has M (or N) a multiple of 8
// and is a single segment.
bool nt16_ok(const GemmDesc& d) {
  if (d.prec != Prec::F16 && d.prec != Prec::BF16) return false;
  if (d.a_src != Src::F16 || d.b_src != Src::F16 || d.ext.kext > 0 || d.b_src == Src::NF4) return false;
  if (d.K % 64 != 0 || d.lda % 8 != 0 || d.ldb % 8 != 0) return false;
  if ((uintptr_t)d.a % 16 != 0) return false;
  for (int s = 0; s < d.b.nseg; ++s)
    if ((uintptr_t)d.b.p[s] % 16 != 0) return false;
  if (d.layout == Layout::TN && (d.M % 8 != 0 || d.M < 8)) return false;
  if (d.layout != Layout::NT && (d.N % 8 != 0 || d.N < 8 || d.b.nseg != 1)) return false;
  return true;
}

// 16-byte epilogue stores: every output row (segment base and stride),
// the residual and the split-K partials start 16-byte aligned and N and
// the diagonal-block width are multiples of 4.
bool out_vec4(const GemmDesc& d, const Grid& g) {
  if (d.N % 4 != 0 || d.ldc % 4 != 0 || d.c_cols_blockdiag % 4 != 0) return false;
  for (int s = 0; s < d.c.nseg; ++s)
    if ((uintptr_t)d.c.p[s] % 16 != 0) return false;
  if (d.r && ((uintptr_t)d.r % 16 != 0 || d.ldr % 4 != 0)) return false;
  if (g.splits > 1 && (uintptr_t)d.ws % 16 != 0) return false;
  if (d.c16 && ((uintptr_t)d.c16 % 8 != 0 || d.ldc16 % 4 != 0)) return false;
  return true;
}

// Big-tile width: 192 instead of 256 (K-major B only) when it takes fewer
// CU-rounds x tile width, i.e. when 256-wide tiles leave many CUs idle.
int big_bn(const GemmDesc& d) {
  if (!Nt16Big::narrow || d.layout != Layout::NT) return Nt16Big::bn;
  const int64_t tm = ceil_div(d.M, 256);
  const int64_t r256 = ceil_div(tm * ceil_div(d.N, 256), kTargetWgs);
  const int64_t r192 = ceil_div(tm * ceil_div(d.N, 192), kTargetWgs);
  return r192 * 192 < r256 * 256 ? 192 : 256;
}

Grid plan(const GemmDesc& d, size_t ws_bytes) {
  if (nt16_ok(d)) {
    const bool big = nt16_big(d);
    const int bn = big ? big_bn(d) : Nt16Small::bn;
    // split K only as far as one workgroup per CU (kTargetWgs): at the
    // seq-512 Qwen3-4B products a second split's partial sums cost more
    // than a second workgroup per CU gains, once the lone workgroup keeps
    // three tiles of copies in flight (e.g. 512 x 2560 x 9728: 3 splits
    // with three stages 36 us, 6 splits with two 40 us)
    Grid g = big ? plan_tiles(d, ws_bytes, Nt16Big::bm, bn, 64, -kTargetWgs)
                 : plan_tiles(d, ws_bytes, Nt16Small::bm, Nt16Small::bn, 64, -kTargetWgs);
    g.bn = bn;
    g.deep = !big && g.tiles_m * g.tiles_n * g.splits <= kTargetWgs;
    g.vec = out_vec4(d, g);
    // weight gradients (TN): the N tiles of one A tile on neighbouring
    // workgroups, so that the long A operand is read about once while the
    // short B operand stays in L2 (fewer bytes fetched past L2)
    g.nfast = big && d.layout == Layout::TN;
    return g;
  }
  const int bk = d.prec == Prec::F16 ? PT<Prec::F16>::BK : PT<Prec::F32>::BK;
  if (reg_small_tiles(d)) return plan_tiles(d, ws_bytes, 64, 64, bk, kRegTargetSmall);
  return plan_tiles(d, ws_bytes, 128, 128, bk, kRegTargetBig);
}

// The fused NF4 kernel applies to fp16 A (K-major, 16-byte aligned rows),
// NF4 B with ldb a multiple of 64 (every 64-element block inside one
// storage row), K a multiple of 64, for NN N a multiple of 32 and B's
// segment boundaries on 64-row tiles, and no diagonal-block output.
bool nf4_fused_ok(const GemmDesc& d) {
  if (d.prec != Prec::F16 || d.a_src != Src::F16 || d.b_src != Src::NF4) return false;
  if (d.layout == Layout::TN || d.ext.kext > 0 || d.c_cols_blockdiag > 0) return false;
  if (d.K % 64 != 0 || d.K == 0 || d.lda % 8 != 0 || d.ldb % 64 != 0 || (uintptr_t)d.a % 16 != 0) return false;
  for (int s = 0; s < d.b.nseg; ++s)
    if ((uintptr_t)d.nf4.codes[s] % 16 != 0 || (uintptr_t)d.nf4.scales[s] % 4 != 0) return false;
  if (d.layout == Layout::NN) {
    if (d.N % 32 != 0) return false;
    for (int s = 1; s < d.b.nseg; ++s)
      if (d.b.start[s] % 64 != 0) return false;
  }
  if (d.ext16_a) {
    if (!d.ext16_b || d.ext16_lda % 8 != 0 || d.ext16_ldb % 8 != 0 || (uintptr_t)d.ext16_a % 16 != 0 ||
        (uintptr_t)d.ext16_b % 16 != 0)
      return false;
    if (d.layout == Layout::NN && d.N % 32 != 0) return false;
  }
  return true;
}

// Split count of the fused NF4 kernel: a product with fewer tiles than
// workgroup slots (two per CU) leaves CUs with a single workgroup, whose
// MFMA pipe then idles through the decode and barrier phases. The split
// minimises an estimate in units of one K tile's time at two workgroups
// per CU: per round of slots, a full round costs 1 and a last round of at
// most one workgroup per CU about 0.6; each split adds the partial sums'
// write and read (M N 8 bytes at about 5 TB/s, with ~1.9 us per K tile
// measured at the Qwen3-4B shapes).
int nf4_splits(int tiles, int nkt, int64_t mn) {
  const int slots = 2 * kTargetWgs;
  int best = 1;
  double best_cost = 1e30;
  for (int sp = 1; sp <= 8 && nkt / sp >= kMinKtPerSplit / 2; ++sp) {
    const int64_t w = (int64_t)tiles * sp;
    const int64_t full = w / slots, rem = w % slots;
    const double rounds = (double)full + (rem == 0 ? 0.0 : rem <= kTargetWgs ? 0.6 : 1.0);
    const double cost = (double)ceil_div(nkt, sp) * rounds + (sp > 1 ? sp * (double)mn * 8.0 / 5e12 / 1.9e-6 : 0.0);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

// 256 x 256 tiles once M spans at least two of them (an NN product's N is
// a multiple of 32 only, so its B shares may clamp at the edge as the
// 128-wide tiles do).
bool nf4_big(const GemmDesc& d) { return d.M >= 512; }

Grid plan_nf4(const GemmDesc& d, size_t ws_bytes) {
  Grid g;
  const bool big = nf4_big(d);
  const int t = big ? 256 : 128;
  g.tiles_m = (int)ceil_div(d.M, t);
  g.tiles_n = (int)ceil_div(d.N, t);
  const int nkt = d.K / 64 + (d.ext16_a ? 1 : 0);
  int splits = big ? std::max(1, std::min(kTargetWgs / (g.tiles_m * g.tiles_n), nkt / kMinKtPerSplit))
                   : nf4_splits(g.tiles_m * g.tiles_n, nkt, (int64_t)d.M * d.N);
  if (splits > 1 && (size_t)splits * d.M * d.N * sizeof(float) > ws_bytes) splits = 1;
  const int kt_per = (int)ceil_div(nkt, splits);
  g.splits = std::max(1, (int)ceil_div(nkt, kt_per));
  g.kchunk = kt_per * 64;
  g.vec = out_vec4(d, g);
  return g;
}

int finish_splits(const GemmDesc& d, const Grid& g, hipStream_t st);

int launch_nf4(const GemmDesc& d, hipStream_t st) {
  const Grid g = plan_nf4(d, d.ws ? d.ws_bytes : 0);
  const unsigned nwg = (unsigned)(g.tiles_m * g.tiles_n * g.splits);
  if (nf4_big(d)) {
    if (d.layout == Layout::NT)
      hipLaunchKernelGGL((gemm_nf4_kernel<false, 256, 256, 4, 2>), dim3(nwg), dim3(512), 0, st, d, g);
    else
      hipLaunchKernelGGL((gemm_nf4_kernel<true, 256, 256, 4, 2>), dim3(nwg), dim3(512), 0, st, d, g);
  } else {
    if (d.layout == Layout::NT)
      hipLaunchKernelGGL((gemm_nf4_kernel<false, 128, 128, 2, 2>), dim3(nwg), dim3(256), 0, st, d, g);
    else
      hipLaunchKernelGGL((gemm_nf4_kernel<true, 128, 128, 2, 2>), dim3(nwg), dim3(256), 0, st, d, g);
  }
  QBLK_TRY(check_launch("gemm_nf4_kernel"));
  return finish_splits(d, g, st);
}

int finish_splits(const GemmDesc& d, const Grid& g, hipStream_t st) {
  if (g.splits > 1) {
    const dim3 grid((unsigned)ceil_div(d.N, 1024), (unsigned)std::min(d.M, 65535));
    if (out_vec4(d, g) && d.c_cols_blockdiag == 0 && ceil_div(d.M, 4) <= 65535) {
      const int threads = (int)std::min<int64_t>(256, ceil_div(ceil_div(d.N, 4), 64) * 64);
      const bool one = d.M <= 65535;  // grid.y limit
      const dim3 rgrid((unsigned)ceil_div(d.N, 4 * threads), (unsigned)ceil_div(d.M, one ? 1 : 4));
      if (one)
        hipLaunchKernelGGL(splitk_reduce_rows_kernel<1>, rgrid, dim3(threads), 0, st, d, g.splits);
      else
        hipLaunchKernelGGL(splitk_reduce_rows_kernel<4>, rgrid, dim3(threads), 0, st, d, g.splits);
    } else {
      hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(256), 0, st, d, g.splits, (int)out_vec4(d, g));
    }
    QBLK_TRY(check_launch("splitk_reduce_kernel"));
  }
  return 0;
}

// fp8 operands: NT, 8-bit storage of both, K a multiple of 128 (one
// 128-byte K tile), lda and ldb multiples of 16 and 16-byte aligned rows,
// a single B segment and no K extension.
bool f8_ok(const GemmDesc& d) {
  if (d.prec != Prec::FP8 || d.a_src != Src::F8 || d.b_src != Src::F8 || d.layout != Layout::NT) return false;
  if (d.K % 128 != 0 || d.K == 0 || d.lda % 16 != 0 || d.ldb % 16 != 0 || d.b.nseg != 1) return false;
  if ((uintptr_t)d.a % 16 != 0 || (uintptr_t)d.b.p[0] % 16 != 0 || d.ext.kext > 0) return false;
  return (unsigned)d.f8_a_e5m2 <= 1 && (unsigned)d.f8_b_e5m2 <= 1;
}

// The fp8 product runs on the 128 x 128 direct-to-LDS kernel with the
// descriptor in 16-bit units; planning (tiles, split-K) is that of a
// 16-bit product of half the K.
GemmDesc f8_units(const GemmDesc& d) {
  GemmDesc u = d;
  u.K = d.K / 2;
  u.lda = d.lda / 2;
  u.ldb = d.ldb / 2;
  return u;
}

int launch_f8(const GemmDesc& d, hipStream_t st) {
  const GemmDesc u = f8_units(d);
  Grid g = plan_tiles(u, u.ws ? u.ws_bytes : 0, F8Cfg::bm, F8Cfg::bn, 64, -2 * kTargetWgs);
  g.bn = F8Cfg::bn;
  g.vec = out_vec4(u, g);
  F8Cfg::launch8(u, g, st);
  QBLK_TRY(check_launch("gemm_dma_kernel (fp8)"));
  return finish_splits(u, g, st);
}

// fp32 products on the direct-to-LDS kernel: K a multiple of 32, lda and
// ldb multiples of 4, 16-byte aligned rows, no K extension; for NN and TN
// the M/N-contiguous operands' widths multiples of 4 and a single B
// segment. The descriptor goes over in 16-bit units (K, lda, ldb doubled),
// so tiles, copies and the K-major fragment reads are the 16-bit kernel's
// (each 16-byte fragment holds 4 fp32 K values); M/N-contiguous operands
// take DmaOperandF32MN.
bool f32dma_fits(const GemmDesc& d) {
  if (d.prec != Prec::F32 || d.a_src != Src::F32 || d.b_src != Src::F32) return false;
  if (d.ext.kext > 0 || d.K % 32 != 0 || d.K == 0 || d.lda % 4 != 0 || d.ldb % 4 != 0) return false;
  if ((uintptr_t)d.a % 16 != 0) return false;
  for (int s = 0; s < d.b.nseg; ++s)
    if ((uintptr_t)d.b.p[s] % 16 != 0) return false;
  if (d.layout == Layout::TN && (d.M % 4 != 0 || d.M < 4)) return false;
  if (d.layout != Layout::NT) {
    // M/N-contiguous B: its segments (along K) start on 32-row K tiles
    if (d.N % 4 != 0 || d.N < 4) return false;
    for (int s = 1; s < d.b.nseg; ++s)
      if (d.b.start[s] % 32 != 0) return false;
  }
  return true;
}

GemmDesc f32_units(const GemmDesc& d) {
  GemmDesc u = d;
  u.K = 2 * d.K;
  u.lda = 2 * d.lda;
  u.ldb = 2 * d.ldb;
  return u;
}

Grid plan_f32dma(const GemmDesc& u, size_t ws_bytes) {
  Grid g = plan_tiles(u, ws_bytes, Nt16Small::bm, Nt16Small::bn, 64, -kTargetWgs);
  g.bn = Nt16Small::bn;
  g.deep = g.tiles_m * g.tiles_n * g.splits <= kTargetWgs;
  g.vec = out_vec4(u, g);
  return g;
}

// fp32 products that fit the direct-to-LDS kernel run on it, with 128 x 128
// tiles when they give at least two rounds of workgroups or at least 4096
// K per workgroup (the LM head: the fill per FLOP halves), else with 64 x 64
// tiles of 4 waves split over K up to one workgroup per CU. Measured (one
// MI355X) against the register-staged kernel's 64-wide tiles: the
// vocabulary-151936 LM head 1.47 -> 1.28 ms (logits, NT), 1.55-1.60 ->
// 1.23 ms (dX, NN, 32 tiles in 8 splits), 1.69 -> 1.31 ms (dW, TN), where
// 64 x 64 tiles took 1.43, 1.32-1.49 and 1.43 ms; every product of a
// seq-1024 layer of the 36-layer stack faster on 64 x 64 tiles (NN 1024 x
// 512 x 768 23.3 -> 16.1 us, TN 768 x 512 x 1024 25.4 -> 18.3 us, NN 1024
// x 512 x 2816 51.6 -> 34 us; the twelve 321 -> 294 us), which also beat
// 128 x 128 tiles on them (NT 1024 x 2816 x 512 35.6-38.9 -> 33.8 us).
Grid plan_f32dma64(const GemmDesc& u, size_t ws_bytes) {
  Grid g = plan_tiles(u, ws_bytes, F32Small::bm, F32Small::bn, 64, -kTargetWgs);
  g.bn = F32Small::bn;
  g.deep = 0;
  g.vec = out_vec4(u, g);
  return g;
}

// 0: register-staged kernel; 1: 64 x 64 direct-to-LDS tiles; 2: 128 x 128
// (decided on the unlimited-workspace plan, so that gemm_workspace and the
// launch agree whatever workspace the caller then passes).
int f32dma_kind(const GemmDesc& d, size_t ws_bytes) {
  if (!f32dma_fits(d)) return 0;
  const Grid g = plan_f32dma(f32_units(d), ws_bytes);
  const bool rounds2 = g.tiles_m * g.tiles_n * g.splits >= 2 * kTargetWgs;
  return rounds2 || g.kchunk / 2 >= 4096 ? 2 : 1;
}

int launch_f32dma64(const GemmDesc& d, hipStream_t st) {
  const GemmDesc u = f32_units(d);
  const Grid g = plan_f32dma64(u, u.ws ? u.ws_bytes : 0);
  F32Small::launch32(u, g, st);
  QBLK_TRY(check_launch("gemm_dma_kernel (fp32, 64 x 64)"));
  return finish_splits(u, g, st);
}

int launch_f32dma(const GemmDesc& d, hipStream_t st) {
  const GemmDesc u = f32_units(d);
  const Grid g = plan_f32dma(u, u.ws ? u.ws_bytes : 0);
  if (g.deep) Nt16Deep::launch32(u, g, st);
  else Nt16Small::launch32(u, g, st);
  QBLK_TRY(check_launch("gemm_dma_kernel (fp32)"));
  return finish_splits(u, g, st);
}

int launch_nt16(const GemmDesc& d, hipStream_t st) {
  const Grid g = plan(d, d.ws ? d.ws_bytes : 0);
  if (nt16_big(d)) Nt16Big::launch(d, g, st);
  else if (g.deep) Nt16Deep::launch(d, g, st);
  else Nt16Small::launch(d, g, st);
  QBLK_TRY(check_launch("gemm_dma_kernel"));
  return finish_splits(d, g, st);
}

template <Prec P, Layout L, Src AS, Src BS, bool EXT>
int launch(const GemmDesc& d, hipStream_t st) {
  const Grid g = plan(d, d.ws ? d.ws_bytes : 0);
  const unsigned nwg = (unsigned)(g.tiles_m * g.tiles_n * g.splits);
  if (reg_small_tiles(d))
    hipLaunchKernelGGL((gemm_kernel<P, L, AS, BS, EXT, 2, 2, 1, 1, PT<P>::BK>), dim3(nwg), dim3(256), 0, st, d, g);
  else
    hipLaunchKernelGGL((gemm_kernel<P, L, AS, BS, EXT, 2, 2, 2, 2, PT<P>::BK>), dim3(nwg), dim3(256), 0, st, d, g);
  QBLK_TRY(check_launch("gemm_kernel"));
  return finish_splits(d, g, st);
}

template <Prec P, Layout L>
int dispatch_src(const GemmDesc& d, hipStream_t st) {
  const bool ext = d.ext.kext > 0;
  if (nf4_fused_ok(d)) return launch_nf4(d, st);
  if (d.b_src == Src::NF4) {
    if constexpr (L == Layout::TN || P == Prec::F32) {
      return fail(QBLK_EUNSUPPORTED, "gemm: NF4 operand needs an NT/NN fp16 contraction");
    } else {
      if (d.a_src != Src::F32) return fail(QBLK_EUNSUPPORTED, "gemm: NF4 B needs fp32 A");
      return ext ? launch<P, L, Src::F32, Src::NF4, true>(d, st)
                 : launch<P, L, Src::F32, Src::NF4, false>(d, st);
    }
  }
  if (ext) {
    if constexpr (L == Layout::TN || P == Prec::F32) {
      return fail(QBLK_EUNSUPPORTED, "gemm: K extension needs an NT/NN fp16 contraction");
    } else {
      if (d.a_src != Src::F32 || d.b_src != Src::F32)
        return fail(QBLK_EUNSUPPORTED, "gemm: K extension needs fp32 operands");
      return launch<P, L, Src::F32, Src::F32, true>(d, st);
    }
  }
  if (d.a_src == Src::F32 && d.b_src == Src::F32) return launch<P, L, Src::F32, Src::F32, false>(d, st);
  if constexpr (P == Prec::F16) {
    if (d.a_src == Src::F16 && d.b_src == Src::F32) return launch<P, L, Src::F16, Src::F32, false>(d, st);
    if (d.a_src == Src::F32 && d.b_src == Src::F16) return launch<P, L, Src::F32, Src::F16, false>(d, st);
    if (d.a_src == Src::F16 && d.b_src == Src::F16) {
      if (nt16_ok(d)) return launch_nt16(d, st);
      return launch<P, L, Src::F16, Src::F16, false>(d, st);
    }
  }
  return fail(QBLK_EUNSUPPORTED, "gemm: operand storage combination (fp16 storage needs fp16 contraction)");
}

int elems16(Src s) { return s == Src::F32 ? 4 : s == Src::F8 ? 16 : 8; }

}  // namespace

namespace {
__global__ void c16_copy_kernel(int M, int N, const float* __restrict__ c, int64_t ldc, f16* __restrict__ c16,
                                int64_t ldc16, int bf16) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= (int64_t)M * N) return;
  const int64_t r = e / N, col = e % N;
  c16[r * ldc16 + col] = to_16(c[r * ldc + col], bf16);
}
}  // namespace

int gemm(const GemmDesc& d, hipStream_t st) {
  if (d.c16) {
    if (d.c.nseg != 1 || d.c_cols_blockdiag > 0)
      return fail(QBLK_EINVAL, "gemm: the fp16 output copy needs a single C segment");
    if (!nt16_ok(d) && !nf4_fused_ok(d)) {  // kernels without the fp16 epilogue: copy afterwards
      GemmDesc e = d;
      e.c16 = nullptr;
      QBLK_TRY(gemm(e, st));
      const int64_t mn = (int64_t)d.M * d.N;
      hipLaunchKernelGGL(c16_copy_kernel, dim3((unsigned)ceil_div(mn, 256)), dim3(256), 0, st, d.M, d.N,
                         (const float*)d.c.p[0], d.ldc, d.c16, d.ldc16, (int)(d.prec == Prec::BF16));
      return check_launch("c16_copy_kernel");
    }
  }
  if (d.M <= 0 || d.N <= 0 || d.K < 0) return fail(QBLK_EINVAL, "gemm: bad shape %d x %d x %d", d.M, d.N, d.K);
  if (d.K == 0 && d.ext.kext == 0) return fail(QBLK_EINVAL, "gemm: empty contraction");
  // Contiguous dimensions and leading dimensions are read in 16-byte chunks.
  const bool a_rows = d.layout != Layout::TN;
  const int ea = elems16(d.a_src), eb = elems16(d.b_src);
  if ((a_rows ? d.K : d.M) % ea != 0 || d.lda % ea != 0)
    return fail(QBLK_EINVAL, "gemm: A contiguous dim and lda must be multiples of %d", ea);
  if ((d.layout == Layout::NT ? d.K : d.N) % eb != 0 || d.ldb % eb != 0)
    return fail(QBLK_EINVAL, "gemm: B contiguous dim and ldb must be multiples of %d", eb);
  if (d.ext.kext % 4 != 0) return fail(QBLK_EINVAL, "gemm: K extension must be a multiple of 4");
  if (d.ext.kext > (d.prec == Prec::F16 ? 64 : 32))
    return fail(QBLK_EUNSUPPORTED, "gemm: K extension wider than one K tile");
  if (d.prec == Prec::FP8) {
    if (!f8_ok(d))
      return fail(QBLK_EUNSUPPORTED, "gemm: fp8 operands need NT layout, 8-bit storage of both, K a multiple of "
                                     "128, lda and ldb multiples of 16 and 16-byte aligned rows");
    return launch_f8(d, st);
  }
  if (d.a_src == Src::F8 || d.b_src == Src::F8)
    return fail(QBLK_EINVAL, "gemm: 8-bit storage goes with fp8 operands only");
  if (d.prec == Prec::BF16) {
    if (!nt16_ok(d))
      return fail(QBLK_EUNSUPPORTED, "gemm: bfloat16 operands need 16-bit storage of both operands, K a multiple "
                                     "of 64 and 16-byte aligned rows");
    return launch_nt16(d, st);
  }
  switch (f32dma_kind(d, (size_t)-1)) {  // by shape alone, as gemm_workspace decides
    case 2: return launch_f32dma(d, st);
    case 1: return launch_f32dma64(d, st);
    default: break;
  }
  if (d.prec == Prec::F32) {
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

bool gemm_nf4_fused(const GemmDesc& d) { return nf4_fused_ok(d); }

size_t gemm_nf4_workspace(int M, int N, int k_total) {
  GemmDesc e;
  e.M = M; e.N = N; e.K = k_total;
  const Grid g = plan_nf4(e, (size_t)-1);
  return g.splits > 1 ? (size_t)g.splits * M * N * sizeof(float) : 0;
}

size_t gemm_workspace(const GemmDesc& d) {
  if (d.prec == Prec::FP8) {
    const Grid g = plan_tiles(f8_units(d), (size_t)-1, F8Cfg::bm, F8Cfg::bn, 64, -2 * kTargetWgs);
    return g.splits > 1 ? (size_t)g.splits * d.M * d.N * sizeof(float) : 0;
  }
  const Grid g = nf4_fused_ok(d) ? plan_nf4(d, (size_t)-1)
                 : f32dma_kind(d, (size_t)-1) == 2 ? plan_f32dma(f32_units(d), (size_t)-1)
                 : f32dma_kind(d, (size_t)-1) == 1 ? plan_f32dma64(f32_units(d), (size_t)-1)
                                  : plan(d, (size_t)-1);
  return g.splits > 1 ? (size_t)g.splits * d.M * d.N * sizeof(float) : 0;
}

}  // namespace qblk
