// Shared device and host helpers of libqblk (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace qblk {

typedef _Float16 f16;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ------------------------------------------------------------ error state
// A thread-local message read back through qblk_last_error(). Every entry
// point returns 0 or one of the negative codes of qblk.h.
int fail(int code, const char* fmt, ...);
int check_hip(hipError_t e, const char* what);
int check_launch(const char* what);

#define QBLK_TRY(expr)          \
  do {                          \
    int _rc = (expr);           \
    if (_rc != 0) return _rc;   \
  } while (0)

// ------------------------------------------------------- wave reductions
// Lane exchanges without the LDS crossbar: DPP within rows of 16 lanes
// (quad permutations, then the mirrors within 8 and 16 lanes) and the
// row swaps of v_permlane16/32_swap above. Each step adds a value equal in
// every lane of a group to the other group's; fp addition commutes, so every
// lane of a group ends with bitwise the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + dpp_f<CTRL>(v);
}
// Lane i's value combined with lane i ^ 32's (v_permlane32_swap), the same
// in both lanes.
__device__ __forceinline__ float2 cross_half(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return make_float2(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float cross_half_sum(float v) {
  const float2 r = cross_half(v);
  return r.x + r.y;
}
__device__ __forceinline__ float cross_half_max(float v) {
  const float2 r = cross_half(v);
  return fmaxf(r.x, r.y);
}
// Sum over aligned groups of N lanes (N a power of two, 1..64).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "group size");
  if constexpr (N >= 2) v = dpp_add<0xB1>(v);   // quad_perm 1,0,3,2
  if constexpr (N >= 4) v = dpp_add<0x4E>(v);   // quad_perm 2,3,0,1
  if constexpr (N >= 8) v = dpp_add<0x141>(v);  // row_half_mirror
  if constexpr (N >= 16) v = dpp_add<0x140>(v); // row_mirror
  if constexpr (N >= 32) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  }
  if constexpr (N >= 64) v = cross_half_sum(v);
  return v;
}

// Whole-wave sum; call in uniform control flow (every lane active).
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// fp32 -> fp16 with round-to-nearest-even (v_cvt_f16_f32 under the default
// rounding mode; the packed round-toward-zero conversion is never used).
__device__ __forceinline__ f16 to_f16(float x) { return (f16)x; }

// bfloat16 operands (gemm_precision 2) travel in the same 16-bit buffers as
// fp16 ones: the buffers are typed f16 as plain 16-bit containers and hold
// bfloat16 bit patterns when `bf` is set. fp32 -> bf16 rounds to nearest
// even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16 to_16(float x, bool bf) {
  return bf ? __builtin_bit_cast(f16, (bf16)x) : (f16)x;
}

__device__ __forceinline__ half4 to_half4(float4 v) {
  half4 h;
  h[0] = (f16)v.x;
  h[1] = (f16)v.y;
  h[2] = (f16)v.z;
  h[3] = (f16)v.w;
  return h;
}

// v_mfma_f32_32x32x16_f16, or its bfloat16 twin on the same 16-bit lanes.
template <bool BF>
__device__ __forceinline__ floatx16 mfma16(half8 a, half8 b, floatx16 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half4 to_16x4(float4 v, bool bf) {
  if (!bf) return to_half4(v);
  half4 h;
  h[0] = __builtin_bit_cast(f16, (bf16)v.x);
  h[1] = __builtin_bit_cast(f16, (bf16)v.y);
  h[2] = __builtin_bit_cast(f16, (bf16)v.z);
  h[3] = __builtin_bit_cast(f16, (bf16)v.w);
  return h;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------- direct global -> LDS copies
// global_load_lds_dwordx4: each lane reads 16 bytes at its own global
// address; the wave's 64 results land contiguously (lane order) at one
// wave-uniform LDS address. Completion is counted by vmcnt.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds, 16, 0, 0);
}

// The same copy issued through inline assembly, invisible to the compiler's
// wait-count tracking: with copies the compiler knows to be in flight it
// makes every LDS read's consumer wait for all outstanding LDS reads. The
// caller orders these copies itself (wait_vmcnt, then a barrier, before
// the tile is read); M0 carries the wave-uniform LDS address.
__device__ __forceinline__ void dma16_asm(const void* g, void* lds) {
  // the low 32 bits of a generic LDS address are its LDS offset
  const unsigned m = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(m) : "memory", "m0");
}

// s_waitcnt with only the vector-memory count limited (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace qblk
