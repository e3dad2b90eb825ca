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
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

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

__device__ __forceinline__ half4 to_half4(float4 v) {
  half4 h;
  h[0] = (f16)v.x;
  h[1] = (f16)v.y;
  h[2] = (f16)v.z;
  h[3] = (f16)v.w;
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
