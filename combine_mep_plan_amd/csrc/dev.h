// Device helpers for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mep {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of m strictly below this lane.
__device__ __forceinline__ int bits_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int first_lane(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int lane_value(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

// bf16 halves of a packed dword, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (a in the low half), round to nearest even.
// gfx950 has a packed convert that rounds per the MODE register (round to
// nearest even by default) and quiets NaNs.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  const uint16_t lo = __builtin_bit_cast(uint16_t, (__bf16)a);
  const uint16_t hi = __builtin_bit_cast(uint16_t, (__bf16)b);
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Four fp32 -> four OCP E4M3 codes packed in a dword (a in the low byte),
// round to nearest even.  gfx950's packed FP8 convert produces the OCP
// encoding; callers only pass |v| <= 448 * (1 + 2^-23).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ void store_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(u32x2* p, u32x2 v) { __builtin_nontemporal_store(v, p); }

}  // namespace mep
