// Payload conversions shared by the dispatch kernels: how a token row becomes
// the bytes of a received row.  A lane owns one 16-byte output unit of the
// row: 8 bf16 values, 16 OCP E4M3 codes, or 32 packed E2M1 codes.
//
// Sources: "MORI-EP User Guide" section 3 dispatch() (rows with their scales);
// "Choosing an EP API and backend": OCP E4M3 is the gfx950 FP8 flavour, the
// HIP backend's dispatch can move FP8/FP4 rows that arrive quantized, gfx950
// has FP4 conversion.  The block formats (E4M3 with an fp32 scale per 128 columns;
// OCP MX FP4 with an E8M0 scale per 32 columns) are this library's readings.
#pragma once

#include "dev.h"
#include "mep_internal.h"

namespace mep {

// FP8 block quantisation of one lane's 16 columns (in0: columns 0..7, in1:
// 8..15, bf16) into 16 OCP E4M3 codes: the 8 lanes of a 128-column block share
// scale = amax / 448 (fp32 division); codes are E4M3(x / scale) by correctly
// rounded division and the packed convert (round to nearest even); an all-zero
// block gives scale 0 and signed-zero codes.
__device__ __forceinline__ u32x4 quant16(u32x4 in0, u32x4 in1, float& scale) {
  float f[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(in0[i]);
    f[2 * i + 1] = bf16_hi(in0[i]);
    f[8 + 2 * i] = bf16_lo(in1[i]);
    f[8 + 2 * i + 1] = bf16_hi(in1[i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  const float s = amax / 448.0f;
  scale = s;
  uint32_t w[4];
  if (s == 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = ((__float_as_uint(f[4 * i]) >> 31) << 7) |
             ((__float_as_uint(f[4 * i + 1]) >> 31) << 15) |
             ((__float_as_uint(f[4 * i + 2]) >> 31) << 23) |
             ((__float_as_uint(f[4 * i + 3]) >> 31) << 31);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_e4m3x4(f[4 * i] / s, f[4 * i + 1] / s, f[4 * i + 2] / s, f[4 * i + 3] / s);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// E2M1 code of v (round to nearest, ties to the even code, saturating at 6;
// sign kept): the magnitude code counts the rounding boundaries below |v|,
// with the boundaries that are ties between an odd and an even code belonging
// to the even side.  Magnitudes by code: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 31) << 3);
}

// OCP MX FP4 block of one lane's 32 columns (in[0..3], bf16): shared exponent
// floor(log2(amax)) - 2, clamped to [-127, 127], from amax's exponent field
// (a subnormal or zero amax clamps to -127, so an all-zero block gets scale
// byte 0 and signed-zero codes); codes E2M1(x * 2^-exponent), the product by a
// power of two being exact.  Even column in the low nibble.
__device__ __forceinline__ u32x4 quant_mx4(const u32x4 (&in)[4], uint32_t& e8) {
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[8 * i + 2 * w] = bf16_lo(in[i][w]);
      f[8 * i + 2 * w + 1] = bf16_hi(in[i][w]);
    }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
  const int biased = (int)(__float_as_uint(amax) >> 23);  // amax >= 0: no sign bit
  const int se = max(biased - 127 - 2, -127);
  e8 = (uint32_t)(se + 127);
  const float inv = __uint_as_float((uint32_t)(127 - se) << 23);  // 2^-se, a normal float
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i / 8] |= e2m1_code(f[i] * inv) << (4 * (i % 8));
  return u32x4{w[0], w[1], w[2], w[3]};
}

// One lane's input for one output unit and its conversion.
template <int QUANT>
struct Unit {
  static constexpr int kIn = QUANT == MEP_QUANT_FP8_E4M3_BLOCK128 ? 2
                             : QUANT == MEP_QUANT_MXFP4           ? 4
                                                                  : 1;
  u32x4 in[kIn];

  // Unit v of token t's row (zeros when !on).  Quantising modes read bf16
  // rows (H/8 units); copy modes read rows in the output format.
  __device__ __forceinline__ void load(const void* x, int t, int H, int v, bool on) {
    const int row_units = kIn > 1 ? H / 8 : payload_units(QUANT, H);
    const u32x4* src = reinterpret_cast<const u32x4*>(x) + (size_t)t * row_units + (size_t)v * kIn;
#pragma unroll
    for (int i = 0; i < kIn; ++i) in[i] = on ? src[i] : u32x4{0, 0, 0, 0};
  }

  // The output unit; scale (FP8, shared by 8 lanes) or e8 (MXFP4, this lane's
  // block).  Every lane of the wave must call it (FP8 shuffles).
  __device__ __forceinline__ u32x4 convert(float& scale, uint32_t& e8) const {
    if constexpr (QUANT == MEP_QUANT_FP8_E4M3_BLOCK128) return quant16(in[0], in[1], scale);
    else if constexpr (QUANT == MEP_QUANT_MXFP4) return quant_mx4(in, e8);
    else return in[0];
  }
};

// The scales that belong to output unit v of a row written at `row`.
template <int QUANT>
__device__ __forceinline__ void store_unit_scale(float* scales, size_t row, int H, int v,
                                                 float scale, uint32_t e8) {
  if constexpr (QUANT == MEP_QUANT_FP8_E4M3_BLOCK128) {
    if ((v & 7) == 0) scales[row * (H / 128) + (v >> 3)] = scale;
  } else if constexpr (QUANT == MEP_QUANT_MXFP4) {
    reinterpret_cast<uint8_t*>(scales)[row * (H / 32) + v] = (uint8_t)e8;
  }
}

// Carry modes: the caller's scale words of token t, copied by one wave.
__device__ __forceinline__ void copy_scale_row(float* dst, size_t row, const float* src, int t,
                                               int words, int lane) {
  for (int i = lane; i < words; i += kWave)
    dst[row * words + i] = src[(size_t)t * words + i];
}

}  // namespace mep
