// Payload conversions shared by the dispatch kernels: how a token row becomes
// the bytes of a received row.  A lane owns one output item of the row: 16
// bytes of 8 bf16 values, 16 OCP E4M3 codes or 32 carried E2M1 codes, or, for
// MX FP4, 8 bytes of 16 packed E2M1 codes (half an MX block).
//
// Sources: "MORI-EP User Guide" section 3 dispatch() (rows with their scales);
// "Choosing an EP API and backend": OCP E4M3 is the gfx950 FP8 flavour, the
// HIP backend's dispatch can move FP8/FP4 rows that arrive quantized, gfx950
// has FP4 conversion.  The block formats (E4M3 with an fp32 scale per 128 columns;
// OCP MX FP4 with an E8M0 scale per 32 columns) are this library's readings.
#pragma once

#include <type_traits>

#include "dev.h"
#include "mep_internal.h"

namespace mep {

// x / b rounded to nearest even in fp32, from y = 1/b rounded to nearest:
// q1 = x*y is within a few ulps of x/b; one correction with the exact
// remainder x - q*b (a fused multiply-add) makes it faithful and a second
// one makes it the correctly rounded quotient (Markstein's theorem, which
// holds while the remainders stay normal: the caller keeps b >= 2^-60, where
// every quotient of magnitude >= 2^-11 has a normal remainder).  The sign of
// a zero quotient is x's.  Three fused multiply-adds and two multiplies
// instead of an IEEE division each.
__device__ __forceinline__ float div_by_recip(float x, float b, float y) {
  const float q1 = x * y;
  const float r1 = __builtin_fmaf(-q1, b, x);
  const float q2 = __builtin_fmaf(r1, y, q1);
  const float r2 = __builtin_fmaf(-q2, b, x);
  return __builtin_copysignf(__builtin_fmaf(r2, y, q2), x);
}

// FP8 block quantisation of one lane's 16 columns (in0: columns 0..7, in1:
// 8..15, bf16) into 16 OCP E4M3 codes: the 8 lanes of a 128-column block share
// scale = amax / 448 (fp32 division); codes are E4M3(x / scale) with the
// quotient correctly rounded and the packed convert (round to nearest even);
// an all-zero block gives scale 0 and signed-zero codes.
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
  } else if (s >= 0x1p-60f) {
    const float y = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_e4m3x4(div_by_recip(f[4 * i], s, y), div_by_recip(f[4 * i + 1], s, y),
                         div_by_recip(f[4 * i + 2], s, y), div_by_recip(f[4 * i + 3], s, y));
  } else {  // blocks with amax below 448 * 2^-60
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_e4m3x4(f[4 * i] / s, f[4 * i + 1] / s, f[4 * i + 2] / s, f[4 * i + 3] / s);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// OCP MX FP4 encoding of half a block: this lane's 16 columns (in0: columns
// 0..7, in1: 8..15, bf16 pairs); the lane holding the block's other half is
// lane ^ 1, so every lane of the wave must call this.  Shared exponent
// floor(log2(amax)) - 2 over the block's 32 columns, clamped to [-127, 127],
// from amax's exponent field (a subnormal or zero amax clamps to -127, so an
// all-zero block gets scale byte 0 and signed-zero codes); codes
// E2M1(x / 2^exponent), round to nearest with ties to the even code,
// saturating at 6, sign kept.  Even column in the low nibble.
//
// amax is taken on the bf16 bit patterns: for finite values |x| orders like
// its bits with the sign cleared, two columns per packed 16-bit max.  The
// codes come from gfx950's scaled packed-bf16 -> FP4 convert, which divides
// each value by the scale and rounds as above (checked on the GPU against the
// rule for every finite bf16 value under every scale 2^-127 .. 2^127); each
// call fills one byte (two columns) of an output word.  Its bf16 pairs are
// taken by shuffles of the input viewed as 8 bf16 values: a bit cast of each
// 32-bit word compiled to the first word for all four calls.
__device__ __forceinline__ u32x2 quant_mx4_half(u32x4 in0, u32x4 in1, uint32_t& e8) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m2 = {0, 0};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, in0[w] & 0x7fff7fffu));
    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, in1[w] & 0x7fff7fffu));
  }
  const int half = m2[0] > m2[1] ? m2[0] : m2[1];
  const int other = __shfl_xor(half, 1);
  const uint32_t amax = (uint32_t)(half > other ? half : other);  // bf16 bits of the block's amax
  const int biased = (int)(amax >> 7);
  const int se = max(biased - 127 - 2, -127);
  e8 = (uint32_t)(se + 127);
  // 2^se as an fp32 value (2^-127 is the subnormal with only mantissa bit 22 set)
  const float scale = __uint_as_float(se > -127 ? (uint32_t)(se + 127) << 23 : 0x00400000u);
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, i == 0 ? in0 : in1);
    uint32_t o = 0u;
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_shufflevector(x, x, 0, 1), scale, 0);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_shufflevector(x, x, 2, 3), scale, 1);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_shufflevector(x, x, 4, 5), scale, 2);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_shufflevector(x, x, 6, 7), scale, 3);
    w[i] = o;
  }
  return u32x2{w[0], w[1]};
}

// One lane's input for one output item (lane_items per row) and its
// conversion: 16 bytes out (bf16 copy, E4M3, carried rows) or 8 (MXFP4).
template <int QUANT>
struct Unit {
  static constexpr bool kQuantizes =
      QUANT == MEP_QUANT_FP8_E4M3_BLOCK128 || QUANT == MEP_QUANT_MXFP4;
  static constexpr int kIn = kQuantizes ? 2 : 1;  // 16 bf16 columns in
  using Out = typename std::conditional<QUANT == MEP_QUANT_MXFP4, u32x2, u32x4>::type;
  u32x4 in[kIn];

  // Item v of token t's row (zeros when !on).  Quantising modes read bf16
  // rows (H/8 units); copy modes read rows in the output format.  NT: with
  // non-temporal loads -- the standard-MoE scatter's choice (its call 70.3 ->
  // 69.0 us at 4096 x 7168 on 32 ranks); the rank-major dispatch keeps cached
  // loads (non-temporal ones cost its fused FP8 call 0.7 us).
  template <bool NT = false>
  __device__ __forceinline__ void load(const void* x, int t, int H, int v, bool on) {
    const int row_units = kIn > 1 ? H / 8 : payload_units(QUANT, H);
    const u32x4* src = reinterpret_cast<const u32x4*>(x) + (size_t)t * row_units + (size_t)v * kIn;
#pragma unroll
    for (int i = 0; i < kIn; ++i) {
      if (NT) in[i] = on ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
      else in[i] = on ? src[i] : u32x4{0, 0, 0, 0};
    }
  }

  // The output item; scale (FP8, shared by 8 lanes) or e8 (MXFP4, shared by
  // 2 lanes).  Every lane of the wave must call it (both shuffle).
  __device__ __forceinline__ Out convert(float& scale, uint32_t& e8) const {
    if constexpr (QUANT == MEP_QUANT_FP8_E4M3_BLOCK128) return quant16(in[0], in[1], scale);
    else if constexpr (QUANT == MEP_QUANT_MXFP4) return quant_mx4_half(in[0], in[1], e8);
    else return in[0];
  }
};

// The scales that belong to output item v of a row written at `row`.
template <int QUANT>
__device__ __forceinline__ void store_unit_scale(float* scales, size_t row, int H, int v,
                                                 float scale, uint32_t e8) {
  if constexpr (QUANT == MEP_QUANT_FP8_E4M3_BLOCK128) {
    if ((v & 7) == 0) scales[row * (H / 128) + (v >> 3)] = scale;
  } else if constexpr (QUANT == MEP_QUANT_MXFP4) {
    if ((v & 1) == 0) reinterpret_cast<uint8_t*>(scales)[row * (H / 32) + (v >> 1)] = (uint8_t)e8;
  }
}

// Carry modes: the caller's scale words of token t, copied by one wave.
__device__ __forceinline__ void copy_scale_row(float* dst, size_t row, const float* src, int t,
                                               int words, int lane) {
  for (int i = lane; i < words; i += kWave)
    dst[row * words + i] = src[(size_t)t * words + i];
}

}  // namespace mep
