// Combine: gather each token's k expert-output rows back to token order as a
// weighted sum.
//
// Source: "MORI-EP User Guide", section 3 combine() (expert outputs, weights
// "for weighted combination", indices as for dispatch; output rows at the
// tokens' original positions) and section 4 combine_standard_moe() for the
// expert-major input; "Choosing an EP API and backend": gather combine in
// BF16/FP32.  Arithmetic: fp32 accumulator starting at +0, one fused
// multiply-add per top-k position in order j = 0..k-1, then bf16 round to
// nearest even -- a fixed order, so the result does not depend on timing.
//
// A row is cut into slices of 2 x 16 bytes per lane (2 KiB per wave); one wave
// handles one (token, slice), so a 4096-token batch runs ~29k short waves.
// Each distinct expert-output row is loaded once (positions that share a rank
// row reuse its registers) with non-temporal loads -- the rows are read
// exactly once -- and all of a slice's loads are issued before the FMAs.
#include "dev.h"
#include "mep_internal.h"

namespace mep {

namespace {

constexpr int kUnitsPerLane = 2;

template <int KMAX, bool DEDUPE>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = g / a.slices, sl = g - t * a.slices;
  if (t >= a.T) return;
  const int nv = a.H / 8;
  int row[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    row[j] = j < a.k ? a.rows[(size_t)t * a.k + j] : -1;
    w[j] = j < a.k ? a.w[(size_t)t * a.k + j] : 0.0f;
  }
  // src[j]: first top-k position holding the same row as j (uniform)
  int src[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    src[j] = j;
    if (DEDUPE) {
#pragma unroll
      for (int jj = KMAX - 1; jj >= 0; --jj)
        if (jj < j && row[jj] == row[j]) src[j] = jj;
    }
  }
  const u32x4* y = reinterpret_cast<const u32x4*>(a.y);
  u32x4* out = reinterpret_cast<u32x4*>(a.out) + (size_t)t * nv;
  const int v0 = sl * (kWave * kUnitsPerLane) + lane;
  u32x4 in[kUnitsPerLane][KMAX];
#pragma unroll
  for (int u = 0; u < kUnitsPerLane; ++u) {
    const int v = v0 + u * kWave;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      in[u][j] = u32x4{0, 0, 0, 0};
      if (row[j] >= 0 && src[j] == j && v < nv)
        in[u][j] = __builtin_nontemporal_load(y + (size_t)row[j] * nv + v);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnitsPerLane; ++u) {
    const int v = v0 + u * kWave;
    if (v >= nv) continue;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (row[j] < 0) continue;  // uniform: position skipped (token not dispatched)
      u32x4 x = in[u][j];
      if (DEDUPE) {
#pragma unroll
        for (int jj = 0; jj < j; ++jj)
          if (src[j] == jj) x = in[u][jj];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(w[j], bf16_lo(x[i]), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(w[j], bf16_hi(x[i]), acc[2 * i + 1]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16_rne(acc[2 * i], acc[2 * i + 1]);
    store_nt(out + v, o);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a0, hipStream_t s) {
  if (a0.T == 0) return hipSuccess;
  CombineArgs a = a0;
  const int per = kWave * kUnitsPerLane;
  a.slice_units = per;
  a.slices = (a.H / 8 + per - 1) / per;
  const int blocks = (int)(((int64_t)a.T * a.slices + 3) / 4);
  if (a.k <= 8) {
    if (a.distinct_rows) combine_kernel<8, false><<<blocks, 256, 0, s>>>(a);
    else combine_kernel<8, true><<<blocks, 256, 0, s>>>(a);
  } else {
    combine_kernel<kMaxTopk, false><<<blocks, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mep
