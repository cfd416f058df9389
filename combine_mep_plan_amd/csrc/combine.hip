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
// One wavefront per token; each lane owns 8 columns (16 bytes) of every row.
// For each column group all k row loads are issued before the k FMAs, so a
// wave keeps k * 1 KiB of loads in flight.  A rank row shared by two top-k
// positions is loaded twice; the second load is served by the cache, so HBM
// reads stay one per (token, rank).
#include "dev.h"
#include "mep_internal.h"

namespace mep {

namespace {

template <int KMAX, int UNROLL>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  t = first_lane(t);
  const int nv = a.H / 8;
  int row[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    row[j] = j < a.k ? a.rows[(size_t)t * a.k + j] : -1;
    w[j] = j < a.k ? a.w[(size_t)t * a.k + j] : 0.0f;
  }
  const u32x4* y = reinterpret_cast<const u32x4*>(a.y);
  u32x4* out = reinterpret_cast<u32x4*>(a.out) + (size_t)t * nv;
  for (int v0 = 0; v0 < nv; v0 += kWave * UNROLL) {
    u32x4 in[UNROLL][KMAX];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int v = v0 + u * kWave + lane;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (row[j] >= 0 && v < nv) in[u][j] = y[(size_t)row[j] * nv + v];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int v = v0 + u * kWave + lane;
      if (v >= nv) continue;
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (row[j] < 0) continue;  // uniform
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = __builtin_fmaf(w[j], bf16_lo(in[u][j][i]), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(w[j], bf16_hi(in[u][j][i]), acc[2 * i + 1]);
        }
      }
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16_rne(acc[2 * i], acc[2 * i + 1]);
      store_nt(out + v, o);
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int blocks = (a.T + 3) / 4;
  if (a.k <= 8) combine_kernel<8, 2><<<blocks, 256, 0, s>>>(a);
  else combine_kernel<kMaxTopk, 1><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mep
