// Expert-major expert outputs back to the rank-major combine input.
//
// Source: "MORI-EP User Guide", section 4 Standard MoE Compatibility:
// convert_combine_input() takes the experts' packed (expert-major) outputs,
// their source info and layout range, and gives back the rows combine()
// takes.  The pages pass no weights to it; this library's reading: a
// converted row (rank r, slot s) is the fp32 chain, in top-k order, of
// fmaf(w_j, y_j, acc) over the token's positions j on rank r that are the
// first naming their expert, w_j the dispatched weight of position j (the
// receive row's own weight copy) and y_j that expert's expert-major row,
// rounded once to bf16.  One merged row per (token, rank) can carry a top-k
// weighted sum only if each weight is applied before the merge; the combine
// of converted rows (MEP_RANK_SUM) then adds the rank rows unweighted.
//
// Where the rows are: the plan's receive row of each (token, top-k position)
// groups the positions by rank (equal receive rows), and the expert-major
// conversion's row of each position locates its expert output (-1 for a
// position repeating an earlier position's expert, or dropped past cap_em).
//
// Up to top-8, one wave per (token, 512-byte slice of its rows), a token's
// waves in one workgroup (two beyond 8192 columns): every expert-major row of
// the token is loaded once with non-temporal loads (each is read by exactly
// one wave), all loads before the multiply-adds, and each rank row is written
// once with non-temporal stores.  At 4096 x 7168 on 32 ranks: 170.5 us,
// against 171.2 us with the same slices in four-wave workgroups (tokens cut
// across workgroups) and 175.0 us with 1 KiB slices either way; 179 us with
// 2 KiB slices and 182 us with one wave per (token, rank, slice).  Beyond
// top-8 the positions are taken rank by rank with ordinary loads, 1 KiB
// slices in four-wave workgroups.
#include <type_traits>

#include "dev.h"
#include "mep_internal.h"

namespace mep {

namespace {

constexpr int kUnits = 1;  // beyond top-8: 16-byte units per lane per wave (8 bf16 each)

constexpr int kConvLaneBytes = 8;  // top-8: bytes of each row per lane
constexpr int kConvMaxWaves = 16;

template <int KMAX, int LB>
__global__ __launch_bounds__(kConvMaxWaves * 64) void convert_kernel(ConvertArgs a) {
  using V = typename std::conditional<LB == 16, u32x4, u32x2>::type;
  constexpr int NW = LB / 4;  // bf16 pairs per lane
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x / a.wg_per_tok;
  const int sl = (blockIdx.x - t * a.wg_per_tok) * a.waves_per_wg + first_lane(threadIdx.x >> 6);
  if (t >= a.T || sl >= a.slices) return;
  const uint32_t first = a.ufirst[t];  // positions owning their rank's row
  if (first == 0) return;              // token not dispatched
  const int nv = a.H * 2 / LB;
  int rr[KMAX], er[KMAX], lead[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rr[j] = j < a.k ? a.rrow[(size_t)t * a.k + j] : -1;
    er[j] = j < a.k ? a.em_row[(size_t)t * a.k + j] : -1;
  }
  // lead[j]: the position owning j's rank row (uniform)
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    lead[j] = j;
#pragma unroll
    for (int jj = KMAX - 1; jj >= 0; --jj)
      if (jj < j && rr[jj] == rr[j]) lead[j] = jj;
  }
  const V* y = reinterpret_cast<const V*>(a.y_em);
  const int v = sl * kWave + lane;
  V in[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    w[j] = er[j] >= 0 ? a.recv_w[(size_t)rr[j] * a.k + j] : 0.0f;
    in[j] = V{};
    if (er[j] >= 0 && v < nv) in[j] = __builtin_nontemporal_load(y + (size_t)er[j] * nv + v);
  }
  if (v >= nv) return;
  V* out = reinterpret_cast<V*>(a.y);
#pragma unroll
  for (int L = 0; L < KMAX; ++L) {
    if (!((first >> L) & 1u)) continue;  // uniform: L owns a rank row
    float acc[2 * NW];
#pragma unroll
    for (int i = 0; i < 2 * NW; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = L; j < KMAX; ++j) {
      if (lead[j] != L || er[j] < 0) continue;  // uniform
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        acc[2 * i] = __builtin_fmaf(w[j], bf16_lo(in[j][i]), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(w[j], bf16_hi(in[j][i]), acc[2 * i + 1]);
      }
    }
    V o;
#pragma unroll
    for (int i = 0; i < NW; ++i) o[i] = pack_bf16_rne(acc[2 * i], acc[2 * i + 1]);
    store_nt(out + (size_t)rr[L] * nv + v, o);
  }
}

// Beyond top-8: rank by rank, each rank's positions loaded in turn (ordinary
// loads; the route entries are re-read from the caches).
__global__ __launch_bounds__(256) void convert_wide_kernel(ConvertArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = g / a.slices, sl = g - t * a.slices;
  if (t >= a.T) return;
  const uint32_t first = a.ufirst[t];
  const int nv = a.H / 8;
  const int32_t* rr = a.rrow + (size_t)t * a.k;
  const int32_t* er = a.em_row + (size_t)t * a.k;
  const u32x4* y = reinterpret_cast<const u32x4*>(a.y_em);
  u32x4* out = reinterpret_cast<u32x4*>(a.y);
  const int v0 = sl * (kWave * kUnits) + lane;
  for (uint32_t m = first; m; m &= m - 1) {  // uniform
    const int L = __builtin_ctz(m);
    const int row = rr[L];
    float acc[kUnits][8];
#pragma unroll
    for (int u = 0; u < kUnits; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
    for (int j = L; j < a.k; ++j) {
      const int e = er[j];
      if (rr[j] != row || e < 0) continue;  // uniform
      const float wj = a.recv_w[(size_t)row * a.k + j];
#pragma unroll
      for (int u = 0; u < kUnits; ++u) {
        const int v = v0 + u * kWave;
        const u32x4 x = v < nv ? y[(size_t)e * nv + v] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[u][2 * i] = __builtin_fmaf(wj, bf16_lo(x[i]), acc[u][2 * i]);
          acc[u][2 * i + 1] = __builtin_fmaf(wj, bf16_hi(x[i]), acc[u][2 * i + 1]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int v = v0 + u * kWave;
      if (v >= nv) continue;
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16_rne(acc[u][2 * i], acc[u][2 * i + 1]);
      store_nt(out + (size_t)row * nv + v, o);
    }
  }
}

}  // namespace

hipError_t launch_convert_combine_input(const ConvertArgs& a0, hipStream_t s) {
  if (a0.T == 0) return hipSuccess;
  ConvertArgs a = a0;
  if (a.k > 8) {
    const int per = kWave * kUnits;
    a.slices = (a.H / 8 + per - 1) / per;
    const int blocks = (int)(((int64_t)a.T * a.slices + 3) / 4);
    convert_wide_kernel<<<blocks, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  // a token's waves in as few workgroups as possible
  a.slices = (a.H * 2 / kConvLaneBytes + kWave - 1) / kWave;
  a.wg_per_tok = (a.slices + kConvMaxWaves - 1) / kConvMaxWaves;
  a.waves_per_wg = (a.slices + a.wg_per_tok - 1) / a.wg_per_tok;
  const int64_t blocks = (int64_t)a.T * a.wg_per_tok;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  convert_kernel<8, kConvLaneBytes><<<(unsigned)blocks, kWave * a.waves_per_wg, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mep
