// Combine: gather each token's k expert-output rows back to token order as a
// weighted sum.
//
// Source: "MORI-EP User Guide", section 3 combine() (expert outputs, the
// weights that scale each expert's contribution, indices as for dispatch;
// output rows at the tokens' original positions) and section 4
// combine_standard_moe() for the expert-major input; "Choosing an EP API and
// backend": the HIP backend's combine gathers in BF16 or FP32.  Arithmetic: fp32 accumulator starting at +0, one fused
// multiply-add per top-k position in order j = 0..k-1, then bf16 round to
// nearest even -- a fixed order, so the result does not depend on timing.
//
// Up to top-8 a row is cut into slices of 16 bytes per lane (1 KiB per wave;
// 8 bytes when a token's rows are all distinct, see kDistinctLaneBytes) and
// one workgroup takes one token, a wave per slice (14 waves at 7168 columns;
// rows wider than 16 KiB, 8 KiB at 8 bytes per lane, split over as few
// workgroups as possible): the pieces of each row the token gathers are then
// fetched together by one CU.  At 4096 x 7168 on 8 ranks the combine took
// 60.7 us this way, against 63.8 us with 2 KiB per wave and four waves per
// workgroup (tokens cut across workgroups) and 164 us with 1 KiB per wave in
// four-wave workgroups.  Each distinct expert-output row is loaded once (positions that share a rank row
// reuse its registers) with non-temporal loads -- the rows are read exactly
// once -- and all of a slice's loads are issued before the FMAs.  Wider
// top-k takes the positions in groups of 8, 2 KiB per wave (see below), and
// so does the E4M3 rounding in flight.
//
// Converted rank rows ("MORI-EP User Guide", section 4 convert_combine_input():
// each row already holds its rank's weighted expert outputs): the same kernel
// adds a token's distinct rank rows with unit weights, in the order of their
// first top-k position.
//
// FP8 direct-cast payload ("MORI-EP User Guide", section 10 Tuning: the
// intra-node tuning matrix pairs quant type fp8_direct_cast with a bf16
// combine; the cast rule -- OCP E4M3, no scale, round to nearest even,
// saturating at 448 -- is this library's reading): a cast launch turns the
// routed bf16 expert-output rows into E4M3 rows, and the E4M3 combine decodes
// each value exactly to fp32 and accumulates as above.
// A lane owns 16 columns there: one 16-byte E4M3 unit in, two bf16 units out.
// On one device the cast and the combine can also meet in registers: the bf16
// combine with ROUND takes every value of each loaded row through the same
// E4M3 encode and decode before the multiply-adds -- bit for bit the
// two-launch result, with the bf16 rows read once and no E4M3 rows written.
#include <type_traits>

#include "dev.h"
#include "mep_internal.h"

namespace mep {

namespace {

constexpr int kUnitsPerLane = 2;   // beyond top-8: 2 KiB of each row per wave
constexpr int kMaxWavesPerWg = 16;  // 1024 threads
// Top-8 combine of distinct rows (expert-major rows, converted rank rows):
// 8 bytes of each row per lane, so a wave keeps 8 x 512 bytes in flight.  At
// 4096 x 7168, eight expert-major rows per token, the combine took 88.1 us
// this way against 91.7 us with 16 bytes per lane (8 KiB per wave); the rank
// rows of a deduplicated combine (5.3 distinct per token at top-8 on 8
// ranks) keep 16 bytes per lane: 61.5 us against 72.5 us with 8.
constexpr int kDistinctLaneBytes = 8;
// The E4M3 rounding in flight converts every loaded value, so its waves stay
// busy longer after their loads: 2 KiB per wave keeps more bytes in flight
// (prefill step with it 114.5 us against 118.8 us with 1 KiB).
constexpr int kRoundUnitsPerLane = 2;

typedef float f32x2 __attribute__((ext_vector_type(2)));

// E4M3 of a bf16 pair's values, clamped to +-448 first so that the convert
// saturates.
__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Two values after the E4M3 direct cast and back (exact decode).
__device__ __forceinline__ void round_e4m3_pair(float& a, float& b) {
  const int p = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  const f32x2 r = __builtin_amdgcn_cvt_pk_f32_fp8(p, false);
  a = r.x;
  b = r.y;
}

// A unit of 8 bf16 values after the E4M3 direct cast and back, packed again as
// bf16: every E4M3 value is a bf16 value, so the repacking is exact.  Applied
// once to each loaded row, not once per top-k position using it.
__device__ __forceinline__ void round_e4m3_unit(u32x4& x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = bf16_lo(x[i]), hi = bf16_hi(x[i]);
    round_e4m3_pair(lo, hi);
    x[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
}

// SUM: the rows are converted rank rows that already carry the weights; each
// token's distinct rank rows (the positions owning them) are added with unit
// weight -- fmaf(1, y, acc) is acc + y with one rounding.
template <int KMAX, bool DEDUPE, bool ROUND, bool SUM = false, int UPL = 1, int LB = 16>
__global__ __launch_bounds__(kMaxWavesPerWg * 64) void combine_kernel(CombineArgs a) {
  static_assert(LB == 16 || (LB == 8 && !ROUND && !DEDUPE), "8-byte lanes: distinct rows only");
  using V = typename std::conditional<LB == 16, u32x4, u32x2>::type;
  constexpr int NW = LB / 4;  // bf16 pairs per lane unit
  constexpr int kUnitsPerLane = UPL;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x / a.wg_per_tok;
  const int part = blockIdx.x - t * a.wg_per_tok;  // which of the token's workgroups
  const int sl = part * a.waves_per_wg + first_lane(threadIdx.x >> 6);
  if (t >= a.T || sl >= a.slices) return;
  const int nv = a.H * 2 / LB;
  const uint32_t own = SUM ? a.ufirst[t] : 0xFFFFFFFFu;
  int row[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    row[j] = j < a.k && ((own >> j) & 1u) ? a.rows[(size_t)t * a.k + j] : -1;
    w[j] = SUM ? 1.0f : j < a.k ? a.w[(size_t)t * a.k + j] : 0.0f;
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
  const V* y = reinterpret_cast<const V*>(a.y);
  V* out = reinterpret_cast<V*>(a.out) + (size_t)t * nv;
  const int v0 = sl * (kWave * kUnitsPerLane) + lane;
  V in[kUnitsPerLane][KMAX];
#pragma unroll
  for (int u = 0; u < kUnitsPerLane; ++u) {
    const int v = v0 + u * kWave;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      in[u][j] = V{};
      if (row[j] >= 0 && src[j] == j && v < nv)
        in[u][j] = __builtin_nontemporal_load(y + (size_t)row[j] * nv + v);
    }
  }
  if constexpr (ROUND) {
#pragma unroll
    for (int u = 0; u < kUnitsPerLane; ++u)
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (row[j] >= 0 && src[j] == j) round_e4m3_unit(in[u][j]);
  }
#pragma unroll
  for (int u = 0; u < kUnitsPerLane; ++u) {
    const int v = v0 + u * kWave;
    if (v >= nv) continue;
    float acc[2 * NW];
#pragma unroll
    for (int i = 0; i < 2 * NW; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (row[j] < 0) continue;  // uniform: position skipped (token not dispatched)
      V x = in[u][j];
      if (DEDUPE) {
#pragma unroll
        for (int jj = 0; jj < j; ++jj)
          if (src[j] == jj) x = in[u][jj];
      }
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const float lo = bf16_lo(x[i]), hi = bf16_hi(x[i]);
        acc[2 * i] = __builtin_fmaf(w[j], lo, acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(w[j], hi, acc[2 * i + 1]);
      }
    }
    V o;
#pragma unroll
    for (int i = 0; i < NW; ++i) o[i] = pack_bf16_rne(acc[2 * i], acc[2 * i + 1]);
    store_nt(out + v, o);
  }
}

// Top-k beyond 8: the positions go in groups of 8, in order, each group
// loaded and accumulated before the next (registers for 8 rows per group
// instead of 32); inside a group, positions that share a rank row reuse its
// registers.  acc carries the fp32 chain across the groups, so the
// multiply-adds still run in j order.  A rank row named again in a later
// group is loaded again; the loads are ordinary cached ones so that such
// repeats can hit the caches (at top-16 on 8 ranks: 100 us against 116 us
// with non-temporal loads).
template <bool DEDUPE, bool ROUND, bool SUM = false>
__global__ __launch_bounds__(256) void combine_wide_kernel(CombineArgs a) {
  constexpr int G = 8;
  const int lane = threadIdx.x & 63;
  const int g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = g / a.slices, sl = g - t * a.slices;
  if (t >= a.T) return;
  const int nv = a.H / 8;
  const uint32_t own = SUM ? a.ufirst[t] : 0xFFFFFFFFu;
  const u32x4* y = reinterpret_cast<const u32x4*>(a.y);
  const int v0 = sl * (kWave * kUnitsPerLane) + lane;
  float acc[kUnitsPerLane][8];
#pragma unroll
  for (int u = 0; u < kUnitsPerLane; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
  for (int j0 = 0; j0 < a.k; j0 += G) {  // uniform
    int row[G], src[G];
    float w[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const int j = j0 + q;
      row[q] = j < a.k && ((own >> j) & 1u) ? a.rows[(size_t)t * a.k + j] : -1;
      w[q] = SUM ? 1.0f : j < a.k ? a.w[(size_t)t * a.k + j] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      src[q] = q;
      if (DEDUPE) {
#pragma unroll
        for (int qq = G - 1; qq >= 0; --qq)
          if (qq < q && row[qq] == row[q]) src[q] = qq;
      }
    }
    u32x4 in[kUnitsPerLane][G];
#pragma unroll
    for (int u = 0; u < kUnitsPerLane; ++u) {
      const int v = v0 + u * kWave;
#pragma unroll
      for (int q = 0; q < G; ++q) {
        in[u][q] = u32x4{0, 0, 0, 0};
        if (row[q] >= 0 && src[q] == q && v < nv)
          in[u][q] = y[(size_t)row[q] * nv + v];
      }
    }
    if (ROUND) {
#pragma unroll
      for (int u = 0; u < kUnitsPerLane; ++u)
#pragma unroll
        for (int q = 0; q < G; ++q)
          if (row[q] >= 0 && src[q] == q) round_e4m3_unit(in[u][q]);
    }
#pragma unroll
    for (int u = 0; u < kUnitsPerLane; ++u) {
#pragma unroll
      for (int q = 0; q < G; ++q) {
        if (row[q] < 0) continue;  // uniform
        u32x4 x = in[u][q];
        if (DEDUPE) {
#pragma unroll
          for (int qq = 0; qq < q; ++qq)
            if (src[q] == qq) x = in[u][qq];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = bf16_lo(x[i]), hi = bf16_hi(x[i]);
          acc[u][2 * i] = __builtin_fmaf(w[q], lo, acc[u][2 * i]);
          acc[u][2 * i + 1] = __builtin_fmaf(w[q], hi, acc[u][2 * i + 1]);
        }
      }
    }
  }
  u32x4* out = reinterpret_cast<u32x4*>(a.out) + (size_t)t * nv;
#pragma unroll
  for (int u = 0; u < kUnitsPerLane; ++u) {
    const int v = v0 + u * kWave;
    if (v >= nv) continue;
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16_rne(acc[u][2 * i], acc[u][2 * i + 1]);
    store_nt(out + v, o);
  }
}

// Up to top-8, each distinct row is loaded once.  Positions sharing a rank
// row (DEDUPE) read it back from LDS: every lane parks the units of the rows
// that later positions repeat in its own LDS slots (at most KMAX/2 per wave)
// and reads them at a uniform slot.  (Selecting among loaded registers, as
// the bf16 kernel does, here compiled to a dynamic register index with a
// wait after every load.)  Whether a position loads is folded into the lane's
// column bound, so the loads are masked instructions in straight-line code.
template <int KMAX, bool DEDUPE>
__global__ __launch_bounds__(256) void combine_fp8_kernel(CombineArgs a) {
  constexpr int kSlots = DEDUPE ? KMAX / 2 : 1;  // repeated rows per wave
  __shared__ u32x4 stage[4 * kSlots][kWave];
  const int lane = threadIdx.x & 63;
  const int g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = g / a.slices, sl = g - t * a.slices;
  if (t >= a.T) return;
  const int nv8 = a.H / 16;  // 16-byte E4M3 units per row
  int row[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    row[j] = j < a.k ? a.rows[(size_t)t * a.k + j] : -1;
    w[j] = j < a.k ? a.w[(size_t)t * a.k + j] : 0.0f;
  }
  // src[j]: first top-k position holding the same row as j; need: positions
  // whose row a later one repeats (both uniform)
  int src[KMAX];
  uint32_t need = 0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    src[j] = j;
    if (DEDUPE) {
#pragma unroll
      for (int jj = KMAX - 1; jj >= 0; --jj)
        if (jj < j && row[jj] == row[j]) src[j] = jj;
      if (src[j] != j) need |= 1u << src[j];
    }
  }
  const u32x4* y = reinterpret_cast<const u32x4*>(a.y);
  const int v = sl * kWave + lane;
  u32x4 in[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    in[j] = u32x4{0, 0, 0, 0};
    const int lim = row[j] >= 0 && src[j] == j ? nv8 : 0;
    if (v < lim) in[j] = __builtin_nontemporal_load(y + (size_t)row[j] * nv8 + v);
  }
  if (v >= nv8) return;
  u32x4(*mine)[kWave] = stage + (threadIdx.x >> 6) * kSlots;  // this wave's slots
  if (DEDUPE) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if ((need >> j) & 1u) mine[__popc(need & ((1u << j) - 1u))][lane] = in[j];
  }
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (row[j] < 0) continue;  // uniform
    u32x4 x = in[j];
    if (DEDUPE && src[j] != j) x = mine[__popc(need & ((1u << src[j]) - 1u))][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[i], false);  // bytes 0, 1
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[i], true);   // bytes 2, 3
      acc[4 * i] = __builtin_fmaf(w[j], lo.x, acc[4 * i]);
      acc[4 * i + 1] = __builtin_fmaf(w[j], lo.y, acc[4 * i + 1]);
      acc[4 * i + 2] = __builtin_fmaf(w[j], hi.x, acc[4 * i + 2]);
      acc[4 * i + 3] = __builtin_fmaf(w[j], hi.y, acc[4 * i + 3]);
    }
  }
  u32x4 o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0[i] = pack_bf16_rne(acc[2 * i], acc[2 * i + 1]);
    o1[i] = pack_bf16_rne(acc[8 + 2 * i], acc[8 + 2 * i + 1]);
  }
  u32x4* out = reinterpret_cast<u32x4*>(a.out) + (size_t)t * (a.H / 8) + 2 * v;
  store_nt(out, o0);
  store_nt(out + 1, o1);
}

// The E4M3 combine beyond top-8: positions in groups of 8, in order, each
// group's loads issued before its multiply-adds (cached loads, so that rank
// rows named again can come from the caches); acc carries the chain.
__global__ __launch_bounds__(256) void combine_fp8_wide_kernel(CombineArgs a) {
  constexpr int G = 8;
  const int lane = threadIdx.x & 63;
  const int g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = g / a.slices, sl = g - t * a.slices;
  if (t >= a.T) return;
  const int nv8 = a.H / 16;  // 16-byte E4M3 units per row
  const u32x4* y = reinterpret_cast<const u32x4*>(a.y);
  const int v = sl * kWave + lane;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  for (int j0 = 0; j0 < a.k; j0 += G) {  // uniform
    int row[G];
    float w[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const int j = j0 + q;
      row[q] = j < a.k ? a.rows[(size_t)t * a.k + j] : -1;
      w[q] = j < a.k ? a.w[(size_t)t * a.k + j] : 0.0f;
    }
    u32x4 in[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      in[q] = u32x4{0, 0, 0, 0};
      if (row[q] >= 0 && v < nv8) in[q] = y[(size_t)row[q] * nv8 + v];
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (row[q] < 0) continue;  // uniform
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)in[q][i], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)in[q][i], true);
        acc[4 * i] = __builtin_fmaf(w[q], lo.x, acc[4 * i]);
        acc[4 * i + 1] = __builtin_fmaf(w[q], lo.y, acc[4 * i + 1]);
        acc[4 * i + 2] = __builtin_fmaf(w[q], hi.x, acc[4 * i + 2]);
        acc[4 * i + 3] = __builtin_fmaf(w[q], hi.y, acc[4 * i + 3]);
      }
    }
  }
  if (v >= nv8) return;
  u32x4 o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0[i] = pack_bf16_rne(acc[2 * i], acc[2 * i + 1]);
    o1[i] = pack_bf16_rne(acc[8 + 2 * i], acc[8 + 2 * i + 1]);
  }
  u32x4* out = reinterpret_cast<u32x4*>(a.out) + (size_t)t * (a.H / 8) + 2 * v;
  store_nt(out, o0);
  store_nt(out + 1, o1);
}

// One wave per (token, 512 bytes of E4M3 output per row); the token's
// distinct rows in groups of 8, all loads of a group issued before its
// converts.  Lane l takes 8-column unit l of the wave's 64, so every load
// (1 KiB) and every store (512 bytes) is contiguous across the wave.  At 4096
// x 7168 on 8 ranks: 84.4 us, against 84.9 us with two units per lane (l and
// l + 64), 89.7 us with each lane's 16 columns adjacent (32-byte strided
// loads and stores) and 88.5 us with a token's waves in one workgroup.
template <bool RANK_MAJOR>
__global__ __launch_bounds__(256) void cast_fp8_kernel(CastArgs a) {
  constexpr int G = 8;
  typedef uint32_t u32x2c __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const int g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = g / a.slices, sl = g - t * a.slices;
  if (t >= a.T) return;
  const int nv = a.H / 8;  // 16-byte bf16 units per row (8 columns each)
  const int u = sl * kWave + lane;  // this lane's unit
  const bool on = u < nv;
  const uint32_t own = RANK_MAJOR ? a.ufirst[t] : 0xFFFFFFFFu;  // uniform
  const u32x4* y = reinterpret_cast<const u32x4*>(a.y);
  u32x2c* y8 = reinterpret_cast<u32x2c*>(a.y8);  // 8-byte units: 8 E4M3 columns
  if (!on) return;
  for (int j0 = 0; j0 < a.k; j0 += G) {
    int row[G];
    u32x4 in[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const int j = j0 + q;
      row[q] = (j < a.k && (own >> j & 1u)) ? a.rows[(size_t)t * a.k + j] : -1;
      in[q] = u32x4{0, 0, 0, 0};
      if (row[q] >= 0) in[q] = __builtin_nontemporal_load(y + (size_t)row[q] * nv + u);
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (row[q] < 0) continue;
      const u32x4 x = in[q];
      u32x2c o;
      o[0] = pack_e4m3x4(clamp448(bf16_lo(x[0])), clamp448(bf16_hi(x[0])), clamp448(bf16_lo(x[1])),
                         clamp448(bf16_hi(x[1])));
      o[1] = pack_e4m3x4(clamp448(bf16_lo(x[2])), clamp448(bf16_hi(x[2])), clamp448(bf16_lo(x[3])),
                         clamp448(bf16_hi(x[3])));
      __builtin_nontemporal_store(o, y8 + (size_t)row[q] * nv + u);
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a0, hipStream_t s) {
  if (a0.T == 0) return hipSuccess;
  CombineArgs a = a0;
  if (a.k > 8) {  // groups of 8 positions, 2 KiB per wave, four waves per workgroup
    const int per = kWave * kUnitsPerLane;
    a.slice_units = per;
    a.slices = (a.H / 8 + per - 1) / per;
    const int blocks = (int)(((int64_t)a.T * a.slices + 3) / 4);
    const bool dedupe = !a.distinct_rows && !a.sum_rows;
    if (a.sum_rows) combine_wide_kernel<false, false, true><<<blocks, 256, 0, s>>>(a);
    else if (a.round_e4m3) {
      if (dedupe) combine_wide_kernel<true, true><<<blocks, 256, 0, s>>>(a);
      else combine_wide_kernel<false, true><<<blocks, 256, 0, s>>>(a);
    } else {
      if (dedupe) combine_wide_kernel<true, false><<<blocks, 256, 0, s>>>(a);
      else combine_wide_kernel<false, false><<<blocks, 256, 0, s>>>(a);
    }
    return hipGetLastError();
  }
  // 1 KiB of each row per wave when rows are shared (dedupe), 512 bytes when
  // a token's rows are all distinct, 2 KiB with the E4M3 rounding; a token's
  // waves in as few workgroups as possible
  const bool dedupe = !a.distinct_rows && !a.sum_rows;
  const bool narrow = a.sum_rows || (!a.round_e4m3 && !dedupe);  // the 8-byte-lane kernels
  const int lane_bytes = narrow ? kDistinctLaneBytes : 16;
  const int upl = a.round_e4m3 ? kRoundUnitsPerLane : 1;
  a.slice_units = kWave * upl;
  a.slices = (a.H * 2 / lane_bytes + a.slice_units - 1) / a.slice_units;
  a.wg_per_tok = (a.slices + kMaxWavesPerWg - 1) / kMaxWavesPerWg;
  a.waves_per_wg = (a.slices + a.wg_per_tok - 1) / a.wg_per_tok;
  const int64_t blocks = (int64_t)a.T * a.wg_per_tok;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block((unsigned)(kWave * a.waves_per_wg));
  if (a.sum_rows)  // converted rank rows: the owning positions' rows are distinct
    combine_kernel<8, false, false, true, 1, kDistinctLaneBytes><<<grid, block, 0, s>>>(a);
  else if (a.round_e4m3) {
    if (dedupe) combine_kernel<8, true, true, false, kRoundUnitsPerLane><<<grid, block, 0, s>>>(a);
    else combine_kernel<8, false, true, false, kRoundUnitsPerLane><<<grid, block, 0, s>>>(a);
  } else {
    if (dedupe) combine_kernel<8, true, false><<<grid, block, 0, s>>>(a);
    else combine_kernel<8, false, false, false, 1, kDistinctLaneBytes><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_combine_fp8(const CombineArgs& a0, hipStream_t s) {
  if (a0.T == 0) return hipSuccess;
  CombineArgs a = a0;
  a.slice_units = kWave;
  a.slices = (a.H / 16 + kWave - 1) / kWave;
  const int blocks = (int)(((int64_t)a.T * a.slices + 3) / 4);
  if (a.k <= 8) {
    if (a.distinct_rows) combine_fp8_kernel<8, false><<<blocks, 256, 0, s>>>(a);
    else combine_fp8_kernel<8, true><<<blocks, 256, 0, s>>>(a);
  }
  else combine_fp8_wide_kernel<<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_cast_fp8(const CastArgs& a0, hipStream_t s) {
  if (a0.T == 0) return hipSuccess;
  CastArgs a = a0;
  a.slices = (a.H / 8 + kWave - 1) / kWave;
  const int blocks = (int)(((int64_t)a.T * a.slices + 3) / 4);
  if (a.ufirst) cast_fp8_kernel<true><<<blocks, 256, 0, s>>>(a);
  else cast_fp8_kernel<false><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mep
