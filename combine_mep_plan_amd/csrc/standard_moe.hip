// Standard-MoE dispatch: token rows routed straight into the expert-major
// layout, without the rank-major receive buffers in between.
//
// Source: "MORI-EP User Guide", section 4 Standard MoE Compatibility:
// dispatch_standard_moe() combines dispatch and the format conversion of
// convert_dispatch_output().  The result equals dispatch followed by the
// expert-major conversion: experts in global order, each expert's rows in
// ascending token order (receive slots are token-ascending), segments padded
// to multiples of 128 rows, padding not written; a token naming an expert id
// outside [0, E) is not dispatched; a token naming an expert twice gets one
// row, mapped from the first top-k position naming it.
//
// Launches:
//   count:   one wave per 64-token chunk counts, in an LDS histogram, the
//            chunk's tokens naming each expert (a token counts once per expert);
//   route:   one workgroup per chunk places the chunk's rows: it takes the
//            per-expert totals and the chunk's prefixes from the histograms,
//            scans the totals padded to 128 rows into segment offsets, and
//            gives the (token, expert) pairs of the chunk their rows in token
//            order (LDS bit masks of the tokens naming each expert); it writes
//            the row of every top-k position and the source of every row;
//   scatter: one wave per (token, 64 lane units of its row) reads and, for FP8,
//            quantises its slice once, then writes it to the token's rows.
// When the histograms are large (chunks x experts above 32768), one workgroup
// first turns them into prefixes and offsets ("offsets" below) and the route
// workgroups read those instead of summing the histograms each.
#include "payload.h"
#include "route.h"

namespace mep {

namespace {

// Token t's expert ids (k <= KMAX); returns false for a token with a bad id.
template <int KMAX>
__device__ __forceinline__ bool load_ids(const SmArgs& a, int t, int (&ids)[KMAX]) {
  const int32_t* p = a.idx + (size_t)t * a.k;
  bool ok = true;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ids[j] = j < a.k ? p[j] : -1;
    if (j < a.k && (ids[j] < 0 || ids[j] >= a.E)) ok = false;
  }
  return ok;
}

template <int KMAX>
__global__ __launch_bounds__(64) void sm_count_kernel(SmArgs a) {
  extern __shared__ int32_t hist[];  // [E]
  const int lane = threadIdx.x;
  const int c = blockIdx.x;
  // the next status word starts clean (the overflow bits come later, from the
  // route launch)
  if (c == 0 && lane == 0) *a.status_next = 0u;
  for (int e = lane; e < a.E; e += kWave) hist[e] = 0;
  __syncthreads();
  const int t = c * kChunk + lane;
  int ids[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) ids[j] = -1;
  uint32_t st = 0;
  bool valid = false;
  if (t < a.T) {
    valid = load_ids<KMAX>(a, t, ids);
    if (!valid) st |= MEP_DEV_BAD_INDEX;
    if (valid) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j >= a.k) continue;
        bool first = true;
#pragma unroll
        for (int jj = 0; jj < j; ++jj) first &= ids[jj] != ids[j];
        if (first) atomicAdd(&hist[ids[j]], 1);
        else st |= MEP_DEV_DUP_EXPERT;
      }
    }
  }
  report_status(a.status, a.tok_status, t, a.T, st);
  __syncthreads();
  for (int e = lane; e < a.E; e += kWave) a.chunk_hist[(size_t)c * a.E + e] = hist[e];
}

constexpr int kOffThreads = 1024;
constexpr int kOffItems = 4096;  // >= max(kOffThreads, E)
static_assert(kOffItems >= kMaxRanks * kMaxEpr && kOffItems >= kOffThreads, "offsets items");

// Exclusive prefixes over chunks (in place), per-expert totals and the padded
// scan into segment offsets, in one workgroup.  Work item i = g * E + e takes
// expert e's chunks [g*Cg, (g+1)*Cg): G items per expert, G the largest power
// of two with G * E <= 1024 (1 when E > 1024), so that a thread's loads are
// few and all in flight.  Also runs alone for an empty batch (C = 0).
__global__ __launch_bounds__(kOffThreads) void sm_offsets_kernel(SmArgs a) {
  __shared__ int32_t item_sum[kOffItems];
  __shared__ int32_t padded[kOffItems];
  __shared__ int32_t part[kOffThreads];
  const int tid = threadIdx.x;
  if (tid == 0) *a.status_next = 0u;  // the next reset epoch starts clean
  const int E = a.E;
  const int C = (a.T + kChunk - 1) / kChunk;
  int G = 1;
  while (2 * G * E <= kOffThreads) G *= 2;
  const int Cg = (C + G - 1) / G;
  const int items = G * E;
  int32_t* hist = a.chunk_hist;
  // pass 1: each item's sum over its chunk range
  for (int i = tid; i < items; i += kOffThreads) {
    const int g = i / E, e = i - g * E;
    const int c0 = min(g * Cg, C), c1 = min(c0 + Cg, C);
    int sum = 0;
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hist[(size_t)(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; c < c1; ++c) sum += hist[(size_t)c * E + e];
    item_sum[i] = sum;
  }
  __syncthreads();
  // pass 2: rewrite each range with exclusive prefixes; the last item of an
  // expert produces its total
  for (int i = tid; i < items; i += kOffThreads) {
    const int g = i / E, e = i - g * E;
    int run = 0;
    for (int gg = 0; gg < g; ++gg) run += item_sum[gg * E + e];
    const int c0 = min(g * Cg, C), c1 = min(c0 + Cg, C);
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hist[(size_t)(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        hist[(size_t)(c + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; c < c1; ++c) {
      const int v = hist[(size_t)c * E + e];
      hist[(size_t)c * E + e] = run;
      run += v;
    }
    if (g == G - 1) {
      a.em_counts[e] = run;
      padded[e] = (run + 127) / 128 * 128;
    }
  }
  __syncthreads();
  // pass 3: padded scan over experts, per consecutive experts per thread
  const int per = (E + kOffThreads - 1) / kOffThreads;
  const int lo = min(tid * per, E), hi = min(lo + per, E);
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += padded[e];
  part[tid] = sum;
  __syncthreads();
  for (int d = 1; d < kOffThreads; d <<= 1) {
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int off = part[tid] - sum;
  for (int e = lo; e < hi; ++e) {
    a.em_offsets[e] = off;
    off += padded[e];
  }
  if (tid == kOffThreads - 1) a.em_offsets[E] = part[tid];
}

constexpr int kRouteThreads = 256;
constexpr int64_t kRouteFusedMax = 32768;  // chunks x experts summed per route workgroup
constexpr int kRouteFusedMaxExperts = 2048;
constexpr int kHistBatch = 64;  // histogram loads per round: 4096 tokens in one round

// LDS of a route workgroup: token masks [E] u64, row bases [E] i32 and, when
// the offsets are computed here, padded totals [E] i32.
__host__ __device__ constexpr size_t route_lds_bytes(int E, bool fused) {
  return (size_t)E * (sizeof(uint64_t) + sizeof(int32_t) + (fused ? sizeof(int32_t) : 0));
}

template <int KMAX, bool FUSED>
__global__ __launch_bounds__(kRouteThreads) void sm_route_kernel(SmArgs a) {
  extern __shared__ __align__(8) unsigned char smem[];
  __shared__ int32_t wsum[kRouteThreads / kWave];
  const int E = a.E;
  uint64_t* mask = reinterpret_cast<uint64_t*>(smem);  // tokens of the chunk naming e
  int32_t* base = reinterpret_cast<int32_t*>(mask + E);  // first row of the chunk for e
  int32_t* pad = base + E;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = blockIdx.x;
  const int C = (a.T + kChunk - 1) / kChunk;
  // the chunk's tokens, one per lane of the first wave; their ids go out first
  const int t = c * kChunk + lane;
  const bool mine = tid < kWave && t < a.T;
  int ids[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) ids[j] = -1;
  const bool valid = mine && load_ids<KMAX>(a, t, ids);
  const int32_t* hist = a.chunk_hist;
  if (FUSED) {
    // per expert: total over all chunks and prefix over the chunks before c
    // (kHistBatch independent loads in flight per thread)
    for (int e = tid; e < E; e += kRouteThreads) {
      int tot = 0, pre = 0;
      int cc = 0;
      for (; cc + kHistBatch <= C; cc += kHistBatch) {
        int v[kHistBatch];
#pragma unroll
        for (int u = 0; u < kHistBatch; ++u) v[u] = hist[(size_t)(cc + u) * E + e];
#pragma unroll
        for (int u = 0; u < kHistBatch; ++u) {
          tot += v[u];
          pre += cc + u < c ? v[u] : 0;
        }
      }
      for (; cc < C; ++cc) {
        const int v = hist[(size_t)cc * E + e];
        tot += v;
        pre += cc < c ? v : 0;
      }
      if (c == 0) a.em_counts[e] = tot;
      pad[e] = (tot + 127) / 128 * 128;
      base[e] = pre;
      mask[e] = 0ull;
    }
    __syncthreads();
    // padded totals scanned into segment offsets, consecutive experts per
    // thread: within the wave by shuffles, then across the waves
    const int per = (E + kRouteThreads - 1) / kRouteThreads;
    const int lo = min(tid * per, E), hi = min(lo + per, E);
    int sum = 0;
    for (int e = lo; e < hi; ++e) sum += pad[e];
    int inc = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(inc, d);
      if (lane >= d) inc += v;
    }
    if (lane == kWave - 1) wsum[w] = inc;
    __syncthreads();
    int off = inc - sum;
    for (int ww = 0; ww < w; ++ww) off += wsum[ww];
    for (int e = lo; e < hi; ++e) {
      if (c == 0) a.em_offsets[e] = off;
      base[e] += off;
      off += pad[e];
    }
    if (c == 0 && tid == kRouteThreads - 1) a.em_offsets[E] = off;
  } else {
    // prefixes and offsets from the offsets workgroup
    for (int e = tid; e < E; e += kRouteThreads) {
      base[e] = a.em_offsets[e] + hist[(size_t)c * E + e];
      mask[e] = 0ull;
    }
  }
  __syncthreads();
  uint32_t firsts = 0;  // top-k positions that own a row
  if (valid) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= a.k) continue;
      bool first = true;
#pragma unroll
      for (int jj = 0; jj < j; ++jj) first &= ids[jj] != ids[j];
      if (first) {
        firsts |= 1u << j;
        atomicOr(reinterpret_cast<unsigned long long*>(&mask[ids[j]]), 1ull << lane);
      }
    }
  }
  __syncthreads();
  if (mine) {
    const uint64_t below = (1ull << lane) - 1ull;
    bool over = false;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= a.k) continue;
      int32_t row = -1;
      if (firsts >> j & 1u) {
        const int e = ids[j];
        const int64_t pos = (int64_t)base[e] + __popcll(mask[e] & below);
        if (pos < a.cap_em) {
          row = (int32_t)pos;
          a.em_src_pos[pos] = a.spos_base + t;
        } else {
          over = true;
        }
      }
      a.em_row[(size_t)t * a.k + j] = row;
    }
    if (over) atomicOr(a.status, (uint32_t)MEP_DEV_EM_OVERFLOW);
  }
}

template <int QUANT, int KMAX>
__global__ __launch_bounds__(256) void sm_scatter_kernel(SmArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = g / a.slices, sl = g - t * a.slices;
  if (t >= a.T) return;
  // this wave's slice of the row: loads go out first
  const int nu = lane_items(QUANT, a.H);
  const int v = sl * kWave + lane;
  const bool on = v < nu;
  Unit<QUANT> unit;
  unit.template load<true>(a.x, t, a.H, v, on);
  // the token's rows, placed by the route launch (-1: no row)
  int rows[KMAX];
  const int32_t* rr = a.em_row + (size_t)t * a.k;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) rows[j] = j < a.k ? rr[j] : -1;
  float scale = 0.0f;
  uint32_t e8 = 0;
  const typename Unit<QUANT>::Out q = unit.convert(scale, e8);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int pos = rows[j];
    if (pos < 0) continue;
    if (on) {
      store_nt(reinterpret_cast<typename Unit<QUANT>::Out*>(a.em_x) + (size_t)pos * nu + v, q);
      store_unit_scale<QUANT>(a.em_scales, (size_t)pos, a.H, v, scale, e8);
    }
    if (is_carry(QUANT) && sl == 0)
      copy_scale_row(a.em_scales, (size_t)pos, a.x_scales, t, a.scale_dim, lane);
  }
}

template <int QUANT>
hipError_t launch_scatter(const SmArgs& a0, hipStream_t s) {
  SmArgs a = a0;
  a.slices = (lane_items(QUANT, a.H) + kWave - 1) / kWave;
  const int blocks = (int)(((int64_t)a.T * a.slices + 3) / 4);
  if (a.k <= 8) sm_scatter_kernel<QUANT, 8><<<blocks, 256, 0, s>>>(a);
  else sm_scatter_kernel<QUANT, kMaxTopk><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_route(const SmArgs& a, int C, hipStream_t s) {
  const size_t lds = route_lds_bytes(a.E, FUSED);
  if (a.k <= 8) sm_route_kernel<8, FUSED><<<C, kRouteThreads, lds, s>>>(a);
  else sm_route_kernel<kMaxTopk, FUSED><<<C, kRouteThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch_standard_moe(const SmArgs& a, hipStream_t s) {
  if (a.T == 0) {
    sm_offsets_kernel<<<1, kOffThreads, 0, s>>>(a);
    return hipGetLastError();
  }
  const int C = (a.T + kChunk - 1) / kChunk;
  const size_t lds = (size_t)a.E * sizeof(int32_t);
  if (a.k <= 8) sm_count_kernel<8><<<C, 64, lds, s>>>(a);
  else sm_count_kernel<kMaxTopk><<<C, 64, lds, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool fused = (int64_t)C * a.E <= kRouteFusedMax && a.E <= kRouteFusedMaxExperts;
  if (fused) {
    e = launch_route<true>(a, C, s);
  } else {
    sm_offsets_kernel<<<1, kOffThreads, 0, s>>>(a);
    e = hipGetLastError();
    if (e == hipSuccess) e = launch_route<false>(a, C, s);
  }
  if (e != hipSuccess) return e;
  switch (a.quant) {
    case MEP_QUANT_FP8_E4M3_BLOCK128: return launch_scatter<MEP_QUANT_FP8_E4M3_BLOCK128>(a, s);
    case MEP_QUANT_FP8_CARRY: return launch_scatter<MEP_QUANT_FP8_CARRY>(a, s);
    case MEP_QUANT_FP4_CARRY: return launch_scatter<MEP_QUANT_FP4_CARRY>(a, s);
    case MEP_QUANT_MXFP4: return launch_scatter<MEP_QUANT_MXFP4>(a, s);
    default: return launch_scatter<MEP_QUANT_NONE>(a, s);
  }
}

}  // namespace mep
