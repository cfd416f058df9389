// Standard-MoE (expert-major) conversion of the dispatch output.
//
// Source: "MORI-EP User Guide", section 4 Standard MoE Compatibility:
// convert_dispatch_output() turns the 2-D receive buffer into per-expert
// packed rows with per-expert counts and source info.  This library's
// layout: experts in global order, each expert's rows in ascending receive
// slot, each expert segment starting at a multiple of 128 rows; padding rows
// are not written.
//
// Three launches:
//   count:   one wave per (rank, 64-row chunk) builds each receive row's mask of
//            the rank's local experts and the chunk's per-expert row counts (one
//            ballot per local expert); it also clears the (token, top-k) ->
//            expert-major row map;
//   offsets: one workgroup; each thread sums a group of chunks for one expert
//            (independent loads), and the padded experts are scanned through
//            LDS into segment offsets;
//   scatter: one wave per (receive row, slice of the row); the row's place
//            inside an expert segment is the segment offset, plus the rows of
//            the rank's earlier chunks naming that expert (one load per lane
//            and a wave reduction), plus a ballot count of the earlier rows of
//            its own chunk.  Each slice is copied with 16-byte-per-lane loads
//            and non-temporal stores.
#include "dev.h"
#include "mep_internal.h"

namespace mep {

namespace {

__device__ __forceinline__ int clamp_count(const EmArgs& a, int r) {
  return min(max(a.recv_counts[r], 0), a.cap);
}

__global__ __launch_bounds__(256) void em_count_kernel(EmArgs a) {
  // clear the (t, j) -> expert-major row map
  const int64_t nmap = (int64_t)a.T * a.k;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nmap;
       i += (int64_t)gridDim.x * blockDim.x)
    a.em_row[i] = -1;

  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int r = g / a.CR, c = g % a.CR;
  if (r >= a.R) return;
  const int cnt = clamp_count(a, r);
  if (c * kChunk >= cnt) return;  // whole wave
  const int s = c * kChunk + lane;
  const int E = a.R * a.epr;
  uint64_t lm = 0;
  if (s < cnt) {
    const size_t row = (size_t)r * a.cap + s;
    const int32_t* ids = a.recv_idx + row * a.k;
    for (int j = 0; j < a.k; ++j) {
      const int e = ids[j];
      if (e >= 0 && e < E && e / a.epr == r) lm |= 1ull << (e - r * a.epr);
    }
    a.lmask[row] = lm;
  }
  int mine = 0;
  for (int l = 0; l < a.epr; ++l) {
    const uint64_t b = ballot((lm >> l) & 1ull);
    if (lane == l) mine = __popcll(b);
  }
  if (lane < a.epr) a.ccnt[((size_t)r * a.CR + c) * a.epr + lane] = mine;
}

constexpr int kOffThreads = 1024;
constexpr int kMaxExperts = kMaxRanks * kMaxEpr;
// 16-byte units per lane per scatter wave.  Each wave first finds its row's
// rank, local experts and in-chunk position, so fewer, larger waves pay that
// less often: at 4096 x 7168 FP8 on 32 ranks the conversion took 129, 95.5,
// 91.6 and 94.8 us with 1, 2, 3 and 4 units per lane.
constexpr int kEmUnitsPerLane = 3;

// Chunks [c0, c1) of expert e's rank that thread group `grp` of G covers.
__device__ __forceinline__ void group_chunks(const EmArgs& a, int e, int grp, int G, int& r,
                                             int& l, int& c0, int& c1) {
  r = e / a.epr;
  l = e - r * a.epr;
  const int nch = (clamp_count(a, r) + kChunk - 1) / kChunk;
  const int per = (nch + G - 1) / G;
  c0 = min(grp * per, nch);
  c1 = min(c0 + per, nch);
}

__device__ __forceinline__ int group_rows(const EmArgs& a, int r, int l, int c0, int c1) {
  int acc[4] = {0, 0, 0, 0};
  int c = c0;
  for (; c + 4 <= c1; c += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += a.ccnt[((size_t)r * a.CR + c + u) * a.epr + l];
  }
  for (; c < c1; ++c) acc[0] += a.ccnt[((size_t)r * a.CR + c) * a.epr + l];
  return acc[0] + acc[1] + acc[2] + acc[3];
}

// Threads are (expert, chunk group) pairs, G groups per expert (G a power of
// two, G * E <= 1024 where possible); experts beyond one pass take more passes.
__global__ __launch_bounds__(kOffThreads) void em_offsets_kernel(EmArgs a, int G) {
  __shared__ int32_t part[kOffThreads];
  __shared__ int32_t seg[kMaxExperts];
  const int E = a.R * a.epr;
  const int tid = threadIdx.x;
  const int slots = kOffThreads / G;  // experts per pass
  const int passes = (E + slots - 1) / slots;
  // 1: rows per expert
  for (int p = 0; p < passes; ++p) {
    const int e = p * slots + tid / G, grp = tid % G;
    int r = 0, l = 0, c0 = 0, c1 = 0;
    if (e < E) group_chunks(a, e, grp, G, r, l, c0, c1);
    part[tid] = e < E ? group_rows(a, r, l, c0, c1) : 0;
    __syncthreads();
    if (e < E && grp == 0) {
      int n = 0;
      for (int q = 0; q < G; ++q) n += part[tid + q];
      seg[e] = n;
    }
    __syncthreads();
  }
  // 2: counts, segment sizes padded to 128 rows, exclusive scan over experts
  for (int e = tid; e < E; e += kOffThreads) a.em_counts[e] = seg[e];
  const int perT = (E + kOffThreads - 1) / kOffThreads;
  const int lo = min(tid * perT, E), hi = min(lo + perT, E);
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += (seg[e] + 127) / 128 * 128;
  __syncthreads();
  part[tid] = sum;
  __syncthreads();
  for (int d = 1; d < kOffThreads; d <<= 1) {
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int e = lo; e < hi; ++e) {
    const int n = seg[e];
    seg[e] = run;  // now the segment offset
    a.em_offsets[e] = run;
    run += (n + 127) / 128 * 128;
  }
  if (tid == kOffThreads - 1) {
    a.em_offsets[E] = part[tid];
  }
  __syncthreads();
}

// Rows of the same rank's earlier chunks that name local expert l: lane c'
// loads chunk c''s count, then a wave reduction (chunks beyond 64 in steps).
__device__ __forceinline__ int rows_before_chunk(const EmArgs& a, int r, int c, int l,
                                                 int lane) {
  int n = 0;
  for (int c0 = 0; c0 < c; c0 += kWave) {
    const int cc = c0 + lane;
    if (cc < c) n += a.ccnt[((size_t)r * a.CR + cc) * a.epr + l];
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) n += __shfl_xor(n, d);
  return n;
}

template <int UPL>
__global__ __launch_bounds__(256) void em_scatter_kernel(EmArgs a) {
  __shared__ int32_t prefix[kMaxRanks + 1];
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < kWave) {  // rank prefix of the receive counts, one lane per rank
    const int n = lane < a.R ? clamp_count(a, lane) : 0;
    int inc = n;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(inc, d);
      if (lane >= d) inc += v;
    }
    if (lane < a.R) prefix[lane + 1] = inc;
    if (lane == 0) prefix[0] = 0;
  }
  __syncthreads();
  const int g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int u = g / a.slices, sl = g - u * a.slices;
  if (u >= prefix[a.R]) return;
  int lo = 0, hi = a.R;  // largest r with prefix[r] <= u (uniform)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= u) lo = mid; else hi = mid;
  }
  const int r = lo;
  const int s = u - prefix[r];
  const int cnt = prefix[r + 1] - prefix[r];
  const size_t row = (size_t)r * a.cap + s;
  const int nv = a.row_units;  // 16-byte units per row
  // row slice first: its loads do not depend on the placement
  const u32x4* src = reinterpret_cast<const u32x4*>(a.recv_x) + row * nv;
  u32x4 val[UPL];
#pragma unroll
  for (int q = 0; q < UPL; ++q) {
    const int v = (sl * UPL + q) * kWave + lane;
    val[q] = v < nv ? src[v] : u32x4{0, 0, 0, 0};
  }
  const int c = s / kChunk, sc = s % kChunk;
  const int peer = c * kChunk + lane;
  const uint64_t lm_lane = peer < cnt ? a.lmask[(size_t)r * a.cap + peer] : 0ull;
  const uint64_t lm_self =
      ((uint64_t)(uint32_t)lane_value((int)(uint32_t)lm_lane, sc)) |
      ((uint64_t)(uint32_t)lane_value((int)(uint32_t)(lm_lane >> 32), sc) << 32);
  int pos_code = 0, t = -1, myid = -1;
  if (sl == 0) {
    pos_code = a.spos[row];
    t = pos_code - a.spos_base;
    if (lane < a.k) myid = a.recv_idx[row * a.k + lane];
  }
  u32x4* dst_x = reinterpret_cast<u32x4*>(a.em_x);
  for (uint64_t m = lm_self; m; m &= m - 1) {
    const int l = __builtin_ctzll(m);
    const uint64_t b = ballot(lane < sc && ((lm_lane >> l) & 1ull));
    const int64_t pos = (int64_t)a.em_offsets[r * a.epr + l] +
                        rows_before_chunk(a, r, c, l, lane) + __popcll(b);
    if (pos >= a.cap_em) {
      if (lane == 0) atomicOr(a.status, (uint32_t)MEP_DEV_EM_OVERFLOW);
      continue;
    }
#pragma unroll
    for (int q = 0; q < UPL; ++q) {
      const int v = (sl * UPL + q) * kWave + lane;
      if (v < nv) store_nt(dst_x + (size_t)pos * nv + v, val[q]);
    }
    if (sl == 0)  // the row's scale columns, one per lane
      for (int i = lane; i < a.nb; i += kWave)
        a.em_scales[(size_t)pos * a.nb + i] = a.recv_scales[row * a.nb + i];
    if (sl == 0) {
      const int e = r * a.epr + l;
      const uint64_t hit = ballot(myid == e);  // top-k position naming e
      if (lane == 0) {
        a.em_src_pos[pos] = pos_code;
        if (t >= 0 && t < a.T && hit) a.em_row[(size_t)t * a.k + __builtin_ctzll(hit)] = (int32_t)pos;
      }
    }
  }
}

}  // namespace

hipError_t launch_to_expert_major(const EmArgs& a0, hipStream_t s) {
  EmArgs a = a0;
  const int waves = a.R * a.CR;
  em_count_kernel<<<(waves + 3) / 4, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int E = a.R * a.epr;
  int G = 1;
  while (G * 2 * E <= kOffThreads && G < 64) G *= 2;
  em_offsets_kernel<<<1, kOffThreads, 0, s>>>(a, G);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one wave per (receive row, kEmUnits x 64 units); rows <= T * min(k, R)
  const int nv = a.row_units;
  const int per = kEmUnitsPerLane * kWave;
  a.slices = (nv + per - 1) / per;
  const int64_t rows = (int64_t)a.T * std::min(a.k, a.R);
  const int64_t waves2 = rows * a.slices;
  if (waves2 == 0) return hipSuccess;
  em_scatter_kernel<kEmUnitsPerLane><<<(unsigned)((waves2 + 3) / 4), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mep
