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
//            the rank's local experts it names and the chunk's per-expert row
//            counts (one ballot per local expert); it also clears the
//            (token, top-k) -> expert-major row map;
//   offsets: one workgroup sums the chunk counts per expert, pads to 128,
//            scans them into segment offsets and gives every chunk the first
//            row of its run inside each expert segment;
//   scatter: waves stride over all received rows; a row's place inside its
//            expert segment is its chunk base plus a ballot count of the
//            earlier rows of its chunk naming that expert.  Each row is copied
//            with 16-byte-per-lane coalesced loads and stores.
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

__global__ __launch_bounds__(kOffThreads) void em_offsets_kernel(EmArgs a) {
  __shared__ int32_t padded[kMaxRanks * kMaxEpr];
  __shared__ int32_t part[kOffThreads];
  const int E = a.R * a.epr;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kOffThreads) {
    const int r = e / a.epr, l = e - r * a.epr;
    const int nch = (clamp_count(a, r) + kChunk - 1) / kChunk;
    int n = 0;
    for (int c = 0; c < nch; ++c) n += a.ccnt[((size_t)r * a.CR + c) * a.epr + l];
    a.em_counts[e] = n;
    padded[e] = (n + 127) / 128 * 128;
  }
  __syncthreads();
  // exclusive scan of padded[0..E): contiguous per-thread segments, then a
  // Hillis-Steele scan of the segment sums
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
  int run = part[tid] - sum;  // exclusive prefix of this segment
  for (int e = lo; e < hi; ++e) {
    const int p = padded[e];
    padded[e] = run;  // now the segment offset
    a.em_offsets[e] = run;
    run += p;
  }
  if (tid == kOffThreads - 1) {
    a.em_offsets[E] = part[tid];
    if ((int64_t)part[tid] > a.cap_em) atomicOr(a.status, (uint32_t)MEP_DEV_EM_OVERFLOW);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kOffThreads) {
    const int r = e / a.epr, l = e - r * a.epr;
    const int nch = (clamp_count(a, r) + kChunk - 1) / kChunk;
    int run2 = padded[e];
    for (int c = 0; c < nch; ++c) {
      const size_t i = ((size_t)r * a.CR + c) * a.epr + l;
      a.cbase[i] = run2;
      run2 += a.ccnt[i];
    }
  }
}

template <int UNROLL>
__global__ __launch_bounds__(256) void em_scatter_kernel(EmArgs a) {
  __shared__ int32_t prefix[kMaxRanks + 1];
  if (threadIdx.x == 0) {
    int run = 0;
    for (int r = 0; r < a.R; ++r) { prefix[r] = run; run += clamp_count(a, r); }
    prefix[a.R] = run;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int total = prefix[a.R];
  const int nwaves = gridDim.x * 4;
  const int nv = a.H * a.elem_bytes / 16;  // 16-byte vectors per row
  const u32x4* src_x = reinterpret_cast<const u32x4*>(a.recv_x);
  u32x4* dst_x = reinterpret_cast<u32x4*>(a.em_x);
  for (int u = blockIdx.x * 4 + (threadIdx.x >> 6); u < total; u += nwaves) {
    int r = 0;
    while (prefix[r + 1] <= u) ++r;  // uniform: u is per wave
    const int s = u - prefix[r];
    const int cnt = prefix[r + 1] - prefix[r];
    const int c = s / kChunk, sl = s % kChunk;
    const int peer = c * kChunk + lane;
    const uint64_t lm_lane = peer < cnt ? a.lmask[(size_t)r * a.cap + peer] : 0ull;
    const uint64_t lm_self = ((uint64_t)(uint32_t)lane_value((int)(uint32_t)lm_lane, sl)) |
                             ((uint64_t)(uint32_t)lane_value((int)(uint32_t)(lm_lane >> 32), sl) << 32);
    const size_t row = (size_t)r * a.cap + s;
    const int pos_code = a.spos[row];
    const int t = pos_code - a.spos_base;
    for (uint64_t m = lm_self; m; m &= m - 1) {
      const int l = __builtin_ctzll(m);
      const uint64_t b = ballot(lane < sl && ((lm_lane >> l) & 1ull));
      const int64_t pos = (int64_t)a.cbase[((size_t)r * a.CR + c) * a.epr + l] + __popcll(b);
      if (pos >= a.cap_em) {
        if (lane == 0) atomicOr(a.status, (uint32_t)MEP_DEV_EM_OVERFLOW);
        continue;
      }
      for (int v0 = 0; v0 < nv; v0 += kWave * UNROLL) {
        u32x4 buf[UNROLL];
#pragma unroll
        for (int k2 = 0; k2 < UNROLL; ++k2) {
          const int v = v0 + k2 * kWave + lane;
          if (v < nv) buf[k2] = src_x[row * nv + v];
        }
#pragma unroll
        for (int k2 = 0; k2 < UNROLL; ++k2) {
          const int v = v0 + k2 * kWave + lane;
          if (v < nv) store_nt(dst_x + (size_t)pos * nv + v, buf[k2]);
        }
      }
      for (int i = lane; i < a.nb; i += kWave)
        a.em_scales[(size_t)pos * a.nb + i] = a.recv_scales[row * a.nb + i];
      if (lane == 0) {
        a.em_src_pos[pos] = pos_code;
        if (t >= 0 && t < a.T) {
          const int e = r * a.epr + l;
          const int32_t* ids = a.recv_idx + row * a.k;
          for (int j = 0; j < a.k; ++j)
            if (ids[j] == e) { a.em_row[(size_t)t * a.k + j] = (int32_t)pos; break; }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_to_expert_major(const EmArgs& a, hipStream_t s) {
  const int waves = a.R * a.CR;
  em_count_kernel<<<(waves + 3) / 4, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  em_offsets_kernel<<<1, kOffThreads, 0, s>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.R * a.cap;
  const int blocks = (int)std::min<int64_t>((rows + 3) / 4, 4096);
  em_scatter_kernel<8><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mep
