// Routing plan: per-token destination-rank dedupe, per-rank counts and a
// deterministic receive slot for every (token, rank) pair.
//
// Source: "MORI-EP User Guide", section 3 Operator API -- dispatch() returns
// the received rows and recv_num_token; get_dispatch_src_token_pos() encodes a
// row's origin as src_rank * (world_size * max_num_inp_token_per_rank) +
// token.  ROCm/mori issue #57: the design removes redundant transfer, so a
// token travels once to each distinct destination rank.  Inside a rank the
// rows are in ascending token order (the only order that needs no atomics and
// is reproducible run to run).
//
// Work unit: a chunk of 64 tokens = one wave, one token per lane.  For a
// chunk, one ballot per rank gives the chunk's row count for that rank
// (popcount) and each lane's offset among the chunk's tokens going there
// (popcount of the ballot below the lane).  The ballots and the chunk's
// per-rank base are put in LDS, so every lane finds the slot of each of its
// top-k entries with one LDS read and a popcount -- no per-rank loop per lane.
//
// The per-rank base of a chunk is the exclusive prefix over earlier chunks,
// built in two levels: inside a block of chunks (4 up to 4096 tokens, 16
// beyond) through LDS, across blocks by summing block totals.  Up to 1024
// tokens one workgroup does everything in a single launch; beyond that, a
// count launch writes the block-level prefixes and a slot launch (one wave per
// chunk) finishes.
#include "route.h"

namespace mep {

namespace {

constexpr int kBlockChunks = 16;  // chunks (waves) of the single-workgroup plan; most per count block

// Slot phase for one chunk.  `base` in lane r is the number of rows rank r got
// from all earlier tokens.  bal/bas are this wave's LDS scratch (64 entries).
// Writes src_token_pos, the flat receive row of each (t, j) and the
// first-occurrence bits.  Returns, in lane r, the rank-r count of the chunk.
template <int KMAX>
__device__ __forceinline__ int chunk_slots(const PlanArgs& a, int c, int lane, int base,
                                           const int (&ids)[KMAX], uint64_t mask,
                                           uint64_t* bal, int* bas) {
  uint64_t mybal = 0;
  for (int r = 0; r < a.R; ++r) {
    const uint64_t b = ballot((mask >> r) & 1ull);
    if (lane == r) mybal = b;
  }
  if (lane < a.R) { bal[lane] = mybal; bas[lane] = base; }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int t = c * kChunk + lane;
  if (t < a.T) {
    int32_t* rr = a.rrow + (size_t)t * a.k;
    if (mask == 0) {
      for (int j = 0; j < a.k; ++j) rr[j] = -1;
      a.ufirst[t] = 0;
    } else {
      uint64_t seen = 0;
      uint32_t first = 0;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < a.k) {
          const int r = (int)a.rdiv((uint32_t)ids[j]);
          const int s = bas[r] + bits_below(bal[r]);
          rr[j] = r * a.cap + s;
          if (!((seen >> r) & 1ull)) {
            first |= 1u << j;
            a.spos[(size_t)r * a.cap + s] = a.spos_base + t;
          }
          seen |= 1ull << r;
        }
      }
      a.ufirst[t] = first;
    }
  }
  return __popcll(mybal);
}

// Whole plan in one workgroup of 16 waves (T <= 1024).
template <int KMAX>
__global__ __launch_bounds__(1024) void plan_single_kernel(PlanArgs a) {
  __shared__ int cnt[kBlockChunks][kMaxRanks];
  __shared__ uint64_t bal[kBlockChunks][kWave];
  __shared__ int bas[kBlockChunks][kWave];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) *a.status_next = 0u;
  const int t = w * kChunk + lane;
  int ids[KMAX];
  uint32_t st = 0;
  const uint64_t mask = t < a.T ? load_token<KMAX>(a.indices, t, a.k, a.E, a.rdiv, ids, st) : 0ull;
  const int mine = ranks_popcount(mask, a.R, lane);
  if (lane < a.R) cnt[w][lane] = mine;
  report_status(a.status, a.tok_status, t, a.T, st);
  __syncthreads();
  int base = 0;
  if (lane < a.R) {
    for (int ww = 0; ww < w; ++ww) base += cnt[ww][lane];
    if (w == kBlockChunks - 1) {
      a.recv_counts[lane] = base + mine;
    }
  }
  if (w * kChunk < a.T) chunk_slots<KMAX>(a, w, lane, base, ids, mask, bal[w], bas[w]);
}

// Count launch: per block of a.blk_chunks chunks (one wave each), the exclusive
// prefix of every chunk inside the block (chunk_cnt[c][r]) and the block
// totals (block_cnt[b][r]).
template <int KMAX>
__global__ __launch_bounds__(1024) void plan_count_kernel(PlanArgs a) {
  __shared__ int cnt[kBlockChunks][kMaxRanks];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int c = b * a.blk_chunks + w;
  const int C = (a.T + kChunk - 1) / kChunk;
  if (b == 0 && threadIdx.x == 0) *a.status_next = 0u;
  const int t = c * kChunk + lane;
  int ids[KMAX];
  uint32_t st = 0;
  const uint64_t mask = t < a.T ? load_token<KMAX>(a.indices, t, a.k, a.E, a.rdiv, ids, st) : 0ull;
  if (t < a.T) a.mask[t] = mask;
  const int mine = ranks_popcount(mask, a.R, lane);
  if (lane < a.R) cnt[w][lane] = mine;
  report_status(a.status, a.tok_status, t, a.T, st);
  __syncthreads();
  if (lane < a.R) {
    int pre = 0;
    for (int ww = 0; ww < w; ++ww) pre += cnt[ww][lane];
    if (c < C) a.chunk_cnt[(size_t)c * a.R + lane] = pre;
    if (w == a.blk_chunks - 1) a.block_cnt[(size_t)b * a.R + lane] = pre + mine;
  }
}

// Slot launch: one wave per chunk.
template <int KMAX>
__global__ __launch_bounds__(256) void plan_slot_kernel(PlanArgs a) {
  __shared__ uint64_t bal[4][kWave];
  __shared__ int bas[4][kWave];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 4 + w;
  const int C = (a.T + kChunk - 1) / kChunk;
  if (c >= C) return;  // whole wave; no block barrier below
  const int b = c / a.blk_chunks;
  int base = 0;
  if (lane < a.R) {
    base = a.chunk_cnt[(size_t)c * a.R + lane];
    int acc[4] = {0, 0, 0, 0};
    int bb = 0;
    for (; bb + 4 <= b; bb += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += a.block_cnt[(size_t)(bb + u) * a.R + lane];
    }
    for (; bb < b; ++bb) acc[0] += a.block_cnt[(size_t)bb * a.R + lane];
    base += acc[0] + acc[1] + acc[2] + acc[3];
  }
  const int t = c * kChunk + lane;
  int ids[KMAX];
  uint64_t mask = 0;
  if (t < a.T) {
    const int32_t* p = a.indices + (size_t)t * a.k;
    if (KMAX == 8 && a.k == 8) {
      const int4 v0 = reinterpret_cast<const int4*>(p)[0];
      const int4 v1 = reinterpret_cast<const int4*>(p)[1];
      ids[0] = v0.x; ids[1] = v0.y; ids[2] = v0.z; ids[3] = v0.w;
      ids[4] = v1.x; ids[5] = v1.y; ids[6] = v1.z; ids[7] = v1.w;
    } else {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) ids[j] = j < a.k ? p[j] : 0;
    }
    mask = a.mask[t];
  }
  const int mine = chunk_slots<KMAX>(a, c, lane, base, ids, mask, bal[w], bas[w]);
  if (c == C - 1 && lane < a.R) a.recv_counts[lane] = base + mine;
}

__global__ void zero_counts_kernel(PlanArgs a) {
  const int i = threadIdx.x;
  if (i == 0) *a.status_next = 0u;
  if (i < a.R) a.recv_counts[i] = 0;
}

template <int KMAX>
hipError_t launch_plan_k(const PlanArgs& a, hipStream_t s) {
  const int C = (a.T + kChunk - 1) / kChunk;
  if (C <= kBlockChunks) {
    plan_single_kernel<KMAX><<<1, 1024, 0, s>>>(a);
    return hipGetLastError();
  }
  PlanArgs b = a;
  b.blk_chunks = count_block_chunks(C);
  hipError_t e = launch_plan_counts(b, s);
  if (e != hipSuccess) return e;
  plan_slot_kernel<KMAX><<<(C + 3) / 4, 256, 0, s>>>(b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan_counts(const PlanArgs& a, hipStream_t s) {
  const int C = (a.T + kChunk - 1) / kChunk;
  const int n = a.blk_chunks;
  if (n != count_block_chunks(C)) return hipErrorInvalidValue;
  const int B = (C + n - 1) / n;
  if (a.k <= 8) plan_count_kernel<8><<<B, 64 * n, 0, s>>>(a);
  else plan_count_kernel<kMaxTopk><<<B, 64 * n, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  if (a.T == 0) {
    zero_counts_kernel<<<1, 64, 0, s>>>(a);
    return hipGetLastError();
  }
  return a.k <= 8 ? launch_plan_k<8>(a, s) : launch_plan_k<kMaxTopk>(a, s);
}

}  // namespace mep
