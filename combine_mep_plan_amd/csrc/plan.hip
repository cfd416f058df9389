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
// Two launches over 64-token chunks (one wave per chunk):
//   count: each wave builds its tokens' destination-rank masks and, with one
//          ballot per rank, the chunk's per-rank row counts;
//   slot:  each wave sums the counts of the chunks before it (exclusive
//          prefix, from L2), then ranks its own tokens with ballot + mbcnt,
//          writes src_token_pos, the flat receive row of every (t, j) and the
//          first-occurrence bits.  The last chunk also writes recv_counts.
#include "dev.h"
#include "mep_internal.h"

namespace mep {

__global__ __launch_bounds__(256) void plan_count_kernel(PlanArgs a) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int C = (a.T + kChunk - 1) / kChunk;
  if (c >= C) return;  // whole wave
  const int t = c * kChunk + lane;
  uint64_t mask = 0;
  uint32_t st = 0;
  if (t < a.T) {
    const int32_t* ids = a.indices + (size_t)t * a.k;
    bool bad = false, dup = false;
    for (int j = 0; j < a.k; ++j) {
      const int e = ids[j];
      if (e < 0 || e >= a.E) {
        bad = true;
      } else {
        mask |= 1ull << a.rdiv((uint32_t)e);
        for (int jj = 0; jj < j; ++jj) dup |= (ids[jj] == e);
      }
    }
    if (bad) { mask = 0; st |= MEP_DEV_BAD_INDEX; }
    else if (dup) st |= MEP_DEV_DUP_EXPERT;
    a.mask[t] = mask;
  }
  int mine = 0;
  for (int r = 0; r < a.R; ++r) {
    const uint64_t b = ballot((mask >> r) & 1ull);
    if (lane == r) mine = __popcll(b);
  }
  if (lane < a.R) a.chunk_cnt[(size_t)c * a.R + lane] = mine;
  const uint64_t any_bad = ballot(st & MEP_DEV_BAD_INDEX);
  const uint64_t any_dup = ballot(st & MEP_DEV_DUP_EXPERT);
  if (lane == 0 && (any_bad | any_dup)) {
    atomicOr(a.status, (any_bad ? MEP_DEV_BAD_INDEX : 0u) | (any_dup ? MEP_DEV_DUP_EXPERT : 0u));
  }
}

// LDS: per wave, the slot each lane's token got on each rank it goes to.
__global__ __launch_bounds__(64) void plan_slot_kernel(PlanArgs a) {
  __shared__ int32_t slot_of[kMaxRanks][kWave];
  const int lane = threadIdx.x;
  const int c = blockIdx.x;
  const int C = (a.T + kChunk - 1) / kChunk;
  // exclusive prefix over earlier chunks, lane r holding rank r
  int base = 0;
  if (lane < a.R) {
    for (int cc = 0; cc < c; ++cc) base += a.chunk_cnt[(size_t)cc * a.R + lane];
    if (c == C - 1) a.recv_counts[lane] = base + a.chunk_cnt[(size_t)c * a.R + lane];
  }
  const int t = c * kChunk + lane;
  const bool valid = t < a.T;
  const uint64_t mask = valid ? a.mask[t] : 0ull;
  for (int r = 0; r < a.R; ++r) {
    const uint64_t b = ballot((mask >> r) & 1ull);
    if (b == 0) continue;  // uniform
    const int s = lane_value(base, r) + bits_below(b);
    if ((mask >> r) & 1ull) {
      slot_of[r][lane] = s;
      a.spos[(size_t)r * a.cap + s] = a.spos_base + t;
    }
  }
  if (!valid) return;  // no barrier below: each lane reads only its own column
  int32_t* rr = a.rrow + (size_t)t * a.k;
  if (mask == 0) {
    for (int j = 0; j < a.k; ++j) rr[j] = -1;
    a.ufirst[t] = 0;
    return;
  }
  const int32_t* ids = a.indices + (size_t)t * a.k;
  uint64_t seen = 0;
  uint32_t first = 0;
  for (int j = 0; j < a.k; ++j) {
    const int r = (int)a.rdiv((uint32_t)ids[j]);
    rr[j] = r * a.cap + slot_of[r][lane];
    if (!((seen >> r) & 1ull)) first |= 1u << j;
    seen |= 1ull << r;
  }
  a.ufirst[t] = first;
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  if (a.T == 0) {
    zero_i32_kernel<<<1, 64, 0, s>>>(a.recv_counts, a.R);
    return hipGetLastError();
  }
  const int C = (a.T + kChunk - 1) / kChunk;
  plan_count_kernel<<<(C + 3) / 4, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  plan_slot_kernel<<<C, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mep
