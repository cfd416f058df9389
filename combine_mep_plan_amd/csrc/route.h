// Token routing helpers shared by the plan and the fused plan+dispatch kernels.
//
// A token's destination ranks are the distinct ranks of its top-k experts
// (expert e lives on rank e / num_experts_per_rank); ROCm/mori issue #57: a
// token is sent once per destination rank.  A token naming an expert id
// outside [0, E) is not dispatched.
#pragma once

#include "dev.h"
#include "mep_internal.h"

namespace mep {

// Load token t's top-k ids (k <= KMAX).
template <int KMAX>
__device__ __forceinline__ void load_ids(const int32_t* indices, int t, int k, int (&ids)[KMAX]) {
  const int32_t* p = indices + (size_t)t * k;
  if (KMAX == 8 && k == 8) {
    const int4 v0 = reinterpret_cast<const int4*>(p)[0];
    const int4 v1 = reinterpret_cast<const int4*>(p)[1];
    ids[0] = v0.x; ids[1] = v0.y; ids[2] = v0.z; ids[3] = v0.w;
    ids[4] = v1.x; ids[5] = v1.y; ids[6] = v1.z; ids[7] = v1.w;
  } else {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ids[j] = j < k ? p[j] : 0;
  }
}

// A token's destination-rank mask from its ids; 0 for a token with a bad id.
// Sets MEP_DEV_* bits in st.
template <int KMAX>
__device__ __forceinline__ uint64_t token_mask(const int (&ids)[KMAX], int k, int E, RankDiv rdiv,
                                               uint32_t& st) {
  uint64_t mask = 0;
  bool bad = false, dup = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int e = ids[j];
    if (j < k) {
      if (e < 0 || e >= E) {
        bad = true;
      } else {
        mask |= 1ull << rdiv((uint32_t)e);
#pragma unroll
        for (int jj = 0; jj < j; ++jj) dup |= (ids[jj] == e);
      }
    }
  }
  if (bad) { st |= MEP_DEV_BAD_INDEX; return 0; }
  if (dup) st |= MEP_DEV_DUP_EXPERT;
  return mask;
}

// Both: token t's ids and destination-rank mask.
template <int KMAX>
__device__ __forceinline__ uint64_t load_token(const int32_t* indices, int t, int k, int E,
                                               RankDiv rdiv, int (&ids)[KMAX], uint32_t& st) {
  load_ids<KMAX>(indices, t, k, ids);
  return token_mask<KMAX>(ids, k, E, rdiv, st);
}

// Lane r receives the number of lanes whose mask has bit r (0 in lanes >= R).
__device__ __forceinline__ int ranks_popcount(uint64_t mask, int R, int lane) {
  int mine = 0;
  for (int r = 0; r < R; ++r) {
    const uint64_t b = ballot((mask >> r) & 1ull);
    if (lane == r) mine = __popcll(b);
  }
  return mine;
}

// Wave-wide OR of status bits into the device status word (one atomic).
__device__ __forceinline__ void or_status(uint32_t* status, uint32_t st) {
  const uint64_t any_bad = ballot(st & MEP_DEV_BAD_INDEX);
  const uint64_t any_dup = ballot(st & MEP_DEV_DUP_EXPERT);
  if (lane_id() == 0 && (any_bad | any_dup))
    atomicOr(status, (any_bad ? MEP_DEV_BAD_INDEX : 0u) | (any_dup ? MEP_DEV_DUP_EXPERT : 0u));
}

// A plan kernel's report of its tokens' bits (st: this lane's token t).
// Outside graph capture the wave ORs them into the status word (sticky until
// reset).  In a captured iteration (tok_status set) every token's bits are
// stored in its own byte -- each replay rewrites all of them, so nothing has
// to be cleared first and no extra launch is captured.  Whole-wave call.
__device__ __forceinline__ void report_status(uint32_t* status, uint8_t* tok_status, int t, int T,
                                              uint32_t st) {
  if (tok_status) {
    if (t < T) tok_status[t] = (uint8_t)st;
  } else {
    or_status(status, st);
  }
}

__device__ __forceinline__ uint64_t lane_value64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)lane_value((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)lane_value((int)(uint32_t)(v >> 32), lane);
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

}  // namespace mep
