// Standard-MoE (expert-major) conversion of the dispatch output.
//
// Source: "MORI-EP User Guide", section 4 Standard MoE Compatibility:
// convert_dispatch_output() turns the 2-D receive buffer into per-expert
// packed rows with per-expert counts and source info.  This library's
// layout: experts in global order, each expert's rows in ascending receive
// slot, each expert segment starting at a multiple of 128 rows; padding rows
// are not written.
//
// Two launches:
//   count:   one workgroup per rank; its 16 waves take consecutive runs of the
//            rank's 64-row receive chunks.  Per row: the mask of the rank's
//            local experts it names; per chunk: one ballot per local expert
//            gives the chunk's rows naming it.  Each wave keeps running sums
//            (one lane per local expert), the waves' totals meet in LDS, and
//            the launch writes every expert's row count and, per (chunk,
//            expert), the rows of the rank's earlier chunks naming it -- an
//            expert's rows all come from its own rank, so no other workgroup
//            is involved -- and, with every segment padded to 128 rows, each
//            expert's offset among its rank's segments and the rank's total.
//            It also clears the (token, top-k) -> expert-major row map;
//   scatter: one wave per (receive row, slice of the row).  Each wave scans
//            the R receive counts and the R padded rank totals across its
//            lanes, which gives its row's rank and the start of that rank's
//            segments (no LDS, no barrier; workgroup 0 also writes the
//            segment offsets out).  The row's place inside an expert segment
//            is that start, plus the expert's offset inside the rank, plus
//            the rows of the rank's earlier chunks naming that expert, plus a
//            ballot count of the earlier rows of its own chunk.  Each slice
//            is copied with 16-byte-per-lane loads and non-temporal stores.
#include "dev.h"
#include "route.h"

namespace mep {

namespace {

__device__ __forceinline__ int clamp_count(const EmArgs& a, int r) {
  return min(max(a.recv_counts[r], 0), a.cap);
}

constexpr int kCountWaves = 16;

template <int KMAX>
__global__ __launch_bounds__(kCountWaves * 64) void em_count_kernel(EmArgs a) {
  __shared__ int32_t wtot[kCountWaves][kMaxEpr];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = blockIdx.x;
  // Loads go out before any store (a wait for a load issued after stores
  // also waits for those stores): the rank's receive count and, on the guess
  // that the rank received at most 16 chunks (one per wave), the ids of chunk
  // w's rows -- all inside the receive buffer; rows at or past the count are
  // ignored below.
  int spec[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) spec[j] = -1;
  const int spec_s = w * kChunk + lane;
  if (spec_s < a.cap) load_ids<KMAX>(a.recv_idx, r * a.cap + spec_s, a.k, spec);
  const int cnt = clamp_count(a, r);
  // clear the (t, j) -> expert-major row map
  const int64_t nmap = (int64_t)a.T * a.k;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nmap;
       i += (int64_t)gridDim.x * blockDim.x)
    a.em_row[i] = -1;

  const int nch = (cnt + kChunk - 1) / kChunk;
  const int per = (nch + kCountWaves - 1) / kCountWaves;
  const int c0 = min(w * per, nch), c1 = min(c0 + per, nch);
  const int E = a.R * a.epr;
  // chunk c's local-expert masks (stored per row) and, in lane l, its rows
  // naming local expert l
  auto count_chunk = [&](int c, const int (&ids)[KMAX]) {
    const int s = c * kChunk + lane;
    uint64_t lm = 0;
    if (s < cnt) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const int e = ids[j];
        if (j < a.k && e >= 0 && e < E && (int)a.rdiv((uint32_t)e) == r) lm |= 1ull << (e - r * a.epr);
      }
      a.lmask[(size_t)r * a.cap + s] = lm;
    }
    int mine = 0;
    for (int l = 0; l < a.epr; ++l) {
      const uint64_t b = ballot((lm >> l) & 1ull);
      if (lane == l) mine = __popcll(b);
    }
    return mine;
  };
  constexpr int B = KMAX <= 8 ? 4 : 1;  // chunks whose ids are loaded together
  int run = 0;  // lane l: rows of this wave's earlier chunks naming local expert l
  int pre0[B];  // the first batch's prefixes, stored once the base is known
#pragma unroll
  for (int q = 0; q < B; ++q) pre0[q] = 0;
  if (per == 1) {  // chunk c0 == w, whose ids are already here
    if (c0 < c1) run = count_chunk(c0, spec);
  } else {
    for (int cb = c0; cb < c1; cb += B) {  // uniform
      int ids[B][KMAX];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int s = (cb + q) * kChunk + lane;
        if (cb + q < c1 && s < cnt) load_ids<KMAX>(a.recv_idx, r * a.cap + s, a.k, ids[q]);
      }
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int c = cb + q;
        if (c >= c1) break;  // uniform
        const int mine = count_chunk(c, ids[q]);
        if (cb == c0) pre0[q] = run;
        else if (lane < a.epr) a.ccnt[((size_t)r * a.CR + c) * a.epr + lane] = run;
        run += mine;
      }
    }
  }
  if (lane < a.epr) wtot[w][lane] = run;
  __syncthreads();
  int tot = 0;
  if (lane < a.epr) {
    int base = 0;
#pragma unroll
    for (int ww = 0; ww < kCountWaves; ++ww) {
      const int v = wtot[ww][lane];
      tot += v;
      base += ww < w ? v : 0;
    }
    if (w == 0) a.em_counts[r * a.epr + lane] = tot;
#pragma unroll
    for (int q = 0; q < B; ++q)
      if (c0 + q < c1) a.ccnt[((size_t)r * a.CR + c0 + q) * a.epr + lane] = pre0[q] + base;
    if (base)  // chunks past the first batch (more than B per wave)
      for (int c = c0 + B; c < c1; ++c) a.ccnt[((size_t)r * a.CR + c) * a.epr + lane] += base;
  }
  if (w == 0) {
    // the rank's experts' segments, each padded to a multiple of 128 rows:
    // their in-rank offsets and the rank's total
    const int pad = (tot + 127) / 128 * 128;
    int inc = pad;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(inc, d);
      if (lane >= d) inc += v;
    }
    if (lane < a.epr) a.seg_inrank[r * a.epr + lane] = inc - pad;
    if (lane == kWave - 1) a.seg_rank[r] = inc;
  }
}

// 16-byte units per lane per scatter wave.  Each wave first finds its row's
// rank, local experts and in-chunk position, so larger waves pay that less
// often, while smaller ones keep more rows in flight: at 4096 x 7168 FP8 on
// 32 ranks the conversion took 99.5, 84.5, 86.0 and 87.9 us with 1, 2, 3 and
// 4 units per lane (with the segment offsets still scanned in LDS by every
// workgroup: 129, 95.5, 91.6 and 94.8 us).
constexpr int kEmUnitsPerLane = 2;

template <int UPL>
__global__ __launch_bounds__(256) void em_scatter_kernel(EmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = first_lane(blockIdx.x * 4 + w);
  const int u = g / a.slices, sl = g - u * a.slices;
  // lane q < R: rank q's receive rows and its experts' padded segment rows,
  // both scanned across the lanes
  int n = 0, p = 0;
  if (lane < a.R) {
    n = clamp_count(a, lane);
    p = a.seg_rank[lane];
  }
  int n_inc = n, p_inc = p;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int vn = __shfl_up(n_inc, d), vp = __shfl_up(p_inc, d);
    if (lane >= d) {
      n_inc += vn;
      p_inc += vp;
    }
  }
  if (blockIdx.x == 0) {
    // segment offsets: expert e of rank q starts after the padded segments of
    // the ranks before q and of q's earlier experts
    const int E = a.R * a.epr;
    const int p_exc = p_inc - p;
    for (int e0 = w * kWave; e0 < E; e0 += 4 * kWave) {  // uniform
      const int e = e0 + lane;
      const int q = e < E ? (int)a.rdiv((uint32_t)e) : 0;
      const int base = __shfl(p_exc, q);
      if (e < E) a.em_offsets[e] = base + a.seg_inrank[e];
    }
    if (tid == 0) a.em_offsets[E] = lane_value(p_inc, a.R - 1);
  }

  // this wave's receive row u (in rank-major order over the received rows):
  // its rank is the number of ranks whose rows all come before u
  const bool live = u < lane_value(n_inc, a.R - 1);
  if (!live) return;
  const int r = __popcll(ballot(lane < a.R && n_inc <= u));
  const int seg_base = r > 0 ? lane_value(p_inc, r - 1) : 0;
  const int s = u - (r > 0 ? lane_value(n_inc, r - 1) : 0);
  const int cnt = lane_value(n, r);
  const size_t row = (size_t)r * a.cap + s;
  const int nv = a.row_units;  // 16-byte units per row
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
  // lane l: rows of the rank's earlier chunks naming local expert l, and the
  // start of local expert l's segment inside the rank's segments
  int pre = 0, inr = 0;
  if (lane < a.epr) {
    pre = a.ccnt[((size_t)r * a.CR + c) * a.epr + lane];
    inr = a.seg_inrank[r * a.epr + lane];
  }
  int pos_code = 0, t = -1, myid = -1;
  float scw = 0.0f;  // the row's first 64 scale words, one per lane
  if (sl == 0) {
    pos_code = a.spos[row];
    t = pos_code - a.spos_base;
    if (lane < a.k) myid = a.recv_idx[row * a.k + lane];
    if (lane < a.nb) scw = a.recv_scales[row * a.nb + lane];
  }

  const uint64_t lm_self =
      ((uint64_t)(uint32_t)lane_value((int)(uint32_t)lm_lane, sc)) |
      ((uint64_t)(uint32_t)lane_value((int)(uint32_t)(lm_lane >> 32), sc) << 32);
  u32x4* dst_x = reinterpret_cast<u32x4*>(a.em_x);
  for (uint64_t m = lm_self; m; m &= m - 1) {
    const int l = __builtin_ctzll(m);
    const uint64_t b = ballot(lane < sc && ((lm_lane >> l) & 1ull));
    const int64_t pos =
        (int64_t)seg_base + lane_value(inr, l) + lane_value(pre, l) + __popcll(b);
    if (pos >= a.cap_em) {
      if (lane == 0) atomicOr(a.status, (uint32_t)MEP_DEV_EM_OVERFLOW);
      continue;
    }
#pragma unroll
    for (int q = 0; q < UPL; ++q) {
      const int v = (sl * UPL + q) * kWave + lane;
      if (v < nv) store_nt(dst_x + (size_t)pos * nv + v, val[q]);
    }
    if (sl == 0) {  // the row's scale columns, one per lane
      if (lane < a.nb) a.em_scales[(size_t)pos * a.nb + lane] = scw;
      for (int i = lane + kWave; i < a.nb; i += kWave)  // rows over 64 words
        a.em_scales[(size_t)pos * a.nb + i] = a.recv_scales[row * a.nb + i];
    }
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
  if (a.k <= 8) em_count_kernel<8><<<a.R, kCountWaves * 64, 0, s>>>(a);
  else em_count_kernel<kMaxTopk><<<a.R, kCountWaves * 64, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one wave per (receive row, kEmUnits x 64 units); rows <= T * min(k, R);
  // at least one workgroup, which writes the segment offsets
  const int nv = a.row_units;
  const int per = kEmUnitsPerLane * kWave;
  a.slices = (nv + per - 1) / per;
  const int64_t rows = (int64_t)a.T * std::min(a.k, a.R);
  const int64_t waves = std::max<int64_t>(rows * a.slices, 1);
  em_scatter_kernel<kEmUnitsPerLane><<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mep
