// Dispatch: scatter each token's row (bf16 copy; OCP E4M3 codes with one fp32
// scale per 128 columns; OCP MX FP4 with one E8M0 scale per 32 columns; or an
// already-quantized FP8/FP4 row with the caller's scales) plus its k weights
// and k expert ids into the receive buffer of every distinct destination
// rank, at the token's slot.
//
// Source: "MORI-EP User Guide", section 3 dispatch() (outputs: received rows,
// weights, scales, indices); "Choosing an EP API and backend": the gfx950 FP8
// flavour is OCP E4M3.  The block-scale rule (scale = amax / 448 per 128
// columns, code = E4M3(x / scale), round to nearest even) is this library's
// reading; the pages do not print the format.
//
// Layout of the work: a row is cut into slices of 64 lane items -- each lane
// owns one item of the received row (bf16: 8 columns, 16 bytes; FP8: 16
// columns, 16 bytes, 8 lanes per 128-column scale block; MX FP4: 16 columns,
// 8 bytes, 2 lanes per MX block; carried FP4: 32 columns, 16 bytes) -- and
// one wave handles one (token, slice).  Many small waves keep enough writes in
// flight to approach the HBM write rate; every receive-row store is a
// non-temporal 16- or 8-byte-per-lane store (1 KiB or 512 bytes per wave
// instruction).
//
// Where the destination slots come from:
//   kRoute  : a prior plan's receive row of each (token, top-k position);
//   kCounts : computed here from the count launch's per-chunk prefixes (the
//             wave ballots its 64-token chunk's rank masks), which also writes
//             the plan outputs -- a fused plan+dispatch;
//   kInline : as kCounts, but the prefixes are recomputed from the ids of the
//             earlier chunks, for small batches: plan+dispatch in one launch.
#include "payload.h"
#include "route.h"

namespace mep {

namespace {

enum { kRoute = 0, kCounts = 1, kInline = 2 };

// Where token t's rows go, as seen by one wave (fused modes).
struct WaveRoute {
  uint64_t tok_mask;  // ranks token t goes to (uniform)
  uint64_t mask_l;    // rank mask of token (t's chunk)*64 + lane
  int base;           // lane r: rows rank r received from tokens before t's chunk
  int tl;             // t's lane in its chunk

  // Receive slot of token t on rank r (r uniform, bit r set in tok_mask).
  __device__ __forceinline__ int slot(int r) const {
    const uint64_t b = ballot((mask_l >> r) & 1ull);
    const uint64_t below = tl ? (b & (~0ull >> (64 - tl))) : 0ull;
    return lane_value(base, r) + __popcll(below);
  }
};

template <int MODE, int KMAX>
__device__ __forceinline__ WaveRoute wave_route(const DispatchArgs& a, int t, int lane,
                                                uint32_t& st) {
  WaveRoute w;
  w.tl = t & 63;
  const int c = t >> 6;
  const int tok = c * kChunk + lane;
  w.base = 0;
  if (MODE == kCounts) {
    // the chunk's in-block prefix and the first 16 earlier blocks' totals go
    // out together with the mask load (a rolled loop would wait on each);
    // blocks past the 16th (batches over 16384 tokens) are summed after
    const int nb = c / a.blk_chunks;
    int acc = 0, v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = 0;
    if (lane < a.R) {
      acc = a.chunk_cnt[(size_t)c * a.R + lane];
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (q < nb) v[q] = a.block_cnt[(size_t)q * a.R + lane];
    }
    w.mask_l = tok < a.T ? a.mask[tok] : 0ull;
    if (lane < a.R) {
      for (int b = 16; b < nb; ++b) acc += a.block_cnt[(size_t)b * a.R + lane];
#pragma unroll
      for (int q = 0; q < 16; ++q) acc += v[q];
      w.base = acc;
    }
  } else if (KMAX <= 8) {
    // the token's chunk and the (at most three) earlier chunks: every id load
    // goes out before any mask is formed
    constexpr int kPrev = kInlinePlanTokens / kChunk - 1;
    int ids[KMAX], prev[kPrev][KMAX];
    if (tok < a.T) load_ids<KMAX>(a.idx, tok, a.k, ids);
#pragma unroll
    for (int q = 0; q < kPrev; ++q)
      if (q < c) load_ids<KMAX>(a.idx, q * kChunk + lane, a.k, prev[q]);
#pragma unroll
    for (int q = 0; q < kPrev; ++q) {
      if (q >= c) continue;  // uniform
      uint32_t ignore = 0;
      w.base += ranks_popcount(token_mask<KMAX>(prev[q], a.k, a.E, a.rdiv, ignore), a.R, lane);
    }
    w.mask_l = tok < a.T ? token_mask<KMAX>(ids, a.k, a.E, a.rdiv, st) : 0ull;
  } else {
    int ids[KMAX];
    for (int cc = 0; cc < c; ++cc) {
      uint32_t ignore = 0;
      const uint64_t m = load_token<KMAX>(a.idx, cc * kChunk + lane, a.k, a.E, a.rdiv, ids,
                                          ignore);
      w.base += ranks_popcount(m, a.R, lane);
    }
    w.mask_l = tok < a.T ? load_token<KMAX>(a.idx, tok, a.k, a.E, a.rdiv, ids, st) : 0ull;
  }
  w.tok_mask = lane_value64(w.mask_l, w.tl);
  return w;
}

// Plan outputs for token t (fused modes; one wave per token does this):
// receive row of each top-k position, first-occurrence bits, src_token_pos,
// and -- from the last token's wave -- recv_counts.  e: lane < k holds the
// token's expert id of top-k position lane.
__device__ __forceinline__ void write_route(const DispatchArgs& a, const WaveRoute& w, int t,
                                            int lane, int e) {
  if (w.tok_mask == 0) {
    if (lane < a.k) a.rrow[(size_t)t * a.k + lane] = -1;
    if (lane == 0) a.ufirst[t] = 0u;
  } else {
    const int rj = lane < a.k ? (int)a.rdiv((uint32_t)e) : -1;
    int my = 0;
    uint32_t first = 0;
    for (uint64_t m = w.tok_mask; m; m &= m - 1) {
      const int r = __builtin_ctzll(m);
      const int s = w.slot(r);
      const uint64_t b = ballot(rj == r);  // top-k positions naming rank r
      first |= 1u << __builtin_ctzll(b);
      if (rj == r) my = s;
      if (lane == 0) a.spos[(size_t)r * a.cap + s] = a.spos_base + t;
    }
    if (lane < a.k) a.rrow[(size_t)t * a.k + lane] = rj * a.cap + my;
    if (lane == 0) a.ufirst[t] = first;
  }
  if (t == a.T - 1) {
    const int tot = w.base + ranks_popcount(w.mask_l, a.R, lane);
    if (lane < a.R) a.recv_counts[lane] = tot;
  }
}

// What slice 0 writes with every row of a token besides the payload: its k
// weights and ids and, carrying, the caller's scale words.  Loaded once per
// token, before the stores: on this architecture a wait for a load issued
// after stores also waits for those stores.
struct TokenMeta {
  float w;     // lane < k: weight
  int32_t id;  // lane < k: expert id
  float sc;    // carrying, lane < scale_dim: scale word (the first 64)
};

template <int QUANT>
__device__ __forceinline__ TokenMeta load_meta(const DispatchArgs& a, int t, int sl, int lane) {
  TokenMeta m{0.0f, 0, 0.0f};
  if (sl == 0 && lane < a.k) {
    m.w = a.w[(size_t)t * a.k + lane];
    m.id = a.idx[(size_t)t * a.k + lane];
  }
  if (is_carry(QUANT) && sl == 0 && lane < a.scale_dim)
    m.sc = a.x_scales[(size_t)t * a.scale_dim + lane];
  return m;
}

// QUANT: a MEP_QUANT_* payload mode (see payload.h).
template <int QUANT, int MODE, int KMAX>
__global__ __launch_bounds__(256) void dispatch_kernel(DispatchArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = g / a.slices, sl = g - t * a.slices;
  if (t >= a.T) return;
  if (MODE == kInline && g == 0 && lane == 0) *a.status_next = 0u;

  // this wave's unit of the row: loads go out before the routing work
  const int nu = lane_items(QUANT, a.H);
  const int v = sl * kWave + lane;
  const bool on = v < nu;
  Unit<QUANT> unit;
  unit.load(a.x, t, a.H, v, on);
  // fused modes: the plan outputs need the ids, so the token's metadata goes
  // out with the payload unit
  TokenMeta meta{0.0f, 0, 0.0f};
  if (MODE != kRoute) meta = load_meta<QUANT>(a, t, sl, lane);

  uint32_t first = 0;
  WaveRoute w{};
  if (MODE == kRoute) {
    first = a.ufirst[t];
    if (first == 0) return;  // token not dispatched (bad expert id)
  } else {
    uint32_t st = 0;
    w = wave_route<MODE, KMAX>(a, t, lane, st);
    if (sl == 0) {
      if (MODE == kInline) {
        if (a.tok_status) {
          if (lane == w.tl) a.tok_status[t] = (uint8_t)st;
        } else {
          or_status(a.status, lane == w.tl ? st : 0u);
        }
      }
      write_route(a, w, t, lane, meta.id);
    }
    if (w.tok_mask == 0) return;
  }

  float scale = 0.0f;
  uint32_t e8 = 0;
  const typename Unit<QUANT>::Out q = unit.convert(scale, e8);
  // after a prior plan, loading the metadata and the rows only once the
  // token is known to be dispatched measured faster at large batches than
  // issuing them with the payload unit
  if (MODE == kRoute) meta = load_meta<QUANT>(a, t, sl, lane);
  auto emit = [&](int row) {
    if (on) {
      store_nt(reinterpret_cast<typename Unit<QUANT>::Out*>(a.recv_x) + (size_t)row * nu + v, q);
      store_unit_scale<QUANT>(a.recv_scales, (size_t)row, a.H, v, scale, e8);
    }
    if (sl == 0) {
      if (lane < a.k) {
        a.recv_w[(size_t)row * a.k + lane] = meta.w;
        a.recv_idx[(size_t)row * a.k + lane] = meta.id;
      }
      if (is_carry(QUANT)) {
        if (lane < a.scale_dim) a.recv_scales[(size_t)row * a.scale_dim + lane] = meta.sc;
        for (int i = lane + kWave; i < a.scale_dim; i += kWave)  // rows over 64 words
          a.recv_scales[(size_t)row * a.scale_dim + i] = a.x_scales[(size_t)t * a.scale_dim + i];
      }
    }
  };
  if (MODE == kRoute) {
    // the token's rows, loaded before the first store
    const int32_t* rr = a.rrow + (size_t)t * a.k;
    int rows[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) rows[j] = j < a.k && (first >> j & 1u) ? rr[j] : -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (rows[j] >= 0) emit(rows[j]);
  } else {
    for (uint64_t m = w.tok_mask; m; m &= m - 1) {
      const int r = __builtin_ctzll(m);
      emit(r * a.cap + w.slot(r));
    }
  }
}

template <int QUANT, int MODE>
hipError_t launch_mode(const DispatchArgs& a0, hipStream_t s) {
  DispatchArgs a = a0;
  a.slices = (lane_items(QUANT, a.H) + kWave - 1) / kWave;
  a.slice_units = kWave;
  const int64_t waves = (int64_t)a.T * a.slices;
  const int blocks = (int)((waves + 3) / 4);
  if (a.k <= 8) dispatch_kernel<QUANT, MODE, 8><<<blocks, 256, 0, s>>>(a);
  else dispatch_kernel<QUANT, MODE, kMaxTopk><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_dtype(const DispatchArgs& a, hipStream_t s) {
  switch (a.quant) {
    case MEP_QUANT_FP8_E4M3_BLOCK128: return launch_mode<MEP_QUANT_FP8_E4M3_BLOCK128, MODE>(a, s);
    case MEP_QUANT_FP8_CARRY: return launch_mode<MEP_QUANT_FP8_CARRY, MODE>(a, s);
    case MEP_QUANT_FP4_CARRY: return launch_mode<MEP_QUANT_FP4_CARRY, MODE>(a, s);
    case MEP_QUANT_MXFP4: return launch_mode<MEP_QUANT_MXFP4, MODE>(a, s);
    default: return launch_mode<MEP_QUANT_NONE, MODE>(a, s);
  }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return launch_dtype<kRoute>(a, s);
}

hipError_t launch_plan_dispatch(const PlanArgs& p, const DispatchArgs& a, hipStream_t s) {
  if (a.T == 0) return launch_plan(p, s);
  if (a.T <= kInlinePlanTokens) return launch_dtype<kInline>(a, s);
  const int C = (a.T + kChunk - 1) / kChunk;
  PlanArgs pc = p;
  DispatchArgs ac = a;
  pc.blk_chunks = ac.blk_chunks = count_block_chunks(C);
  hipError_t e = launch_plan_counts(pc, s);
  if (e != hipSuccess) return e;
  return launch_dtype<kCounts>(ac, s);
}

}  // namespace mep
