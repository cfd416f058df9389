// Host side of the C ABI declared in include/mep.h: argument checks, call-order
// state and launch of the gfx950 kernels.  Every check here runs before any
// HIP call, so a rejected call launches nothing.
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "mep_internal.h"

struct mep_handle {
  mep_config cfg;
  unsigned char* ws;
  size_t ws_bytes;
  mep::WsLayout lay;
  mep::RankDiv rdiv;
  bool plan_valid;
  bool em_valid;
  bool planned_since_reset;
  bool captured;   // the last iteration's plan was recorded into a HIP graph
  bool eager_planned;     // a plan has run outside capture
  uint32_t eager_epoch;   // the epoch of the last plan outside capture
  uint32_t epoch;  // selects the status word; advanced by mep_reset
  int32_t plan_T;
};

namespace mep {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const mep_config& c) {
  WsLayout L{};
  const size_t cap = (size_t)c.max_num_inp_token_per_rank, k = (size_t)c.num_experts_per_token;
  const size_t R = (size_t)c.world_size, epr = (size_t)c.num_experts_per_rank;
  const size_t C = (cap + kChunk - 1) / kChunk;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  L.status = take(3 * sizeof(uint32_t));
  L.tok_status = take(cap);
  L.chunk_cnt = take(C * R * sizeof(int32_t));
  L.block_cnt = take((C + mep::kMinBlockChunks - 1) / mep::kMinBlockChunks * R * sizeof(int32_t));
  L.mask = take(cap * sizeof(uint64_t));
  L.rrow = take(cap * k * sizeof(int32_t));
  L.ufirst = take(cap * sizeof(uint32_t));
  L.em_row = take(cap * k * sizeof(int32_t));
  L.em_lmask = take(R * cap * sizeof(uint64_t));
  L.em_ccnt = take(R * C * epr * sizeof(int32_t));
  L.em_seg = take((R + R * epr) * sizeof(int32_t));
  L.sm_hist = take(C * R * epr * sizeof(int32_t));
  L.total = off;
  return L;
}

}  // namespace mep

using mep::WsLayout;

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

namespace mep {

int check_config(const mep_config* c) {
  if (!c) return MEP_ERR_NULL;
  const int64_t H = c->hidden_dim, R = c->world_size, epr = c->num_experts_per_rank;
  const int64_t k = c->num_experts_per_token, cap = c->max_num_inp_token_per_rank;
  if (H <= 0 || H % 8 != 0 || H > (1 << 20)) return MEP_ERR_CONFIG;
  if (R < 1 || R > mep::kMaxRanks) return MEP_ERR_CONFIG;
  if (epr < 1 || epr > mep::kMaxEpr) return MEP_ERR_CONFIG;
  if (k < 1 || k > mep::kMaxTopk || k > R * epr) return MEP_ERR_CONFIG;
  if (cap < 1) return MEP_ERR_CONFIG;
  if (c->rank < 0 || c->rank >= R) return MEP_ERR_CONFIG;
  // flat receive rows and src_token_pos must fit int32
  if (R * cap + (int64_t)c->rank * R * cap > INT32_MAX) return MEP_ERR_CONFIG;
  if (c->quant == MEP_QUANT_NONE) {
    if (c->scale_dim != 0) return MEP_ERR_CONFIG;
  } else if (c->quant == MEP_QUANT_FP8_E4M3_BLOCK128) {
    if (H % 128 != 0 || c->scale_dim != H / 128) return MEP_ERR_CONFIG;
  } else if (c->quant == MEP_QUANT_FP8_CARRY) {
    if (H % 16 != 0 || c->scale_dim < 0 || c->scale_dim > (1 << 16)) return MEP_ERR_CONFIG;
  } else if (c->quant == MEP_QUANT_FP4_CARRY) {
    if (H % 32 != 0 || c->scale_dim < 0 || c->scale_dim > (1 << 16)) return MEP_ERR_CONFIG;
  } else if (c->quant == MEP_QUANT_MXFP4) {
    if (H % 128 != 0 || c->scale_dim != H / 128) return MEP_ERR_CONFIG;
  } else {
    return MEP_ERR_CONFIG;
  }
  return MEP_OK;
}

RankDiv make_rdiv(int32_t epr) {
  RankDiv d;
  d.m = (uint32_t)(((1u << 20) + (uint32_t)epr - 1) / (uint32_t)epr);
  return d;
}

int check_rank_map(const mep_config& c, RankDiv rd) {
  const uint32_t E = (uint32_t)c.world_size * (uint32_t)c.num_experts_per_rank;
  for (uint32_t e = 0; e < E; ++e)
    if (rd(e) != e / (uint32_t)c.num_experts_per_rank) return MEP_ERR_CONFIG;
  return MEP_OK;
}

int check_plan_args(const mep_config& c, const int32_t* indices, int32_t T,
                    const int32_t* recv_counts, const int32_t* src_token_pos) {
  if (!recv_counts || !src_token_pos) return MEP_ERR_NULL;
  if (T < 0 || T > c.max_num_inp_token_per_rank) return MEP_ERR_SHAPE;
  if (T > 0 && !indices) return MEP_ERR_NULL;
  if ((indices && !aligned16(indices)) || !aligned16(recv_counts) || !aligned16(src_token_pos))
    return MEP_ERR_ALIGN;
  return MEP_OK;
}

// Scale columns the payload carries per row (0 for bf16 rows).
static int scale_cols(const mep_config& c) {
  return c.quant == MEP_QUANT_NONE ? 0 : c.scale_dim;
}

int check_dispatch_args(const mep_config& c, int32_t T, const void* x, const float* weights,
                        const float* scales, const int32_t* indices, const void* recv_x,
                        const float* recv_scales, const float* recv_weights,
                        const int32_t* recv_indices) {
  const bool carry = is_carry(c.quant);
  if (!recv_x || !recv_weights || !recv_indices) return MEP_ERR_NULL;
  if (scale_cols(c) > 0 && !recv_scales) return MEP_ERR_NULL;
  if (T > 0 && (!x || !weights || !indices)) return MEP_ERR_NULL;
  if (T > 0 && carry && c.scale_dim > 0 && !scales) return MEP_ERR_NULL;
  if ((x && !aligned16(x)) || (weights && !aligned16(weights)) ||
      (indices && !aligned16(indices)) || !aligned16(recv_x) ||
      (carry && scales && !aligned16(scales)) ||
      (recv_scales && !aligned16(recv_scales)) || !aligned16(recv_weights) ||
      !aligned16(recv_indices))
    return MEP_ERR_ALIGN;
  return MEP_OK;
}

PlanArgs plan_args(const mep_config& c, RankDiv rd, const WsPtrs& w, const int32_t* indices,
                   int32_t T, int32_t* recv_counts, int32_t* src_token_pos) {
  PlanArgs a{};
  a.indices = indices;
  a.recv_counts = recv_counts;
  a.spos = src_token_pos;
  a.status = w.status;
  a.status_next = w.status_next;
  a.tok_status = w.tok_status;
  a.chunk_cnt = w.chunk_cnt;
  a.block_cnt = w.block_cnt;
  a.mask = w.mask;
  a.rrow = w.rrow;
  a.ufirst = w.ufirst;
  a.T = T;
  a.k = c.num_experts_per_token;
  a.R = c.world_size;
  a.E = c.world_size * c.num_experts_per_rank;
  a.cap = c.max_num_inp_token_per_rank;
  a.spos_base = c.rank * c.world_size * c.max_num_inp_token_per_rank;
  a.rdiv = rd;
  return a;
}

DispatchArgs dispatch_args(const mep_config& c, RankDiv rd, const WsPtrs& w, int32_t T,
                           const void* x, const float* weights, const float* scales,
                           const int32_t* indices, void* recv_x, float* recv_scales,
                           float* recv_weights, int32_t* recv_indices) {
  DispatchArgs a{};
  a.x = x;
  a.x_scales = is_carry(c.quant) ? scales : nullptr;
  a.quant = c.quant;
  a.scale_dim = scale_cols(c);
  a.w = weights;
  a.idx = indices;
  a.rrow = w.rrow;
  a.ufirst = w.ufirst;
  a.recv_x = recv_x;
  a.recv_scales = recv_scales;
  a.recv_w = recv_weights;
  a.recv_idx = recv_indices;
  a.mask = w.mask;
  a.chunk_cnt = w.chunk_cnt;
  a.block_cnt = w.block_cnt;
  a.status = w.status;
  a.status_next = w.status_next;
  a.tok_status = w.tok_status;
  a.T = T;
  a.H = c.hidden_dim;
  a.k = c.num_experts_per_token;
  a.R = c.world_size;
  a.E = c.world_size * c.num_experts_per_rank;
  a.cap = c.max_num_inp_token_per_rank;
  a.spos_base = c.rank * c.world_size * c.max_num_inp_token_per_rank;
  a.rdiv = rd;
  return a;
}

}  // namespace mep

using mep::check_config;
using mep::scale_cols;

template <class T>
static T* ws_ptr(mep_handle* h, size_t off) {
  return reinterpret_cast<T*>(h->ws + off);
}

static int hip_rc(hipError_t e) { return e == hipSuccess ? MEP_OK : MEP_ERR_HIP; }

// Status words.  Outside graph capture: the word of the current reset epoch,
// ORed into by the kernels; a plan clears the word of the next epoch, so that
// it is zero when mep_reset moves there, and reset launches nothing.
//
// A replayed graph keeps the pointers it was captured with while mep_reset
// moves only the host epoch, so an iteration whose plan is captured reports
// differently, with nothing to clear beforehand: its plan kernels store each
// token's bad/repeated-id bits in the token's own byte (every replay rewrites
// all of them), and the expert-major overflow bit goes to word 2, which the
// plan's first launch clears (as it clears a next-epoch word) and only later
// launches set.  mep_get_status then ORs word 2 with the planned tokens' bytes.
static uint32_t* status_base(mep_handle* h) { return ws_ptr<uint32_t>(h, h->lay.status); }

static uint32_t* status_word(mep_handle* h) {
  return status_base(h) + (h->captured ? 2u : (h->epoch & 1u));
}

static uint32_t* status_next_word(mep_handle* h) {
  return status_base(h) + (h->captured ? 2u : ((h->epoch + 1u) & 1u));
}

static uint8_t* tok_status(mep_handle* h) {
  return h->captured ? ws_ptr<uint8_t>(h, h->lay.tok_status) : nullptr;
}

// Start of an iteration (a plan, fused plan+dispatch or standard-MoE
// dispatch): note whether the stream is being captured.  Back outside capture,
// the iteration starts in the epoch after the last plan outside capture, whose
// word that plan cleared (no plan outside capture yet: both words still hold
// the zeros of the fresh workspace); nothing is launched.
static int begin_iteration(mep_handle* h, hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return MEP_ERR_HIP;
  const bool capturing = cs == hipStreamCaptureStatusActive;
  if (!capturing) {
    if (h->captured && h->eager_planned) h->epoch = h->eager_epoch + 1u;
    h->eager_planned = true;
    h->eager_epoch = h->epoch;
  }
  h->captured = capturing;
  return MEP_OK;
}

// Expert-major segment offsets are int32 sums of per-expert counts padded to
// 128 rows; T*k rows and 127 padding rows per expert must fit.
static bool em_offsets_fit(const mep_config& c, int32_t T) {
  return (int64_t)T * c.num_experts_per_token +
             127 * (int64_t)c.world_size * c.num_experts_per_rank <= INT32_MAX;
}

extern "C" {

const char* mep_error_string(int code) {
  switch (code) {
    case MEP_OK: return "ok";
    case MEP_ERR_NULL: return "null pointer";
    case MEP_ERR_CONFIG: return "invalid config";
    case MEP_ERR_SHAPE: return "size out of range";
    case MEP_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MEP_ERR_STATE: return "call order violated";
    case MEP_ERR_HIP: return "HIP runtime error";
    case MEP_ERR_DEVICE: return "device status set";
    case MEP_ERR_NOMEM: return "out of host memory";
    default: return "unknown";
  }
}

size_t mep_workspace_bytes(const mep_config* cfg) {
  if (check_config(cfg) != MEP_OK) return 0;
  return mep::ws_layout(*cfg).total;
}

int mep_create(const mep_config* cfg, void* workspace, size_t workspace_bytes, mep_handle** out) {
  if (!out) return MEP_ERR_NULL;
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc != MEP_OK) return rc;
  if (!workspace) return MEP_ERR_NULL;
  if (!aligned16(workspace)) return MEP_ERR_ALIGN;
  const WsLayout lay = mep::ws_layout(*cfg);
  if (workspace_bytes < lay.total) return MEP_ERR_SHAPE;
  const mep::RankDiv rd = mep::make_rdiv(cfg->num_experts_per_rank);
  if (mep::check_rank_map(*cfg, rd) != MEP_OK) return MEP_ERR_CONFIG;
  mep_handle* h = (mep_handle*)calloc(1, sizeof(mep_handle));
  if (!h) return MEP_ERR_NOMEM;
  h->cfg = *cfg;
  h->ws = (unsigned char*)workspace;
  h->ws_bytes = workspace_bytes;
  h->lay = lay;
  h->rdiv = rd;
  *out = h;
  return MEP_OK;
}

int mep_destroy(mep_handle* h) {
  if (!h) return MEP_ERR_NULL;
  free(h);
  return MEP_OK;
}

// The workspace pointers of a handle's next call.
static mep::WsPtrs ws_ptrs(mep_handle* h) {
  mep::WsPtrs w{};
  w.status = status_word(h);
  w.status_next = status_next_word(h);
  w.tok_status = tok_status(h);
  w.chunk_cnt = ws_ptr<int32_t>(h, h->lay.chunk_cnt);
  w.block_cnt = ws_ptr<int32_t>(h, h->lay.block_cnt);
  w.mask = ws_ptr<uint64_t>(h, h->lay.mask);
  w.rrow = ws_ptr<int32_t>(h, h->lay.rrow);
  w.ufirst = ws_ptr<uint32_t>(h, h->lay.ufirst);
  return w;
}

static mep::PlanArgs plan_args(mep_handle* h, const int32_t* indices, int32_t T,
                               int32_t* recv_counts, int32_t* src_token_pos) {
  return mep::plan_args(h->cfg, h->rdiv, ws_ptrs(h), indices, T, recv_counts, src_token_pos);
}

static int check_plan_args(mep_handle* h, const int32_t* indices, int32_t T,
                           const int32_t* recv_counts, const int32_t* src_token_pos) {
  if (!h) return MEP_ERR_NULL;
  return mep::check_plan_args(h->cfg, indices, T, recv_counts, src_token_pos);
}

static int check_dispatch_args(mep_handle* h, int32_t T, const void* x, const float* weights,
                               const float* scales, const int32_t* indices, const void* recv_x,
                               const float* recv_scales, const float* recv_weights,
                               const int32_t* recv_indices) {
  return mep::check_dispatch_args(h->cfg, T, x, weights, scales, indices, recv_x, recv_scales,
                                  recv_weights, recv_indices);
}

static mep::DispatchArgs dispatch_args(mep_handle* h, int32_t T, const void* x,
                                       const float* weights, const float* scales,
                                       const int32_t* indices, void* recv_x, float* recv_scales,
                                       float* recv_weights, int32_t* recv_indices) {
  return mep::dispatch_args(h->cfg, h->rdiv, ws_ptrs(h), T, x, weights, scales, indices, recv_x,
                            recv_scales, recv_weights, recv_indices);
}

int mep_plan(mep_handle* h, const int32_t* indices, int32_t T, int32_t* recv_counts,
             int32_t* src_token_pos, void* stream) {
  int rc = check_plan_args(h, indices, T, recv_counts, src_token_pos);
  if (rc != MEP_OK) return rc;
  h->plan_valid = false;
  h->em_valid = false;
  rc = begin_iteration(h, (hipStream_t)stream);
  if (rc != MEP_OK) return rc;
  const mep::PlanArgs a = plan_args(h, indices, T, recv_counts, src_token_pos);
  rc = hip_rc(mep::launch_plan(a, (hipStream_t)stream));
  if (rc != MEP_OK) return rc;
  h->plan_valid = true;
  h->planned_since_reset = true;
  h->plan_T = T;
  return MEP_OK;
}

int mep_dispatch(mep_handle* h, const void* x, const float* weights, const float* scales,
                 const int32_t* indices, void* recv_x, float* recv_scales, float* recv_weights,
                 int32_t* recv_indices, void* stream) {
  if (!h) return MEP_ERR_NULL;
  if (!h->plan_valid) return MEP_ERR_STATE;
  const int32_t T = h->plan_T;
  int rc = check_dispatch_args(h, T, x, weights, scales, indices, recv_x, recv_scales,
                               recv_weights, recv_indices);
  if (rc != MEP_OK) return rc;
  const mep::DispatchArgs a = dispatch_args(h, T, x, weights, scales, indices, recv_x,
                                            recv_scales, recv_weights, recv_indices);
  return hip_rc(mep::launch_dispatch(a, (hipStream_t)stream));
}

int mep_plan_dispatch(mep_handle* h, const int32_t* indices, int32_t T, int32_t* recv_counts,
                      int32_t* src_token_pos, const void* x, const float* weights,
                      const float* scales, void* recv_x, float* recv_scales,
                      float* recv_weights, int32_t* recv_indices, void* stream) {
  int rc = check_plan_args(h, indices, T, recv_counts, src_token_pos);
  if (rc != MEP_OK) return rc;
  rc = check_dispatch_args(h, T, x, weights, scales, indices, recv_x, recv_scales, recv_weights,
                           recv_indices);
  if (rc != MEP_OK) return rc;
  h->plan_valid = false;
  h->em_valid = false;
  rc = begin_iteration(h, (hipStream_t)stream);
  if (rc != MEP_OK) return rc;
  const mep::PlanArgs p = plan_args(h, indices, T, recv_counts, src_token_pos);
  mep::DispatchArgs a = dispatch_args(h, T, x, weights, scales, indices, recv_x, recv_scales,
                                      recv_weights, recv_indices);
  a.recv_counts = recv_counts;
  a.spos = src_token_pos;
  rc = hip_rc(mep::launch_plan_dispatch(p, a, (hipStream_t)stream));
  if (rc != MEP_OK) return rc;
  h->plan_valid = true;
  h->planned_since_reset = true;
  h->plan_T = T;
  return MEP_OK;
}

int mep_to_expert_major(mep_handle* h, const void* recv_x, const float* recv_scales,
                        const int32_t* recv_indices, const int32_t* recv_counts,
                        const int32_t* src_token_pos, void* em_x, float* em_scales,
                        int32_t* em_counts, int32_t* em_offsets, int32_t* em_src_pos,
                        int64_t cap_em, void* stream) {
  if (!h) return MEP_ERR_NULL;
  if (!h->plan_valid) return MEP_ERR_STATE;
  const mep_config& c = h->cfg;
  const int nb = scale_cols(c);
  if (!recv_x || !recv_indices || !recv_counts || !src_token_pos || !em_x || !em_counts ||
      !em_offsets || !em_src_pos)
    return MEP_ERR_NULL;
  if (nb > 0 && (!recv_scales || !em_scales)) return MEP_ERR_NULL;
  if (cap_em < 0 || cap_em > INT32_MAX) return MEP_ERR_SHAPE;
  if (!em_offsets_fit(c, h->plan_T)) return MEP_ERR_SHAPE;
  if (!aligned16(recv_x) || !aligned16(recv_indices) || !aligned16(recv_counts) ||
      !aligned16(src_token_pos) || !aligned16(em_x) || !aligned16(em_counts) ||
      !aligned16(em_offsets) || !aligned16(em_src_pos) ||
      (recv_scales && !aligned16(recv_scales)) || (em_scales && !aligned16(em_scales)))
    return MEP_ERR_ALIGN;
  mep::EmArgs a{};
  a.recv_x = recv_x;
  a.recv_scales = nb > 0 ? recv_scales : nullptr;
  a.recv_idx = recv_indices;
  a.recv_counts = recv_counts;
  a.spos = src_token_pos;
  a.rrow = ws_ptr<int32_t>(h, h->lay.rrow);
  a.em_x = em_x;
  a.em_scales = nb > 0 ? em_scales : nullptr;
  a.em_counts = em_counts;
  a.em_offsets = em_offsets;
  a.em_src_pos = em_src_pos;
  a.em_row = ws_ptr<int32_t>(h, h->lay.em_row);
  a.lmask = ws_ptr<uint64_t>(h, h->lay.em_lmask);
  a.ccnt = ws_ptr<int32_t>(h, h->lay.em_ccnt);
  a.seg_rank = ws_ptr<int32_t>(h, h->lay.em_seg);
  a.seg_inrank = a.seg_rank + c.world_size;
  a.status = status_word(h);
  a.cap_em = cap_em;
  a.T = h->plan_T;
  a.H = c.hidden_dim;
  a.k = c.num_experts_per_token;
  a.R = c.world_size;
  a.rdiv = h->rdiv;
  a.epr = c.num_experts_per_rank;
  a.cap = c.max_num_inp_token_per_rank;
  a.CR = (c.max_num_inp_token_per_rank + mep::kChunk - 1) / mep::kChunk;
  a.nb = nb;
  a.row_units = mep::payload_units(c.quant, c.hidden_dim);
  a.spos_base = c.rank * c.world_size * c.max_num_inp_token_per_rank;
  h->em_valid = false;
  int rc = hip_rc(mep::launch_to_expert_major(a, (hipStream_t)stream));
  if (rc != MEP_OK) return rc;
  h->em_valid = true;
  return MEP_OK;
}

int mep_dispatch_standard_moe(mep_handle* h, const int32_t* indices, int32_t T, const void* x,
                              const float* scales, void* em_x, float* em_scales,
                              int32_t* em_counts, int32_t* em_offsets, int32_t* em_src_pos,
                              int64_t cap_em, void* stream) {
  if (!h) return MEP_ERR_NULL;
  const mep_config& c = h->cfg;
  const int nb = scale_cols(c);
  const bool carry = mep::is_carry(c.quant);
  if (T < 0 || T > c.max_num_inp_token_per_rank) return MEP_ERR_SHAPE;
  if (cap_em < 0 || cap_em > INT32_MAX || !em_offsets_fit(c, T)) return MEP_ERR_SHAPE;
  if (!em_x || !em_counts || !em_offsets || !em_src_pos) return MEP_ERR_NULL;
  if (nb > 0 && !em_scales) return MEP_ERR_NULL;
  if (T > 0 && (!indices || !x)) return MEP_ERR_NULL;
  if (T > 0 && carry && nb > 0 && !scales) return MEP_ERR_NULL;
  if ((indices && !aligned16(indices)) || (x && !aligned16(x)) ||
      (carry && scales && !aligned16(scales)) || !aligned16(em_x) ||
      (em_scales && !aligned16(em_scales)) || !aligned16(em_counts) ||
      !aligned16(em_offsets) || !aligned16(em_src_pos))
    return MEP_ERR_ALIGN;
  h->plan_valid = false;  // no rank-major plan: only the expert-major combine follows
  h->em_valid = false;
  int rc = begin_iteration(h, (hipStream_t)stream);
  if (rc != MEP_OK) return rc;
  mep::SmArgs a{};
  a.x = x;
  a.x_scales = carry ? scales : nullptr;
  a.idx = indices;
  a.em_x = em_x;
  a.em_scales = nb > 0 ? em_scales : nullptr;
  a.em_counts = em_counts;
  a.em_offsets = em_offsets;
  a.em_src_pos = em_src_pos;
  a.em_row = ws_ptr<int32_t>(h, h->lay.em_row);
  a.chunk_hist = ws_ptr<int32_t>(h, h->lay.sm_hist);
  a.status = status_word(h);
  a.status_next = status_next_word(h);
  a.tok_status = tok_status(h);
  a.cap_em = cap_em;
  a.T = T;
  a.H = c.hidden_dim;
  a.k = c.num_experts_per_token;
  a.E = c.world_size * c.num_experts_per_rank;
  a.quant = c.quant;
  a.scale_dim = nb;
  a.spos_base = c.rank * c.world_size * c.max_num_inp_token_per_rank;
  rc = hip_rc(mep::launch_dispatch_standard_moe(a, (hipStream_t)stream));
  if (rc != MEP_OK) return rc;
  h->em_valid = true;
  h->planned_since_reset = true;
  h->plan_T = T;
  return MEP_OK;
}

// Layout and call-order checks shared by the combine-side entry points.
static int check_combine_layout(mep_handle* h, int32_t layout, bool sum_ok) {
  const bool sum = layout == MEP_RANK_SUM;
  if (layout != MEP_RANK_MAJOR && layout != MEP_EXPERT_MAJOR && !(sum && sum_ok))
    return MEP_ERR_SHAPE;
  if ((layout == MEP_RANK_MAJOR || sum) && !h->plan_valid) return MEP_ERR_STATE;
  if (layout == MEP_EXPERT_MAJOR && !h->em_valid) return MEP_ERR_STATE;
  return MEP_OK;
}

// kind: 0 bf16 rows, 1 E4M3 rows, 2 bf16 rows rounded through E4M3 in flight
static int combine_common(mep_handle* h, int32_t layout, const void* y, const float* weights,
                          void* out, void* stream, int kind) {
  const bool fp8 = kind == 1;
  if (!h) return MEP_ERR_NULL;
  int rc = check_combine_layout(h, layout, kind == 0);
  if (rc != MEP_OK) return rc;
  const bool sum = layout == MEP_RANK_SUM;
  if (fp8 && h->cfg.hidden_dim % 16 != 0) return MEP_ERR_SHAPE;
  const int32_t T = h->plan_T;
  if (!out) return MEP_ERR_NULL;
  if (T > 0 && (!y || (!weights && !sum))) return MEP_ERR_NULL;
  if ((y && !aligned16(y)) || (weights && !aligned16(weights)) || !aligned16(out))
    return MEP_ERR_ALIGN;
  mep::CombineArgs a{};
  a.y = y;
  a.w = sum ? nullptr : weights;
  a.rows = ws_ptr<int32_t>(h, layout == MEP_EXPERT_MAJOR ? h->lay.em_row : h->lay.rrow);
  a.ufirst = ws_ptr<uint32_t>(h, h->lay.ufirst);
  a.distinct_rows = layout == MEP_EXPERT_MAJOR ? 1 : 0;
  a.sum_rows = sum ? 1 : 0;
  a.out = out;
  a.T = T;
  a.H = h->cfg.hidden_dim;
  a.k = h->cfg.num_experts_per_token;
  a.round_e4m3 = kind == 2 ? 1 : 0;
  return hip_rc(fp8 ? mep::launch_combine_fp8(a, (hipStream_t)stream)
                    : mep::launch_combine(a, (hipStream_t)stream));
}

int mep_combine(mep_handle* h, int32_t layout, const void* y, const float* weights, void* out,
                void* stream) {
  return combine_common(h, layout, y, weights, out, stream, 0);
}

int mep_combine_fp8(mep_handle* h, int32_t layout, const void* y8, const float* weights,
                    void* out, void* stream) {
  return combine_common(h, layout, y8, weights, out, stream, 1);
}

int mep_combine_fp8_direct(mep_handle* h, int32_t layout, const void* y, const float* weights,
                           void* out, void* stream) {
  return combine_common(h, layout, y, weights, out, stream, 2);
}

int mep_cast_fp8_direct(mep_handle* h, int32_t layout, const void* y, void* y8, void* stream) {
  if (!h) return MEP_ERR_NULL;
  int rc = check_combine_layout(h, layout, false);
  if (rc != MEP_OK) return rc;
  if (h->cfg.hidden_dim % 16 != 0) return MEP_ERR_SHAPE;
  const int32_t T = h->plan_T;
  if (T > 0 && (!y || !y8)) return MEP_ERR_NULL;
  if ((y && !aligned16(y)) || (y8 && !aligned16(y8))) return MEP_ERR_ALIGN;
  mep::CastArgs a{};
  a.y = y;
  a.y8 = y8;
  const bool rm = layout == MEP_RANK_MAJOR;
  a.rows = ws_ptr<int32_t>(h, rm ? h->lay.rrow : h->lay.em_row);
  a.ufirst = rm ? ws_ptr<uint32_t>(h, h->lay.ufirst) : nullptr;
  a.T = T;
  a.H = h->cfg.hidden_dim;
  a.k = h->cfg.num_experts_per_token;
  return hip_rc(mep::launch_cast_fp8(a, (hipStream_t)stream));
}

int mep_convert_combine_input(mep_handle* h, const void* em_y, const float* recv_weights,
                              void* y, void* stream) {
  if (!h) return MEP_ERR_NULL;
  if (!h->plan_valid || !h->em_valid) return MEP_ERR_STATE;
  const int32_t T = h->plan_T;
  if (T > 0 && (!em_y || !recv_weights || !y)) return MEP_ERR_NULL;
  if ((em_y && !aligned16(em_y)) || (recv_weights && !aligned16(recv_weights)) ||
      (y && !aligned16(y)))
    return MEP_ERR_ALIGN;
  mep::ConvertArgs a{};
  a.y_em = em_y;
  a.recv_w = recv_weights;
  a.rrow = ws_ptr<int32_t>(h, h->lay.rrow);
  a.em_row = ws_ptr<int32_t>(h, h->lay.em_row);
  a.ufirst = ws_ptr<uint32_t>(h, h->lay.ufirst);
  a.y = y;
  a.T = T;
  a.H = h->cfg.hidden_dim;
  a.k = h->cfg.num_experts_per_token;
  return hip_rc(mep::launch_convert_combine_input(a, (hipStream_t)stream));
}

int mep_reset(mep_handle* h, void* stream) {
  if (!h) return MEP_ERR_NULL;
  (void)stream;  // nothing to launch: the last plan cleared the next status word
  if (h->planned_since_reset) h->epoch++;
  h->planned_since_reset = false;
  h->plan_valid = false;
  h->em_valid = false;
  return MEP_OK;
}

int mep_get_status(mep_handle* h, void* stream, int32_t* device_status) {
  if (!h || !device_status) return MEP_ERR_NULL;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, status_word(h), sizeof(v),
                                hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess && h->captured && h->plan_T > 0) {
    // a captured iteration: OR in the per-token bits of its planned tokens,
    // copied in pieces through a host buffer on the stack
    const uint8_t* src = ws_ptr<uint8_t>(h, h->lay.tok_status);
    uint8_t buf[4096];
    for (int64_t i = 0; e == hipSuccess && i < h->plan_T; i += (int64_t)sizeof(buf)) {
      const size_t n = (size_t)std::min<int64_t>(sizeof(buf), h->plan_T - i);
      e = hipMemcpyAsync(buf, src + i, n, hipMemcpyDeviceToHost, (hipStream_t)stream);
      if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
      for (size_t j = 0; e == hipSuccess && j < n; ++j) v |= buf[j];
    }
  }
  if (e != hipSuccess) return MEP_ERR_HIP;
  *device_status = (int32_t)v;
  return v ? MEP_ERR_DEVICE : MEP_OK;
}

int mep_get_route(mep_handle* h, int32_t* recv_row, int32_t* em_row, void* stream) {
  if (!h || (!recv_row && !em_row)) return MEP_ERR_NULL;
  if (recv_row && !h->plan_valid) return MEP_ERR_STATE;
  if (em_row && !h->em_valid) return MEP_ERR_STATE;
  if ((recv_row && !aligned16(recv_row)) || (em_row && !aligned16(em_row))) return MEP_ERR_ALIGN;
  const int64_t n = (int64_t)h->plan_T * h->cfg.num_experts_per_token;
  int rc = MEP_OK;
  if (recv_row)
    rc = hip_rc(mep::launch_copy_i32(ws_ptr<int32_t>(h, h->lay.rrow), recv_row, n,
                                     (hipStream_t)stream));
  if (rc == MEP_OK && em_row)
    rc = hip_rc(mep::launch_copy_i32(ws_ptr<int32_t>(h, h->lay.em_row), em_row, n,
                                     (hipStream_t)stream));
  return rc;
}

int mep_probe_e4m3(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n < 0) return MEP_ERR_SHAPE;
  if (n > 0 && (!in || !out)) return MEP_ERR_NULL;
  if (n > 0 && (!aligned16(in) || !aligned16(out))) return MEP_ERR_ALIGN;
  return hip_rc(mep::launch_probe_e4m3(in, out, n, (hipStream_t)stream));
}

int mep_probe_bf16(const float* in, uint16_t* out, int64_t n, void* stream) {
  if (n < 0) return MEP_ERR_SHAPE;
  if (n > 0 && (!in || !out)) return MEP_ERR_NULL;
  if (n > 0 && (!aligned16(in) || !aligned16(out))) return MEP_ERR_ALIGN;
  return hip_rc(mep::launch_probe_bf16(in, out, n, (hipStream_t)stream));
}

int mep_probe_fp8_block(const uint16_t* in, uint8_t* q, float* scales, int64_t nblocks,
                        void* stream) {
  if (nblocks < 0 || nblocks > ((int64_t)1 << 28)) return MEP_ERR_SHAPE;
  if (nblocks > 0 && (!in || !q || !scales)) return MEP_ERR_NULL;
  if (nblocks > 0 && (!aligned16(in) || !aligned16(q) || !aligned4(scales))) return MEP_ERR_ALIGN;
  return hip_rc(mep::launch_probe_fp8_block(in, q, scales, nblocks, (hipStream_t)stream));
}

int mep_probe_mxfp4(const uint16_t* in, uint8_t* q, uint8_t* e8, int64_t nblocks,
                    void* stream) {
  if (nblocks < 0 || nblocks > ((int64_t)1 << 32)) return MEP_ERR_SHAPE;
  if (nblocks > 0 && (!in || !q || !e8)) return MEP_ERR_NULL;
  if (nblocks > 0 && (!aligned16(in) || !aligned16(q))) return MEP_ERR_ALIGN;
  return hip_rc(mep::launch_probe_mxfp4(in, q, e8, nblocks, (hipStream_t)stream));
}

int mep_probe_stream(const void* src, void* dst, int64_t waves, int64_t rd_units,
                     int64_t wr_units, void* stream) {
  const int64_t kMaxUnits = (int64_t)1 << 30;  // 1 TiB either way
  if (waves < 0 || rd_units < 0 || wr_units < 0) return MEP_ERR_SHAPE;
  if (rd_units > kMaxUnits || wr_units > kMaxUnits) return MEP_ERR_SHAPE;
  if (waves == 0) return (rd_units || wr_units) ? MEP_ERR_SHAPE : MEP_OK;
  if (waves > ((int64_t)1 << 24)) return MEP_ERR_SHAPE;  // 256-thread blocks: 2^32 threads
  if ((rd_units + waves - 1) / waves > mep::stream_probe_max_units()) return MEP_ERR_SHAPE;
  if ((rd_units && !src) || !dst) return MEP_ERR_NULL;  // a read-only wave may store
  if ((src && !aligned16(src)) || !aligned16(dst)) return MEP_ERR_ALIGN;
  return hip_rc(mep::launch_stream_probe(src, dst, waves, rd_units, wr_units,
                                         (hipStream_t)stream));
}

}  // extern "C"
