// Internal declarations shared by the host ABI (mep_abi.cpp) and the kernels.
// Not installed; the public interface is include/mep.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mep.h"

namespace mep {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kMaxRanks = 64;    // a token's destination ranks fit one 64-bit mask
constexpr int kMaxTopk = 32;     // first-occurrence bits of a token fit 32 bits
constexpr int kMaxEpr = 64;      // a row's local experts fit one 64-bit mask
constexpr int kChunk = 64;       // tokens (or receive rows) per scan chunk = one wave

// Chunks per block of the plan's count launch for a batch of C chunks: small
// blocks (4 chunks, 256 threads) start and finish sooner, but every later
// chunk sums the totals of all earlier blocks, so batches over 64 chunks
// (4096 tokens) take blocks of 16 chunks; either way a batch of up to 16384
// tokens has at most 16 earlier blocks.  The workspace holds blocks of the
// smaller size.
__host__ __device__ constexpr int count_block_chunks(int C) { return C <= 64 ? 4 : 16; }
constexpr int kMinBlockChunks = 4;

// 16-byte units per received row of a payload mode: 8 bf16 values, 16 E4M3
// codes or 32 packed E2M1 codes per unit.
__host__ __device__ constexpr int payload_units(int quant, int H) {
  return quant == MEP_QUANT_NONE ? H / 8
         : (quant == MEP_QUANT_FP4_CARRY || quant == MEP_QUANT_MXFP4) ? H / 32
                                                                       : H / 16;
}

// Items of a received row that the dispatch waves take one per lane: the
// 16-byte units above, except MXFP4, whose lanes take 16 columns (8 code
// bytes, half an MX block) so that a row's waves stay full.
__host__ __device__ constexpr int lane_items(int quant, int H) {
  return quant == MEP_QUANT_MXFP4 ? H / 16 : payload_units(quant, H);
}

// Modes whose rows arrive already quantised, with the caller's scale words.
__host__ __device__ constexpr bool is_carry(int quant) {
  return quant == MEP_QUANT_FP8_CARRY || quant == MEP_QUANT_FP4_CARRY;
}

// Expert id -> rank without a hardware divide: for e < 4096 and epr <= 64,
// (e * m) >> 20 with m = ceil(2^20 / epr) equals e / epr (checked on the host
// for every expert id when a handle is created).
struct RankDiv {
  uint32_t m;
  __host__ __device__ inline uint32_t operator()(uint32_t e) const { return (e * m) >> 20; }
};

// Byte offsets of the workspace sections (each 256-byte aligned).
struct WsLayout {
  size_t status;     // uint32 [3]: sticky MEP_DEV_* bits, one word per reset epoch [0, 1];
                     // the expert-major overflow word of captured iterations [2]
  size_t tok_status; // uint8 [cap]: bad/repeated-id bits of each token of a captured plan
  size_t chunk_cnt;  // int32 [C][R]: rows earlier chunks of the same count block send to each rank
  size_t block_cnt;  // int32 [ceil(C/4)][R]: rows each count block (4 or 16 chunks) sends to each rank
  size_t mask;       // uint64 [cap]: destination-rank mask of each token (0 = dropped)
  size_t rrow;       // int32 [cap][k]: flat receive row r*cap+slot of (t, j), -1 if dropped
  size_t ufirst;     // uint32 [cap]: bit j set when top-k position j owns its rank's row
  size_t em_row;     // int32 [cap][k]: expert-major row of (t, j), -1 if none
  size_t em_lmask;   // uint64 [R*cap]: local experts named by each receive row
  size_t em_ccnt;    // int32 [R][CR][epr]: per 64-row chunk, rows per local expert
  size_t em_seg;     // int32 [R + R*epr]: padded segment rows of each rank's experts, then
                     // each expert's padded in-rank offset
  size_t sm_hist;    // int32 [C][E]: standard-MoE dispatch, per-chunk expert counts / prefixes
  size_t total;
};

WsLayout ws_layout(const mep_config& c);

struct PlanArgs {
  const int32_t* indices;  // [T,k]
  int32_t* recv_counts;    // [R]
  int32_t* spos;           // [R,cap]
  uint32_t* status;       // this epoch's status word
  uint32_t* status_next;  // the other epoch's word, cleared by the plan
  uint8_t* tok_status;    // captured iteration: per-token bits stored here instead
  int32_t* chunk_cnt;
  int32_t* block_cnt;
  uint64_t* mask;
  int32_t* rrow;
  uint32_t* ufirst;
  int32_t T, k, R, E, cap, spos_base;  // spos_base = rank * R * cap
  RankDiv rdiv;
  int32_t blk_chunks;  // chunks per count block (count_block_chunks), set at launch
};

struct DispatchArgs {
  const void* x;           // [T,H] bf16, or E4M3 bytes when carried
  const float* x_scales;   // [T,scale_dim] carried scales (MEP_QUANT_FP8_CARRY)
  const float* w;          // [T,k]
  const int32_t* idx;      // [T,k]
  int32_t* rrow;           // [T,k] receive row of (t, j): read after a plan, written when fused
  uint32_t* ufirst;        // [T] first-occurrence bits: likewise
  void* recv_x;            // [R*cap, H] bf16 or e4m3
  float* recv_scales;      // [R*cap, H/128]
  float* recv_w;           // [R*cap, k]
  int32_t* recv_idx;       // [R*cap, k]
  // fused plan+dispatch only
  const uint64_t* mask;    // per-token rank masks from the count launch
  const int32_t* chunk_cnt;
  const int32_t* block_cnt;
  int32_t* recv_counts;    // [R]
  int32_t* spos;           // [R,cap]
  uint32_t* status;
  uint32_t* status_next;
  uint8_t* tok_status;     // as PlanArgs
  int32_t T, H, k, R, E, cap, spos_base;
  int32_t quant, scale_dim;
  RankDiv rdiv;
  int32_t blk_chunks;      // fused: chunks per count block (count_block_chunks)
  int32_t slices, slice_units;  // waves per token and 16-byte lane units per wave
};

// Batches up to this many tokens plan inside the dispatch launch itself.
constexpr int kInlinePlanTokens = 256;

struct CombineArgs {
  const void* y;           // bf16 rows
  const float* w;          // [T,k]; unused when sum_rows
  const int32_t* rows;     // [T,k] row of (t, j) in y, -1 = skip
  const uint32_t* ufirst;  // [T] positions owning a rank row (sum_rows only)
  void* out;               // [T,H] bf16
  int32_t T, H, k;
  int32_t distinct_rows;   // 1: the k rows of a token are distinct (no dedupe needed)
  int32_t sum_rows;        // 1: add the token's distinct rank rows, no weights
  int32_t round_e4m3;      // 1: each value rounded through E4M3 (direct cast) before use
  int32_t slices, slice_units;  // waves per token and lane units (16 or 8 bytes) per wave
  int32_t wg_per_tok, waves_per_wg;  // top-8 kernel: workgroups per token, waves in each
};

struct CastArgs {           // E4M3 direct cast of the routed expert-output rows
  const void* y;             // bf16 rows
  void* y8;                  // E4M3 rows, same row indices
  const int32_t* rows;       // [T,k] row of (t, j), -1 = none
  const uint32_t* ufirst;    // [T] positions owning a distinct row (rank-major), or null
  int32_t T, H, k, slices;
};

struct ConvertArgs {         // expert-major expert outputs back to rank-major rows
  const void* y_em;          // [cap_em,H] bf16
  const float* recv_w;       // [R*cap,k] dispatched weights
  const int32_t* rrow;       // [T,k] receive row of (t, j)
  const int32_t* em_row;     // [T,k] expert-major row of (t, j), -1 = none
  const uint32_t* ufirst;    // [T] positions owning a rank row
  void* y;                   // [R*cap,H] bf16
  int32_t T, H, k, slices;
  int32_t wg_per_tok, waves_per_wg;  // top-8: workgroups per token, waves per workgroup
};

struct EmArgs {
  const void* recv_x;
  const float* recv_scales;
  const int32_t* recv_idx;      // [R*cap, k]
  const int32_t* recv_counts;   // [R]
  const int32_t* spos;          // [R*cap]
  const int32_t* rrow;          // plan rows, to find dropped tokens
  void* em_x;
  float* em_scales;
  int32_t* em_counts;           // [E]
  int32_t* em_offsets;          // [E+1]
  int32_t* em_src_pos;          // [cap_em]
  int32_t* em_row;              // [T,k]
  uint64_t* lmask;              // [R*cap]
  int32_t* ccnt;                // [R][CR][epr]
  int32_t* seg_rank;            // [R]: padded segment rows of rank r's experts
  int32_t* seg_inrank;          // [E]: padded rows of the same rank's earlier experts
  uint32_t* status;
  RankDiv rdiv;                 // expert id -> rank
  int64_t cap_em;
  int32_t T, H, k, R, epr, cap, CR, nb, row_units, spos_base;  // row_units: 16-byte units per row
  int32_t slices;  // scatter: waves per receive row
};

struct SmArgs {                // standard-MoE dispatch
  const void* x;                // [T,H] bf16, or E4M3 bytes when carried
  const float* x_scales;        // [T,scale_dim] carried scales
  const int32_t* idx;           // [T,k]
  void* em_x;                   // [cap_em,H]
  float* em_scales;             // [cap_em,scale_dim]
  int32_t* em_counts;           // [E]
  int32_t* em_offsets;          // [E+1]
  int32_t* em_src_pos;          // [cap_em]
  int32_t* em_row;              // [T,k] expert-major row of (t, j)
  int32_t* chunk_hist;          // [C][E]
  uint32_t* status;
  uint32_t* status_next;
  uint8_t* tok_status;          // as PlanArgs
  int64_t cap_em;
  int32_t T, H, k, E, quant, scale_dim, spos_base, slices;
};

// Workspace pointers one call uses: a handle's workspace, or the library's own
// scratch in the entry point that allocates nothing.
struct WsPtrs {
  uint32_t* status;       // status bits ORed in
  uint32_t* status_next;  // the word the plan clears
  uint8_t* tok_status;    // per-token status bytes (captured iterations), or null
  int32_t* chunk_cnt;
  int32_t* block_cnt;
  uint64_t* mask;
  int32_t* rrow;
  uint32_t* ufirst;
};

// Host-side checks and argument packing shared by the entry points
// (mep_abi.cpp); each check returns MEP_OK or a MEP_ERR_* code.
int check_config(const mep_config* c);
RankDiv make_rdiv(int32_t epr);
int check_rank_map(const mep_config& c, RankDiv rd);  // the divide-free map is exact
int check_plan_args(const mep_config& c, const int32_t* indices, int32_t T,
                    const int32_t* recv_counts, const int32_t* src_token_pos);
int check_dispatch_args(const mep_config& c, int32_t T, const void* x, const float* weights,
                        const float* scales, const int32_t* indices, const void* recv_x,
                        const float* recv_scales, const float* recv_weights,
                        const int32_t* recv_indices);
PlanArgs plan_args(const mep_config& c, RankDiv rd, const WsPtrs& w, const int32_t* indices,
                   int32_t T, int32_t* recv_counts, int32_t* src_token_pos);
DispatchArgs dispatch_args(const mep_config& c, RankDiv rd, const WsPtrs& w, int32_t T,
                           const void* x, const float* weights, const float* scales,
                           const int32_t* indices, void* recv_x, float* recv_scales,
                           float* recv_weights, int32_t* recv_indices);

// Launchers (return hipError_t of the launch).
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_plan_counts(const PlanArgs& a, hipStream_t s);  // count launch only, T > 0
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
hipError_t launch_plan_dispatch(const PlanArgs& p, const DispatchArgs& a, hipStream_t s);
hipError_t launch_dispatch_standard_moe(const SmArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_combine_fp8(const CombineArgs& a, hipStream_t s);  // y holds E4M3 rows
hipError_t launch_cast_fp8(const CastArgs& a, hipStream_t s);
hipError_t launch_to_expert_major(const EmArgs& a, hipStream_t s);
hipError_t launch_convert_combine_input(const ConvertArgs& a, hipStream_t s);
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t s);
hipError_t launch_probe_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t s);
hipError_t launch_probe_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s);
hipError_t launch_probe_fp8_block(const uint16_t* in, uint8_t* q, float* scales, int64_t nblocks,
                                  hipStream_t s);
hipError_t launch_probe_mxfp4(const uint16_t* in, uint8_t* q, uint8_t* e8, int64_t nblocks,
                              hipStream_t s);
hipError_t launch_stream_probe(const void* src, void* dst, int64_t waves, int64_t rd_units,
                               int64_t wr_units, hipStream_t s);
int stream_probe_max_units();  // read units (1 KiB each) one probe wave can take

}  // namespace mep
