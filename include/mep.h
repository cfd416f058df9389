/*
 * mep.h -- C ABI of libmep: MoE token dispatch and combine on one gfx950 GPU.
 *
 * The operation is the MORI-EP intra-node dispatch/combine ("MORI-EP User
 * Guide", sections 2 Configuration and 3 Operator API; standard-MoE layout in
 * section 4), restated for one device: the receive buffers of R "virtual
 * ranks" are ordinary device buffers in local HBM, and this device's T tokens
 * are routed into them.  Ranks own contiguous expert blocks: expert e lives on
 * rank e / num_experts_per_rank.
 *
 * Conventions (every entry point):
 *   - Pointers named x, scales, recv_*, y, y8, out, em_*, indices, weights,
 *     recv_counts, src_token_pos and workspace are DEVICE pointers, caller-owned, borrowed
 *     only for the duration of the asynchronous call on `stream`
 *     (a hipStream_t passed as void*; NULL = the null stream).  The library
 *     never allocates or frees device memory and never synchronises, except
 *     in mep_get_status.
 *   - All device pointers must be 16-byte aligned (MEP_ERR_ALIGN otherwise).
 *   - Errors a host can see (null pointers, bad shapes, alignment, call order)
 *     return a negative MEP_ERR_* code synchronously and launch nothing.
 *     Data errors only the device can see (an expert id out of range, a
 *     repeated expert in one token, expert-major overflow) set bits of a
 *     sticky device status word (MEP_DEV_*), read by mep_get_status.
 *   - A handle is not thread-safe; use one handle per stream.  Calls on one
 *     handle must be issued on one stream (or externally ordered).
 *   - Layouts are row-major and dense: [T,H] means row t at offset t*H.
 *   - Apart from mep_get_status, the calls launch kernels only (no memset,
 *     copy or host wait), so a sequence of them can be captured into a HIP
 *     graph; a replay reuses the handle state of the capture (its plan).  An
 *     iteration whose plan (mep_plan, mep_plan_dispatch or
 *     mep_dispatch_standard_moe) is captured keeps its MEP_DEV_* bits apart
 *     (per planned token, and one word for the expert-major overflow that its
 *     plan clears), so every replay starts clean without an extra launch:
 *     mep_get_status returns the bits of the latest replay (of its last plan,
 *     if it holds several), mep_reset between replays is allowed and changes
 *     nothing there.  The next plan issued outside capture starts a new reset
 *     epoch.
 */
#ifndef MEP_H
#define MEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------- */
#define MEP_OK 0
#define MEP_ERR_NULL (-1)    /* a required pointer is NULL                     */
#define MEP_ERR_CONFIG (-2)  /* config fields out of range or inconsistent      */
#define MEP_ERR_SHAPE (-3)   /* a size argument out of range                    */
#define MEP_ERR_ALIGN (-4)   /* a device pointer is not 16-byte aligned         */
#define MEP_ERR_STATE (-5)   /* call order violated (e.g. dispatch before plan) */
#define MEP_ERR_HIP (-6)     /* the HIP runtime reported an error               */
#define MEP_ERR_DEVICE (-7)  /* mep_get_status: device status word is non-zero  */
#define MEP_ERR_NOMEM (-8)   /* mep_create: the host heap could not hold a handle */

/* ---- device status bits (sticky until mep_reset) ------------------------- */
#define MEP_DEV_BAD_INDEX 1   /* an expert id outside [0, E): that token is not
                                 dispatched and combines to +0                  */
#define MEP_DEV_DUP_EXPERT 2  /* a token names one expert twice (still routed)  */
#define MEP_DEV_EM_OVERFLOW 4 /* expert-major rows exceed cap_em; rows past it
                                 are dropped                                    */

/* ---- payload and layout selectors --------------------------------------- */
#define MEP_QUANT_NONE 0              /* dispatch payload: bf16 bit copy        */
#define MEP_QUANT_FP8_E4M3_BLOCK128 1 /* dispatch payload: OCP E4M3 codes with
                                         one fp32 scale per 128 columns          */
#define MEP_QUANT_FP8_CARRY 2         /* dispatch payload arrives already as OCP
                                         E4M3 bytes with scale_dim fp32 scales
                                         per row; both are carried unchanged
                                         ("Choosing an EP API and backend": the
                                         HIP backend's dispatch can move FP8
                                         rows that arrive quantized)             */
#define MEP_QUANT_FP4_CARRY 3         /* as MEP_QUANT_FP8_CARRY for FP4 rows: H/2
                                         bytes per row (two E2M1 codes a byte),
                                         scale_dim 32-bit scale words per row,
                                         both carried unchanged (same passage) */
#define MEP_QUANT_MXFP4 4             /* dispatch payload: OCP MX FP4 -- per 32
                                         columns an E8M0 scale byte, shared
                                         exponent floor(log2(amax)) - 2 clamped
                                         to [-127, 127]; codes E2M1(x / 2^exp),
                                         round to nearest even, saturating at 6,
                                         even column in the low nibble; all-zero
                                         block: scale byte 0.  Rows of H/2
                                         bytes; the H/32 scale bytes of a row
                                         fill its H/128 scale words ("Choosing
                                         an EP API and backend": FP4 conversion
                                         kernels on gfx950; the block format is
                                         this library's reading)                */
#define MEP_RANK_MAJOR 0              /* combine input: [R, cap, H] bf16         */
#define MEP_EXPERT_MAJOR 1            /* combine input: [cap_em, H] bf16         */
#define MEP_RANK_SUM 2                /* combine input: [R, cap, H] bf16 rows from
                                         mep_convert_combine_input, which already
                                         carry the weights                       */

/*
 * Configuration.  Fields follow EpDispatchCombineConfig ("MORI-EP User Guide",
 * section 2 Configuration); the multi-node fields (gpu_per_node,
 * rdma_block_num, num_qp_per_pe, kernel_type) and launch geometry have no
 * meaning on one device and are absent.
 */
typedef struct mep_config {
  int32_t hidden_dim;                 /* H: > 0, multiple of 8; of 128 when quantising, of
                                         16 when carrying E4M3, of 32 when carrying FP4  */
  int32_t scale_dim;                  /* 32-bit scale words per row: 0 for bf16; H/128
                                         when quantising; any >= 0 when carrying         */
  int32_t num_experts_per_rank;       /* epr: 1..64                                       */
  int32_t num_experts_per_token;      /* k: 1..32, k <= R*epr                              */
  int32_t max_num_inp_token_per_rank; /* cap: receive rows per rank and the largest T, >= 1 */
  int32_t world_size;                 /* R virtual ranks: 1..64                           */
  int32_t rank;                       /* source rank used in src_token_pos: 0..R-1        */
  int32_t quant;                      /* MEP_QUANT_*  (the pages' data_type choice)        */
} mep_config;

typedef struct mep_handle mep_handle;

/* Human-readable name of a MEP_OK / MEP_ERR_* code (static string). */
const char *mep_error_string(int code);

/* Bytes of device workspace a handle needs for this config, or 0 if the config
 * is invalid.  The workspace holds the routing plan (receive row of every
 * (token, top-k slot)), the expert-major maps and the status word. */
size_t mep_workspace_bytes(const mep_config *cfg);

/* Check the config and bind it to a caller-owned device workspace of at least
 * mep_workspace_bytes(cfg) bytes, which must be zero-filled before its first
 * use (it holds the status words).  Host-only: launches nothing, makes no HIP
 * call.  *out receives a host-heap handle freed by mep_destroy.  One
 * workspace serves one handle at a time. */
int mep_create(const mep_config *cfg, void *workspace, size_t workspace_bytes,
               mep_handle **out);
int mep_destroy(mep_handle *h);

/*
 * Routing plan ("MORI-EP User Guide" section 3: dispatch() returns
 * recv_num_token; get_dispatch_src_token_pos() gives each received row's
 * origin).  For T tokens with top-k expert ids indices[T,k] (int32):
 *   - each token is sent once to each distinct rank among its experts (the
 *     first top-k position naming that rank owns the row; later positions on
 *     the same rank share it);
 *   - recv_counts[r] (int32, R entries) = rows rank r receives;
 *   - inside a rank, rows are in ascending token order, and
 *     src_token_pos[r*cap + s] (int32, [R,cap]) = rank*(R*cap) + t for the
 *     token t in slot s < recv_counts[r]; entries past the count are not
 *     written.
 * The plan is kept in the workspace and stays valid (for any number of
 * dispatch/combine calls: routing replay) until mep_reset or the next plan.
 * 0 <= T <= cap.
 */
int mep_plan(mep_handle *h, const int32_t *indices, int32_t T, int32_t *recv_counts,
             int32_t *src_token_pos, void *stream);

/*
 * Dispatch ("MORI-EP User Guide" section 3 dispatch(input, weights, scales,
 * indices)): every planned (token, rank) row receives
 *   recv_x[r, s, :]       the token row: x[T,H] bf16 copied bit for bit
 *                         (MEP_QUANT_NONE, recv_x is [R,cap,H] bf16); or its
 *                         OCP E4M3 codes (MEP_QUANT_FP8_E4M3_BLOCK128, recv_x is
 *                         [R,cap,H] bytes): per 128 columns b, scale =
 *                         amax_b / 448 (fp32) and code =
 *                         E4M3_rne_satfinite(x / scale), signed zero when
 *                         amax_b == 0; or, MEP_QUANT_FP8_CARRY, the E4M3 bytes
 *                         of x[T,H] copied;
 *   recv_scales[r, s, :]  the block scales ([R,cap,H/128] fp32), or the carried
 *                         scales[t, :] ([R,cap,scale_dim]); NULL for bf16;
 * MEP_QUANT_MXFP4 writes [R,cap,H/2] packed E2M1 bytes and [R,cap,H/32] E8M0
 * bytes (= H/128 words; x finite: NaN/Inf inputs are not supported);
 * MEP_QUANT_FP4_CARRY copies H/2 bytes of x and the
 * scale_dim words of scales[t, :];
 *   recv_weights[r, s, :] the token's k weights (fp32 [R,cap,k]);
 *   recv_indices[r, s, :] the token's k expert ids (int32 [R,cap,k]).
 * scales is the caller's [T,scale_dim] 32-bit input for the carry modes and is
 * ignored otherwise.  Rows past recv_counts[r] are not written.  Needs a
 * valid plan; x, weights, scales and indices hold the planned T tokens.
 */
int mep_dispatch(mep_handle *h, const void *x, const float *weights, const float *scales,
                 const int32_t *indices, void *recv_x, float *recv_scales, float *recv_weights,
                 int32_t *recv_indices, void *stream);

/*
 * Fused routing plan + dispatch: the same outputs as mep_plan followed by
 * mep_dispatch (recv_counts, src_token_pos, the receive rows, scales, weights
 * and ids, and a valid plan in the handle), in fewer launches -- one launch up
 * to 256 tokens, else two.  The pages pair the two steps the same way:
 * dispatch() itself returns recv_num_token ("MORI-EP User Guide" section 3).
 */
int mep_plan_dispatch(mep_handle *h, const int32_t *indices, int32_t T, int32_t *recv_counts,
                      int32_t *src_token_pos, const void *x, const float *weights,
                      const float *scales, void *recv_x, float *recv_scales,
                      float *recv_weights, int32_t *recv_indices, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * outputs as mep_plan_dispatch (recv_counts, src_token_pos, the receive rows,
 * scales, weights and ids, with the same argument layouts, alignment and
 * host-side checks) with no handle and no workspace.  The plan's scratch is a
 * 2 MiB device array inside the library, one per GPU, held until the process
 * ends; its address on the stream's GPU is looked up on the first call there
 * (hipGetSymbolAddress, no allocation).  The batch must fit it: 179 KiB
 * for 4096 tokens at top-8 on 8 ranks, roughly T*(12 + 4k) + (T/64)*R*5
 * bytes in general (each section rounded up to 256 bytes); MEP_ERR_SHAPE
 * beyond 2 MiB
 * (no launch).  Every call on one GPU shares that scratch, so calls that
 * overlap on one GPU (concurrent streams, or threads) race; calls ordered on
 * one stream do not.  Tokens with bad expert ids are not dispatched, as in
 * mep_plan_dispatch, but no status word is kept for mep_get_status.  No plan
 * is left behind: combine needs a handle and its own plan.
 */
int mep_plan_dispatch_noalloc(const mep_config *cfg, const int32_t *indices, int32_t T,
                              int32_t *recv_counts, int32_t *src_token_pos, const void *x,
                              const float *weights, const float *scales, void *recv_x,
                              float *recv_scales, float *recv_weights, int32_t *recv_indices,
                              void *stream);

/*
 * Standard-MoE layout ("MORI-EP User Guide" section 4,
 * convert_dispatch_output(): packed rows, per-expert counts, source info).
 * From the dispatch outputs (recv_x, recv_scales or NULL, recv_indices,
 * recv_counts, and the plan's src_token_pos), for every expert e in global
 * order:
 *   em_counts[e]        rows naming expert e (int32, E = R*epr entries);
 *   em_offsets[e]       first row of e's segment; segments are padded to
 *                       multiples of 128 rows (int32, E+1 entries,
 *                       em_offsets[E] = rows used);
 *   em_x[em_offsets[e] + i, :]      the i-th such receive row (ascending
 *                       receive slot), in the row format of recv_x;
 *   em_scales[...]      its scale words (scale_dim per row; NULL when 0);
 *   em_src_pos[...]     its src_token_pos.
 * Padding rows are not written.  cap_em is the row capacity of em_x /
 * em_scales / em_src_pos; T*k + 127*E always suffices.  Rows past cap_em are
 * dropped and set MEP_DEV_EM_OVERFLOW.  Needs a valid plan.  MEP_ERR_SHAPE if
 * T*k + 127*E exceeds INT32_MAX (the int32 offsets could not hold the
 * padded segments).
 */
int mep_to_expert_major(mep_handle *h, const void *recv_x, const float *recv_scales,
                        const int32_t *recv_indices, const int32_t *recv_counts,
                        const int32_t *src_token_pos, void *em_x, float *em_scales,
                        int32_t *em_counts, int32_t *em_offsets, int32_t *em_src_pos,
                        int64_t cap_em, void *stream);

/*
 * Standard-MoE dispatch ("MORI-EP User Guide" section 4,
 * dispatch_standard_moe(): dispatch and format conversion combined): the same
 * em_x / em_scales / em_counts / em_offsets / em_src_pos as mep_plan +
 * mep_dispatch + mep_to_expert_major would produce for these T tokens (rows of
 * each expert in ascending token order, segments padded to 128 rows, padding
 * not written), but written straight from x without the rank-major receive
 * buffers.  A token naming one expert twice gets one row (mapped from the
 * first position naming it).  Leaves the handle ready for
 * mep_combine(MEP_EXPERT_MAJOR) and mep_get_route(NULL, em_row); the
 * rank-major calls need a new mep_plan.  scales as for mep_dispatch.
 * 0 <= T <= cap; cap_em (and the T*k + 127*E bound) as for
 * mep_to_expert_major.
 */
int mep_dispatch_standard_moe(mep_handle *h, const int32_t *indices, int32_t T, const void *x,
                              const float *scales, void *em_x, float *em_scales,
                              int32_t *em_counts, int32_t *em_offsets, int32_t *em_src_pos,
                              int64_t cap_em, void *stream);

/*
 * Combine ("MORI-EP User Guide" section 3 combine(): expert outputs gathered
 * back to token order as a weighted combination; section 4
 * combine_standard_moe() for the expert-major input; "Choosing an EP API and
 * backend": the HIP backend's combine gathers in BF16 or FP32).  For every
 * planned token t:
 *   out[t, h] = bf16_rne(acc),  acc = +0.0f, then for j = 0..k-1 in order
 *               acc = fmaf(weights[t, j], y_j[h], acc)
 * where y_j is the bf16 expert-output row holding (t, expert j):
 *   MEP_RANK_MAJOR:   y is [R,cap,H]; y_j = y[rank of expert j, slot of t];
 *                     a row shared by two experts is used once per expert;
 *   MEP_EXPERT_MAJOR: y is [cap_em,H] in the layout mep_to_expert_major or
 *                     mep_dispatch_standard_moe produced (needs one of them
 *                     after the current plan).
 * weights are token-major fp32 [T,k]; out is [T,H] bf16.  Tokens that were
 * not dispatched (bad expert id) produce +0.
 *   MEP_RANK_SUM:     y is [R,cap,H] rows written by mep_convert_combine_input
 *                     (each already weighted); out[t, h] = bf16_rne(acc),
 *                     acc = +0, then acc = acc + y_r[h] over t's distinct
 *                     destination ranks r in the order of their first top-k
 *                     position (one fp32 rounding per addition); weights is
 *                     not read and may be NULL.  Needs a valid plan.
 */
int mep_combine(mep_handle *h, int32_t layout, const void *y, const float *weights, void *out,
                void *stream);

/*
 * FP8 direct-cast combine payload ("MORI-EP User Guide", section 10 Tuning:
 * the intra-node tuning matrix pairs quant type fp8_direct_cast with a bf16
 * combine):
 * mep_cast_fp8_direct writes y8 = OCP E4M3 of each bf16 value of the rows the
 * current plan routes (round to nearest even, saturating at +-448, no scale;
 * NaN inputs are not supported), y and y8 in the layout of mep_combine with 1
 * byte per value (y8 is [R,cap,H] or [cap_em,H] bytes; other rows are not
 * touched).  mep_combine_fp8 is mep_combine on such E4M3 rows: each value is
 * decoded exactly to fp32 and accumulated as above.  Same state rules as
 * mep_combine.
 */
int mep_cast_fp8_direct(mep_handle *h, int32_t layout, const void *y, void *y8, void *stream);
int mep_combine_fp8(mep_handle *h, int32_t layout, const void *y8, const float *weights,
                    void *out, void *stream);

/*
 * The same payload rounding without the E4M3 rows (one device: source and
 * destination of the cast are the same): mep_combine on the bf16 rows y with
 * each value cast to E4M3 and decoded back before its multiply-add.  out is
 * bit for bit what mep_cast_fp8_direct followed by mep_combine_fp8 gives, the
 * bf16 rows being read once.  Same state rules and layouts as mep_combine.
 */
int mep_combine_fp8_direct(mep_handle *h, int32_t layout, const void *y, const float *weights,
                           void *out, void *stream);

/*
 * Standard-MoE expert outputs back to the combine input ("MORI-EP User
 * Guide" section 4, convert_combine_input(packed rows, source info, layout
 * range): the experts' expert-major outputs turned into the rows combine()
 * takes).  em_y is [cap_em,H] bf16 in the layout of the last
 * mep_to_expert_major (whose source info and segments this handle keeps);
 * recv_weights is the dispatch's [R,cap,k] fp32 output.  For every received
 * row (rank r, slot s < recv_counts[r]) of token t:
 *   y[r, s, h] = bf16_rne(acc), acc = +0, then for j = 0..k-1 in order, over
 *   t's positions whose expert lives on rank r and is not named by an earlier
 *   position: acc = fmaf(recv_weights[r, s, j], em_y[row of (t, j)][h], acc).
 * The pages pass no weights to this step; applying the dispatched weights
 * here is this library's reading -- a row merging several local experts can
 * carry their weighted sum only if the weights go in before the merge -- so
 * the combine that follows is mep_combine(MEP_RANK_SUM), which adds rank rows
 * without weights.  y is [R,cap,H] bf16; rows past recv_counts[r] are not
 * written; a position whose expert-major row was dropped (MEP_DEV_EM_OVERFLOW)
 * adds nothing.  Needs a valid plan and mep_to_expert_major after it.
 */
int mep_convert_combine_input(mep_handle *h, const void *em_y, const float *recv_weights,
                              void *y, void *stream);

/*
 * Reset between iterations ("MORI-EP User Guide" section 3 reset()):
 * invalidates the plan (and the expert-major maps) and starts a new status
 * epoch, whose status word the last plan already cleared on the device, so no
 * kernel is launched and `stream` is unused.  Caller buffers are not touched:
 * the library writes a caller buffer only during the call that names it.
 */
int mep_reset(mep_handle *h, void *stream);

/* Synchronise `stream`, then copy the device status word (MEP_DEV_* bits) to
 * *device_status.  Returns MEP_ERR_DEVICE if any bit is set, else MEP_OK. */
int mep_get_status(mep_handle *h, void *stream, int32_t *device_status);

/*
 * Inspection of the current plan (for verification, "MORI-EP User Guide"
 * section 3 get_dispatch_src_token_pos()): copies, on `stream`, the flat
 * receive row r*cap + slot of every (token, top-k position) into
 * recv_row[T,k] (int32, -1 for tokens not dispatched; needs a rank-major
 * plan), and/or the expert-major row of each (token, top-k position) into
 * em_row[T,k] (-1 where none; needs mep_to_expert_major or
 * mep_dispatch_standard_moe).  Either pointer may be NULL, not both.
 */
int mep_get_route(mep_handle *h, int32_t *recv_row, int32_t *em_row, void *stream);

/*
 * Codec probes: run, over n values, exactly the device conversions the
 * kernels use.  in is fp32 [n]; mep_probe_e4m3 writes OCP E4M3 codes (uint8
 * [n]) of in[i] (no scaling; values must satisfy |v| <= 464), mep_probe_bf16
 * writes bf16 round-to-nearest-even bits (uint16 [n]).
 */
int mep_probe_e4m3(const float *in, uint8_t *out, int64_t n, void *stream);
int mep_probe_bf16(const float *in, uint16_t *out, int64_t n, void *stream);

/*
 * FP8 block probe: the dispatch's MEP_QUANT_FP8_E4M3_BLOCK128 block encoder
 * over nblocks blocks of 128 bf16 values (in: uint16 bit patterns
 * [nblocks,128], finite values only), writing each block's 128 E4M3 codes (q:
 * uint8 [nblocks,128]) and its fp32 scale (scales [nblocks]).  in and q
 * 16-byte aligned, scales 4-byte aligned; nblocks <= 2^28.
 */
int mep_probe_fp8_block(const uint16_t *in, uint8_t *q, float *scales, int64_t nblocks,
                        void *stream);

/*
 * MX FP4 block probe: the dispatch's MEP_QUANT_MXFP4 block encoder over
 * nblocks blocks of 32 bf16 values (in: uint16 bit patterns [nblocks,32],
 * finite values only), writing each block's 16 packed E2M1 code bytes (q:
 * uint8 [nblocks,16], even column in the low nibble) and its E8M0 scale byte
 * (e8: uint8 [nblocks]).  in and q 16-byte aligned; nblocks <= 2^32.
 */
int mep_probe_mxfp4(const uint16_t *in, uint8_t *q, uint8_t *e8, int64_t nblocks, void *stream);

/*
 * Streaming probe (measurement, not part of the path): what HBM gives a mix of
 * reads and writes spread over a number of waves, for comparing a kernel with
 * plain streams of its own byte mix.  `waves` 64-lane waves share rd_units
 * reads of src and wr_units writes of dst, each unit 1 KiB (16 bytes per
 * lane), as evenly as the counts allow; each wave's share of src and of dst is
 * one contiguous run, its loads are non-temporal and all issued before its
 * non-temporal stores.  src holds rd_units KiB and dst wr_units KiB (at least
 * 16 bytes when wr_units is 0: a never-taken store keeps read-only waves'
 * loads live).  MEP_ERR_SHAPE when a wave would take more than 16 read units,
 * for more than 2^24 waves or more than 2^30 units.  The values written are
 * unspecified.
 */
int mep_probe_stream(const void *src, void *dst, int64_t waves, int64_t rd_units,
                     int64_t wr_units, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MEP_H */
