/*
 * mep_oracle.c -- plain, slow, single-threaded CPU reference for MoE token
 * dispatch and combine (the MORI-EP intra-node path, restated for R virtual
 * ranks held in one address space).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this file's library.  The GPU library never links,
 * includes or calls it, and it shares no code, header or table with the GPU
 * kernels.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * No FMA contraction: every fused multiply-add below is an explicit fmaf().
 *
 * Sources (web pages; cited by title and section):
 *   [Guide]    "MORI-EP User Guide"  (rocm.github.io/mori/MORI-EP-GUIDE.html)
 *   [Backends] "Choosing an EP API and backend" (rocm.github.io/mori/ep_backends.html)
 *   [Issue57]  ROCm/mori issue #57, maintainer answer on the design
 *   [README]   MORI README, "Benchmarks / MORI-EP"
 *
 * Readings taken where the pages leave a step open (each is repeated at the
 * function that applies it):
 *   R1 expert e lives on rank e / num_experts_per_rank (contiguous blocks:
 *      [Guide] section 2, whose DeepSeek-V3 example gives each of 8 GPUs 32
 *      of the 256 experts).
 *   R2 a token is sent once per destination rank; the first j (in top-k
 *      order) naming that rank owns the row, later j on the same rank share it
 *      ([Issue57]: the design removes redundant transfer).
 *   R3 inside a rank, received rows are in ascending source-token order.
 *   R4 src_token_pos = src_rank * (world_size * max_num_inp_token_per_rank)
 *      + token ([Guide] section 3, get_dispatch_src_token_pos()).
 *   R5 FP8 block quantisation: per 128 columns, scale = amax / 448 (fp32,
 *      IEEE division), code = OCP E4M3 of fp32(x) / scale (IEEE division,
 *      round to nearest, ties to even code, saturating at 448); amax == 0
 *      gives scale 0 and signed-zero codes.  OCP E4M3 is the gfx950 FP8
 *      flavour ([Backends], restrictions list).
 *   R6 combine: out[t] = bf16_rne( fp32 sum over j = 0..k-1, in that order,
 *      acc = fmaf(w[t][j], y_j, acc), acc starting at +0 ), where y_j is the
 *      expert-output row holding (t, expert j) -- a rank row shared by two
 *      experts is used once per expert ([Guide] section 3 combine(): the
 *      weights scale each expert's output; [Backends]: the HIP backend's
 *      combine gathers in BF16 or FP32).
 *   R7 expert-major layout: experts in global order; each expert's rows in
 *      ascending receive slot; each segment starts at a multiple of 128 rows;
 *      padding rows are not written ([Guide] section 4,
 *      convert_dispatch_output()).
 *   R8 a token naming an expert id outside [0, E) is not dispatched (all its
 *      slots are -1, status bit 1) and combines to +0; a token naming the
 *      same expert twice sets status bit 2 and is otherwise handled as usual.
 *   R9 an already-quantized FP8 payload ([Backends]: the HIP backend carries
 *      one) is a row of E4M3 bytes plus the caller's fp32 scale row of any
 *      width; both travel unchanged.
 *   R10 standard-MoE dispatch ([Guide] section 4, dispatch_standard_moe():
 *      dispatch and convert_dispatch_output() in one call) produces exactly
 *      what the two steps produce one after the other; it is not a function
 *      of its own here.
 *   R11 FP4 payloads ([Backends]: FP4 conversion kernels on gfx950; the
 *      block format is not given): OCP Microscaling MXFP4 -- blocks of 32
 *      columns, E2M1 elements, one E8M0 scale per block.  Per the OCP MX
 *      conversion: shared exponent = floor(log2(amax)) - 2 (2 = the largest
 *      E2M1 exponent), clamped to [-127, 127]; scale byte = exponent + 127;
 *      element = E2M1(x / 2^exponent), round to nearest, ties to the even
 *      code, saturating at 6, sign kept; an all-zero block gets scale byte 0.
 *      Two elements per byte, the even column in the low nibble; the H/32
 *      scale bytes of a row fill H/128 32-bit scale words.  A carried FP4
 *      payload is H/2 bytes per row with the caller's scale words.
 *   R12 FP8 direct-cast combine payload ("MORI-EP User Guide", section 10
 *      Tuning, intra-node tuning matrix: quant type fp8_direct_cast with a bf16
 *      combine): each expert-output value is cast
 *      to OCP E4M3 with no scale (round to nearest even, saturating at 448);
 *      the combine accumulates the decoded values exactly as R6.
 *   R21 standard-MoE expert outputs back to the combine input ([Guide]
 *      section 4, convert_combine_input(packed rows, source info, layout
 *      range), which takes no weights): one bf16 row per received row (rank
 *      r, slot s), the fp32 chain acc = fmaf(w_j, y_j, acc) from +0 over the
 *      top-k positions j of that row whose expert lives on rank r and that are
 *      the first naming their expert, in j order, rounded once; w_j is the
 *      dispatched weight (recv weights [r][s][j]) and y_j the expert-major row
 *      of expert j whose source info is the row's src_token_pos.  The weights
 *      are applied here because one merged row per (token, rank) can carry a
 *      top-k weighted sum only if each expert's weight is applied before the
 *      merge; the combine of converted rows therefore adds a token's distinct
 *      rank rows without weights, in the order of their first top-k position,
 *      one fp32 rounding per addition, then bf16.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_ST_BAD_INDEX 1
#define ORACLE_ST_DUP_EXPERT 2
#define ORACLE_ST_EM_OVERFLOW 4

/* ------------------------------------------------------------------------ */
/* bfloat16: the upper half of an IEEE binary32.                             */
/* ------------------------------------------------------------------------ */

float oracle_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Value of a bfloat16 magnitude code (no sign), as a double.  Code 0x7F80 is
 * taken as 2^128, the value the next binade would start at, so that the
 * rounding rule below can send values past the largest finite code to inf. */
static double bf16_mag_value(uint32_t m) {
  uint32_t e = m >> 7, f = m & 0x7F;
  if (e == 0) return ldexp((double)f, -126 - 7);
  return ldexp(128.0 + (double)f, (int)e - 127 - 7);
}

/* Round a finite float to the nearest bfloat16, ties to the even code. */
uint16_t oracle_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t sign = u & 0x80000000u;
  if (isnan(f)) return (uint16_t)((sign >> 16) | 0x7FC0);
  if (isinf(f)) return (uint16_t)((sign >> 16) | 0x7F80);
  double a = fabs((double)f);
  uint32_t lo = (u & 0x7FFFFFFFu) >> 16; /* largest code with value <= a */
  uint32_t hi = lo + 1;
  double vlo = bf16_mag_value(lo), vhi = bf16_mag_value(hi);
  uint32_t pick;
  if (a == vlo) pick = lo;
  else if (a - vlo < vhi - a) pick = lo; /* both differences exact: a, vlo, vhi share a binade */
  else if (a - vlo > vhi - a) pick = hi;
  else pick = (lo & 1) ? hi : lo;
  return (uint16_t)((sign >> 16) | pick);
}

/* ------------------------------------------------------------------------ */
/* OCP E4M3 (OFP8): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.      */
/* Exponent field 0 is subnormal (m/8 * 2^-6).  No infinities; S.1111.111 is */
/* NaN, so the largest finite magnitude is 1.75 * 2^8 = 448 (code 0x7E).     */
/* ------------------------------------------------------------------------ */

double oracle_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Encode v to the nearest finite E4M3 value, ties to the even code, values
 * beyond 448 saturating to 448, the sign kept (so -0 and tiny negatives give
 * 0x80).  Magnitude codes 0x00..0x7E are increasing in value; the search walks
 * them to the first code not below |v| and compares |v| with the midpoint to
 * the code before it (midpoints are exact in double). */
uint8_t oracle_e4m3_encode(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  if (isnan(v)) return (uint8_t)(sign | 0x7F);
  double a = fabs((double)v);
  int c = 0;
  while (c < 0x7E && oracle_e4m3_decode((uint8_t)c) < a) c++;
  /* now decode(c) >= a, or c == 0x7E (a above the largest code: saturate) */
  if (c > 0 && oracle_e4m3_decode((uint8_t)c) >= a) {
    double lo = oracle_e4m3_decode((uint8_t)(c - 1)), hi = oracle_e4m3_decode((uint8_t)c);
    double mid = 0.5 * (lo + hi);
    if (a < mid) c = c - 1;
    else if (a == mid && (c & 1)) c = c - 1; /* tie: keep the even code */
  }
  return (uint8_t)(sign | c);
}

void oracle_e4m3_encode_array(const float *v, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_bf16_rne_array(const float *v, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_rne(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Routing plan ([Guide] section 3 dispatch(): recv_num_token, and           */
/* get_dispatch_src_token_pos(); [Issue57] for the dedupe; readings R1-R4,   */
/* R8).                                                                      */
/*                                                                          */
/* recv_counts[R]        rows each rank receives                             */
/* src_token_pos[R*cap]  for s < recv_counts[r]: R4 encoding of the token    */
/*                       in receive slot s of rank r (other entries untouched)*/
/* slot[T*k]             receive slot of (t, j) on rank idx[t][j]/epr; -1 for */
/*                       a token that is not dispatched                      */
/* Returns the status bits (R8).                                             */
/* ------------------------------------------------------------------------ */
int32_t oracle_plan(const int32_t *idx, int32_t T, int32_t k, int32_t R, int32_t epr,
                    int32_t cap, int32_t src_rank, int32_t *recv_counts,
                    int32_t *src_token_pos, int32_t *slot) {
  int32_t E = R * epr, status = 0;
  for (int32_t r = 0; r < R; r++) recv_counts[r] = 0;
  for (int32_t t = 0; t < T; t++) {
    const int32_t *e = idx + (int64_t)t * k;
    int32_t *sl = slot + (int64_t)t * k;
    int bad = 0;
    for (int32_t j = 0; j < k; j++)
      if (e[j] < 0 || e[j] >= E) bad = 1;
    for (int32_t j = 0; j < k && !bad; j++)
      for (int32_t jj = 0; jj < j; jj++)
        if (e[jj] == e[j]) status |= ORACLE_ST_DUP_EXPERT;
    if (bad) {
      status |= ORACLE_ST_BAD_INDEX;
      for (int32_t j = 0; j < k; j++) sl[j] = -1;
      continue;
    }
    for (int32_t j = 0; j < k; j++) {
      int32_t r = e[j] / epr;
      int32_t first = -1;
      for (int32_t jj = 0; jj < j; jj++)
        if (e[jj] / epr == r) { first = jj; break; }
      if (first >= 0) {
        sl[j] = sl[first]; /* R2: the rank already holds this token's row */
      } else {
        int32_t s = recv_counts[r]++; /* R3: tokens arrive in ascending order */
        sl[j] = s;
        src_token_pos[(int64_t)r * cap + s] = src_rank * (R * cap) + t; /* R4 */
      }
    }
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* Dispatch ([Guide] section 3 dispatch(): the received rows carry the token */
/* row, its k weights, its scales and its k expert ids; reading R5 for the   */
/* FP8 payload).                                                             */
/*                                                                          */
/* w, idx [T,k]; slot [T,k] from oracle_plan.                               */
/* quant == 0: x [T,H] bf16 bits; recv_x is [R,cap,H] bf16 (bit copy),      */
/*             recv_scales unused.                                           */
/* quant == 1: x [T,H] bf16 bits; recv_x is [R,cap,H] E4M3 bytes,           */
/*             recv_scales [R,cap,H/128] (reading R5).                       */
/* quant == 2: x [T,H] E4M3 bytes with xs [T,sd] fp32 scales, both copied    */
/*             into recv_x [R,cap,H] bytes and recv_scales [R,cap,sd]        */
/*             ([Backends]: the HIP backend's dispatch can move FP8 rows     */
/*             that arrive quantized; reading R9).                           */
/* quant == 3: as 2 for FP4 rows of H/2 bytes (reading R11).                 */
/* quant == 4: x [T,H] bf16 bits quantised to MXFP4: recv_x [R,cap,H/2]      */
/*             bytes, recv_scales [R,cap,H/128] words of E8M0 bytes (R11).   */
/* recv_w [R,cap,k] f32, recv_idx [R,cap,k] i32.  Only written rows change.  */
/* ------------------------------------------------------------------------ */

/* ------------------------------------------------------------------------ */
/* E2M1, the OCP MX FP4 element: sign, 2 exponent bits (bias 1), 1 mantissa */
/* bit; no inf or NaN.  Code bits 0..2 give the magnitudes 0, 0.5, 1, 1.5,  */
/* 2, 3, 4, 6; bit 3 is the sign.                                            */
/* ------------------------------------------------------------------------ */
double oracle_e2m1_decode(uint8_t c) {
  int e = (c >> 1) & 3, m = c & 1;
  double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return (c & 8) ? -mag : mag;
}

/* Nearest E2M1 code of v (a double), ties to the even code, saturating at 6;
 * the sign is kept, zero included. */
uint8_t oracle_e2m1_encode(double v) {
  uint8_t sign = signbit(v) ? 8 : 0;
  double a = fabs(v);
  int c = 0;
  while (c < 7 && oracle_e2m1_decode((uint8_t)c) < a) c++;
  if (c > 0 && oracle_e2m1_decode((uint8_t)c) >= a) {
    double lo = oracle_e2m1_decode((uint8_t)(c - 1)), hi = oracle_e2m1_decode((uint8_t)c);
    double mid = 0.5 * (lo + hi);
    if (a < mid) c = c - 1;
    else if (a == mid && (c & 1)) c = c - 1;
  }
  return (uint8_t)(sign | c);
}

/* R11 for one token row: q[H/2] packed codes, e8[H/32] scale bytes. */
void oracle_mx4_quant_row(const uint16_t *x, int32_t H, uint8_t *q, uint8_t *e8) {
  for (int32_t b = 0; b < H / 32; b++) {
    double amax = 0.0;
    for (int32_t i = 0; i < 32; i++) {
      double v = fabs((double)oracle_bf16_to_f32(x[b * 32 + i]));
      if (v > amax) amax = v;
    }
    int se = -127;
    if (amax > 0.0) {
      int ex;
      frexp(amax, &ex); /* amax = m * 2^ex, m in [0.5, 1): floor(log2(amax)) = ex - 1 */
      se = ex - 1 - 2;
      if (se < -127) se = -127;
      if (se > 127) se = 127;
    }
    e8[b] = (uint8_t)(se + 127);
    for (int32_t i = 0; i < 32; i += 2) {
      uint8_t c0, c1;
      double v0 = oracle_bf16_to_f32(x[b * 32 + i]), v1 = oracle_bf16_to_f32(x[b * 32 + i + 1]);
      if (amax == 0.0) {
        c0 = signbit(v0) ? 8 : 0;
        c1 = signbit(v1) ? 8 : 0;
      } else {
        c0 = oracle_e2m1_encode(ldexp(v0, -se));
        c1 = oracle_e2m1_encode(ldexp(v1, -se));
      }
      q[(b * 32 + i) / 2] = (uint8_t)(c0 | (c1 << 4));
    }
  }
}

/* R11 decoding of one packed row: out[H] as doubles. */
void oracle_mx4_decode_row(const uint8_t *q, const uint8_t *e8, int32_t H, double *out) {
  for (int32_t i = 0; i < H; i++) {
    uint8_t c = (q[i / 2] >> ((i & 1) * 4)) & 0xF;
    out[i] = ldexp(oracle_e2m1_decode(c), (int)e8[i / 32] - 127);
  }
}

/* R12: E4M3 direct cast (no scale) of n bf16 values. */
void oracle_cast_fp8_direct(const uint16_t *y, int64_t n, uint8_t *y8) {
  for (int64_t i = 0; i < n; i++) y8[i] = oracle_e4m3_encode(oracle_bf16_to_f32(y[i]));
}

/* R5 for one token row: fills q[H] and scale[H/128]. */
void oracle_quant_row(const uint16_t *x, int32_t H, uint8_t *q, float *scale) {
  for (int32_t b = 0; b < H / 128; b++) {
    float amax = 0.0f;
    for (int32_t i = 0; i < 128; i++) {
      float v = fabsf(oracle_bf16_to_f32(x[b * 128 + i]));
      if (v > amax) amax = v;
    }
    float s = amax / 448.0f;
    scale[b] = s;
    for (int32_t i = 0; i < 128; i++) {
      float xf = oracle_bf16_to_f32(x[b * 128 + i]);
      if (s == 0.0f) q[b * 128 + i] = signbit(xf) ? 0x80 : 0x00;
      else q[b * 128 + i] = oracle_e4m3_encode(xf / s);
    }
  }
}

void oracle_dispatch(const void *x, const float *xs, int32_t sd, const float *w,
                     const int32_t *idx, const int32_t *slot, int32_t T, int32_t H, int32_t k,
                     int32_t R, int32_t epr, int32_t cap, int32_t quant, void *recv_x,
                     float *recv_scales, float *recv_w, int32_t *recv_idx,
                     uint8_t *q_tmp /* [H] */, float *s_tmp /* [scale words] */) {
  /* bytes per received row, 32-bit scale words per row */
  int64_t rowb = quant == 0 ? 2 * (int64_t)H : (quant >= 3 ? H / 2 : H);
  int32_t nb = (quant == 1 || quant == 4) ? H / 128 : (quant == 0 ? 0 : sd);
  (void)R;
  for (int32_t t = 0; t < T; t++) {
    const int32_t *e = idx + (int64_t)t * k;
    const int32_t *sl = slot + (int64_t)t * k;
    if (sl[0] < 0) continue; /* R8: token not dispatched */
    const uint16_t *xr = (const uint16_t *)x + (int64_t)t * H;
    if (quant == 1) {
      oracle_quant_row(xr, H, q_tmp, s_tmp);
    } else if (quant == 2 || quant == 3) {
      memcpy(q_tmp, (const uint8_t *)x + (int64_t)t * rowb, (size_t)rowb);
      if (sd > 0) memcpy(s_tmp, xs + (int64_t)t * sd, sizeof(float) * (size_t)sd);
    } else if (quant == 4) {
      oracle_mx4_quant_row(xr, H, q_tmp, (uint8_t *)s_tmp);
    }
    for (int32_t j = 0; j < k; j++) {
      int32_t r = e[j] / epr;
      int first = 1;
      for (int32_t jj = 0; jj < j; jj++)
        if (e[jj] / epr == r) first = 0;
      if (!first) continue; /* R2: one row per destination rank */
      int64_t row = (int64_t)r * cap + sl[j];
      if (quant) {
        memcpy((uint8_t *)recv_x + row * rowb, q_tmp, (size_t)rowb);
        if (nb > 0) memcpy(recv_scales + row * nb, s_tmp, sizeof(float) * (size_t)nb);
      } else {
        memcpy((uint16_t *)recv_x + row * H, xr, sizeof(uint16_t) * (size_t)H);
      }
      memcpy(recv_w + row * k, w + (int64_t)t * k, sizeof(float) * (size_t)k);
      memcpy(recv_idx + row * k, e, sizeof(int32_t) * (size_t)k);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Combine from the rank-major receive layout ([Guide] section 3 combine(); */
/* reading R6).  y [R,cap,H] bf16 bits; out [T,H] bf16 bits.                 */
/* ------------------------------------------------------------------------ */
void oracle_combine(const uint16_t *y, const float *w, const int32_t *idx,
                    const int32_t *slot, int32_t T, int32_t H, int32_t k, int32_t epr,
                    int32_t cap, uint16_t *out) {
  for (int32_t t = 0; t < T; t++) {
    for (int32_t h = 0; h < H; h++) {
      float acc = 0.0f;
      for (int32_t j = 0; j < k; j++) {
        int32_t s = slot[(int64_t)t * k + j];
        if (s < 0) continue;
        int64_t row = (int64_t)(idx[(int64_t)t * k + j] / epr) * cap + s;
        acc = fmaf(w[(int64_t)t * k + j], oracle_bf16_to_f32(y[row * H + h]), acc);
      }
      out[(int64_t)t * H + h] = oracle_bf16_rne(acc);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Expert-major conversion ([Guide] section 4, convert_dispatch_output():    */
/* packed rows, per-expert counts and source info; reading R7).              */
/*                                                                          */
/* elem_bytes: 1 (E4M3 payload) or 2 (bf16).  nb: scale columns (0 = none).  */
/* em_counts[E], em_offsets[E+1], em_x [cap_em,H], em_scales [cap_em,nb],    */
/* em_src_pos [cap_em]; tok_em_row [T,k] gets the expert-major row holding   */
/* (t, expert j) (-1 if none).  Returns status bit 4 if the padded segments  */
/* need more than cap_em rows (rows past cap_em are then dropped).           */
/* ------------------------------------------------------------------------ */
int32_t oracle_to_expert_major(const void *recv_x, const float *recv_scales,
                               const int32_t *recv_idx, const int32_t *recv_counts,
                               const int32_t *src_token_pos, int32_t R, int32_t epr,
                               int32_t cap, int32_t H, int32_t nb, int32_t k,
                               int32_t elem_bytes, int32_t src_rank, int32_t T,
                               int64_t cap_em, void *em_x, float *em_scales,
                               int32_t *em_counts, int32_t *em_offsets,
                               int32_t *em_src_pos, int32_t *tok_em_row) {
  int32_t E = R * epr, status = 0;
  int64_t rowbytes = (int64_t)H * elem_bytes;
  for (int64_t i = 0; i < (int64_t)T * k; i++) tok_em_row[i] = -1;
  em_offsets[0] = 0;
  for (int32_t e = 0; e < E; e++) {
    int32_t r = e / epr, n = 0;
    for (int32_t s = 0; s < recv_counts[r]; s++) {
      const int32_t *ids = recv_idx + ((int64_t)r * cap + s) * k;
      int32_t jhit = -1;
      for (int32_t j = 0; j < k; j++)
        if (ids[j] == e) { jhit = j; break; }
      if (jhit < 0) continue;
      int64_t dst = (int64_t)em_offsets[e] + n;
      n++;
      if (dst >= cap_em) { status |= ORACLE_ST_EM_OVERFLOW; continue; }
      int64_t src = (int64_t)r * cap + s;
      memcpy((uint8_t *)em_x + dst * rowbytes, (const uint8_t *)recv_x + src * rowbytes,
             (size_t)rowbytes);
      if (nb > 0) memcpy(em_scales + dst * nb, recv_scales + src * nb, sizeof(float) * (size_t)nb);
      int32_t pos = src_token_pos[src];
      em_src_pos[dst] = pos;
      int32_t t = pos - src_rank * (R * cap);
      if (t >= 0 && t < T) tok_em_row[(int64_t)t * k + jhit] = (int32_t)dst;
    }
    em_counts[e] = n;
    em_offsets[e + 1] = em_offsets[e] + ((n + 127) / 128) * 128;
  }
  return status;
}

/* Combine from the expert-major layout ([Guide] section 4,
 * combine_standard_moe(); reading R6 with y_j = y_em[tok_em_row[t][j]]). */
void oracle_combine_em(const uint16_t *y_em, const float *w, const int32_t *tok_em_row,
                       int32_t T, int32_t H, int32_t k, uint16_t *out) {
  for (int32_t t = 0; t < T; t++) {
    for (int32_t h = 0; h < H; h++) {
      float acc = 0.0f;
      for (int32_t j = 0; j < k; j++) {
        int32_t row = tok_em_row[(int64_t)t * k + j];
        if (row < 0) continue;
        acc = fmaf(w[(int64_t)t * k + j], oracle_bf16_to_f32(y_em[(int64_t)row * H + h]), acc);
      }
      out[(int64_t)t * H + h] = oracle_bf16_rne(acc);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Expert stand-ins (harness, not part of the path).  The identity expert of */
/* [Guide] section 7 returns the received rows unchanged; for FP8 payloads   */
/* the stand-in dequantises: y = bf16_rne((fp32(decode(q)) * scale) * mult). */
/* ------------------------------------------------------------------------ */
void oracle_expert_dequant(const uint8_t *q, const float *scales, int64_t rows, int32_t H,
                           float mult, uint16_t *y) {
  int32_t nb = H / 128;
  for (int64_t i = 0; i < rows; i++)
    for (int32_t h = 0; h < H; h++) {
      float p = (float)oracle_e4m3_decode(q[i * H + h]) * scales[i * nb + h / 128];
      p = p * mult;
      y[i * H + h] = oracle_bf16_rne(p);
    }
}

/* ------------------------------------------------------------------------ */
/* Expert-major expert outputs back to the rank-major combine input          */
/* ([Guide] section 4, convert_combine_input(): standard-MoE rows, their      */
/* source info and layout, turned into the rows the combine takes; reading   */
/* R21).                                                                     */
/*                                                                          */
/* y_em [cap_em,H] bf16 expert outputs in the layout em_counts/em_offsets/   */
/* em_src_pos describe; recv_w, recv_idx [R,cap,k], recv_counts [R] and      */
/* src_token_pos [R,cap] from the dispatch.  For every received row (r, s),  */
/* s < recv_counts[r], with source position p = src_token_pos[r][s]:         */
/*   y_rm[r][s][h] = bf16_rne(acc), acc = +0, then for j = 0..k-1 in order,  */
/*   over positions whose expert e lives on rank r and that are the first    */
/*   naming e: acc = fmaf(recv_w[r][s][j], y_em[i][h], acc), i the row of    */
/*   e's segment whose source info is p.                                     */
/* Rows past recv_counts[r] are not written.  A position whose expert-major  */
/* row is absent (dropped past cap_em) adds nothing.  em_of_j: [k] scratch.  */
/* ------------------------------------------------------------------------ */
void oracle_convert_combine_input(const uint16_t *y_em, int64_t cap_em, const int32_t *em_counts,
                                  const int32_t *em_offsets, const int32_t *em_src_pos,
                                  const float *recv_w, const int32_t *recv_idx,
                                  const int32_t *recv_counts, const int32_t *src_token_pos,
                                  int32_t R, int32_t epr, int32_t cap, int32_t H, int32_t k,
                                  uint16_t *y_rm, int64_t *em_of_j) {
  int32_t E = R * epr;
  for (int32_t r = 0; r < R; r++) {
    for (int32_t s = 0; s < recv_counts[r]; ++s) {
      int64_t row = (int64_t)r * cap + s;
      const int32_t *ids = recv_idx + row * k;
      int32_t pos = src_token_pos[row];
      for (int32_t j = 0; j < k; j++) {
        int32_t e = ids[j];
        em_of_j[j] = -1;
        if (e < 0 || e >= E) continue;
        if (e / epr != r) continue; /* the expert lives on another rank */
        int first = 1;
        for (int32_t jj = 0; jj < j; jj++)
          if (ids[jj] == e) first = 0;
        if (!first) continue; /* a repeated expert has one row */
        int64_t end = (int64_t)em_offsets[e] + em_counts[e];
        if (end > cap_em) end = cap_em;
        for (int64_t i = em_offsets[e]; i < end; i++)
          if (em_src_pos[i] == pos) { em_of_j[j] = i; break; }
      }
      for (int32_t h = 0; h < H; h++) {
        float acc = 0.0f;
        for (int32_t j = 0; j < k; j++) {
          if (em_of_j[j] < 0) continue;
          acc = fmaf(recv_w[row * k + j], oracle_bf16_to_f32(y_em[em_of_j[j] * H + h]), acc);
        }
        y_rm[row * H + h] = oracle_bf16_rne(acc);
      }
    }
  }
}

/* Combine of converted rows (reading R21): for every token t,
 *   out[t][h] = bf16_rne(acc), acc = +0, then over t's destination ranks in
 *   the order of their first top-k position: acc = acc + y_rm[r][slot][h]
 *   (one fp32 rounding per addition, no weights: the converted rows already
 *   carry them).  Tokens that were not dispatched give +0.
 * rank_of_j: [k] scratch. */
void oracle_combine_rank_sum(const uint16_t *y_rm, const int32_t *idx, const int32_t *slot,
                             int32_t T, int32_t H, int32_t k, int32_t epr, int32_t cap,
                             uint16_t *out, int64_t *row_of_j) {
  for (int32_t t = 0; t < T; t++) {
    const int32_t *e = idx + (int64_t)t * k;
    for (int32_t j = 0; j < k; j++) {
      int32_t s = slot[(int64_t)t * k + j];
      int32_t r = e[j] / epr;
      row_of_j[j] = -1;
      if (s < 0) continue;
      int first = 1;
      for (int32_t jj = 0; jj < j; jj++)
        if (e[jj] / epr == r) first = 0;
      if (first) row_of_j[j] = (int64_t)r * cap + s; /* one row per destination rank */
    }
    for (int32_t h = 0; h < H; h++) {
      float acc = 0.0f;
      for (int32_t j = 0; j < k; j++) {
        if (row_of_j[j] < 0) continue;
        acc = acc + oracle_bf16_to_f32(y_rm[row_of_j[j] * H + h]);
      }
      out[(int64_t)t * H + h] = oracle_bf16_rne(acc);
    }
  }
}
