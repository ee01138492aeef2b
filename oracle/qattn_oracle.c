/*
 * qattn_oracle.c -- plain, slow CPU oracle for the quantized attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * cpu_baseline leg may load this library.  It shares no code, header, table or
 * constant generator with the HIP library; the two are written independently from
 * the same numeric contract.
 *
 * Build: gcc -O3 -march=x86-64-v3 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no FMA contraction, no reassociation: every fp32 rounding below is explicit).
 *
 * Method (from the pages):
 *   - K smoothing, Q/K INT8 and V FP8 preparation: "H3 Performance Roadmap",
 *     section "Measured GB10 Baseline" (SageAttention 2.2.0 internals table) and
 *     section "Phase 4: Dense Sage-Compatible Attention" (items 2 and 3: per-warp
 *     INT8 Q/K quantization, FP8 V policy, K smoothing).
 *   - Per-tile order QK -> update m, d, O -> accumulate d -> convert P to 8 bit -> PV:
 *     "Sage2 SM89 Temporal Pair Experiment", section "Candidate".
 *   - Prefill over an int8 KV cache with per-token scales: Strata #2092 (description
 *     and the "qsa_prompt_attn_parity (int8 KV)" table).
 * Where the pages leave a step open, the reading taken is stated at the function.
 *
 * Parity pins: every function here is checked by tests/test_oracle_*.py against
 * closed forms, invariants, brute force or library routines (see each function).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_TILE 64 /* KV tile = 64 keys; also the Q/K scale block (64 rows) */

/* ------------------------------------------------------------------------- */
/* scalar helpers                                                            */
/* ------------------------------------------------------------------------- */

static float f_of_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of_f(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits. */
float orc_bf16_to_f32(uint16_t h) { return f_of_bits((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest even (output rounding of the epilogue). */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u = bits_of_f(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, exponent field 0 encodes subnormals m * 2^-9.
 * Decoding straight from that definition. */
double orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Table of the 127 non-negative finite values, ascending with the code. */
static double g_e4m3_pos[127];
static int g_e4m3_ready = 0;
static void e4m3_init(void) {
  if (g_e4m3_ready) return;
  for (int c = 0; c < 127; ++c) g_e4m3_pos[c] = orc_e4m3_decode((uint8_t)c);
  g_e4m3_ready = 1;
}

/* Encode fp32 -> E4M3: magnitude clamped to 448 (the largest finite value), then the
 * nearest representable value, ties to the code with an even mantissa; the sign is
 * kept (so -0 encodes as 0x80).  NaN -> 0x7F.  Reading of "quantize V to FP8 e4m3"
 * (pages silent on rounding and overflow): round to nearest even, saturate. */
uint8_t orc_e4m3_encode(float x) {
  e4m3_init();
  uint32_t u = bits_of_f(x);
  uint8_t sign = (uint8_t)((u >> 31) << 7);
  if (x != x) return 0x7f;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7e;
  /* largest code lo with value <= a (binary search over the ascending table) */
  int lo = 0, hi = 126;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (g_e4m3_pos[mid] <= a) lo = mid; else hi = mid - 1;
  }
  int code = lo;
  if (g_e4m3_pos[lo] != a && lo < 126) {
    double dlo = a - g_e4m3_pos[lo], dhi = g_e4m3_pos[lo + 1] - a;
    if (dhi < dlo || (dhi == dlo && ((lo + 1) & 1) == 0)) code = lo + 1;
  }
  return sign | (uint8_t)code;
}

/* 2^x rounded to the nearest fp32.  Evaluated as (float)exp2((double)x): the double
 * result is within one double ulp of 2^x, so the final rounding is the correct one
 * unless 2^x lies within ~2^-52 (relative) of an fp32 rounding midpoint.  The tests
 * check, for every grid argument the softmax below can produce, that this agrees with
 * a second route through long double (so the rounding is settled) and with
 * high-precision decimal arithmetic on samples.  The pages leave the exponential
 * unspecified; the reading taken is the correctly rounded one. */
float orc_exp2(float x) { return (float)exp2((double)x); }

/* P' of a grid argument u: 2^(u - 80) rounded once to fp32 (u - 80 is exact in double;
 * for u in [40, 160] it is also exact in fp32, so this is orc_exp2(u - 80) there). */
float orc_p_of_u(float u) { return (float)exp2((double)u - 80.0); }

/* INT8 code of one value: round half to even of fl32(x * r), clamped to [-127, 127]. */
static int8_t i8_code(float x, float r) {
  float t = x * r;
  float q = rintf(t); /* default rounding mode: to nearest, ties to even */
  if (q > 127.0f) q = 127.0f;
  if (q < -127.0f) q = -127.0f;
  return (int8_t)q;
}

/* ------------------------------------------------------------------------- */
/* a1: K channel mean ("K smoothing")                                         */
/* ------------------------------------------------------------------------- */
/* H3 Performance Roadmap, "Measured GB10 Baseline" (K smoothing row) and "Phase 4"
 * item 3.  Reading: mean over all N tokens of each (b, h, channel), summed in fp64,
 * one rounding to fp32; it is subtracted and not added back (softmax is invariant to
 * a per-row constant shift of the scores).  Returns the number of fp64 additions that
 * were inexact (TwoSum error != 0); 0 means the sum is exact, so the result does not
 * depend on summation order.
 * k: bf16 [B, N, H, D] with element strides str = {sb, sn, sh}, d stride 1.
 * mean: fp32 [B, H, D]. */
long orc_k_mean(const uint16_t* k, const int64_t* str, int B, int H, int N, int D, float* mean) {
  long inexact = 0;
  double* s = (double*)malloc(sizeof(double) * D);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      for (int c = 0; c < D; ++c) s[c] = 0.0;
      /* each channel's sum runs over n = 0, 1, ..., N-1 in order */
      for (int n = 0; n < N; ++n) {
        const uint16_t* row = k + b * str[0] + (int64_t)n * str[1] + h * str[2];
        for (int c = 0; c < D; ++c) {
          double x = (double)orc_bf16_to_f32(row[c]);
          double t = s[c] + x;
          /* TwoSum error term */
          double bp = t - s[c];
          double err = (s[c] - (t - bp)) + (x - bp);
          if (err != 0.0) inexact++;
          s[c] = t;
        }
      }
      for (int c = 0; c < D; ++c) mean[((int64_t)b * H + h) * D + c] = (float)(s[c] / (double)N);
    }
  free(s);
  return inexact;
}

/* ------------------------------------------------------------------------- */
/* a2: INT8 per-block quantization of Q and of smoothed K                     */
/* ------------------------------------------------------------------------- */
/* H3 Performance Roadmap, "Measured GB10 Baseline" (Q/K INT8 quantization row) and
 * "Phase 4" item 2 (per-warp INT8 Q/K quantization).  Reading: symmetric INT8 with one
 * fp32 scale per block of 64 consecutive rows of one (b, h); a = max |x| over the
 * block's valid rows; s = fl32(a / 127); r = min(fl32(127 / a), FLT_MAX);
 * code = clamp(rne(fl32(x * r))); a = 0 gives s = 0 and zero codes; rows N..N_pad-1
 * are zero codes.  (The clamp of r only acts when a < 127 / FLT_MAX, where the
 * reciprocal would overflow; the pages are silent on it.)
 * With mean != NULL the value quantized is x' = fl32(x - mean[b,h,c]) (smoothing).
 * x: bf16 [B, N, H, D] strided; codes: int8 [B, H, N_pad, D]; scales: [B, H, N_pad/64]. */
void orc_quant_i8_blocks(const uint16_t* x, const int64_t* str, const float* mean, int B, int H, int N, int D,
                         int8_t* codes, float* scales) {
  int npad = (N + ORC_TILE - 1) / ORC_TILE * ORC_TILE;
  int nblk = npad / ORC_TILE;
  float* buf = (float*)malloc(sizeof(float) * ORC_TILE * D);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int blk = 0; blk < nblk; ++blk) {
        int r0 = blk * ORC_TILE;
        int rows = N - r0 < ORC_TILE ? N - r0 : ORC_TILE;
        float a = 0.0f;
        for (int r = 0; r < rows; ++r)
          for (int c = 0; c < D; ++c) {
            float v = orc_bf16_to_f32(x[b * str[0] + (int64_t)(r0 + r) * str[1] + h * str[2] + c]);
            if (mean) v = v - mean[((int64_t)b * H + h) * D + c];
            buf[r * D + c] = v;
            float av = fabsf(v);
            if (av > a) a = av;
          }
        float s = 0.0f, rcp = 0.0f;
        if (a > 0.0f) {
          s = a / 127.0f;
          rcp = fminf(127.0f / a, FLT_MAX);
        }
        scales[((int64_t)b * H + h) * nblk + blk] = s;
        int8_t* out = codes + (((int64_t)b * H + h) * npad + r0) * D;
        for (int r = 0; r < ORC_TILE; ++r)
          for (int c = 0; c < D; ++c)
            out[r * D + c] = (r < rows && a > 0.0f) ? i8_code(buf[r * D + c], rcp) : (int8_t)0;
      }
  free(buf);
}

/* ------------------------------------------------------------------------- */
/* f4: appending tokens to an INT8 KV cache with per-token scales             */
/* ------------------------------------------------------------------------- */
/* Strata #2092 runs its prompt attention on an int8 KV cache with one fp32 scale per
 * (head, token) and leaves the quantizer that fills it unstated.  Reading: the same
 * symmetric INT8 quantizer as the Q/K blocks, with a block of one (token, head) row:
 * a = max |x| over the D channels, s = fl32(a / 127), r = min(fl32(127 / a), FLT_MAX),
 * code = clamp(rne(fl32(x * r))); a = 0 gives s = 0 and zero codes.
 * x: bf16 [Nnew, H, D] with element strides str = {sn, sh}; token n goes to cache row
 * pos + n: cache int8 [H, Nmax, D], tok_scale f32 [H, Nmax]; other rows are untouched. */
void orc_kv_append_i8(const uint16_t* x, const int64_t* str, int Nnew, int H, int D, int8_t* cache,
                      float* tok_scale, int Nmax, int pos) {
  float* buf = (float*)malloc(sizeof(float) * D);
  for (int n = 0; n < Nnew; ++n)
    for (int h = 0; h < H; ++h) {
      float a = 0.0f;
      for (int c = 0; c < D; ++c) {
        buf[c] = orc_bf16_to_f32(x[(int64_t)n * str[0] + (int64_t)h * str[1] + c]);
        if (fabsf(buf[c]) > a) a = fabsf(buf[c]);
      }
      float s = 0.0f, rcp = 0.0f;
      if (a > 0.0f) {
        s = a / 127.0f;
        rcp = fminf(127.0f / a, FLT_MAX);
      }
      int64_t row = (int64_t)h * Nmax + pos + n;
      tok_scale[row] = s;
      for (int c = 0; c < D; ++c) cache[row * D + c] = a > 0.0f ? i8_code(buf[c], rcp) : (int8_t)0;
    }
  free(buf);
}

/* ------------------------------------------------------------------------- */
/* a3: V FP8 per-channel quantization (V stored transposed)                   */
/* ------------------------------------------------------------------------- */
/* H3 Performance Roadmap, "Measured GB10 Baseline" (V FP8 quantization row: a combined
 * V transpose and FP8 quantization) and "Phase 4" item 2 (FP8 V policy).  Reading: one
 * fp32 scale per (b, h, channel) over all valid tokens: a = max |v|; s = fl32(a / 448);
 * r = min(fl32(448 / a), FLT_MAX); code = E4M3(fl32(v * r)); a = 0 gives s = 0 and 0x00
 * codes.  (As for INT8, the clamp of r only acts when the reciprocal would overflow.)  Output is
 * channel-major (transposed): v8t [B, H, D, N_pad] with zero codes for n >= N.
 * vf: fp32 values [B, H, N, D] already gathered (bf16 inputs or dequantized cache). */
static void quant_v_f32(const float* vf, int B, int H, int N, int D, uint8_t* v8t, float* vscale) {
  int npad = (N + ORC_TILE - 1) / ORC_TILE * ORC_TILE;
  float* a = (float*)malloc(sizeof(float) * D);
  float* rcp = (float*)malloc(sizeof(float) * D);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const float* src = vf + ((int64_t)b * H + h) * (int64_t)N * D;
      uint8_t* out = v8t + ((int64_t)b * H + h) * D * (int64_t)npad;
      for (int c = 0; c < D; ++c) a[c] = 0.0f;
      for (int n = 0; n < N; ++n)
        for (int c = 0; c < D; ++c) {
          float av = fabsf(src[(int64_t)n * D + c]);
          if (av > a[c]) a[c] = av;
        }
      for (int c = 0; c < D; ++c) {
        float sc = 0.0f;
        rcp[c] = 0.0f;
        if (a[c] > 0.0f) {
          sc = a[c] / 448.0f;
          rcp[c] = fminf(448.0f / a[c], FLT_MAX);
        }
        vscale[((int64_t)b * H + h) * D + c] = sc;
      }
      for (int n = 0; n < npad; ++n)
        for (int c = 0; c < D; ++c)
          out[(int64_t)c * npad + n] =
              (n < N && a[c] > 0.0f) ? orc_e4m3_encode(src[(int64_t)n * D + c] * rcp[c]) : (uint8_t)0;
    }
  free(a);
  free(rcp);
}

/* v: bf16 [B, N, H, D] strided -> v8t [B, H, D, N_pad], vscale [B, H, D]. */
void orc_quant_v(const uint16_t* v, const int64_t* str, int B, int H, int N, int D, uint8_t* v8t, float* vscale) {
  float* vf = (float*)malloc(sizeof(float) * (size_t)B * H * N * D);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int n = 0; n < N; ++n)
        for (int c = 0; c < D; ++c)
          vf[(((int64_t)b * H + h) * N + n) * D + c] =
              orc_bf16_to_f32(v[b * str[0] + (int64_t)n * str[1] + h * str[2] + c]);
  quant_v_f32(vf, B, H, N, D, v8t, vscale);
  free(vf);
}

/* Int8 KV cache V (per-token scales) -> per-channel E4M3.  Strata #2092 keeps V as int8
 * with one scale per token; the method's PV runs in FP8, so each cached value is first
 * dequantized exactly as fl32(code * s_tok) and then quantized as above (reading: one
 * requantization per call, channel scales over all Nk cached tokens).
 * v_cache: int8 [H, Nk, D]; v_tok_scale: [H, Nk] -> v8t [H, D, Nk_pad], vscale [H, D]. */
void orc_requant_v_cache(const int8_t* v_cache, const float* v_tok_scale, int H, int Nk, int D, uint8_t* v8t,
                         float* vscale) {
  float* vf = (float*)malloc(sizeof(float) * (size_t)H * Nk * D);
  for (int h = 0; h < H; ++h)
    for (int n = 0; n < Nk; ++n) {
      float s = v_tok_scale[(int64_t)h * Nk + n];
      for (int c = 0; c < D; ++c)
        vf[((int64_t)h * Nk + n) * D + c] = (float)v_cache[((int64_t)h * Nk + n) * D + c] * s;
    }
  quant_v_f32(vf, 1, H, Nk, D, v8t, vscale);
  free(vf);
}

/* ------------------------------------------------------------------------- */
/* a4-a6: INT8 QK, tile-ordered online softmax, FP8 PV, epilogue              */
/* ------------------------------------------------------------------------- */
/* Sage2 SM89 Temporal Pair Experiment, "Candidate": every query row keeps its own
 * running max m, denominator d and fp32 output accumulator, and each KV tile runs
 * QK -> update m, d, O -> accumulate d -> convert P to 8 bit -> PV, in that order.
 * Readings where the pages are silent:
 *   - tile = 64 keys, tiles in ascending key order, one pass;
 *   - scores in the log2 domain: c = fl32(fl32(s_q * s_k) * lambda), lambda = softmax
 *     scale * log2(e) (default fl32(fl32(1/sqrt(D)) * fl32(log2 e)));
 *     S_j = fl32(f32(acc_j) * c) is what the running max sees;
 *   - the exponent of each P is formed on a fixed grid:
 *         b  = fl32(88 - m_s)               (m_s = new max, or 0 if it is -inf)
 *         u  = fl32(f32(acc_j) * c + b)     (one rounding: fused multiply-add)
 *         P' = 2^(u - 80)  (correctly rounded fp32) = 256 * P
 *     (u - 80 = S_j - m_s + 8, rounded to the grid of u) so P' carries the exact 2^8
 *     pre-scale that keeps FP8 P in the normal range, and its exponent u - 80 is a
 *     multiple of 2^-17 whenever S_j - m_s is in [-24, 40) (u in [64, 128)), which
 *     holds for every P' with a nonzero e4m3 code;
 *   - alpha = 1 if the max did not change, else 2^(fl32(m - m_s)) (0 when m = -inf);
 *   - d' = fl32(alpha * d') + sum_j P'   (fp32; d is accumulated from P before the 8-bit
 *     conversion, as the page's order says; d' = 256 d);
 *   - P8_j = E4M3(P'_j);  O_c = fl32(alpha * O_c) + sum_j dec(P8_j) * dec(v8[c][j]);
 *   - masked keys (beyond Nk, or causal) have S = -inf and P' = 0;
 *   - epilogue: out_c = fl32(fl32(O_c * s_v[c]) / d'), 0 if d' = 0.
 * fp32 sums of d' and O are formed here key by key in ascending order; their order is
 * not part of the contract (the GPU result is compared within a tolerance).
 *
 * orc_attn_rows_part runs the tiles t_lo <= t < t_hi only and returns, per row, the
 * unnormalized O (D values), the running max m (-inf if none of its keys is visible)
 * and d'; orc_attn_rows runs all tiles and applies the epilogue.
 *
 * Computes rows i0..i1-1 of one (b, h).
 *   q8:  int8 [Nq_pad, D] rows of this (b, h);  qs: fp32 [Nq_pad/64]
 *   k8:  int8 rows of this (b, h), row stride D (at least Nk rows);
 *   ks:  per 64-key block [Nk_pad/64] (ks_per_token = 0) or per key [Nk] (= 1)
 *   v8t: E4M3 [D][ldv] (channel-major, ldv >= Nk);  vs: fp32 [D]
 *   causal: key j visible iff j <= i + pos_off (pos_off = Nk - Nq for bottom-right
 *           alignment, = pos0 for a prefill chunk starting at position pos0)
 *   out: fp32 [i1 - i0][D]. */
void orc_attn_rows_part(const int8_t* q8, const float* qs, const int8_t* k8, const float* ks, int ks_per_token,
                        const uint8_t* v8t, int64_t ldv, int Nq, int Nk, int D, float lambda, int causal,
                        int64_t pos_off, int i0, int i1, int t_lo, int t_hi, float* o_out, float* m_out,
                        float* d_out) {
  (void)Nq;
  e4m3_init();
  int ntile = (Nk + ORC_TILE - 1) / ORC_TILE;
  if (t_hi > ntile) t_hi = ntile;
  float* O = (float*)malloc(sizeof(float) * D);
  float* Pp = (float*)malloc(sizeof(float) * ORC_TILE);
  float* Sv = (float*)malloc(sizeof(float) * ORC_TILE);
  int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * ORC_TILE);
  uint8_t* P8 = (uint8_t*)malloc(ORC_TILE);
  float dec_tab[256];
  for (int c = 0; c < 256; ++c) dec_tab[c] = (float)orc_e4m3_decode((uint8_t)c);
  /* the decoded V values of the keys these tiles cover, token-major [key][c] (decoded once
   * per call rather than once per row: a table of exact values, no arithmetic) */
  int64_t j_lo = (int64_t)t_lo * ORC_TILE, j_hi = (int64_t)t_hi * ORC_TILE;
  if (j_hi > Nk) j_hi = Nk;
  if (j_lo > j_hi) j_lo = j_hi;
  float* vdec = (float*)malloc(sizeof(float) * (size_t)(j_hi - j_lo + 1) * D);
  for (int64_t j = j_lo; j < j_hi; ++j)
    for (int c = 0; c < D; ++c) vdec[(j - j_lo) * D + c] = dec_tab[v8t[(int64_t)c * ldv + j]];

  for (int i = i0; i < i1; ++i) {
    const int8_t* qrow = q8 + (int64_t)i * D;
    float sq = qs[i / ORC_TILE];
    float m = -INFINITY, d = 0.0f;
    for (int c = 0; c < D; ++c) O[c] = 0.0f;
    for (int t = t_lo; t < t_hi; ++t) {
      int j0 = t * ORC_TILE;
      /* skip tiles with no visible key for this row (a no-op for m, d and O) */
      int64_t last_vis = causal ? (int64_t)i + pos_off : (int64_t)Nk - 1;
      if (last_vis > Nk - 1) last_vis = Nk - 1;
      if ((int64_t)j0 > last_vis) break;
      /* QK: exact INT32 dot products; scores in the log2 domain */
      float mt = -INFINITY;
      for (int jj = 0; jj < ORC_TILE; ++jj) {
        int j = j0 + jj;
        if (j > last_vis) { Sv[jj] = -INFINITY; continue; }
        const int8_t* krow = k8 + (int64_t)j * D;
        int32_t a = 0;
        for (int c = 0; c < D; ++c) a += (int32_t)qrow[c] * (int32_t)krow[c];
        acc[jj] = a;
        float sk = ks_per_token ? ks[j] : ks[j / ORC_TILE];
        float cc = (sq * sk) * lambda;
        Sv[jj] = (float)a * cc;
        if (Sv[jj] > mt) mt = Sv[jj];
      }
      /* update m, d, O */
      float mnew = mt > m ? mt : m;
      float ms = (mnew == -INFINITY) ? 0.0f : mnew;
      float alpha = (mnew == m) ? 1.0f : orc_exp2(m - ms);
      d = alpha * d;
      for (int c = 0; c < D; ++c) O[c] = alpha * O[c];
      /* P' and accumulate d (fp32 P, before the 8-bit conversion) */
      float bconst = 88.0f - ms;
      for (int jj = 0; jj < ORC_TILE; ++jj) {
        if (Sv[jj] == -INFINITY) { Pp[jj] = 0.0f; continue; }
        int j = j0 + jj;
        float sk = ks_per_token ? ks[j] : ks[j / ORC_TILE];
        float cc = (sq * sk) * lambda;
        float u = fmaf((float)acc[jj], cc, bconst);
        Pp[jj] = orc_p_of_u(u);
      }
      for (int jj = 0; jj < ORC_TILE; ++jj) d = d + Pp[jj];
      /* convert P to 8 bit */
      for (int jj = 0; jj < ORC_TILE; ++jj) P8[jj] = orc_e4m3_encode(Pp[jj]);
      /* PV: products of two E4M3 values are exact in fp32 */
      for (int jj = 0; jj < ORC_TILE; ++jj) {
        if (Sv[jj] == -INFINITY) continue;
        float p = dec_tab[P8[jj]];
        if (p == 0.0f) continue; /* adds exact zeros */
        const float* vrow = vdec + ((int64_t)(j0 + jj) - j_lo) * D;
        for (int c = 0; c < D; ++c) O[c] = O[c] + p * vrow[c];
      }
      m = mnew;
    }
    float* o = o_out + (int64_t)(i - i0) * D;
    for (int c = 0; c < D; ++c) o[c] = O[c];
    m_out[i - i0] = m;
    d_out[i - i0] = d;
  }
  free(O); free(Pp); free(Sv); free(acc); free(P8); free(vdec);
}

/* All tiles, then the epilogue out_c = fl32(fl32(O_c * s_v[c]) / d'), 0 if d' = 0. */
void orc_attn_rows(const int8_t* q8, const float* qs, const int8_t* k8, const float* ks, int ks_per_token,
                   const uint8_t* v8t, int64_t ldv, const float* vs, int Nq, int Nk, int D, float lambda,
                   int causal, int64_t pos_off, int i0, int i1, float* out) {
  int n = i1 - i0;
  float* O = (float*)malloc(sizeof(float) * (size_t)n * D);
  float* mv = (float*)malloc(sizeof(float) * (size_t)n);
  float* dv = (float*)malloc(sizeof(float) * (size_t)n);
  orc_attn_rows_part(q8, qs, k8, ks, ks_per_token, v8t, ldv, Nq, Nk, D, lambda, causal, pos_off, i0, i1, 0,
                     (Nk + ORC_TILE - 1) / ORC_TILE, O, mv, dv);
  for (int r = 0; r < n; ++r)
    for (int c = 0; c < D; ++c)
      out[(int64_t)r * D + c] = (dv[r] == 0.0f) ? 0.0f : (O[(int64_t)r * D + c] * vs[c]) / dv[r];
  free(O); free(mv); free(dv);
}

/* Split-KV combine (the reading taken for splitting the key range of few-query prefill;
 * the pages' kernels run one pass): the key tiles [0, T) are cut into S contiguous
 * ranges [s T / S, (s + 1) T / S); each range runs the loop above from m = -inf,
 * d' = 0, O = 0 and leaves (O_s, m_s, d'_s).  Per row, in split order s = 0 .. S-1:
 *     M = max_s m_s                          (all -inf: the row outputs zeros)
 *     w_s = 2^(fl32(m_s - M)) correctly rounded (0 when m_s = -inf)
 *     d' = sum_s fl32(w_s * d'_s),  O_c = sum_s fl32(w_s * O_s,c)   (fp32, in order)
 *     out_c = fl32(fl32(O_c * s_v[c]) / d'), 0 if d' = 0.
 * o_part [S][n][D], m_part and d_part [S][n]; out [n][D]. */
void orc_combine_rows(int S, const float* o_part, const float* m_part, const float* d_part, const float* vs, int n,
                      int D, float* out) {
  for (int r = 0; r < n; ++r) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s)
      if (m_part[(int64_t)s * n + r] > M) M = m_part[(int64_t)s * n + r];
    float* o = out + (int64_t)r * D;
    if (M == -INFINITY) {
      for (int c = 0; c < D; ++c) o[c] = 0.0f;
      continue;
    }
    float d = 0.0f;
    for (int c = 0; c < D; ++c) o[c] = 0.0f;
    for (int s = 0; s < S; ++s) {
      float ms = m_part[(int64_t)s * n + r];
      float w = (ms == -INFINITY) ? 0.0f : orc_exp2(ms - M);
      d = d + w * d_part[(int64_t)s * n + r];
      const float* os = o_part + ((int64_t)s * n + r) * D;
      for (int c = 0; c < D; ++c) o[c] = o[c] + w * os[c];
    }
    for (int c = 0; c < D; ++c) o[c] = (d == 0.0f) ? 0.0f : (o[c] * vs[c]) / d;
  }
}

/* Default lambda for head dim D: fl32(fl32(1/sqrt(D)) * fl32(log2 e)). */
float orc_default_lambda(int D) {
  float inv = (float)(1.0 / sqrt((double)D));
  float log2e = (float)1.4426950408889634;
  return inv * log2e;
}

/* Number of grid arguments u in [lo_bits, hi_bits) (fp32 bit patterns) for which
 * P' = 2^(u - 80) rounds differently through double and through long double; used by
 * the tests to settle the rounding of orc_p_of_u over the whole grid domain. */
long orc_exp2_check_grid(uint32_t lo_bits, uint32_t hi_bits) {
  long bad = 0;
  for (uint32_t ub = lo_bits; ub < hi_bits; ++ub) {
    float u = f_of_bits(ub);
    float a = (float)exp2((double)u - 80.0);
    float b = (float)exp2l((long double)u - 80.0L);
    if (bits_of_f(a) != bits_of_f(b)) bad++;
  }
  return bad;
}

/* E4M3 codes of P' = 2^(u - 80) for all u with bit patterns in [lo_bits, hi_bits):
 * the P8 code the softmax produces for every grid argument. */
void orc_p8_codes_grid(uint32_t lo_bits, uint32_t hi_bits, uint8_t* codes) {
  for (uint32_t ub = lo_bits; ub < hi_bits; ++ub) codes[ub - lo_bits] = orc_e4m3_encode(orc_p_of_u(f_of_bits(ub)));
}

/* Array forms of the scalar codecs (for the tests). */
void orc_e4m3_encode_n(const float* x, long n, uint8_t* out) {
  for (long i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}
void orc_exp2_n(const float* x, long n, float* out) {
  for (long i = 0; i < n; ++i) out[i] = orc_exp2(x[i]);
}
