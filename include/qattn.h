/*
 * qattn.h -- C ABI of the quantized attention forward for MI355X (gfx950).
 *
 * The method: K smoothing, INT8 Q/K with per-block scales, FP8 e4m3 V with per-channel
 * scales, INT8 Q.K^T with INT32 accumulation, a tile-ordered online softmax whose P is
 * converted to FP8, and FP8 P.V with a fused V-scale epilogue ("H3 Performance Roadmap",
 * sections "Measured GB10 Baseline" and "Phase 4: Dense Sage-Compatible Attention";
 * "Sage2 SM89 Temporal Pair Experiment", section "Candidate").  Prefill over an INT8 KV
 * cache with per-token scales follows Strata #2092 (description).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  Nothing is allocated
 *     or freed by the library.  Shape and stride arrays are HOST pointers.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream) and returns before the GPU work completes.
 *   - Arguments are validated before any HIP call; on failure the call returns a negative
 *     qattn_status and launches nothing.  QATTN_EHIP reports a failed launch.
 *   - Strides are in elements; the innermost (D) stride is always 1.
 *   - D (head dimension) must be 64 or 128 (QATTN_EUNSUPPORTED otherwise).
 *   - bf16 inputs: base 16-byte aligned, strides multiples of 8 elements.
 *     Code buffers (q8, k8, v8t, vbf) and the workspace: 256-byte aligned.
 *     Scale buffers: 4-byte aligned.  Outputs: base and strides aligned to 4 elements.
 *   - N_pad = ceil(N / 64) * 64.  Code layouts are zero-padded to N_pad rows/columns.
 *   - Results are bitwise deterministic run to run (no atomics).
 *   - NaN/Inf inputs are outside the contract (their codes are unspecified).
 *   - Calls on different streams that share output buffers race.  Apart from the
 *     scratch array of qattn_fwd_i8kv_noalloc (shared by that call on each GPU; see
 *     there), the library holds no global mutable state, so calls are otherwise
 *     thread-safe.
 */
#ifndef QATTN_H
#define QATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QATTN_OK = 0,
  QATTN_EINVAL = -1,        /* null pointer, bad size, misalignment, bad stride, pos0 out of range */
  QATTN_EUNSUPPORTED = -2,  /* D not in {64, 128} */
  QATTN_EWORKSPACE = -3,    /* workspace smaller than qattn_fwd_i8kv_workspace_bytes() */
  QATTN_EHIP = -4,          /* a kernel launch failed */
  QATTN_ESCRATCH = -5       /* qattn_fwd_i8kv_noalloc: the call needs more than QATTN_NOALLOC_SCRATCH_BYTES */
} qattn_status;

typedef enum { QATTN_OUT_BF16 = 0, QATTN_OUT_F32 = 1 } qattn_out_dtype;

/* Step 1 -- K smoothing and INT8 Q/K quantization ("H3 Performance Roadmap", "Measured
 * GB10 Baseline": K smoothing and Q/K INT8 quantization rows; "Phase 4" items 2-3).
 *   q: bf16 [B, Nq, H, D] view with element strides q_str = {sb, sn, sh};
 *   k: bf16 [B, Nk, H, D] view with strides k_str.
 *   k_mean  f32 [B, H, D]: mu = fl32(fp64 sum over the Nk tokens / Nk);
 *   q8      int8 [B, H, Nq_pad, D], q_scale f32 [B, H, Nq_pad/64];
 *   k8      int8 [B, H, Nk_pad, D] of fl32(K - mu), k_scale f32 [B, H, Nk_pad/64].
 * Per (b, h) block of 64 rows: a = max|x|, scale = fl32(a/127), code =
 * clamp(rne(fl32(x * min(fl32(127/a), FLT_MAX))), -127, 127); a = 0 gives scale 0 and
 * zero codes; padding rows are zero.  k8 doubles as scratch for the fp64 partial sums
 * during the call (its final contents are the codes). */
int qattn_quant_qk(const void* q, const int64_t q_str[3], const void* k, const int64_t k_str[3], int B, int H,
                   int Nq, int Nk, int D, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, float* k_mean,
                   void* stream);

/* Step 2 -- V FP8 quantization with transpose ("H3 Performance Roadmap", "Measured GB10
 * Baseline": V transpose/FP8 quantization row; "Phase 4" item 2).
 *   v: bf16 [B, Nk, H, D] view with strides v_str.
 *   v8t     OCP e4m3fn bytes, channel-major [B, H, D, Nk_pad] (tokens >= Nk are 0x00);
 *   v_scale f32 [B, H, D].
 * Per (b, h, channel): a = max|v| over the Nk tokens, scale = fl32(a/448), code =
 * E4M3(fl32(v * min(fl32(448/a), FLT_MAX))) rounded to nearest even, saturated at 448,
 * sign kept; a = 0 gives scale 0 and 0x00 codes.  v8t and v_scale are used as scratch
 * during the call.
 *   vbf (optional, may be NULL): bf16 [B, H, D, Nk_pad] (256-byte aligned), the exact
 *   values of the v8t codes (every e4m3 value is a bf16 value; padding tokens 0) -- the
 *   form of V the fused loop reads. */
int qattn_quant_v(const void* v, const int64_t v_str[3], int B, int H, int Nk, int D, uint8_t* v8t,
                  float* v_scale, uint16_t* vbf, void* stream);

/* Steps 1-2 in one call ("H3 Performance Roadmap", "Phase 4" item 2: a single
 * preparation pass over the strided inputs in place of separate quantizer and layout
 * kernels): the outputs of qattn_quant_qk followed by qattn_quant_v, byte for byte, from
 * four launches instead of eight.  Q is read once; K and V twice (the channel mean and
 * the channel absmax need every token before any token is coded).  Arguments, layouts
 * and alignment are those of the two calls; either v8t or vbf (not both) may be NULL,
 * so a caller that runs qattn_fwd only needs vbf.  k8, and v8t (or vbf when v8t is
 * NULL), hold partial results during the call.  Returns QATTN_EINVAL /
 * QATTN_EUNSUPPORTED before any launch on a bad argument. */
int qattn_prep(const void* q, const int64_t q_str[3], const void* k, const int64_t k_str[3], const void* v,
               const int64_t v_str[3], int B, int H, int Nq, int Nk, int D, int8_t* q8, float* q_scale, int8_t* k8,
               float* k_scale, float* k_mean, uint8_t* v8t, float* v_scale, uint16_t* vbf, void* stream);

/* Steps 3-5 -- fused INT8 QK, online softmax with FP8 P, PV and epilogue ("Sage2 SM89
 * Temporal Pair Experiment", "Candidate": per 64-key tile QK -> update m, d, O ->
 * accumulate d -> P to 8 bit -> PV), on the outputs of steps 1-2 (same layouts).
 * PV sums the exact products of the e4m3 values of P and V in fp32 (no truncation of
 * small products).  V enters as vbf, the bf16 values of the step-2 codes (qattn_quant_v's
 * vbf output), so the loop reads V tiles that its matrix instructions take as they are.
 *   scale_log2: softmax scale times log2(e); <= 0 selects fl32(fl32(1/sqrt(D)) * log2e).
 *   causal: key j visible to query i iff j <= i + (Nk - Nq) (bottom-right aligned); a
 *           query with no visible key outputs zeros.
 *   out: [B, Nq, H, D] view with strides out_str, dtype out_dtype (token-major NHD).
 * Output = fl32(O * s_v / d') with fp32 accumulation; bf16 output is its RNE rounding.
 * Score domain: every finite input whose log2-domain scores S = acc * c stay below 2^28
 * in magnitude, including the P codes that saturate at 448 once |S| reaches about 2^22
 * (the oracle's encoder saturates the same way).  Beyond 2^28 the fp32 sum d' itself may
 * overflow (the method's arithmetic, not this kernel's): outside the contract. */
int qattn_fwd(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale, const uint16_t* vbf,
              const float* v_scale, int B, int H, int Nq, int Nk, int D, float scale_log2, int causal, void* out,
              const int64_t out_str[3], int out_dtype, void* stream);

/* Prefill over an INT8 KV cache with per-token scales (Strata #2092, description and
 * the "qsa_prompt_attn_parity (int8 KV)" table); the loop is the one of qattn_fwd, with
 * the same score domain.
 *   q: bf16 [Nq, H, D] view with strides q_str = {sn, sh}; query i sits at absolute
 *      position pos0 + i and sees keys 0 .. pos0 + i (0 <= pos0, pos0 + Nq <= Nk).
 *   k_cache, v_cache: int8 [H, Nk, D] contiguous; k_tok_scale, v_tok_scale: f32 [H, Nk]
 *      (one scale per head and token: value = code * scale).
 *   workspace: >= qattn_fwd_i8kv_workspace_bytes(H, Nq, Nk, D, kv_splits) bytes (kv_splits
 *      resolved), 256-byte aligned;
 *      receives the per-channel e4m3 requantization of V (fl32(code * scale) quantized
 *      as in step 2 over all Nk tokens), held as the bf16 values of its codes, and the
 *      INT8 blocks of q (as in step 1, no smoothing).  Sections, each starting on a
 *      256-byte boundary: V scales f32 [H, D]; q codes int8 [H, Nq_pad, D]; q scales f32
 *      [H, Nq_pad / 64]; V values bf16 [H, D, Nk_pad]; for kv_splits > 1 the partial O
 *      f32 [S, H, Nq_pad, D] and (m, d') f32 [S, H, Nq_pad, 2].
 *   kv_splits: split-KV for few queries over a long context.  The key tiles
 *      [0, T), T = ceil(min(Nk, pos0 + Nq) / 64), are cut into kv_splits contiguous ranges
 *      [s T / S, (s + 1) T / S); each range runs the loop above on its own (from
 *      m = -inf, d' = 0, O = 0) and a second kernel combines the ranges of every row in
 *      range order: M = max m_s, w_s = 2^(m_s - M), out = (sum w_s O_s) * s_v /
 *      (sum w_s d'_s).  1 = one pass; 0 = the count qattn_fwd_i8kv_kv_splits returns;
 *      at most 64.
 *   out: [Nq, H, D] view with strides out_str = {sn, sh}.
 * K codes are used as stored, with c_j = fl32(fl32(s_q * s_k[j]) * scale_log2). */
int qattn_fwd_i8kv(const void* q, const int64_t q_str[2], const int8_t* k_cache, const float* k_tok_scale,
                   const int8_t* v_cache, const float* v_tok_scale, int H, int Nq, int Nk, int D, int pos0,
                   float scale_log2, int kv_splits, void* workspace, size_t workspace_bytes, void* out,
                   const int64_t out_str[2], int out_dtype, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, hosts that forbid hipMalloc): qattn_fwd_i8kv with the same arguments
 * minus the workspace, which lives instead in a device array of the library holding
 * QATTN_NOALLOC_SCRATCH_BYTES bytes on each GPU it runs on (kept until the process ends).
 * The call allocates nothing.  Returns QATTN_ESCRATCH, before any launch, when the call
 * would need a larger workspace than that (qattn_fwd_i8kv_workspace_bytes with the
 * resolved kv_splits), e.g. 32 heads of D = 128 and 512 or 1,024 queries over 28K or
 * more cached tokens;
 * every other argument is checked as by qattn_fwd_i8kv.  All calls on one GPU share its
 * array: calls that overlap on one GPU (other streams, other threads) race and give
 * undefined results.  A call leaves its intermediates in the array; nothing needs to be
 * cleared between calls. */
#define QATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int qattn_fwd_i8kv_noalloc(const void* q, const int64_t q_str[2], const int8_t* k_cache, const float* k_tok_scale,
                           const int8_t* v_cache, const float* v_tok_scale, int H, int Nq, int Nk, int D, int pos0,
                           float scale_log2, int kv_splits, void* out, const int64_t out_str[2], int out_dtype,
                           void* stream);

/* Workspace size in bytes for qattn_fwd_i8kv(H, Nq, Nk, D, ..., kv_splits, ...) with
 * kv_splits key ranges (1 .. 64; resolve 0 with qattn_fwd_i8kv_kv_splits first):
 * H*D*4 (V scales) + H*Nq_pad*D (q codes) +
 * H*Nq_pad/64*4 (q scales) + H*D*Nk_pad*2 (bf16 values of the V codes), and for
 * kv_splits > 1 the partial results
 * kv_splits*H*Nq_pad*D*4 (O) + kv_splits*H*Nq_pad*8 (m, d'), each section rounded up to
 * 256 bytes.  Returns 0 for invalid sizes. */
size_t qattn_fwd_i8kv_workspace_bytes(int H, int Nq, int Nk, int D, int kv_splits);

/* The key-range count qattn_fwd_i8kv uses for kv_splits = 0 (host only, no GPU call):
 * ceil(256 / (H * ceil(Nq / 256))) -- one workgroup per CU -- capped so that every
 * range holds at least 16 key tiles and at 64, at least 1.  Returns 0 for invalid sizes
 * (0 <= pos0, pos0 + Nq <= Nk). */
int qattn_fwd_i8kv_kv_splits(int H, int Nq, int Nk, int pos0);

/* Appends tokens to an INT8 KV cache with per-token scales, the layout qattn_fwd_i8kv
 * reads (Strata #2092 runs its prompt attention on such a cache; the quantizer that
 * fills it is not stated there, and the one taken is step 1's INT8 quantizer with a
 * block of one (token, head) row).
 *   x: bf16 [Nnew, H, D] view with strides x_str = {sn, sh} (16-byte aligned, strides
 *      multiples of 8 elements), e.g. one projection of a packed [N, 3, H, D] tensor;
 *   cache: int8 [H, Nmax, D] contiguous (8-byte aligned); tok_scale: f32 [H, Nmax].
 * Token n of x goes to row pos + n of every head: a = max |x| over its D channels,
 * tok_scale = fl32(a / 127), code = clamp(rne(fl32(x * min(fl32(127 / a), FLT_MAX))),
 * -127, 127); a = 0 gives scale 0 and zero codes.  Other rows are not touched.
 * 0 <= pos, pos + Nnew <= Nmax.  Call once for K and once for V. */
int qattn_kv_append_i8(const void* x, const int64_t x_str[2], int Nnew, int H, int D, int8_t* cache,
                       float* tok_scale, int Nmax, int pos, void* stream);

/* Static description of a status code. */
const char* qattn_status_string(int status);

/* ---- Self-test hook: not part of the attention interface ---------------------------
 * codes[i] = the FP8 code of P' = 2^(u[i] - 80) as the fused kernel's softmax forms it
 * for the exponent argument u[i] (the kernel's own device functions: the hardware
 * exponential of u, then the FP8 conversion with the exact 2^80 scale), so that a test
 * can compare it with the correctly rounded, saturating E4M3 of 2^(u - 80) over every
 * argument the softmax can produce.
 *   saturating = 0: the ordinary form, used while every row of a wave has |m| < 2^22
 *     (m = running maximum of the log2-domain scores).  There u <= 88.375 + 2^-17.  The
 *     conversion itself does not saturate: u >= 88.86 (a power of 464 or more) would give
 *     the NaN code 0x7F.
 *   saturating = 1: the large-score form (some row with |m| >= 2^22), where u is
 *     unbounded above: the conversion input is clamped to 448 * 2^80, so every u above
 *     88.81 (and an infinite power) gives 0x7E.
 * u: f32 [n], codes: u8 [n], device pointers; n > 0. */
int qattn_selftest_p8_codes(const float* u, uint8_t* codes, int64_t n, int saturating, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QATTN_H */
