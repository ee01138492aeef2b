// Internal device helpers and launcher declarations for libqattn (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qattn {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBlk = 64;  // rows per Q/K scale block, keys per KV tile
constexpr float kFltMax = 3.40282346638528859812e+38f;
// Word 3 of a raw (stride 0) buffer resource on gfx9-family GPUs: 32-bit data format,
// bounds checked against num_records (out-of-range loads return zero).
constexpr int kRsrcWord3 = 0x00020000;

// A wave-uniform pointer moved to scalar registers (both halves via readfirstlane), so
// buffer resources built from it need no per-lane waterfall.
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Unpack 8 bf16 values held in a 16-byte vector into fp32 (exact).
__device__ __forceinline__ void unpack_bf16x8(const v4i& w, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo((uint32_t)w[i]);
    f[2 * i + 1] = bf16_hi((uint32_t)w[i]);
  }
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Workgroup id -> work item so that each of the 8 XCDs (workgroups are dealt to XCDs
// round-robin by id) receives one contiguous range of work items.  Neighbouring work
// items share K/V, so the K/V tiles they stream stay in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  constexpr int X = 8;
  const int x = id % X, slot = id / X;
  const int q = n / X, r = n % X;
  return x * q + (x < r ? x : r) + slot;
}

// ---------------------------------------------------------------------------------
// launchers (defined in quant.hip / attn_fwd.hip); all asynchronous on `st`
// ---------------------------------------------------------------------------------
struct BshdView {
  const void* p;
  int64_t sb, sn, sh;  // element strides; d stride is 1
};

hipError_t launch_k_mean(BshdView k, int B, int H, int N, int D, int npad, int8_t* scratch, float* mean,
                         hipStream_t st);
hipError_t launch_quant_i8(BshdView x, const float* mean, int B, int H, int N, int D, int npad, int8_t* codes,
                           float* scales, hipStream_t st);
// V: bf16 view (cache == nullptr) or int8 cache [H, N, D] with per-token scales (B must be 1)
hipError_t launch_quant_v(BshdView v, const int8_t* cache, const float* tok_scale, int B, int H, int N, int D,
                          int npad, uint8_t* v8t, float* v_scale, uint16_t* vbf, hipStream_t st);

// Fused preparation (pass 1, final, pass 2, scale).  Dense form: q, k, v bf16 views with
// k8 != nullptr; prefill form: q view (b = 0) and the int8 V cache with per-token scales,
// k8 == nullptr.  v8t or vbf may be null (not both).  Partial results live in the k8 and
// v8t (else vbf) regions until pass 2 writes them.
struct PrepArgs {
  BshdView q, k, v;
  int B, H, Nq, Nk;
  int8_t* q8;
  float* q_scale;
  int8_t* k8;
  float* k_scale;
  float* k_mean;
  const int8_t* v_cache;
  const float* v_tok_scale;
  uint8_t* v8t;
  float* v_scale;
  uint16_t* vbf;
};
hipError_t launch_prep(const PrepArgs& p, int D, hipStream_t st);

struct FwdArgs {
  const int8_t* q8;
  const float* q_scale;
  const int8_t* k8;
  const float* k_scale;
  const uint16_t* vbf;  // bf16 values of the V^T e4m3 codes [B*H][D][ldv]
  const float* v_scale;
  void* out;
  int64_t q8_bh, qs_bh, k8_bh, ks_bh, vbf_bh, ldv;  // per-(b,h) element strides
  int64_t out_sb, out_sn, out_sh;
  int B, H, Nq, Nk, nq_pad, k_rows;
  float lambda;
  int64_t pos_off;  // causal: key j visible to query i iff j <= i + pos_off
  int causal, per_token, out_bf16;
  // Split-KV: the key tiles [0, tiles_total) are cut into kv_splits contiguous ranges
  // [s T / S, (s + 1) T / S); with kv_splits > 1 each (b, h, query block, range) writes
  // its unnormalized O and (m, d') to part_o / part_md and the combine kernel forms the
  // output.  kv_splits = 1: one pass over all tiles, output written directly.
  int kv_splits, tiles_total;
  float* part_o;   // [kv_splits][B*H][nq_pad][D]
  float* part_md;  // [kv_splits][B*H][nq_pad][2]: m (log2 domain, -inf if none), d'
};
hipError_t launch_kv_append_i8(const void* x, int64_t sn, int64_t sh, int Nnew, int H, int D, int8_t* cache,
                               float* tok_scale, int Nmax, int pos, hipStream_t st);
hipError_t launch_attn_fwd(const FwdArgs& a, int D, hipStream_t st);  // both kernels when split
hipError_t launch_p8_codes(const float* u, uint8_t* codes, int64_t n, int saturating, hipStream_t st);

// The prefill call (qattn_fwd_i8kv) in two parts: validation of everything but the
// workspace (resolves *kv_splits, returns the workspace size in *need; no HIP call), and
// the launches into a workspace of at least that size, 256-byte aligned.  Both return a
// qattn_status.
int i8kv_check(const void* q, const int64_t q_str[2], const int8_t* k_cache, const float* k_tok_scale,
               const int8_t* v_cache, const float* v_tok_scale, int H, int Nq, int Nk, int D, int pos0,
               float scale_log2, int* kv_splits, const void* out, const int64_t out_str[2], int out_dtype,
               size_t* need);
int i8kv_launch(const void* q, const int64_t q_str[2], const int8_t* k_cache, const float* k_tok_scale,
                const int8_t* v_cache, const float* v_tok_scale, int H, int Nq, int Nk, int D, int pos0,
                float scale_log2, int kv_splits, void* workspace, void* out, const int64_t out_str[2],
                int out_dtype, void* stream);

}  // namespace qattn
