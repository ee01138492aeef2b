// Preparation kernels: K channel mean, INT8 per-64-row blocks of Q and smoothed K, and
// per-channel e4m3 V written channel-major ("H3 Performance Roadmap", "Measured GB10
// Baseline": K smoothing, Q/K INT8 quantization, V transpose + FP8 quantization;
// "Phase 4" items 2-3).  All of them stream their input once or twice from HBM; each
// thread moves 16-byte vectors, workgroups cover 64-row blocks or 256-token chunks.
#include "common.h"

namespace qattn {
namespace detail {

constexpr int kThreads = 256;
constexpr int kChunk = 256;  // tokens per partial-reduction workgroup

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------------
// a1: K channel mean.  Pass 1 sums each 256-token chunk in fp64 (the sum of bf16 values
// is exact in fp64 for these magnitudes, so the order is immaterial) into scratch that
// lives in the k8 region of the same (b, h); pass 2 adds the chunks and divides once.
// ---------------------------------------------------------------------------------
template <int D>
struct KSumLds {
  double red[kThreads / (D / 8)][D];
};
template <int D>
__device__ __forceinline__ void k_mean_partial_body(BshdView k, int H, int N, int64_t region, int8_t* scratch, int chunk,
                                                    int h, int b, KSumLds<D>& lds) {
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int RPP = kThreads / CPR;  // rows per pass
  auto& red = lds.red;
  const int t = threadIdx.x, cg = t % CPR, rl = t / CPR;
  const int n0 = chunk * kChunk, n1 = min(N, n0 + kChunk);
  const uint16_t* base = (const uint16_t*)k.p + b * k.sb + h * k.sh + cg * 8;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  // unrolled so that several rows' loads are in flight at once (the additions into each
  // acc[i] stay in token order)
#pragma unroll 4
  for (int n = n0 + rl; n < n1; n += RPP) {
    v4i w = *(const v4i*)(base + (int64_t)n * k.sn);
    float f[8];
    unpack_bf16x8(w, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += (double)f[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rl][cg * 8 + i] = acc[i];
  __syncthreads();
  if (t < D) {
    double s = 0.0;
    for (int r = 0; r < RPP; ++r) s += red[r][t];
    double* part = (double*)(scratch + (int64_t)(b * H + h) * region);
    part[chunk * D + t] = s;
  }
}
template <int D>
__global__ __launch_bounds__(kThreads) void k_mean_partial(BshdView k, int H, int N, int64_t region, int8_t* scratch) {
  __shared__ KSumLds<D> lds;
  k_mean_partial_body<D>(k, H, N, region, scratch, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// The final reductions run kFinalThreads threads per (b, h): kFinalThreads / D per
// channel.  Thread j of channel c folds chunks j, j + J, j + 2 J, ... in that order, then
// the J partial results are folded in j order through LDS: a fixed order, shared by the
// separate and the fused preparation.
constexpr int kFinalThreads = 1024;
template <int D>
__device__ __forceinline__ void k_mean_of_chunks(const double* part, int nchunk, int N, double* red, float* mean) {
  constexpr int J = kFinalThreads / D;
  const int c = threadIdx.x % D, j = threadIdx.x / D;
  double s = 0.0;
#pragma unroll 4
  for (int i = j; i < nchunk; i += J) s += part[i * D + c];
  red[threadIdx.x] = s;
  __syncthreads();
  if (j == 0) {
    double t = red[c];
#pragma unroll
    for (int r = 1; r < J; ++r) t += red[r * D + c];
    mean[c] = (float)(t / (double)N);
  }
}
template <int D>
__global__ __launch_bounds__(kFinalThreads) void k_mean_final(int N, int nchunk, int64_t region, const int8_t* scratch,
                                                              float* mean) {
  __shared__ double red[kFinalThreads];
  const int bh = blockIdx.x;
  k_mean_of_chunks<D>((const double*)(scratch + (int64_t)bh * region), nchunk, N, red, mean + (int64_t)bh * D);
}

// ---------------------------------------------------------------------------------
// a2: INT8 blocks of 64 rows: a = max|x|, s = a/127, code = rne(x * min(127/a, FLT_MAX)).
// One workgroup per (block, h, b); each thread keeps its 8-channel slices in registers.
// ---------------------------------------------------------------------------------
// wmax: kThreads / 64 floats of LDS, not reused by the workgroup until a barrier has
// followed this call
template <int D, bool SMOOTH>
__device__ __forceinline__ void quant_i8_block_body(BshdView x, const float* mean, int H, int N, int npad,
                                                    int8_t* codes, float* scales, int blk, int h, int b,
                                                    float* wmax) {
  constexpr int CPR = D / 8, RPP = kThreads / CPR, PASSES = kBlk / RPP;
  const int t = threadIdx.x, cg = t % CPR, rl = t / CPR;
  const int r0 = blk * kBlk;
  const int64_t bh = (int64_t)b * H + h;
  const uint16_t* base = (const uint16_t*)x.p + b * x.sb + h * x.sh + cg * 8;
  float mu[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mu[i] = SMOOTH ? mean[bh * D + cg * 8 + i] : 0.0f;
  float v[PASSES][8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int n = r0 + rl + p * RPP;
    if (n < N) {
      v4i w = *(const v4i*)(base + (int64_t)n * x.sn);
      float f[8];
      unpack_bf16x8(w, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[p][i] = SMOOTH ? f[i] - mu[i] : f[i];
        amax = fmaxf(amax, fabsf(v[p][i]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[p][i] = 0.0f;
    }
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  float a = wmax[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) a = fmaxf(a, wmax[w]);
  float s = 0.0f, r = 0.0f;
  if (a > 0.0f) {
    s = a / 127.0f;
    r = fminf(127.0f / a, kFltMax);
  }
  if (t == 0) scales[bh * (npad / kBlk) + blk] = s;
  int8_t* out = codes + (bh * npad + r0) * D + cg * 8;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    uint32_t wd[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = __builtin_rintf(v[p][i] * r);
      q = fminf(fmaxf(q, -127.0f), 127.0f);
      wd[i >> 2] |= ((uint32_t)(int)q & 0xffu) << (8 * (i & 3));
    }
    *(uint2*)(out + (int64_t)(rl + p * RPP) * D) = make_uint2(wd[0], wd[1]);
  }
}
template <int D, bool SMOOTH>
__global__ __launch_bounds__(kThreads) void quant_i8_blocks(BshdView x, const float* mean, int H, int N, int npad,
                                                            int8_t* codes, float* scales) {
  __shared__ float wmax[kThreads / 64];
  quant_i8_block_body<D, SMOOTH>(x, mean, H, N, npad, codes, scales, blockIdx.x, blockIdx.y, blockIdx.z, wmax);
}

// ---------------------------------------------------------------------------------
// a3: per-channel e4m3 V.  Pass 1: per-chunk channel absmax into scratch inside v8t;
// pass 2: the channel absmax is parked in v_scale; pass 3: encode 64-token tiles and
// write them channel-major (each lane codes eight tokens of its channels, so no transpose
// buffer is needed); pass 4: v_scale = absmax / 448.
// The input is either a bf16 view or an int8 cache with per-token scales, dequantized
// as fl32(code * scale).
// ---------------------------------------------------------------------------------
// Channels per lane of the V passes: every lane moves 16 bytes per row, i.e. 8 bf16
// channels or 16 int8 cache channels.
template <bool CACHE>
constexpr int v_ch() { return CACHE ? 16 : 8; }

// Row n of V for channel group cg as raw words: 16 bytes, and (cache) the token's scale;
// padding rows (n >= N) read as zeros.  value_of decodes channel i: fl32(code * scale)
// for a cache, the bf16 value otherwise.
template <int D, bool CACHE>
__device__ __forceinline__ void load_v_raw(BshdView v, const int8_t* cache, const float* tok_scale, int b, int h,
                                           int N, int n, int cg, v4i& raw, float& sc) {
  raw = v4i{0, 0, 0, 0};
  sc = 0.0f;
  if (n < N) {
    if constexpr (CACHE) {
      raw = *(const v4i*)(cache + ((int64_t)h * N + n) * D + cg * 16);
      sc = tok_scale[(int64_t)h * N + n];
    } else {
      raw = *(const v4i*)((const uint16_t*)v.p + b * v.sb + (int64_t)n * v.sn + h * v.sh + cg * 8);
    }
  }
}
template <bool CACHE>
__device__ __forceinline__ float value_of(const v4i& raw, float sc, int i) {
  if constexpr (CACHE) {
    return (float)(int8_t)(raw[i >> 2] >> (8 * (i & 3))) * sc;  // fl32(code * scale)
  } else {
    const uint32_t w = (uint32_t)raw[i >> 1];
    return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
}

template <int D, bool CACHE>
struct VMaxLds {
  float red[kThreads / (D / v_ch<CACHE>())][D];
};
template <int D, bool CACHE>
__device__ __forceinline__ void v_amax_partial_body(BshdView v, const int8_t* cache, const float* tok_scale, int H,
                                                    int N, int64_t region, uint8_t* scratch, int chunk, int h, int b,
                                                    VMaxLds<D, CACHE>& lds) {
  constexpr int CH = v_ch<CACHE>(), CPR = D / CH, RPP = kThreads / CPR;
  auto& red = lds.red;
  const int t = threadIdx.x, cg = t % CPR, rl = t / CPR;
  const int n0 = chunk * kChunk, n1 = min(N, n0 + kChunk);
  float mx[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) mx[i] = 0.0f;
  // unrolled so that several rows' loads are in flight at once
#pragma unroll 4
  for (int n = n0 + rl; n < n1; n += RPP) {
    v4i raw;
    float sc;
    load_v_raw<D, CACHE>(v, cache, tok_scale, b, h, N, n, cg, raw, sc);
#pragma unroll
    for (int i = 0; i < CH; ++i) mx[i] = fmaxf(mx[i], fabsf(value_of<CACHE>(raw, sc, i)));
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) red[rl][cg * CH + i] = mx[i];
  __syncthreads();
  if (t < D) {
    float m = 0.0f;
    for (int r = 0; r < RPP; ++r) m = fmaxf(m, red[r][t]);
    float* part = (float*)(scratch + ((int64_t)b * H + h) * region);
    part[chunk * D + t] = m;
  }
}
template <int D, bool CACHE>
__global__ __launch_bounds__(kThreads) void v_amax_partial(BshdView v, const int8_t* cache, const float* tok_scale,
                                                           int H, int N, int64_t region, uint8_t* scratch) {
  __shared__ VMaxLds<D, CACHE> lds;
  v_amax_partial_body<D, CACHE>(v, cache, tok_scale, H, N, region, scratch, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

template <int D>
__device__ __forceinline__ void v_amax_of_chunks(const float* part, int nchunk, float* red, float* amax) {
  constexpr int J = kFinalThreads / D;
  const int c = threadIdx.x % D, j = threadIdx.x / D;
  float m = 0.0f;
#pragma unroll 4
  for (int i = j; i < nchunk; i += J) m = fmaxf(m, part[i * D + c]);
  red[threadIdx.x] = m;
  __syncthreads();
  if (j == 0) {
    float t = red[c];
#pragma unroll
    for (int r = 1; r < J; ++r) t = fmaxf(t, red[r * D + c]);
    amax[c] = t;
  }
}
template <int D>
__global__ __launch_bounds__(kFinalThreads) void v_amax_final(int nchunk, int64_t region, const uint8_t* scratch,
                                                              float* v_scale) {
  __shared__ float red[kFinalThreads];
  const int bh = blockIdx.x;
  // the absmax; converted to the scale after encoding
  v_amax_of_chunks<D>((const float*)(scratch + (int64_t)bh * region), nchunk, red, v_scale + (int64_t)bh * D);
}

// Encode of one 64-token tile, channel-major, without a transpose buffer: lane L of the
// tile owns tokens 8 o .. 8 o + 7 (o = L % 8) of the channel group g = L / 8 (CH
// channels).  It loads its 8 rows, then forms each channel's codes four tokens to a word
// (the e4m3 conversion takes any two values: tokens t, t + 1 into the low half of the
// word, t + 2, t + 3 into the high half), so the codes come out in the order they are
// stored.  Eight lanes of a group store 64 contiguous bytes of codes and 128 of bf16
// values per channel.  Lanes L >= kEncLanes do nothing.
template <int D, bool CACHE>
constexpr int enc_lanes() { return 8 * (D / v_ch<CACHE>()); }

template <int D, bool CACHE>
__device__ __forceinline__ void v_encode_tile(BshdView v, const int8_t* cache, const float* tok_scale, int H, int N,
                                              int npad, const float* v_amax, uint8_t* v8t, uint16_t* vbf, int tile,
                                              int h, int b, int L) {
  constexpr int CH = v_ch<CACHE>();
  if (L >= enc_lanes<D, CACHE>()) return;
  const int o = L & 7, g = L >> 3;
  const int64_t bh = (int64_t)b * H + h;
  const int n0 = tile * kBlk + 8 * o;  // this lane's first token
  float rc[CH];
  bool zc[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const float a = v_amax[bh * D + g * CH + i];
    zc[i] = !(a > 0.0f);
    rc[i] = zc[i] ? 0.0f : fminf(448.0f / a, kFltMax);
  }
  // all eight rows' loads first (raw 16-byte words, and the token scales of a cache),
  // then each channel decoded from them: every load is in flight at once
  v4i raw[8];
  float sc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) load_v_raw<D, CACHE>(v, cache, tok_scale, b, h, N, n0 + r, g, raw[r], sc[r]);
  auto value = [&](int r, int i) { return value_of<CACHE>(raw[r], sc[r], i); };
  uint32_t cw[2][CH];  // [token quad][channel]: the codes of four tokens of one channel
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      // hardware e4m3 conversion: round to nearest even; |f * r| <= 448 (1 + 2^-23)
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(value(4 * hq, i) * rc[i], value(4 * hq + 1, i) * rc[i], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(value(4 * hq + 2, i) * rc[i], value(4 * hq + 3, i) * rc[i], w, true);
      cw[hq][i] = zc[i] ? 0u : (uint32_t)w;  // a zero channel codes as 0x00 (also for -0)
    }
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t row = (bh * D + g * CH + i) * npad + tile * kBlk + 8 * o;
    if (v8t) *(uint2*)(v8t + row) = make_uint2(cw[0][i], cw[1][i]);
    if (vbf) {  // the exact bf16 values of the 8 codes (every e4m3 value is a bf16 value)
      uint32_t bw[4];
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        bw[2 * hq] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hq][i], 1.0f, false));
        bw[2 * hq + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[hq][i], 1.0f, true));
      }
      *(v4i*)(vbf + row) = v4i{(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3]};
    }
  }
}
// Tiles per 256-thread workgroup of the standalone encode launches.
template <int D, bool CACHE>
constexpr int enc_tiles_per_wg() { return kThreads / enc_lanes<D, CACHE>(); }

template <int D, bool CACHE>
__global__ __launch_bounds__(kThreads) void v_encode(BshdView v, const int8_t* cache, const float* tok_scale, int H,
                                                     int N, int npad, const float* v_amax, uint8_t* v8t, uint16_t* vbf) {
  constexpr int TPW = enc_tiles_per_wg<D, CACHE>(), EL = enc_lanes<D, CACHE>();
  const int t = threadIdx.x, tile = blockIdx.x * TPW + t / EL;
  if (tile < npad / kBlk)
    v_encode_tile<D, CACHE>(v, cache, tok_scale, H, N, npad, v_amax, v8t, vbf, tile, blockIdx.y, blockIdx.z, t % EL);
}

__global__ void v_scale_from_amax(float* v_scale, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) v_scale[i] = v_scale[i] / 448.0f;
}

__host__ __device__ inline int nchunks(int N) { return (N + kChunk - 1) / kChunk; }

// ---------------------------------------------------------------------------------
// Fused preparation ("Phase 4" item 2: one preparation pass over the strided inputs
// instead of separate quantizer and layout kernels): the steps above in four launches.
//   pass 1 - per 256-token chunk of one (b, h): the INT8 blocks of Q (the chunk's four
//            64-row blocks), the fp64 partial sums of K and the partial absmax of V;
//   final  - per (b, h): the K channel mean and the V channel absmax (parked in v_scale);
//   pass 2 - per 64-token tile: the INT8 blocks of K - mean, and the e4m3 V tile written
//            channel-major with its bf16 values;
//   scale  - v_scale = absmax / 448.
// Q is read once, K and V twice: a channel's statistics need all of its tokens before
// any of them is coded.  Every value is computed by the same device code as the
// separate kernels, in the same order, so the two paths give identical bytes.
// ---------------------------------------------------------------------------------
template <int D, bool HAS_K, bool CACHE>
__global__ __launch_bounds__(kThreads) void prep_pass1(BshdView q, int Nq, int nqpad, int8_t* q8, float* q_scale,
                                                       BshdView k, BshdView v, const int8_t* v_cache,
                                                       const float* v_tok_scale, int H, int Nk, int64_t region,
                                                       int8_t* k_part, int64_t v_region, uint8_t* v_part) {
  constexpr int QB = kChunk / kBlk;  // Q blocks per chunk
  __shared__ float wmax[QB][kThreads / 64];
  __shared__ KSumLds<D> klds;
  __shared__ VMaxLds<D, CACHE> vlds;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (q8) {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int blk = chunk * QB + j;  // uniform over the workgroup: the barrier inside is safe
      if (blk < nqpad / kBlk) quant_i8_block_body<D, false>(q, nullptr, H, Nq, nqpad, q8, q_scale, blk, h, b, wmax[j]);
    }
  }
  if (chunk < nchunks(Nk)) {
    if (HAS_K) k_mean_partial_body<D>(k, H, Nk, region, k_part, chunk, h, b, klds);
    v_amax_partial_body<D, CACHE>(v, v_cache, v_tok_scale, H, Nk, v_region, v_part, chunk, h, b, vlds);
  }
}

template <int D, bool HAS_K>
__global__ __launch_bounds__(kFinalThreads) void prep_final(int Nk, int nchunk, int64_t region, const int8_t* k_part,
                                                            float* k_mean, int64_t v_region, const uint8_t* v_part,
                                                            float* v_amax) {
  __shared__ double kred[kFinalThreads];
  __shared__ float vred[kFinalThreads];
  const int bh = blockIdx.x;
  if (HAS_K) k_mean_of_chunks<D>((const double*)(k_part + bh * region), nchunk, Nk, kred, k_mean + (int64_t)bh * D);
  v_amax_of_chunks<D>((const float*)(v_part + bh * v_region), nchunk, vred, v_amax + (int64_t)bh * D);
}

// pass 2: blocks [0, nkt) of the dense form code one K block each (all 256 threads);
// the blocks after them encode enc_tiles_per_wg V tiles each
template <int D, bool HAS_K, bool CACHE>
__global__ __launch_bounds__(kThreads) void prep_pass2(BshdView k, const float* k_mean, int8_t* k8, float* k_scale,
                                                       BshdView v, const int8_t* v_cache, const float* v_tok_scale,
                                                       const float* v_amax, uint8_t* v8t, uint16_t* vbf, int H,
                                                       int Nk, int nkpad) {
  constexpr int TPW = enc_tiles_per_wg<D, CACHE>(), EL = enc_lanes<D, CACHE>();
  __shared__ float wmax[kThreads / 64];
  const int t = threadIdx.x, h = blockIdx.y, b = blockIdx.z, nkt = nkpad / kBlk;
  int vb = blockIdx.x;
  if (HAS_K) {
    if (vb < nkt) {  // uniform over the workgroup: the barrier inside is safe
      quant_i8_block_body<D, true>(k, k_mean, H, Nk, nkpad, k8, k_scale, vb, h, b, wmax);
      return;
    }
    vb -= nkt;
  }
  const int tile = vb * TPW + t / EL;
  if (tile < nkt) v_encode_tile<D, CACHE>(v, v_cache, v_tok_scale, H, Nk, nkpad, v_amax, v8t, vbf, tile, h, b, t % EL);
}

template <int D, bool HAS_K, bool CACHE>
static void prep_impl(const PrepArgs& p, hipStream_t st) {
  const int nqp = p.q8 ? (p.Nq + kBlk - 1) / kBlk * kBlk : 0;
  const int nkp = (p.Nk + kBlk - 1) / kBlk * kBlk;
  // partial results live in the output buffers of pass 2 (per (b, h): k8 holds nkp * D
  // bytes; v8t nkp * D, or vbf 2 * nkp * D where there is no v8t)
  const int64_t region = (int64_t)nkp * D;
  const int64_t v_region = p.v8t ? region : 2 * region;
  uint8_t* v_part = p.v8t ? p.v8t : (uint8_t*)p.vbf;
  const int nck = nchunks(p.Nk), ncq = p.q8 ? nchunks(p.Nq) : 0;
  prep_pass1<D, HAS_K, CACHE><<<dim3(max(nck, ncq), p.H, p.B), kThreads, 0, st>>>(
      p.q, p.Nq, nqp, p.q8, p.q_scale, p.k, p.v, p.v_cache, p.v_tok_scale, p.H, p.Nk, region, p.k8, v_region, v_part);
  prep_final<D, HAS_K><<<p.B * p.H, kFinalThreads, 0, st>>>(p.Nk, nck, region, p.k8, p.k_mean, v_region, v_part,
                                                             p.v_scale);
  constexpr int TPW = enc_tiles_per_wg<D, CACHE>();
  const int nkt = nkp / kBlk, nb2 = (HAS_K ? nkt : 0) + (nkt + TPW - 1) / TPW;
  prep_pass2<D, HAS_K, CACHE><<<dim3(nb2, p.H, p.B), kThreads, 0, st>>>(
      p.k, p.k_mean, p.k8, p.k_scale, p.v, p.v_cache, p.v_tok_scale, p.v_scale, p.v8t, p.vbf, p.H, p.Nk, nkp);
  const int64_t n = (int64_t)p.B * p.H * D;
  v_scale_from_amax<<<(int)((n + 255) / 256), 256, 0, st>>>(p.v_scale, n);
}

}  // namespace detail
using namespace detail;

hipError_t launch_k_mean(BshdView k, int B, int H, int N, int D, int npad, int8_t* scratch, float* mean,
                         hipStream_t st) {
  const int64_t region = (int64_t)npad * D;  // bytes of k8 per (b, h)
  const int nc = nchunks(N);
  dim3 g1(nc, H, B);
  if (D == 128) {
    k_mean_partial<128><<<g1, kThreads, 0, st>>>(k, H, N, region, scratch);
    k_mean_final<128><<<B * H, kFinalThreads, 0, st>>>(N, nc, region, scratch, mean);
  } else {
    k_mean_partial<64><<<g1, kThreads, 0, st>>>(k, H, N, region, scratch);
    k_mean_final<64><<<B * H, kFinalThreads, 0, st>>>(N, nc, region, scratch, mean);
  }
  return hipGetLastError();
}

hipError_t launch_quant_i8(BshdView x, const float* mean, int B, int H, int N, int D, int npad, int8_t* codes,
                           float* scales, hipStream_t st) {
  dim3 g(npad / kBlk, H, B);
  if (D == 128) {
    if (mean)
      quant_i8_blocks<128, true><<<g, kThreads, 0, st>>>(x, mean, H, N, npad, codes, scales);
    else
      quant_i8_blocks<128, false><<<g, kThreads, 0, st>>>(x, mean, H, N, npad, codes, scales);
  } else {
    if (mean)
      quant_i8_blocks<64, true><<<g, kThreads, 0, st>>>(x, mean, H, N, npad, codes, scales);
    else
      quant_i8_blocks<64, false><<<g, kThreads, 0, st>>>(x, mean, H, N, npad, codes, scales);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// KV-cache append: each (token, head) row of D channels becomes INT8 codes with its own
// scale, by the same formula as the 64-row blocks (a = max|x|, s = a/127, code =
// rne(x * min(127/a, FLT_MAX))).  D/8 consecutive lanes own one row (8 channels each,
// 16-byte loads, 8-byte stores) and reduce its max with lane exchanges.
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void kv_append_i8(const uint16_t* x, int64_t sn, int64_t sh, int Nnew, int H,
                                                         int8_t* cache, float* tok_scale, int Nmax, int pos) {
  constexpr int CPR = D / 8;  // lanes per row (a power of two dividing 64)
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = t / CPR;  // n * H + h
  const int cg = (int)(t % CPR);
  const bool live = row < (int64_t)Nnew * H;
  const int n = live ? (int)(row / H) : 0, h = live ? (int)(row - (int64_t)n * H) : 0;
  float f[8];
  float amax = 0.0f;
  if (live) {
    const v4i w = *(const v4i*)(x + (int64_t)n * sn + (int64_t)h * sh + cg * 8);
    unpack_bf16x8(w, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  // every lane of the row's group takes part (the group never straddles a wave)
#pragma unroll
  for (int o = CPR / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, CPR));
  if (!live) return;
  float s = 0.0f, r = 0.0f;
  if (amax > 0.0f) {
    s = amax / 127.0f;
    r = fminf(127.0f / amax, kFltMax);
  }
  const int64_t crow = (int64_t)h * Nmax + pos + n;
  if (cg == 0) tok_scale[crow] = s;
  uint32_t wd[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = __builtin_rintf(f[i] * r);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    wd[i >> 2] |= ((uint32_t)(int)q & 0xffu) << (8 * (i & 3));
  }
  *(uint2*)(cache + crow * D + cg * 8) = make_uint2(wd[0], wd[1]);
}

hipError_t launch_kv_append_i8(const void* x, int64_t sn, int64_t sh, int Nnew, int H, int D, int8_t* cache,
                               float* tok_scale, int Nmax, int pos, hipStream_t st) {
  const int64_t threads = (int64_t)Nnew * H * (D / 8);
  const int blocks = (int)((threads + kThreads - 1) / kThreads);
  if (D == 128)
    kv_append_i8<128><<<blocks, kThreads, 0, st>>>((const uint16_t*)x, sn, sh, Nnew, H, cache, tok_scale, Nmax, pos);
  else
    kv_append_i8<64><<<blocks, kThreads, 0, st>>>((const uint16_t*)x, sn, sh, Nnew, H, cache, tok_scale, Nmax, pos);
  return hipGetLastError();
}

template <int D, bool CACHE>
static void quant_v_impl(BshdView v, const int8_t* cache, const float* tok_scale, int B, int H, int N, int npad,
                         uint8_t* v8t, float* v_scale, uint16_t* vbf, hipStream_t st) {
  const int64_t region = (int64_t)npad * D;  // bytes of v8t per (b, h)
  const int nc = nchunks(N);
  v_amax_partial<D, CACHE><<<dim3(nc, H, B), kThreads, 0, st>>>(v, cache, tok_scale, H, N, region, v8t);
  v_amax_final<D><<<B * H, kFinalThreads, 0, st>>>(nc, region, v8t, v_scale);
  constexpr int TPW = enc_tiles_per_wg<D, CACHE>();
  v_encode<D, CACHE><<<dim3((npad / kBlk + TPW - 1) / TPW, H, B), kThreads, 0, st>>>(v, cache, tok_scale, H, N, npad,
                                                                                    v_scale, v8t, vbf);
  const int64_t n = (int64_t)B * H * D;
  v_scale_from_amax<<<(int)((n + 255) / 256), 256, 0, st>>>(v_scale, n);
}

hipError_t launch_quant_v(BshdView v, const int8_t* cache, const float* tok_scale, int B, int H, int N, int D,
                          int npad, uint8_t* v8t, float* v_scale, uint16_t* vbf, hipStream_t st) {
  if (D == 128) {
    if (cache)
      quant_v_impl<128, true>(v, cache, tok_scale, B, H, N, npad, v8t, v_scale, vbf, st);
    else
      quant_v_impl<128, false>(v, cache, tok_scale, B, H, N, npad, v8t, v_scale, vbf, st);
  } else {
    if (cache)
      quant_v_impl<64, true>(v, cache, tok_scale, B, H, N, npad, v8t, v_scale, vbf, st);
    else
      quant_v_impl<64, false>(v, cache, tok_scale, B, H, N, npad, v8t, v_scale, vbf, st);
  }
  return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs& p, int D, hipStream_t st) {
  const bool has_k = p.k8 != nullptr, cache = p.v_cache != nullptr;
  if (has_k == cache) return hipErrorInvalidValue;  // dense Q/K/V, or q and an int8 V cache
  if (!p.v8t && !p.vbf) return hipErrorInvalidValue;
  if (D == 128) {
    if (has_k)
      prep_impl<128, true, false>(p, st);
    else
      prep_impl<128, false, true>(p, st);
  } else {
    if (has_k)
      prep_impl<64, true, false>(p, st);
    else
      prep_impl<64, false, true>(p, st);
  }
  return hipGetLastError();
}

}  // namespace qattn
