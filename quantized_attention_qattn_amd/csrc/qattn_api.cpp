// C-ABI entry points of libqattn: argument validation (before any HIP call) and launch
// sequencing on the caller's stream.  No allocation, no synchronization.
#include <math.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qattn.h"
#include "common.h"

using namespace qattn;

namespace {

constexpr int64_t kMaxN = (int64_t)1 << 28;  // keeps every row index and grid size in range
constexpr int kMaxGridYZ = 65535;
// Split-KV rule for the prefill entry point: enough key ranges for one workgroup per CU
// (256 CUs, one resident workgroup each), each range at least kSplitMinTiles key tiles long.
constexpr int64_t kSplitTargetWorkgroups = 256;
constexpr int64_t kSplitMinTiles = 16;
constexpr int kMaxKvSplits = 64;

inline int64_t npad64(int64_t n) { return (n + kBlk - 1) / kBlk * kBlk; }
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

inline bool bf16_view_ok(const void* p, const int64_t* str, int n) {
  if (!p || !str) return false;
  if (!aligned(p, 16)) return false;
  for (int i = 0; i < n; ++i)
    if (str[i] < 0 || (str[i] & 7) != 0) return false;
  return true;
}

inline bool sizes_ok(int64_t B, int64_t H, int64_t N) {
  return B > 0 && H > 0 && N > 0 && B <= kMaxGridYZ && H <= kMaxGridYZ && N <= kMaxN;
}

// buffer resources of the fused kernel address one (b, h) slice with 32-bit offsets
inline bool slice_ok(int64_t n, int D) { return npad64(n) * D < ((int64_t)1 << 31); }

inline int status_of(hipError_t e) { return e == hipSuccess ? QATTN_OK : QATTN_EHIP; }

inline float resolve_lambda(float scale_log2, int D) {
  if (scale_log2 > 0.0f) return scale_log2;
  const float inv = (float)(1.0 / sqrt((double)D));
  const float log2e = (float)1.4426950408889634;
  return inv * log2e;
}

inline bool out_ok(const void* out, const int64_t* str, int n, int out_dtype) {
  if (!out || !str) return false;
  if (out_dtype != QATTN_OUT_BF16 && out_dtype != QATTN_OUT_F32) return false;
  const int esz = out_dtype == QATTN_OUT_BF16 ? 2 : 4;
  if (!aligned(out, 4 * esz)) return false;
  for (int i = 0; i < n; ++i)
    if (str[i] < 0 || (str[i] & 3) != 0) return false;
  return true;
}

// Key tiles a causal prefill reads: every query sees keys 0 .. pos0 + i.
inline int64_t i8kv_key_tiles(int Nq, int Nk, int pos0) {
  const int64_t last = std::min<int64_t>(Nk, (int64_t)pos0 + Nq);
  return (last + kBlk - 1) / kBlk;
}

}  // namespace

extern "C" {

const char* qattn_status_string(int status) {
  switch (status) {
    case QATTN_OK: return "ok";
    case QATTN_EINVAL: return "invalid argument (null pointer, size, alignment, stride or position)";
    case QATTN_EUNSUPPORTED: return "unsupported head dimension (D must be 64 or 128)";
    case QATTN_EWORKSPACE: return "workspace too small";
    case QATTN_EHIP: return "HIP kernel launch failed";
    case QATTN_ESCRATCH: return "the call needs a larger workspace than the library's static scratch array holds";
    default: return "unknown status";
  }
}

int qattn_quant_qk(const void* q, const int64_t q_str[3], const void* k, const int64_t k_str[3], int B, int H,
                   int Nq, int Nk, int D, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, float* k_mean,
                   void* stream) {
  if (!q8 || !q_scale || !k8 || !k_scale || !k_mean) return QATTN_EINVAL;
  if (!bf16_view_ok(q, q_str, 3) || !bf16_view_ok(k, k_str, 3)) return QATTN_EINVAL;
  if (!sizes_ok(B, H, Nq) || !sizes_ok(B, H, Nk)) return QATTN_EINVAL;
  if (D != 64 && D != 128) return QATTN_EUNSUPPORTED;
  if (!aligned(q8, 256) || !aligned(k8, 256) || !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(k_mean, 4))
    return QATTN_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  const int nqp = (int)npad64(Nq), nkp = (int)npad64(Nk);
  BshdView qv{q, q_str[0], q_str[1], q_str[2]};
  BshdView kv{k, k_str[0], k_str[1], k_str[2]};
  hipError_t e = launch_k_mean(kv, B, H, Nk, D, nkp, k8, k_mean, st);
  if (e != hipSuccess) return QATTN_EHIP;
  e = launch_quant_i8(qv, nullptr, B, H, Nq, D, nqp, q8, q_scale, st);
  if (e != hipSuccess) return QATTN_EHIP;
  e = launch_quant_i8(kv, k_mean, B, H, Nk, D, nkp, k8, k_scale, st);
  return status_of(e);
}

int qattn_quant_v(const void* v, const int64_t v_str[3], int B, int H, int Nk, int D, uint8_t* v8t, float* v_scale,
                  uint16_t* vbf, void* stream) {
  if (!v8t || !v_scale) return QATTN_EINVAL;
  if (vbf && !aligned(vbf, 256)) return QATTN_EINVAL;
  if (!bf16_view_ok(v, v_str, 3)) return QATTN_EINVAL;
  if (!sizes_ok(B, H, Nk)) return QATTN_EINVAL;
  if (D != 64 && D != 128) return QATTN_EUNSUPPORTED;
  if (!aligned(v8t, 256) || !aligned(v_scale, 4)) return QATTN_EINVAL;
  BshdView vv{v, v_str[0], v_str[1], v_str[2]};
  return status_of(launch_quant_v(vv, nullptr, nullptr, B, H, Nk, D, (int)npad64(Nk), v8t, v_scale, vbf,
                                  (hipStream_t)stream));
}

int qattn_prep(const void* q, const int64_t q_str[3], const void* k, const int64_t k_str[3], const void* v,
               const int64_t v_str[3], int B, int H, int Nq, int Nk, int D, int8_t* q8, float* q_scale, int8_t* k8,
               float* k_scale, float* k_mean, uint8_t* v8t, float* v_scale, uint16_t* vbf, void* stream) {
  if (!q8 || !q_scale || !k8 || !k_scale || !k_mean || !v_scale || (!v8t && !vbf)) return QATTN_EINVAL;
  if (!bf16_view_ok(q, q_str, 3) || !bf16_view_ok(k, k_str, 3) || !bf16_view_ok(v, v_str, 3)) return QATTN_EINVAL;
  if (!sizes_ok(B, H, Nq) || !sizes_ok(B, H, Nk)) return QATTN_EINVAL;
  if (D != 64 && D != 128) return QATTN_EUNSUPPORTED;
  if (!aligned(q8, 256) || !aligned(k8, 256) || (v8t && !aligned(v8t, 256)) || (vbf && !aligned(vbf, 256)))
    return QATTN_EINVAL;
  if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(k_mean, 4) || !aligned(v_scale, 4)) return QATTN_EINVAL;
  PrepArgs p{};
  p.q = BshdView{q, q_str[0], q_str[1], q_str[2]};
  p.k = BshdView{k, k_str[0], k_str[1], k_str[2]};
  p.v = BshdView{v, v_str[0], v_str[1], v_str[2]};
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.q8 = q8;
  p.q_scale = q_scale;
  p.k8 = k8;
  p.k_scale = k_scale;
  p.k_mean = k_mean;
  p.v8t = v8t;
  p.v_scale = v_scale;
  p.vbf = vbf;
  return status_of(launch_prep(p, D, (hipStream_t)stream));
}

int qattn_fwd(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale, const uint16_t* vbf,
              const float* v_scale, int B, int H, int Nq, int Nk, int D, float scale_log2, int causal, void* out,
              const int64_t out_str[3], int out_dtype, void* stream) {
  if (!q8 || !q_scale || !k8 || !k_scale || !vbf || !v_scale) return QATTN_EINVAL;
  if (!sizes_ok(B, H, Nq) || !sizes_ok(B, H, Nk)) return QATTN_EINVAL;
  if (D != 64 && D != 128) return QATTN_EUNSUPPORTED;
  if (!aligned(q8, 256) || !aligned(k8, 256) || !aligned(vbf, 256)) return QATTN_EINVAL;
  if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4)) return QATTN_EINVAL;
  if (!out_ok(out, out_str, 3, out_dtype)) return QATTN_EINVAL;
  if (isnan(scale_log2) || isinf(scale_log2)) return QATTN_EINVAL;
  const int64_t nqp = npad64(Nq), nkp = npad64(Nk);
  const int64_t nqb = (Nq + 127) / 128;
  if ((int64_t)B * H * nqb > INT32_MAX || !slice_ok(Nk, D)) return QATTN_EINVAL;
  FwdArgs a{};
  a.q8 = q8;
  a.q_scale = q_scale;
  a.k8 = k8;
  a.k_scale = k_scale;
  a.vbf = vbf;
  a.v_scale = v_scale;
  a.out = out;
  a.q8_bh = nqp * D;
  a.qs_bh = nqp / kBlk;
  a.k8_bh = nkp * D;
  a.ks_bh = nkp / kBlk;
  a.vbf_bh = (int64_t)D * nkp;
  a.ldv = nkp;
  a.out_sb = out_str[0];
  a.out_sn = out_str[1];
  a.out_sh = out_str[2];
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.nq_pad = (int)nqp;
  a.k_rows = (int)nkp;
  a.lambda = resolve_lambda(scale_log2, D);
  a.pos_off = (int64_t)Nk - Nq;
  a.causal = causal ? 1 : 0;
  a.per_token = 0;
  a.out_bf16 = out_dtype == QATTN_OUT_BF16;
  a.kv_splits = 1;
  a.tiles_total = (int)(nkp / kBlk);
  return status_of(launch_attn_fwd(a, D, (hipStream_t)stream));
}

int qattn_fwd_i8kv_kv_splits(int H, int Nq, int Nk, int pos0) {
  if (H <= 0 || Nq <= 0 || Nk <= 0 || pos0 < 0 || (int64_t)pos0 + Nq > Nk) return 0;
  const int64_t wgs = (int64_t)H * ((Nq + 255) / 256);  // workgroups of one pass
  const int64_t T = i8kv_key_tiles(Nq, Nk, pos0);
  int64_t S = (kSplitTargetWorkgroups + wgs - 1) / wgs;
  S = std::min<int64_t>(S, T / kSplitMinTiles);
  S = std::min<int64_t>(S, kMaxKvSplits);
  return (int)std::max<int64_t>(S, 1);
}

size_t qattn_fwd_i8kv_workspace_bytes(int H, int Nq, int Nk, int D, int kv_splits) {
  if (H <= 0 || Nq <= 0 || Nk <= 0 || H > kMaxGridYZ || Nq > kMaxN || Nk > kMaxN) return 0;
  if (D != 64 && D != 128) return 0;
  if (kv_splits < 1 || kv_splits > kMaxKvSplits) return 0;
  const size_t nkp = (size_t)npad64(Nk), nqp = (size_t)npad64(Nq);
  size_t bytes = round256((size_t)H * D * 4) + round256((size_t)H * nqp * D) + round256((size_t)H * (nqp / kBlk) * 4) +
                 round256((size_t)H * D * nkp * 2);
  if (kv_splits > 1)
    bytes += round256((size_t)kv_splits * H * nqp * D * 4) + round256((size_t)kv_splits * H * nqp * 2 * 4);
  return bytes;
}

int qattn_fwd_i8kv(const void* q, const int64_t q_str[2], const int8_t* k_cache, const float* k_tok_scale,
                   const int8_t* v_cache, const float* v_tok_scale, int H, int Nq, int Nk, int D, int pos0,
                   float scale_log2, int kv_splits, void* workspace, size_t workspace_bytes, void* out,
                   const int64_t out_str[2], int out_dtype, void* stream) {
  if (!workspace) return QATTN_EINVAL;
  size_t need = 0;
  const int st = qattn::i8kv_check(q, q_str, k_cache, k_tok_scale, v_cache, v_tok_scale, H, Nq, Nk, D, pos0,
                                   scale_log2, &kv_splits, out, out_str, out_dtype, &need);
  if (st != QATTN_OK) return st;
  if (!aligned(workspace, 256)) return QATTN_EINVAL;
  if (workspace_bytes < need) return QATTN_EWORKSPACE;
  return qattn::i8kv_launch(q, q_str, k_cache, k_tok_scale, v_cache, v_tok_scale, H, Nq, Nk, D, pos0, scale_log2,
                            kv_splits, workspace, out, out_str, out_dtype, stream);
}

int qattn_kv_append_i8(const void* x, const int64_t x_str[2], int Nnew, int H, int D, int8_t* cache,
                       float* tok_scale, int Nmax, int pos, void* stream) {
  if (!cache || !tok_scale) return QATTN_EINVAL;
  if (!bf16_view_ok(x, x_str, 2)) return QATTN_EINVAL;
  if (!sizes_ok(1, H, Nnew) || Nmax <= 0 || Nmax > kMaxN) return QATTN_EINVAL;
  if (D != 64 && D != 128) return QATTN_EUNSUPPORTED;
  if (pos < 0 || (int64_t)pos + Nnew > Nmax) return QATTN_EINVAL;
  if ((int64_t)H * Nmax * D > ((int64_t)1 << 40)) return QATTN_EINVAL;
  if (!aligned(cache, 8) || !aligned(tok_scale, 4)) return QATTN_EINVAL;
  return status_of(launch_kv_append_i8(x, x_str[0], x_str[1], Nnew, H, D, cache, tok_scale, Nmax, pos,
                                       (hipStream_t)stream));
}

int qattn_selftest_p8_codes(const float* u, uint8_t* codes, int64_t n, int saturating, void* stream) {
  if (!u || !codes || n <= 0 || (saturating != 0 && saturating != 1)) return QATTN_EINVAL;
  if (!aligned(u, 4)) return QATTN_EINVAL;
  return status_of(launch_p8_codes(u, codes, n, saturating, (hipStream_t)stream));
}

}  // extern "C"

namespace qattn {

// Validation of a prefill call, everything but the workspace: resolves *kv_splits (0 =
// the rule) and returns the workspace size in *need.
int i8kv_check(const void* q, const int64_t q_str[2], const int8_t* k_cache, const float* k_tok_scale,
               const int8_t* v_cache, const float* v_tok_scale, int H, int Nq, int Nk, int D, int pos0,
               float scale_log2, int* kv_splits, const void* out, const int64_t out_str[2], int out_dtype,
               size_t* need) {
  if (!k_cache || !k_tok_scale || !v_cache || !v_tok_scale || !kv_splits || !need) return QATTN_EINVAL;
  if (!bf16_view_ok(q, q_str, 2)) return QATTN_EINVAL;
  if (!sizes_ok(1, H, Nq) || !sizes_ok(1, H, Nk)) return QATTN_EINVAL;
  if (D != 64 && D != 128) return QATTN_EUNSUPPORTED;
  if (pos0 < 0 || (int64_t)pos0 + Nq > Nk || !slice_ok(Nk, D)) return QATTN_EINVAL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_tok_scale, 4) || !aligned(v_tok_scale, 4))
    return QATTN_EINVAL;
  if (!out_ok(out, out_str, 2, out_dtype)) return QATTN_EINVAL;
  if (isnan(scale_log2) || isinf(scale_log2)) return QATTN_EINVAL;
  int S = *kv_splits;
  if (S == 0) S = qattn_fwd_i8kv_kv_splits(H, Nq, Nk, pos0);
  if (S < 1 || S > kMaxKvSplits) return QATTN_EINVAL;
  if ((int64_t)H * ((Nq + 255) / 256) * S > INT32_MAX) return QATTN_EINVAL;
  *need = qattn_fwd_i8kv_workspace_bytes(H, Nq, Nk, D, S);
  if (*need == 0) return QATTN_EINVAL;
  *kv_splits = S;
  return QATTN_OK;
}

// The launches of a validated prefill call into a workspace of at least the checked size
// (256-byte aligned): the preparation of q and of the cached V, then the fused loop.
int i8kv_launch(const void* q, const int64_t q_str[2], const int8_t* k_cache, const float* k_tok_scale,
                const int8_t* v_cache, const float* v_tok_scale, int H, int Nq, int Nk, int D, int pos0,
                float scale_log2, int kv_splits, void* workspace, void* out, const int64_t out_str[2],
                int out_dtype, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int64_t nkp = npad64(Nk), nqp = npad64(Nq);
  uint8_t* ws = (uint8_t*)workspace;
  float* v_scale = (float*)ws;
  ws += round256((size_t)H * D * 4);
  int8_t* q8 = (int8_t*)ws;
  ws += round256((size_t)H * nqp * D);
  float* q_scale = (float*)ws;
  ws += round256((size_t)H * (nqp / kBlk) * 4);
  uint16_t* vbf = (uint16_t*)ws;
  ws += round256((size_t)H * D * nkp * 2);
  float* part_o = nullptr;
  float* part_md = nullptr;
  if (kv_splits > 1) {
    part_o = (float*)ws;
    ws += round256((size_t)kv_splits * H * nqp * D * 4);
    part_md = (float*)ws;
  }

  // q -> INT8 blocks (no smoothing), V cache -> per-channel e4m3 (channel-major), kept as
  // the bf16 values of the codes (the only form the fused loop reads): the fused
  // preparation with no K and no separate code array
  PrepArgs p{};
  p.q = BshdView{q, 0, q_str[0], q_str[1]};
  p.B = 1;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.q8 = q8;
  p.q_scale = q_scale;
  p.v_cache = v_cache;
  p.v_tok_scale = v_tok_scale;
  p.v_scale = v_scale;
  p.vbf = vbf;
  hipError_t e = launch_prep(p, D, st);
  if (e != hipSuccess) return QATTN_EHIP;

  FwdArgs a{};
  a.q8 = q8;
  a.q_scale = q_scale;
  a.k8 = k_cache;
  a.k_scale = k_tok_scale;
  a.vbf = vbf;
  a.v_scale = v_scale;
  a.out = out;
  a.q8_bh = nqp * D;
  a.qs_bh = nqp / kBlk;
  a.k8_bh = (int64_t)Nk * D;
  a.ks_bh = Nk;
  a.vbf_bh = (int64_t)D * nkp;
  a.ldv = nkp;
  a.out_sb = 0;
  a.out_sn = out_str[0];
  a.out_sh = out_str[1];
  a.B = 1;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.nq_pad = (int)nqp;
  a.k_rows = Nk;
  a.lambda = resolve_lambda(scale_log2, D);
  a.pos_off = pos0;
  a.causal = 1;
  a.per_token = 1;
  a.out_bf16 = out_dtype == QATTN_OUT_BF16;
  a.kv_splits = kv_splits;
  a.tiles_total = (int)i8kv_key_tiles(Nq, Nk, pos0);
  a.part_o = part_o;
  a.part_md = part_md;
  return status_of(launch_attn_fwd(a, D, st));
}


}  // namespace qattn
