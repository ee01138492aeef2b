// The prefill entry point for callers that cannot allocate (code under stream capture,
// serving loops, hosts that forbid device allocation): the workspace of qattn_fwd_i8kv
// lives in a fixed device array of this library, one per GPU, so that the caller passes
// only its inputs and outputs.
#include <mutex>

#include "../../include/qattn.h"
#include "common.h"

namespace {
constexpr int kMaxDevices = 64;
static_assert(QATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
}  // namespace

// The workspace array.  Each GPU the library runs on holds its own copy for the life of
// the process.  In host code this name is only a stand-in for the symbol: the device
// address of a GPU's copy comes from hipGetSymbolAddress, made with that GPU current.
static __device__ __align__(256) uint8_t scratch[QATTN_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of each GPU's copy, looked up once

// Device address of the current GPU's copy of `scratch` (looked up on the first call on
// that GPU, with that GPU current).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QATTN_EHIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return QATTN_EHIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return QATTN_OK;
}
}  // namespace

extern "C" int qattn_fwd_i8kv_noalloc(const void* q, const int64_t q_str[2], const int8_t* k_cache,
                                      const float* k_tok_scale, const int8_t* v_cache, const float* v_tok_scale,
                                      int H, int Nq, int Nk, int D, int pos0, float scale_log2, int kv_splits,
                                      void* out, const int64_t out_str[2], int out_dtype, void* stream) {
  size_t need = 0;
  int st = qattn::i8kv_check(q, q_str, k_cache, k_tok_scale, v_cache, v_tok_scale, H, Nq, Nk, D, pos0, scale_log2,
                             &kv_splits, out, out_str, out_dtype, &need);
  if (st != QATTN_OK) return st;
  if (need > QATTN_NOALLOC_SCRATCH_BYTES) return QATTN_ESCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != QATTN_OK) return st;
  // Every section of the workspace is written by the call before it is read (codes,
  // scales, V values with their zero padding, split partials of every row), so the
  // contents a previous call left need no clearing.
  return qattn::i8kv_launch(q, q_str, k_cache, k_tok_scale, v_cache, v_tok_scale, H, Nq, Nk, D, pos0, scale_log2,
                            kv_splits, ws, out, out_str, out_dtype, stream);
}
