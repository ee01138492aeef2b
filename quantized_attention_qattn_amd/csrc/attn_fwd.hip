// Fused quantized attention forward for gfx950: INT8 MFMA Q.K^T with INT32 accumulation,
// tile-ordered online softmax with FP8 P, P.V over the FP8 values of P and V, fused
// V-scale epilogue.
//
// Per 64-key tile every query row runs QK -> update m, d, O -> accumulate d -> P to FP8
// -> PV ("Sage2 SM89 Temporal Pair Experiment", section "Candidate"), so each row's
// numeric sequence is independent of how rows are grouped into waves.
//
// Layout of the work (CDNA4, 64-wide waves):
//   * a workgroup owns 256 query rows of one (b, h): 8 waves x 32 rows.  Waves w and
//     w + 4 share a SIMD.  Each wave alternates an MFMA phase (QK of tile i and PV of
//     tile i - 1) with a VALU phase (online softmax of tile i); group 1 (waves 4-7) runs
//     one phase behind group 0, so the two waves of a SIMD start each interval in
//     different kinds of phase and one issues matrix instructions while its partner is in
//     the softmax;
//   * scores are computed transposed, S^T = K . Q^T, with v_mfma_i32_32x32x32_i8: the
//     accumulator gives each lane one query (its column) and 32 keys of the tile (16 per
//     32-key block), so the row max and row sum are in-lane plus one exchange with the
//     lane 32 apart;
//   * the key order inside a tile is permuted so that lane half h holds keys 32h..32h+31;
//     its 32 P values then form, 8 keys at a time, the B operand of four
//     v_mfma_f32_32x32x16_bf16 whose A operand (V^T) is read from LDS at the same keys;
//   * P.V runs on the bf16 MFMA over the exact values of the FP8 codes of P and V (every
//     e4m3 value is a bf16 value, every product of two is exact in fp32).  The FP8 MFMA
//     of gfx950 was not used here: it truncates each product to 13 bits below the
//     largest product of its group of 8, which moved outputs by up to 3.1e-3 of their
//     RMS on short key ranges with many heads (1.6e-3 on the long workloads), beyond the
//     2e-3 accuracy bound;
//   * K tiles (INT8) and V^T tiles (the bf16 values of the V codes, written by the V
//     quantizer beside the codes) are loaded straight into LDS, so the MFMA phases read
//     the PV operand as it is;
//   * O^T (D x 32 queries per wave) lives in D/32 accumulators of 16 fp32 per lane;
//   * workgroups are mapped so each XCD walks one contiguous range of (b, h, query block)
//     and keeps the K/V it streams in its own L2.
//
// Tile pipeline: interval i (between two workgroup barriers) holds group 0's MFMA phase i
// and VALU phase i, and group 1's VALU phase i - 1 and MFMA phase i.
//   slot j = {K tile j, bf16 V^T of tile j - 1} sits in buffer j % 3.  Both groups' MFMA
//   phases j read it in interval j.  Group 1, which finishes its interval earlier, issues
//   the loads at the start of interval j - 2 (the buffer's previous slot, j - 3, was read
//   in interval j - 3) and waits for them at the end of interval j - 1.  The per-key
//   scales of a per-token cache follow the same ring (sC[j % 3]): the groups read those of
//   tile j in intervals j and j + 1, before group 1 overwrites them at the end of
//   interval j + 2.
//
// Issue priority: of a SIMD's two waves the hardware favours the older one, group 0, and
// group 1's softmax then advances little while group 0 issues.  So each wave raises its
// priority (s_setprio) for its MFMA phase (2: an MFMA issues as soon as the matrix core
// is free) and group 1 for its softmax (1), which then ends in time for group 1's MFMA
// phase to run beside group 0's softmax (0).
#include <climits>
#include <type_traits>
#include <utility>

#include "common.h"

namespace qattn {
namespace detail {

constexpr int BM = 256;  // query rows per workgroup
[[maybe_unused]] constexpr int BN = 64;   // keys per tile (the numeric contract's tile)
constexpr int NT = 512;  // threads per workgroup (8 waves)
[[maybe_unused]] constexpr int NBUF = 3;  // tile slots in LDS (loads run two slots ahead)
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt_hi[15:14]): vmcnt(n < 16) with the others at their maxima, and lgkmcnt(0).
[[maybe_unused]] constexpr int kVmcntZero = 0x0F70;
constexpr int vmcnt_imm(int n) { return 0x0F70 | n; }
[[maybe_unused]] constexpr int kLgkmcntZero = 0xC07F;
// The softmax works with P'' = 2^u = 2^80 P', u = fl32(acc * c + fl32(88 - m)) being
// the exponent argument on its fixed grid (2^-17 where P' can have a nonzero e4m3
// code): one hardware exponential and no subtraction per key.  The 2^80 is exact and is
// folded out by the FP8 conversion (its scale operand divides, exactly, for every
// input) and once from d'' in the epilogue.  On this grid the e4m3 code of the result
// equals the code of the correctly rounded power (checked over every fp32 u through
// qattn_p8_codes).
constexpr float kPScale = 0x1p80f;     // P'' / P'
constexpr float kPScaleInv = 0x1p-80f;
__device__ __forceinline__ float p_from_u(float u) { return __builtin_amdgcn_exp2f(u); }
// The large-score form (see softmax_tile): the FP8 conversion does not saturate (a value
// of 464 or more gives the NaN code), so its input is clamped to 448 * 2^80, whose code
// is the saturated one (0x7E).
constexpr float kPSat = 448.0f * 0x1p80f;
__device__ __forceinline__ float p_code_input_saturating(float p) { return __builtin_fminf(p, kPSat); }
typedef short v2s_t __attribute__((ext_vector_type(2)));

// e4m3 codes of P' = P'' / 2^80 for four values (bytes 0..3).  Both halves of the word
// are written, so the first conversion may start from any register: `spent` is a value
// that has no other use, whose register the result then takes over in place (a value
// still needed later would cost a copy, a zeroed start a move).
__device__ __forceinline__ int pack_fp8x4(float spent, float a, float b, float c, float d) {
  v2s_t w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s_t, spent), a, b, kPScale, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, kPScale, true);
  return __builtin_bit_cast(int, w);
}

// Puts a wave-uniform value in an SGPR as an opaque operand.  A buffer load's soffset
// (and M0) must be an SGPR or a small inline constant: a value the compiler has folded
// to a larger constant would otherwise reach the assembly below as a literal, and one
// it cannot prove uniform would sit in a VGPR.
__device__ __forceinline__ void sgpr_value(uint32_t& x) {
  x = __builtin_amdgcn_readfirstlane(x);
  asm volatile("" : "+s"(x));
}
__device__ __forceinline__ void sgpr_value(int& x) {
  x = __builtin_amdgcn_readfirstlane(x);
  asm volatile("" : "+s"(x));
}

// Direct global -> LDS load of 16 bytes per lane: lane l of the wave writes LDS bytes
// [lds + OFF + 16 l, lds + OFF + 16 l + 16).  Issued as inline assembly so that the
// compiler does not order the kernel's LDS reads after it (it would have to assume that
// the asynchronous LDS write may alias them); completion is awaited explicitly with
// s_waitcnt vmcnt(0) and a barrier before the buffer is read.  M0 (the LDS address) is
// formed inside the assembly from one base register and the constant OFF, so that no
// register holds a precomputed address per buffer and segment, and is restored after.
template <int OFF>
__device__ __forceinline__ void dma_16B(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, int voffset, int soffset) {
  uint32_t saved;
  sgpr_value(lds);
  sgpr_value(soffset);
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %5\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voffset), "s"(rsrc), "s"(soffset), "i"(OFF)
      : "memory", "scc");
}
// The same with 4 bytes per lane: lane l writes LDS bytes [lds + OFF + 4 l, ... + 4).
// Each dword is range-checked on its own (reads past the end of the resource give 0).
template <int OFF>
__device__ __forceinline__ void dma_4B(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, int voffset, int soffset) {
  uint32_t saved;
  sgpr_value(lds);
  sgpr_value(soffset);
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %5\n\t"
      "buffer_load_dword %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voffset), "s"(rsrc), "s"(soffset), "i"(OFF)
      : "memory", "scc");
}
// Calls f(std::integral_constant<int, I>) for I = 0 .. N - 1.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// wave-uniform LDS byte address of a shared-memory location
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p);
}

// Physical key (within the tile) of A-operand row m of the QK MFMA for 32-key block kb:
// the accumulator row m lands in lane half (m >> 2) & 1, register 4 (m >> 3) + (m & 3).
__device__ __forceinline__ int key_of_row(int kb, int m) {
  return 32 * ((m >> 2) & 1) + 16 * kb + 4 * (m >> 3) + (m & 3);
}

// 16-byte-slot XOR swizzle of the K tile (row pitch D bytes), chosen so that the QK
// reads (lanes of a half wave read 32 key rows through key_of_row at one chunk column)
// hit distinct banks both when 8 lanes share a 128-byte bank cycle and when 16 lanes
// share a 256-byte one.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if (D == 128) return ((row ^ (row >> 2)) & 1) | (row & 2) | (((row >> 5) & 1) << 2);
  return (((row >> 1) ^ (row >> 2)) & 1) | (((row >> 5) & 1) << 1);
}
// bf16 V^T rows are 128 bytes (64 keys); the 16-byte chunk q of row r sits at q ^ vbswz(r).
// The PV reads (32 consecutive rows at one chunk) then hit distinct banks both when 8
// lanes share a 128-byte bank cycle and when 16 lanes share a 256-byte one.
__device__ __forceinline__ int vbswz(int row) { return (row ^ (row >> 3)) & 7; }

// Combine a value with the one held by the lane 32 apart (same query, other key half).
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with the lower 32
// lanes of its second; applied to a value and a copy of it, every lane ends up holding
// {own, partner} in its two registers (in some order), which max and sum combine.  It is
// issued as assembly because the compiler folds the two results of the builtin into one
// when both operands are the same value.  s_nop 1 covers the VALU-write -> permlane-read
// hazard.
__device__ __forceinline__ void own_and_partner(uint32_t x, uint32_t& a, uint32_t& b) {
  a = x;
  asm volatile(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1"
      : "+v"(a), "=&v"(b));
}
__device__ __forceinline__ int max_with_partner(int x) {
  uint32_t a, b;
  own_and_partner((uint32_t)x, a, b);
  return max((int)a, (int)b);
}
__device__ __forceinline__ float fmax_with_partner(float x) {
  uint32_t a, b;
  own_and_partner(__builtin_bit_cast(uint32_t, x), a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  uint32_t a, b;
  own_and_partner(__builtin_bit_cast(uint32_t, x), a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// INT32 accumulators start at the bit pattern of 1.5 * 2^23, so that reading an
// accumulator as fp32 and subtracting 1.5 * 2^23 gives the exact dot product
// (|acc| <= 127 * 127 * 128 < 2^22) with one fast fp32 subtraction.
[[maybe_unused]] constexpr int kAccBias = 0x4B400000;
constexpr float kAccBiasF = 12582912.0f;
__device__ __forceinline__ float acc_f32(int biased) { return __builtin_bit_cast(float, biased) - kAccBiasF; }

// x if key I of the lane's 32 keys is visible (I <= lim), else `masked` (a VGPR: with
// VCC the select may read no other scalar operand), or 0 in the second form: compare
// and select in one piece of assembly.  Written as C++, the compiler computes the 32
// compares of a masked tile ahead of their uses and keeps each result in a 64-bit
// scalar mask register; that pressure makes it spill scalar registers throughout the
// tile loop.  The s_nop gives the two wait states that a VALU write of VCC needs before
// a VALU read of it.
template <int I>
__device__ __forceinline__ int select_visible(int x, int lim, int masked) {
  asm("v_cmp_le_i32 vcc, %2, %1\n\t"
      "s_nop 1\n\t"
      "v_cndmask_b32_e64 %0, %3, %0, vcc"
      : "+v"(x)
      : "v"(lim), "i"(I), "v"(masked)
      : "vcc");
  return x;
}
template <int I>
__device__ __forceinline__ int select_visible_or_zero(int x, int lim) {
  asm("v_cmp_le_i32 vcc, %2, %1\n\t"
      "s_nop 1\n\t"
      "v_cndmask_b32_e64 %0, 0, %0, vcc"
      : "+v"(x)
      : "v"(lim), "i"(I)
      : "vcc");
  return x;
}

// Online-softmax step of one 64-key tile for this lane's query and its 32 keys
// (key0 + i, i = 16 kb + j held in S_kb[j]).  Returns the 32 FP8 codes of P' = 256 P
// packed as the B operand of the PV MFMA; updates m and returns in `tsum` the lane's
// share of the tile's sum of P'' = 2^80 P' (the caller folds it into d'' with the
// factor alpha of the old terms).
template <bool MASKED, bool PER_TOKEN>
__device__ __forceinline__ v8i softmax_tile(const v16i& S0, const v16i& S1, const float* cp, float c_tile,
                                            int key0, int vis_last, float& m, float& tsum, float (&p)[32]) {
  float cvec[32];
  if (PER_TOKEN) {
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float4 c4 = *(const float4*)(cp + i);
      cvec[i] = c4.x;
      cvec[i + 1] = c4.y;
      cvec[i + 2] = c4.z;
      cvec[i + 3] = c4.w;
    }
  }
  // masked tile: key i of this lane is visible iff i <= lim.  A hidden key's
  // accumulator reads as 0 (below every biased accumulator) for the tile max and its
  // exponent argument as -inf, so that its P is exactly 0 whatever the scale.
  const int lim = vis_last - key0;
  const int ninf = (int)0xff800000u;
  int accv[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    accv[i] = S0[i];
    accv[16 + i] = S1[i];
  }
  // exact fp32 dot products.  With per-block scales they are formed first, while the tile
  // max (on the integers) is pending; with per-token scales the max needs them anyway.
  float accf[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) accf[i] = PER_TOKEN ? 0.0f : acc_f32(accv[i]);
  auto af = [&](int i) { return PER_TOKEN ? acc_f32(accv[i]) : accf[i]; };
  float Mt;
  if (PER_TOKEN) {
    Mt = -INFINITY;
    static_for<32>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      float sv = af(i) * cvec[i];
      if (MASKED) sv = __builtin_bit_cast(float, select_visible<i>(__builtin_bit_cast(int, sv), lim, ninf));
      Mt = fmaxf(Mt, sv);
    });
    Mt = fmax_with_partner(Mt);
  } else {
    int am[32];
    static_for<32>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      am[i] = MASKED ? select_visible_or_zero<i>(accv[i], lim) : accv[i];
    });
    // two chains of three-input maxima (v_max3_i32): 17 instructions for 32 values
    int mxa = INT_MIN, mxb = INT_MIN;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      mxa = max(max(mxa, am[i]), am[i + 1]);
      mxb = max(max(mxb, am[16 + i]), am[16 + i + 1]);
    }
    const int mx = max_with_partner(max(mxa, mxb));
    // a visible key's biased accumulator is positive, so a maximum of 0 means that every
    // key of the row is hidden, which only a masked tile can have
    Mt = (MASKED && mx <= 0) ? -INFINITY : acc_f32(mx) * c_tile;
  }
  const float mnew = fmaxf(m, Mt);
  // m stays -inf while every key so far is hidden (masked tiles only: an unmasked
  // tile's maximum is finite)
  const float ms = (MASKED && mnew == -INFINITY) ? 0.0f : mnew;
  const float bconst = 88.0f - ms;  // u = S - m + 88: P' = 2^(u - 80) peaks at 2^8
  m = mnew;
  // four partial sums keep the additions off one dependent chain (the order of the
  // additions into d' is not part of the contract; the result is an fp32 sum of P'',
  // i.e. 2^80 times an fp32 sum of P')
  float ds[4];
  v8i pf;
  float u0[8];
  static_for<32>([&](auto i_c) {
    constexpr int i = decltype(i_c)::value;
    float u = __builtin_fmaf(af(i), PER_TOKEN ? cvec[i] : c_tile, bconst);
    if (MASKED) u = __builtin_bit_cast(float, select_visible<i>(__builtin_bit_cast(int, u), lim, ninf));
    p[i] = p_from_u(u);
    if (i % 4 == 0) u0[i / 4] = u;
    ds[i & 3] = i < 4 ? p[i] : ds[i & 3] + p[i];
  });
#pragma unroll
  for (int w = 0; w < 8; ++w) pf[w] = pack_fp8x4(u0[w], p[4 * w], p[4 * w + 1], p[4 * w + 2], p[4 * w + 3]);
  tsum = (ds[0] + ds[1]) + (ds[2] + ds[3]);
  return pf;
}

// The large-score form of a tile's results from its powers p = 2^u = 2^80 P'.
// u = fl32(acc c + fl32(88 - m_s)) exceeds 88 by at most (ulp(m_s) + ulp(88 - m_s)) / 2
// + ulp(u) / 2, i.e. by at most 0.375 + 2^-17 while |m_s| < 2^22: then P' <= 2^8.375 < 448
// and no code saturates.  Beyond, u may pass 88.81, where P' exceeds 448 and its code
// saturates; for |m_s| < 2^28 (the contract's score domain) u stays below 112 and 2^u is
// finite.  From the first tile where some row of a wave has |m_s| >= 2^22 the wave stays
// in this form: the codes are formed again from min(2^u, 448 * 2^80) and the tile's sum
// from P' = 2^-80 2^u, so d' is kept unscaled (a sum of up to 2^28 values of 2^112 would
// overflow).  It replaces the ordinary form's results, which are formed first.
__device__ __forceinline__ v8i large_score_form(const float (&p)[32], float& tsum) {
  float ds[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ds[j] = p[j] * kPScaleInv;
#pragma unroll
  for (int i = 4; i < 32; ++i) ds[i & 3] = ds[i & 3] + p[i] * kPScaleInv;
  tsum = (ds[0] + ds[1]) + (ds[2] + ds[3]);
  v8i pf;
#pragma unroll
  for (int w = 0; w < 8; ++w)
    pf[w] = pack_fp8x4(p[4 * w], p_code_input_saturating(p[4 * w]), p_code_input_saturating(p[4 * w + 1]),
                       p_code_input_saturating(p[4 * w + 2]), p_code_input_saturating(p[4 * w + 3]));
  return pf;
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Exact bf16 values of four packed e4m3 codes (bytes 0..3 -> elements 0..3 of two words).
__device__ __forceinline__ void fp8x4_to_bf16(int codes, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true));
}

// Workgroup barrier that waits only for this wave's LDS and scalar-memory operations
// (not for the in-flight tile loads, as the fence of __syncthreads would); the
// scheduling barriers keep the compiler from moving work across a phase boundary.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool PER_TOKEN, bool CAUSAL>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(FwdArgs a) {
  // The body uses device-only types (buffer resources); the host pass only needs the
  // kernel's launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NS = D / 32;        // QK k-steps = O accumulator blocks
  constexpr int KCH = D / 16;       // 16-byte chunks per K row
  constexpr int PT = D / 64;        // 16-byte chunks per loading thread per K tile
  constexpr int PTV = D / 32;       // 16-byte chunks per loading thread per bf16 V^T tile
  constexpr int QB = BM / kBlk;     // 64-row Q scale blocks per workgroup
  __shared__ __align__(16) uint8_t sK[NBUF][BN * D];   // K codes, swizzled for the QK reads
  __shared__ __align__(16) uint8_t sVb[NBUF][D * BN * 2];  // bf16 V^T of each slot, swizzled
  __shared__ __align__(16) float sC[NBUF][QB][BN];  // PER_TOKEN: c_j per (buffer, query block, key)
  __shared__ __align__(16) float sKs[NBUF][BN];     // PER_TOKEN: raw K scales of each slot

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it are scalar
  const int grp = wave >> 2;  // group 0 leads by one phase; group 1 loads the tiles
  const int gtid = tid & 255;  // thread index within the group
  const int l32 = lane & 31, hh = lane >> 5;
  const int nqb = (a.Nq + BM - 1) / BM;
  // wave-uniform by construction; readfirstlane lets the compiler keep it in SGPRs
  // work = ((bh * kv_splits + split) * nqb + qblk): workgroups that stream the same key
  // range of one (b, h) are neighbours, so an XCD's L2 serves all their query blocks
  const int work = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, gridDim.x));
  const int rest = __builtin_amdgcn_readfirstlane(work / nqb);
  // causal: the last query blocks see the most keys, so they are dispatched first and the
  // final wave of workgroups is the light one
  const int qblk = CAUSAL ? nqb - 1 - (work - rest * nqb) : work - rest * nqb;
  const int bh = __builtin_amdgcn_readfirstlane(rest / a.kv_splits);
  const int split = rest - bh * a.kv_splits;
  const int q0 = qblk * BM;
  const int qw = q0 + 32 * wave;  // first row of this wave
  const int qrow = qw + l32;      // this lane's query row
  const bool wave_live = qw < a.nq_pad;

  // Q fragment: lane half hh supplies channels [hh*D/2, hh*D/2 + D/2) of its row; QK
  // step s covers bytes [16 s, 16 s + 16) of that half (the same permutation of the
  // contraction index is applied to K below, so the INT32 dot products are unchanged).
  v4i qf[NS];
  if (wave_live) {
    const int8_t* qp = a.q8 + bh * a.q8_bh + (int64_t)qrow * D + hh * (D / 2);
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *(const v4i*)(qp + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = v4i{0, 0, 0, 0};
  }
  const float sq_w = wave_live ? a.q_scale[bh * a.qs_bh + qw / kBlk] : 0.0f;
  // group 1 thread t computes c for query block t / 64 and key t % 64 of each tile
  float sq_mine = 0.0f;
  if (PER_TOKEN && grp == 1 && q0 + kBlk * (gtid >> 6) < a.nq_pad)
    sq_mine = a.q_scale[bh * a.qs_bh + q0 / kBlk + (gtid >> 6)];

  // tiles streamed by the workgroup, and tiles holding a key visible to this wave
  // (absolute tile indices), then restricted to this workgroup's key range: the loop
  // below runs tiles t0 + i, i = 0 .. ntiles - 1
  int ntiles = (a.Nk + BN - 1) / BN;
  int wtiles = wave_live ? ntiles : 0;
  if (CAUSAL) {
    int64_t last = (int64_t)min(q0 + BM, a.Nq) - 1 + a.pos_off;
    if (last > a.Nk - 1) last = a.Nk - 1;
    ntiles = last < 0 ? 0 : (int)(last / BN) + 1;
    int64_t wlast = (int64_t)min(qw + 32, a.Nq) - 1 + a.pos_off;
    if (wlast > a.Nk - 1) wlast = a.Nk - 1;
    wtiles = (!wave_live || wlast < 0) ? 0 : (int)(wlast / BN) + 1;
  }
  const int t0 = __builtin_amdgcn_readfirstlane((int)((int64_t)split * a.tiles_total / a.kv_splits));
  const int t_end = (int)((int64_t)(split + 1) * a.tiles_total / a.kv_splits);
  ntiles = __builtin_amdgcn_readfirstlane(max(0, min(ntiles, t_end) - t0));
  wtiles = __builtin_amdgcn_readfirstlane(max(0, min(wtiles, t_end) - t0));

  // ---- staging: global -> LDS directly (buffer loads with the LDS destination) ----
  // Each group-1 wave fills PT 1 KiB segments of the K tile and PTV of the bf16 V^T tile;
  // lane l of a segment writes LDS slot 64 seg + l (16 bytes), so each lane fetches the
  // global chunk that the swizzled layout keeps in that slot.
  // Buffer resources are per (b, h) with 32-bit offsets; rows past the end of the
  // resource (a KV cache whose length is not a multiple of 64) read as zeros.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(a.k8 + bh * a.k8_bh), (short)0, a.k_rows * D, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(a.vbf + bh * a.vbf_bh),
                                                                       (short)0, (int)(2 * D * a.ldv), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(a.k_scale + bh * a.ks_bh), (short)0, PER_TOKEN ? a.Nk * 4 : 0, kRsrcWord3);
  int koff[PT], voff[PTV];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int slot = 64 * ((wave & 3) * PT + i) + lane;
    const int row = slot / KCH, pc = slot % KCH;
    koff[i] = row * D + 16 * (pc ^ kswz<D>(row));
  }
  // bf16 V^T rows are 128 bytes (8 slots): slot L holds chunk (L & 7) ^ vbswz(row) of
  // channel row L >> 3, i.e. keys 8 q .. 8 q + 7 of that channel
#pragma unroll
  for (int i = 0; i < PTV; ++i) {
    const int slot = 64 * ((wave & 3) * PTV + i) + lane;
    const int row = slot >> 3, q = (slot & 7) ^ vbswz(slot >> 3);
    voff[i] = row * (int)(2 * a.ldv) + 16 * q;
  }
  // Slot t: K tile t and its raw per-token K scales (t < ntiles), and the bf16 V^T of
  // tile t - 1 (t >= 1), into buffer buf = t % NBUF.  Every group-1 wave loads all 64
  // raw scales of the tile itself (the waves write identical bytes), so that its own
  // wait makes them visible to it.  All slot traffic goes through the direct-to-LDS
  // loads: a compiler-visible load whose value is used while tile loads are in flight
  // would make the compiler wait for all of them.
  // LDS byte addresses of the buffers, formed once (wave-uniform)
  // LDS byte addresses of this wave's segments of buffer 0 (wave-uniform); the buffer
  // and segment offsets are immediates of the loads
  const uint32_t ldsK = lds_addr(&sK[0][0]) + 1024u * ((wave & 3) * PT);
  const uint32_t ldsV = lds_addr(&sVb[0][0]) + 1024u * ((wave & 3) * PTV);
  const uint32_t ldsKs = lds_addr(&sKs[0][0]);
  auto stage = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    if (PER_TOKEN && t < ntiles) dma_4B<buf * (4 * BN)>(srs, ldsKs, 4 * lane, 4 * (t0 + t) * BN);
    static_for<PT>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      if (t < ntiles) dma_16B<buf * (BN * D) + 1024 * i>(krs, ldsK, koff[i], (t0 + t) * BN * D);
    });
    static_for<PTV>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      if (t > 0) dma_16B<buf * (2 * D * BN) + 1024 * i>(vrs, ldsV, voff[i], (t0 + t - 1) * BN * 2);
    });
  };
  // wait until at most the loads of slot t are in flight (t > ntiles: none)
  static_assert(PT + PTV + 1 < 64, "vmcnt immediate");
  auto wait_all_but = [&](int t) {
    if (t > ntiles)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else if (t == ntiles)  // last slot: V^T only
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PTV));
    else if (t > 0)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PT + PTV + (PER_TOKEN ? 1 : 0)));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PT + (PER_TOKEN ? 1 : 0)));
  };
  auto scale_store = [&](int t, int buf) {  // c of slot t (buffer buf), after its wait
    if (PER_TOKEN) sC[buf][gtid >> 6][gtid & (BN - 1)] = (sq_mine * sKs[buf][gtid & (BN - 1)]) * a.lambda;
  };
  float m = -INFINITY;  // running max (log2 domain)
  float dsum = 0.0f;    // this lane's share of d'' = 2^80 d' (its 32 keys of every tile)
  bool big = false;     // wave-uniform: the large-score form (see softmax_tile)
  float dscale = kPScaleInv;  // d' / (sum of dsum): 2^-80, or 1 in the large-score form
  v16f O[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[s][r] = 0.0f;
  v16i S0, S1;
  // With per-block K scales the first QK MFMA of each score block reads its start value
  // (the accumulator bias) from this register vector, set once; the empty asm makes it
  // opaque, so the compiler does not rebuild it every tile.  With per-token scales (32
  // more values per lane in registers) there is no room for it: the MFMA phase resets
  // the accumulators instead.
  v16i bias16;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias16[r] = kAccBias;
  if constexpr (!PER_TOKEN) asm volatile("" : "+v"(bias16));
  uint32_t pb[16];  // bf16 P of the last softmax: keys 32 hh + 2 j, 2 j + 1 in word j
#pragma unroll
  for (int j = 0; j < 16; ++j) pb[j] = 0u;

  // the first MFMA phase reads the V^T of slot 0 (no tile: never loaded) with P = 0: it
  // must hold finite values (uninitialized LDS may hold NaN patterns)
  if (16 * tid < 2 * D * BN) *(v4i*)&sVb[0][16 * tid] = v4i{0, 0, 0, 0};
  if (D * BN > 8 * NT) *(v4i*)&sVb[0][16 * (tid + NT)] = v4i{0, 0, 0, 0};
  // Q fragment and scales are in registers before any tile load: otherwise the
  // compiler's waits for them, placed inside the loop, would also wait for the tile
  // loads in flight
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  if (grp == 1 && ntiles > 0) {
    stage(0, std::integral_constant<int, 0>{});
    stage(1, std::integral_constant<int, 1>{});
    wait_all_but(1);
    scale_store(0, 0);
  }
  phase_barrier();

  const int krow0 = key_of_row(0, l32), krow1 = key_of_row(1, l32);
  const __attribute__((address_space(4))) float* ks_const =
      (const __attribute__((address_space(4))) float*)uniform_ptr(a.k_scale + bh * a.ks_bh);
  const int nkb = (a.Nk + BN - 1) / BN;  // K scale blocks
  float ks_next = (!PER_TOKEN && ntiles > 0) ? ks_const[t0] : 0.0f;
  // One interval of the tile loop (between two workgroup barriers) for slot i, which sits
  // in buffer BUF = i % NBUF.  The loop is unrolled NBUF times so that the buffer offsets
  // of every LDS access are immediates: the per-lane addresses stay in registers and no
  // interval recomputes them.
  auto iteration = [&](const int i, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    constexpr int buf1 = (buf + 1) % NBUF, buf2 = (buf + 2) % NBUF;
    // ---- MFMA phase i: S = K_i . Q^T and O^T += V_{i-1}^T . P_{i-1}^T ----
    // The MFMA phase has one branch-free form: the first one runs PV on a zeroed V^T
    // buffer with P = 0, the last one computes a QK that nobody reads, and a wave whose
    // rows see no key of the tile has P = 0 (separate forms would make the compiler copy
    // the O accumulators between register sets every iteration).
    auto mfma_phase = [&]() {
    const uint8_t* tK = sK[buf];
    const uint8_t* tV = sVb[buf];  // bf16 V^T of tile i - 1
    // lane (channel row, half hh) reads the bf16 V^T of keys 32 hh + 8 c .. + 7 of its row
    auto read_v = [&](int s, int c) {
      const int vrow = 32 * s + l32;
      return *(const v8bf*)(tV + vrow * (2 * BN) + 16 * ((4 * hh + c) ^ vbswz(vrow)));
    };
    // The phase is a pipeline of 2 NS QK steps and 4 NS PV steps; step k reads one
    // 16-byte operand from LDS and runs one MFMA on it.  Operands are read kPrefetch steps
    // ahead into a ring of registers, so that every read's latency hides behind the
    // MFMAs before its own.  QK steps alternate the two score blocks; PV steps run
    // chunk-major (each O block accumulates its four key chunks in order, as before).
    constexpr int kQkSteps = 2 * NS, kSteps = kQkSteps + 4 * NS, kPrefetch = 4;
    auto read_op = [&](auto k_c) -> v4i {
      constexpr int k = decltype(k_c)::value;
      if constexpr (k < kQkSteps) {
        const int krow = (k & 1) ? krow1 : krow0;
        const int ch = NS * hh + k / 2;
        return *(const v4i*)(tK + krow * D + 16 * (ch ^ kswz<D>(krow)));
      } else {
        return __builtin_bit_cast(v4i, read_v((k - kQkSteps) % NS, (k - kQkSteps) / NS));
      }
    };
    auto mfma_op = [&](auto k_c, const v4i& op) {
      constexpr int k = decltype(k_c)::value;
      if constexpr (k < kQkSteps) {
        constexpr bool first = !PER_TOKEN && k < 2;
        if constexpr (k & 1)
          S1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(op, qf[k / 2], first ? bias16 : S1, 0, 0, 0);
        else
          S0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(op, qf[k / 2], first ? bias16 : S0, 0, 0, 0);
      } else {
        constexpr int c = (k - kQkSteps) / NS, s = (k - kQkSteps) % NS;
        const v8bf pfrag = __builtin_bit_cast(v8bf, v4i{(int)pb[4 * c], (int)pb[4 * c + 1], (int)pb[4 * c + 2],
                                                        (int)pb[4 * c + 3]});
        O[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, op), pfrag, O[s], 0, 0, 0);
      }
    };
    {
      v4i ring[kPrefetch];
      static_for<kPrefetch>([&](auto k_c) { ring[decltype(k_c)::value] = read_op(k_c); });
      if constexpr (PER_TOKEN) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          S0[r] = kAccBias;
          S1[r] = kAccBias;
        }
      }
      static_for<kSteps>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        const v4i op = ring[k % kPrefetch];
        if constexpr (k + kPrefetch < kSteps) ring[k % kPrefetch] = read_op(std::integral_constant<int, k + kPrefetch>{});
        mfma_op(k_c, op);
      });
      // pin that order: the first reads, then each MFMA followed by the read kPrefetch
      // steps ahead (left alone, the scheduler places most reads right before their MFMA
      // and waits out each latency)
      __builtin_amdgcn_sched_group_barrier(0x100, kPrefetch, 0);
      static_for<kSteps>([&](auto k_c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (decltype(k_c)::value + kPrefetch < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      });
    }
    };

    // ---- VALU phase j: online softmax of tile j (its per-key scales in sC[jbuf]) ----
    auto valu_phase = [&](const int j, const int jbuf) {
    // per-tile K scale of this tile (loaded during the previous VALU phase) and of the
    // next one: uniform addresses read through the constant address space, i.e. scalar
    // loads, issued a phase ahead so that their latency is never waited for
    const float ks_cur = ks_next;
    if (!PER_TOKEN && t0 + j + 1 < nkb) ks_next = ks_const[t0 + j + 1];
    if (j < wtiles) {
      const int ti = t0 + j;  // absolute tile
      const int key0 = ti * BN + 32 * hh;
      const bool masked =
          (ti * BN + BN > a.Nk) || (CAUSAL && (int64_t)ti * BN + BN - 1 > (int64_t)qw + a.pos_off);
      const float c_tile = PER_TOKEN ? 0.0f : (sq_w * ks_cur) * a.lambda;
      const float* cp = &sC[jbuf][wave >> 1][32 * hh];
      float tsum;
      v8i pf;
      const float m_old = m;
      float p[32];
      if (masked) {
        const int vis_last = (int)min(CAUSAL ? (int64_t)qrow + a.pos_off : (int64_t)a.Nk - 1, (int64_t)a.Nk - 1);
        pf = softmax_tile<true, PER_TOKEN>(S0, S1, cp, c_tile, key0, vis_last, m, tsum, p);
      } else {
        pf = softmax_tile<false, PER_TOKEN>(S0, S1, cp, c_tile, key0, 0, m, tsum, p);
      }
      // alpha = 2^(m_old - m) rescales the old terms of d'' and O; it is exactly 1 for a
      // row whose maximum stayed (d'' * 1 = d''), so the exponential, the product and the
      // rescale run only when some row of the wave has a new maximum (then m is finite).
      // The large-score form (large_score_form) is entered on such a tile too: |m_s|
      // grows only with m.
      const bool moved = __ballot(m != m_old) != 0;
      if (moved && !big) {
        const float am = __builtin_fabsf(m);
        big = __ballot(am >= 0x1p22f && am < INFINITY) != 0;
      }
      if (__builtin_expect(big, 0)) pf = large_score_form(p, tsum);
      if (moved) {
        const float alpha = m == m_old ? 1.0f : __builtin_amdgcn_exp2f(m_old - m);
        // entering the large-score form: the sum so far holds P'' = 2^80 P' and is brought
        // to P' (exact for every partial sum above 2^-46; smaller ones lie far below d')
        if (big && dscale != 1.0f) {
          dsum *= kPScaleInv;
          dscale = 1.0f;
        }
        dsum = dsum * alpha + tsum;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int r = 0; r < 16; ++r) O[s][r] *= alpha;
      } else {
        dsum = dsum + tsum;
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) fp8x4_to_bf16(pf[w], pb[2 * w], pb[2 * w + 1]);
    } else {
#pragma unroll
      for (int w = 0; w < 16; ++w) pb[w] = 0u;  // no contribution from this tile
    }
    };

    // Group 0 runs MFMA phase i, then the softmax of tile i; group 1 the softmax of tile
    // i - 1, then MFMA phase i.  So the two waves of a SIMD start the interval in
    // different kinds of phase, and each wave's softmax of tile j precedes its MFMA
    // phase j + 1, which needs the P of tile j.  The priorities are those of the header.
    if (grp == 1 && i + 2 <= ntiles) stage(i + 2, std::integral_constant<int, buf2>{});
    if (grp == 0) {
      __builtin_amdgcn_s_setprio(2);
      mfma_phase();
      __builtin_amdgcn_s_setprio(0);
    } else {
      __builtin_amdgcn_s_setprio(1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0 || i >= 1) valu_phase(grp == 0 ? i : i - 1, grp == 0 ? buf : buf2);
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 1) {
      __builtin_amdgcn_s_setprio(2);
      mfma_phase();
      __builtin_amdgcn_s_setprio(0);
    }
    // group 1: slot i + 1 (issued one interval back) must have landed before the MFMA
    // phases i + 1 read it; its raw K scales give the c of tile i + 1
    if (grp == 1 && i < ntiles) {
      wait_all_but(i + 2);
      if (i + 1 < ntiles) scale_store(i + 1, buf1);
    }
    phase_barrier();
  };
  static_assert(NBUF == 3, "the tile loop is unrolled once per buffer");
  for (int i = 0;;) {
    iteration(i, std::integral_constant<int, 0>{});
    if (++i > ntiles) break;
    iteration(i, std::integral_constant<int, 1>{});
    if (++i > ntiles) break;
    iteration(i, std::integral_constant<int, 2>{});
    if (++i > ntiles) break;
  }

  // ---- epilogue: out = O * s_v / d' ----
  const float dt = sum_with_partner(dsum) * dscale;  // d' = d'' / 2^80 (exact), or d' itself
  if (a.kv_splits > 1) {  // partial result of this key range, combined by attn_combine_kernel
    if (qrow < a.Nq) {
      const int64_t prow = ((int64_t)split * (a.B * a.H) + bh) * a.nq_pad + qrow;
      float* po = a.part_o + prow * D;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = 32 * s + 8 * g + 4 * hh;
          *(float4*)(po + c0) = make_float4(O[s][4 * g], O[s][4 * g + 1], O[s][4 * g + 2], O[s][4 * g + 3]);
        }
      if (hh == 0) *(float2*)(a.part_md + 2 * prow) = make_float2(m, dt);
    }
  } else if (qrow < a.Nq) {
    const int b = bh / a.H, h = bh - b * a.H;
    const int64_t off = b * a.out_sb + (int64_t)qrow * a.out_sn + h * a.out_sh;
    const float* vs = a.v_scale + (int64_t)bh * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * s + 8 * g + 4 * hh;  // channels c0 .. c0 + 3
        float o[4];
        const float svv[4] = {vs[c0], vs[c0 + 1], vs[c0 + 2], vs[c0 + 3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = dt == 0.0f ? 0.0f : (O[s][4 * g + e] * svv[e]) / dt;
        if (a.out_bf16) {
          uint16_t* op = (uint16_t*)a.out + off + c0;
          const uint32_t w0 = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
          const uint32_t w1 = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
          *(uint2*)op = make_uint2(w0, w1);
        } else {
          float* op = (float*)a.out + off + c0;
          *(float4*)op = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// The FP8 code of P' that the softmax produces for exponent argument u: in the ordinary
// form (saturating = 0) and in the large-score form (saturating = 1).
__global__ void p8_codes_kernel(const float* u, uint8_t* codes, int64_t n, int saturating) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float p = p_from_u(u[i]);
    if (saturating) p = p_code_input_saturating(p);
    codes[i] = (uint8_t)(__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s_t{0, 0}, p, 0.0f,
                                                                                            kPScale, false)) &
                         0xff);
  }
}

// Split-KV combine: one thread per (b, h, query row, 4 channels).  Per row, in split
// order: M = max m_s; w_s = 2^(m_s - M) (0 for a range with no visible key); d' =
// sum w_s d'_s and O_c = sum w_s O_s,c in fp32; out_c = (O_c * s_v[c]) / d' (0 if d' = 0).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(FwdArgs a) {
  constexpr int G = D / 4;  // channel groups per row
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)a.B * a.H * a.Nq;
  if (t >= rows * G) return;
  const int g = (int)(t % G);
  const int64_t r = t / G;  // (bh, row)
  const int bh = (int)(r / a.Nq), row = (int)(r - (int64_t)bh * a.Nq);
  const int S = a.kv_splits;
  const int64_t BH = (int64_t)a.B * a.H;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_md[2 * ((s * BH + bh) * a.nq_pad + row)]);
  float d = 0.0f, o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const int64_t prow = (s * BH + bh) * a.nq_pad + row;
      const float2 md = *(const float2*)(a.part_md + 2 * prow);
      const float w = md.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(md.x - M);
      d = d + w * md.y;
      const float4 po = *(const float4*)(a.part_o + prow * D + 4 * g);
      o0 = o0 + w * po.x;
      o1 = o1 + w * po.y;
      o2 = o2 + w * po.z;
      o3 = o3 + w * po.w;
    }
  }
  const int b = bh / a.H, h = bh - b * a.H;
  const int c0 = 4 * g;
  const float* vs = a.v_scale + (int64_t)bh * D;
  const float o[4] = {d == 0.0f ? 0.0f : (o0 * vs[c0]) / d, d == 0.0f ? 0.0f : (o1 * vs[c0 + 1]) / d,
                      d == 0.0f ? 0.0f : (o2 * vs[c0 + 2]) / d, d == 0.0f ? 0.0f : (o3 * vs[c0 + 3]) / d};
  const int64_t off = b * a.out_sb + (int64_t)row * a.out_sn + h * a.out_sh + c0;
  if (a.out_bf16) {
    const uint32_t w0 = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
    const uint32_t w1 = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
    *(uint2*)((uint16_t*)a.out + off) = make_uint2(w0, w1);
  } else {
    *(float4*)((float*)a.out + off) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t st) {
  const int grid = a.B * a.H * ((a.Nq + BM - 1) / BM) * a.kv_splits;
  if (a.per_token) {
    if (a.causal)
      attn_fwd_kernel<D, true, true><<<grid, NT, 0, st>>>(a);
    else
      attn_fwd_kernel<D, true, false><<<grid, NT, 0, st>>>(a);
  } else {
    if (a.causal)
      attn_fwd_kernel<D, false, true><<<grid, NT, 0, st>>>(a);
    else
      attn_fwd_kernel<D, false, false><<<grid, NT, 0, st>>>(a);
  }
  if (a.kv_splits > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)a.B * a.H * a.Nq * (D / 4);
    attn_combine_kernel<D><<<(int)((threads + 255) / 256), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace detail
using namespace detail;

hipError_t launch_attn_fwd(const FwdArgs& a, int D, hipStream_t st) {
  return D == 128 ? launch_d<128>(a, st) : launch_d<64>(a, st);
}

hipError_t launch_p8_codes(const float* u, uint8_t* codes, int64_t n, int saturating, hipStream_t st) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  p8_codes_kernel<<<(int)blocks, 256, 0, st>>>(u, codes, n, saturating);
  return hipGetLastError();
}

}  // namespace qattn
