// prefill_common.hpp -- pieces shared by the prefill kernels: tile size, the key order of the
// QK^T products, and the HBM -> LDS copy, scalar-load and wait primitives.
#pragma once

#include <utility>

#include "attn_common.hpp"

namespace ga {

constexpr int kTileKeys = 2 * kPage;  // 32 keys per tile: P.V runs on 16x16x32 MFMAs

// How raw scores s = q.k enter the softmax (exponentials are base 2):
//   kScorePlain  x = s * scale * log2(e);      weight exp2(x - mu)
//   kScoreFold   x = s (raw; scale > 0, so the max commutes with it); the row max is scaled
//                once, and the weight is exp2(s * scale * log2(e) - mu), one fused multiply-add
//   kScoreCap    x = cap * log2(e) * tanh(s * scale / cap) ([INFLM] Gemma-2 §1);
//                weight exp2(x - mu)
// Masked scores are -inf in every mode; mu is the row's reference on the log2 scale.
constexpr int kScorePlain = 0, kScoreFold = 1, kScoreCap = 2;

template <int SM>
__device__ __forceinline__ float score_in(float s, const ScoreConsts& k) {
  if constexpr (SM == kScoreCap) return softcap_log2(s, k.inv_cap, k.cap_log2);
  else if constexpr (SM == kScoreFold) return s;
  else return s * k.c_scale;
}
// the row max of the x values, on the log2 scale
template <int SM>
__device__ __forceinline__ float score_max(float mx, const ScoreConsts& k) {
  if constexpr (SM == kScoreFold) return mx * k.c_scale;
  else return mx;
}
template <int SM>
__device__ __forceinline__ float score_exp_arg(float x, float mu, const ScoreConsts& k) {
  if constexpr (SM == kScoreFold) return __builtin_fmaf(x, k.c_scale, -mu);
  else return x - mu;
}

// Max of 8 scores and over the 4 lane groups with the NaN-propagating maximum: gfx950 has a
// native three-input form, and unlike fmaxf it needs no quieting of its operands first.  A
// score is NaN only when a visible key or the query holds NaN, and the output row is NaN then
// either way.
__device__ __forceinline__ float fmax_nc(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float max8_nc(const float (&x)[8]) {
  return fmax_nc(fmax_nc(fmax_nc(x[0], x[1]), fmax_nc(x[2], x[3])),
                 fmax_nc(fmax_nc(x[4], x[5]), fmax_nc(x[6], x[7])));
}
__device__ __forceinline__ float max_over_groups_nc(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = fmax_nc(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const uint32_t w = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmax_nc(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Scheduling fence: the compiler moves no instruction across it.  The tile loops are cut into
// chunks with it so that operand reads stay the intended distance ahead of their products.
__device__ __forceinline__ void fence_sched() { __builtin_amdgcn_sched_barrier(0); }

// Compile-time loop: f(integral_constant<int, 0>) .. f(integral_constant<int, N-1>), so that
// every register-array index in the body is a constant whatever the size of the body (an
// unroll pragma gives up on large bodies and leaves the arrays in scratch memory).
template <class F, int... Is>
__device__ __forceinline__ void sfor_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (N > 0) sfor_impl(f, std::make_integer_sequence<int, N>{});
}

// Row of page c16 / 8 that QK^T product m (0, 1) places at MFMA row c16: keys {0-3, 8-11} of
// each page for m = 0 and {4-7, 12-15} for m = 1.
__device__ __forceinline__ int qk_row_key(int c16, int m) {
  return (c16 & 3) + 8 * ((c16 >> 2) & 1) + 4 * m;
}

// One HBM -> LDS copy of 1 KiB from a wave-uniform 64-bit base (scalar registers) plus a
// 32-bit per-lane byte offset: each lane moves 16 bytes to M0 + 16 * lane.  Issued through
// inline assembly so that the compiler does not add waits of its own for the LDS it writes:
// the kernel waits on the vector-memory counter explicitly before the barrier that publishes
// a tile.  No memory clobber: a copy only ever writes a ring stage that no LDS access of the
// same iteration touches, and being volatile it stays ordered with the barriers and explicit
// waits that separate iterations.  An LDS DMA must not issue in the instruction right after
// a scalar write of M0 (one wait state; the compiler pads its own such pairs with s_nop 0),
// hence the nop.  M0 is set inside the statement each time: nothing in these kernels leaves
// a value of the compiler's own in M0 (on this target it uses M0 for LDS DMA, messages and
// indirect register indexing, which the kernels do not ask of it).
__device__ __forceinline__ void lds_copy16_sv(const void* base, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_off)
               : "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace ga
