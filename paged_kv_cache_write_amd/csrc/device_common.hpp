// device_common.hpp -- small device helpers shared by the gfx950 kernels of this library.
//
// Everything here is CDNA4-specific: 64-lane wavefronts, the bf16 matrix-core instructions
// v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x16_bf16 and their register layouts.
//
// MFMA register layouts used throughout (l = lane 0..63, j = l / 16, c = l % 16):
//   16x16x32 bf16:  A[i][k]: lane l holds row i = c, k = 8j .. 8j+7   (8 bf16)
//                   B[k][n]: lane l holds col n = c, k = 8j .. 8j+7   (8 bf16)
//   16x16x16 bf16:  A[i][k]: row i = c, k = 4j .. 4j+3                (4 bf16)
//                   B[k][n]: col n = c, k = 4j .. 4j+3                (4 bf16)
//   output D[i][n] (both): lane l holds D[4j + r][c] in register r = 0..3.
// The contraction index k is only ever used to pair A with B, so any assignment of k-slots
// to actual elements is correct as long as A and B use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace ga {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float float2_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kWave = 64;
constexpr int kPage = 16;  // tokens per page (block_size)

// ------------------------------------------------------------------------ bf16 <-> fp32 ---

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> bf16x2 with the hardware conversion (round to nearest even; NaN stays NaN).
__device__ __forceinline__ bf16x2_t cvt_bf16x2(float lo, float hi) {
  return __builtin_convertvector(float2_t{lo, hi}, bf16x2_t);
}

// The same conversion, packed (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, cvt_bf16x2(lo, hi));
}

// acc + w.x + w.y in fp32 (one dot-product instruction).
__device__ __forceinline__ float sum_bf16x2(bf16x2_t w, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(w, one, acc, false);
}

// double -> bf16 with a single rounding (nearest, ties to even): round to fp32 toward zero,
// make the result sticky (round-to-odd) if anything was dropped, then round to bf16.  fp32
// keeps 16 more bits than bf16, so the second rounding sees the exact tie/no-tie information.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  if (x != x) return (uint16_t)0x7fc0u;
  float fz = __double2float_rz(x);
  uint32_t u = __float_as_uint(fz);
  if ((double)fz != x && (u & 0x7f800000u) != 0x7f800000u) u |= 1u;
  return f32_to_bf16(__uint_as_float(u));
}

// ------------------------------------------------------------------------ K page layout -----
// A K page (16 keys of one kv head) is stored in 16-byte units: unit (row r, x) holds elements
// [x U, x U + U) of key row r, U = 16 / element size (8 for bf16, 4 for fp32), and sits at
// byte 256 x + 16 k_slot(r, x, lp) of the page, lp being the page's logical index
// (position / 16) in its sequence: the 16 rows of one unit column x form one 256-byte run and
// a 1 KiB run holds four consecutive unit columns of all 16 rows.  The rows are rotated by 4
// on pages of odd logical index and again in unit columns whose bit 3 is set.  A 32-key tile
// (an even page, then an odd one) copied to LDS as it is stored is then read without bank
// conflicts both by the score fragments (16 lanes: 8 rows of each page, one unit column) and,
// in the K=V forms, by the transposing value reads (16 lanes: 4 rows of units x and x + 8).
__device__ __forceinline__ int k_slot(int r, int x, int64_t lp) {
  return (r + 4 * (int)(lp & 1) + 4 * ((x >> 3) & 1)) & 15;
}
template <int ESIZE>
__device__ __forceinline__ int64_t k_page_elem(int r, int d, int64_t lp) {
  constexpr int U = 16 / ESIZE;
  const int x = d / U;
  return (int64_t)x * (16 * U) + (int64_t)k_slot(r, x, lp) * U + (d % U);
}

// Block-table column of logical page lp: lp itself, or lp mod max_blocks when the table row is
// a ring (sliding-window page recycling: a sliding layer keeps only the pages its window and
// the current chunk need, and position t reuses the block of position t - 16 max_blocks).
// The page's parity in the K layout above stays that of lp, not of its column.
__device__ __forceinline__ int bt_col(int lp, int max_blocks, int ring) {
  return ring ? (int)((unsigned)lp % (unsigned)max_blocks) : lp;
}

// ------------------------------------------------------------------------ debug checks ------
// Built with GA_DEBUG_BOUNDS, the kernels also check the device-resident metadata they read and
// record what they find as bits of a device word, one per source file (the kernels are compiled
// file by file, without device linking); ga_debug_take_error reads and clears the words.  The
// regular build compiles no check.  Either way every kernel keeps its own clamps, so bad
// metadata never leads to an access outside the buffers it was given.
// (the bits are the kDbg* constants of launch.hpp)
#ifdef GA_DEBUG_BOUNDS
static __device__ uint32_t g_debug_word;
__device__ __forceinline__ void debug_flag(uint32_t bits) { atomicOr(&g_debug_word, bits); }
// host: the word of this source file on the current device, cleared (synchronous)
#define GA_DEBUG_TAKE_DEFINE(fn)                                                             \
  uint32_t fn() {                                                                            \
    uint32_t v = 0;                                                                          \
    const uint32_t zero = 0;                                                                 \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_word), sizeof(v), 0,                      \
                            hipMemcpyDeviceToHost) != hipSuccess ||                          \
        hipMemcpyToSymbol(HIP_SYMBOL(g_debug_word), &zero, sizeof(zero), 0,                  \
                          hipMemcpyHostToDevice) != hipSuccess)                              \
      return kDbgReadFailed;                                                                 \
    return v;                                                                                \
  }
#else
__device__ __forceinline__ void debug_flag(uint32_t) {}
#define GA_DEBUG_TAKE_DEFINE(fn) \
  uint32_t fn() { return 0u; }
#endif

// ------------------------------------------------------------------------ MFMA --------------

__device__ __forceinline__ float4_t mfma_16x16x32(const bf16x8_t& a, const bf16x8_t& b,
                                                  const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4_t mfma_16x16x16(const short4_t& a, const short4_t& b,
                                                  const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}
// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i receives,
// as its element e (0..3), element i % 4 of the four 16-bit elements at the address given by
// lane 4e + i / 4 of the group: if lane 4e + q points at four consecutive columns 4q .. 4q+3
// of row e of a row-major block, lane i gets column i of rows 0..3, the layout of a
// matrix-core operand whose reduction index runs over those rows.  (Layout measured on gfx950
// with an in-bounds probe.)  `lds_byte` is an LDS byte address, 8-byte aligned.
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* lds_byte) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(
          (void*)lds_byte));
  return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ short4_t as_short4(const u32x2_t& v) {
  return __builtin_bit_cast(short4_t, v);
}

// LDS written by this wave is visible to this wave's later LDS reads (and its earlier reads
// have completed): a wave-local barrier with workgroup-scope fences.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ------------------------------------------------------------------------ cross-lane -------

// Max over the 4 lane groups (lanes c, c+16, c+32, c+48) without LDS: the two permlane swaps
// exchange rows of 16 and halves of 32 lanes.
__device__ __forceinline__ float max_over_groups(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const uint32_t w = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Soft cap on the log2 scale: returns cap_log2 * tanh(s * inv_cap), tanh from exp2 with
// saturation (exp2 overflow -> +inf -> tanh = 1).  cap_log2 = cap * log2(e), inv_cap = scale/cap.
__device__ __forceinline__ float softcap_log2(float s, float inv_cap, float cap_log2) {
  const float x = s * inv_cap;
  const float e = __builtin_amdgcn_exp2f(fabsf(x) * 2.8853900817779268f);  // exp(2|x|)
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  return cap_log2 * copysignf(t, x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace ga
