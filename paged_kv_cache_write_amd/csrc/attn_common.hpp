// attn_common.hpp -- device building blocks shared by the decode and prefill kernels.
//
// Work decomposition (bf16).  A "row" is one (query position, query head) pair; the 16 rows of
// one matrix-core column block sit on the 16 columns of a 16x16 MFMA tile:
//   S^T[key][row] = K[key][:] . Q[row][:]        (A = K rows from the page, B = Q^T)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]  (A = V^T rows from the transposed V page,
//                                                 B = P^T straight from the S^T registers)
// so every lane's accumulators belong to one row and the softmax rescale is lane-uniform, the
// probabilities never cross lanes, and only the running max needs two cross-lane steps.
// Scores are kept on the log2 scale (exp2 is the hardware exponential).
#pragma once

#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace ga {

constexpr float kLog2e = 1.4426950408889634f;

struct ScoreConsts {
  float c_scale;   // scale * log2(e)            (no cap)
  float inv_cap;   // scale / cap                (cap)
  float cap_log2;  // cap * log2(e)              (cap)
};

template <bool CAP>
__device__ __forceinline__ float to_log2(float s, const ScoreConsts& k) {
  if constexpr (CAP) return softcap_log2(s, k.inv_cap, k.cap_log2);
  else return s * k.c_scale;
}

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) { return *(const u32x4_t*)p; }
__device__ __forceinline__ u32x2_t ld8(const uint16_t* p) { return *(const u32x2_t*)p; }

template <int D>
struct Acc {
  float4_t o[D / 16];
  float m, l;
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) o[n] = float4_t{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }
};

// Online softmax over NS new log2-domain scores per lane (the lane's row is its column c16;
// its keys are spread over the 4 lane groups, hence the two xor steps for the max).
template <int D, int NS>
__device__ __forceinline__ void softmax_update(Acc<D>& acc, const float (&x)[NS], float (&p)[NS]) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < NS; ++i) mx = fmaxf(mx, x[i]);
  mx = xor_max(mx, 16);
  mx = xor_max(mx, 32);
  const float m_new = fmaxf(acc.m, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2(acc.m - m_use);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    p[i] = fast_exp2(x[i] - m_use);
    sum += p[i];
  }
  acc.l = acc.l * alpha + sum;
  acc.m = m_new;
#pragma unroll
  for (int n = 0; n < D / 16; ++n) acc.o[n] *= alpha;
}

// Mask word for two bf16 slots: keep slot a (bits 0..15) / slot b (bits 16..31).
__device__ __forceinline__ uint32_t keep2(bool a, bool b) {
  return (a ? 0x0000ffffu : 0u) | (b ? 0xffff0000u : 0u);
}

// Row stride (elements) of a wave's LDS page buffer in the K=V path: 16 bytes of padding
// shift consecutive rows by 4 banks so the column-wise reads of 4 rows hit distinct banks.
template <int D>
struct KeqvLds {
  static constexpr int kStride = D + 8;
  static constexpr int kElems = kPage * kStride;  // per wave
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ int64_t clamp_blk(int64_t blk, int64_t nb) {
  return blk < 0 ? 0 : (blk >= nb ? nb - 1 : blk);
}

struct AttnArgs {
  const uint16_t* q;
  const int32_t* cu;  // prefill
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* bt;
  const int32_t* ctx;
  int32_t* ws_pref;   // decode: visible-page prefix over sequences [batch + 1]
  float* ws_o;        // decode: partial outputs [pieces][G][D]
  float* ws_ml;       // decode: partial (max, sum) [pieces][G][2]
  uint16_t* out;
  int64_t num_blocks;
  int32_t max_blocks, batch, max_ctx, Hq, Hkv, G, window;
  int32_t ring;                // block-table rows are rings of max_blocks pages
  int32_t nworkers;            // decode
  int32_t max_q_len, total_q;  // prefill
  ScoreConsts sc;
};

// Keys of sequence b that a decode query at position L-1 sees, and the pages holding them:
// L = min(context_len, max_ctx); keys lo .. L-1; pages p0 .. p0 + npg - 1 ([INFLM] Gemma-3 §3:
// a sliding layer reads only the last min(L, W) keys).
__device__ __forceinline__ void decode_range(const AttnArgs& a, int b, int& L, int& lo, int& p0,
                                             int& npg) {
  L = a.ctx[b];
  L = L > a.max_ctx ? a.max_ctx : L;
  if (L < 1) {
    L = 0; lo = 0; p0 = 0; npg = 0;
    return;
  }
  lo = a.window > 0 ? (L - a.window > 0 ? L - a.window : 0) : 0;
  p0 = lo / kPage;
  npg = (L + kPage - 1) / kPage - p0;
}

AttnArgs make_attn_args(const AttnLaunch& L);

// Q^T fragments of this lane's row: B operand of S^T = K Q^T (k = d, column = row).
template <int D>
__device__ __forceinline__ void load_q(bf16x8_t (&qf)[D / 32], const uint16_t* qrow, bool ok) {
  const int j = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const u32x4_t v = ok ? ld16(qrow + 32 * c + 8 * j) : u32x4_t{0u, 0u, 0u, 0u};
    qf[c] = as_bf16x8(v);
  }
}


}  // namespace ga
