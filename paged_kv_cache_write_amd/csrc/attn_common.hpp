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
  float m, l;  // the reference o and l are scaled to (exp2(-m)), and the weight sum
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) o[n] = float4_t{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }
};

// Lazy online softmax: the reference of a row moves only when a weight exp2(x - m_ref) would
// exceed 2^kLazyLog2.  Weights, row sums and O^T then stay below 2^64, 2^(64+log2 keys) and
// 2^(64+log2 keys+log2 max|v|), far inside fp32 (and bf16) range, and rounding is relative,
// so the size of a weight costs no precision; a large threshold makes the rescale of O^T (one
// multiply per accumulator register) rare: the reference moves about once per row, on its
// first visible keys.
constexpr float kLazyLog2 = 64.0f;

// Online softmax over NS new log2-domain scores per lane (the lane's row is its column c16;
// its keys are spread over the 4 lane groups, hence the max over the groups), with the
// lazily moved reference above: the accumulators are rescaled only in the rare step where
// some lane's reference moves.  The weights come out as packed bf16 pairs (pw[w] holds keys
// 2w, 2w+1), and the row sum adds those same rounded weights, so the numerator and the
// denominator of the output use one set of weights.
template <int D, int NS>
__device__ __forceinline__ void softmax_update(Acc<D>& acc, const float (&x)[NS],
                                               uint32_t (&pw)[NS / 2]) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < NS; ++i) mx = fmaxf(mx, x[i]);
  mx = max_over_groups(mx);
  const bool grow = mx > acc.m + kLazyLog2;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float alpha = grow && acc.m != -INFINITY ? fast_exp2(acc.m - mx) : 1.f;
    acc.l *= alpha;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc.o[n] *= alpha;
    if (grow) acc.m = mx;
  }
  const float mu = acc.m == -INFINITY ? 0.f : acc.m;
  float sum = acc.l;
#pragma unroll
  for (int w = 0; w < NS / 2; ++w) {
    const bf16x2_t b = cvt_bf16x2(fast_exp2(x[2 * w] - mu), fast_exp2(x[2 * w + 1] - mu));
    sum = sum_bf16x2(b, sum);
    pw[w] = __builtin_bit_cast(uint32_t, b);
  }
  acc.l = sum;
}

// Mask word for two bf16 slots: keep slot a (bits 0..15) / slot b (bits 16..31).
__device__ __forceinline__ uint32_t keep2(bool a, bool b) {
  return (a ? 0x0000ffffu : 0u) | (b ? 0xffff0000u : 0u);
}

// One page [16 keys][D] per wave for the K=V value reads, rows padded so that the rows of
// a transposing read (4 keys x 4 columns per 16 lanes) fall 32 bytes apart in the banks.
template <int D>
struct KeqvLds {
  static constexpr int kStride = D + 16;
  static constexpr int kElems = kPage * kStride;  // per wave
};

__device__ __forceinline__ int64_t clamp_blk(int64_t blk, int64_t nb) {
  if (blk < 0 || blk >= nb) {
    debug_flag(kDbgBlockId);
    return blk < 0 ? 0 : nb - 1;
  }
  return blk;
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
  // Exact K=V (k_eq_v = 2, [MNN] §6.2): the cache holds normalised keys without RoPE.  Pair k
  // (dimensions k and k + D/2, k < rope_pairs) of a key at position t turns, for the scores,
  // by 2 pi t rho_k with rho_k = rho0 * rho_step^k revolutions per position (rho0 =
  // 1 / (2 pi rope_scale), rho_step = theta^(-2/D)); values are the stored keys times
  // kv_vw[d] / kv_kw[d] (factor 1 when both are null).
  int32_t kv_mode;     // 0 separate V, 1 K=V, 2 exact K=V
  int32_t rope_pairs;  // 0: no rotation
  double rho0, rho_step;
  const float* kv_kw;
  const float* kv_vw;
};

// cos and sin of 2 pi rev, for a revolution count formed in double: reduced to [0, 1) in
// double, then the hardware sine and cosine (whose argument is in revolutions).
__device__ __forceinline__ void cos_sin_rev(double rev, float& c, float& s) {
  const float fr = (float)__builtin_amdgcn_fract(rev);
  s = __builtin_amdgcn_sinf(fr);
  c = __builtin_amdgcn_cosf(fr);
}

// Exact K=V: rotate the 8 pairs of two bf16 units of one key, unit `a` holding dimensions
// 8x .. 8x+7 (pairs k = 8x + e) and unit `b` their partners k + D/2, for a key at position t:
// a <- a cos - b sin, b <- b cos + a sin.  Each rotated value y goes back as two bf16 terms,
// hi = bf16(y) (into ua / ub) and lo = bf16(y - hi) (into la / lb): the matrix cores take both,
// so the scores see the rotated key to about 16 bits instead of rounding it a second time.
// rho_x = rho0 * rho_step^(8x).
__device__ __forceinline__ void rope_units_exact(u32x4_t& ua, u32x4_t& ub, u32x4_t& la,
                                                 u32x4_t& lb, int x, double rho_x,
                                                 double rho_step, int rope_pairs, int64_t t) {
  double rho = rho_x;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float c[2], s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 8 * x + 2 * w + h;
      if (k < rope_pairs) {
        cos_sin_rev((double)t * rho, c[h], s[h]);
      } else {
        c[h] = 1.f;
        s[h] = 0.f;
      }
      rho *= rho_step;
    }
    const float a0 = __uint_as_float(ua[w] << 16), a1 = __uint_as_float(ua[w] & 0xffff0000u);
    const float b0 = __uint_as_float(ub[w] << 16), b1 = __uint_as_float(ub[w] & 0xffff0000u);
    const float ya0 = a0 * c[0] - b0 * s[0], ya1 = a1 * c[1] - b1 * s[1];
    const float yb0 = b0 * c[0] + a0 * s[0], yb1 = b1 * c[1] + a1 * s[1];
    ua[w] = __builtin_bit_cast(uint32_t, cvt_bf16x2(ya0, ya1));
    ub[w] = __builtin_bit_cast(uint32_t, cvt_bf16x2(yb0, yb1));
    la[w] = __builtin_bit_cast(uint32_t, cvt_bf16x2(ya0 - __uint_as_float(ua[w] << 16),
                                                    ya1 - __uint_as_float(ua[w] & 0xffff0000u)));
    lb[w] = __builtin_bit_cast(uint32_t, cvt_bf16x2(yb0 - __uint_as_float(ub[w] << 16),
                                                    yb1 - __uint_as_float(ub[w] & 0xffff0000u)));
  }
}

// rho0 * rho_step^k in double (the frequency of pair k in revolutions per position).
__device__ __forceinline__ double rope_rho(const double rho0, const double rho_step, int k) {
  double r = rho0, p = rho_step;
  for (int e = k; e > 0; e >>= 1) {  // exponentiation by squaring
    if (e & 1) r *= p;
    p *= p;
  }
  return r;
}

// Keys of sequence b that a decode query at position L-1 sees, and the pages holding them:
// L = min(context_len, max_ctx); keys lo .. L-1; pages p0 .. p0 + npg - 1 ([INFLM] Gemma-3 §3:
// a sliding layer reads only the last min(L, W) keys).
__device__ __forceinline__ void decode_range(const AttnArgs& a, int b, int& L, int& lo, int& p0,
                                             int& npg) {
  L = a.ctx[b];
  if (L > a.max_ctx) {
    debug_flag(kDbgBound);
    L = a.max_ctx;
  }
  if (L < 1) {
    debug_flag(kDbgLength);
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
