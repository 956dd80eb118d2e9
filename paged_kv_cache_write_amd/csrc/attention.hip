// attention.hip -- the fp32 attention path (decode and prefill) and the host-side argument
// packing shared by the bf16 decode and prefill launchers.
//
// Sources: [INFLM] = "Feat/add gemma3 model" (InfiniLM pull request 581): Gemma-2 §1 (soft cap
// of the scaled scores before the softmax), Gemma-3 §3 (band + causal mask; decode reads only
// the last min(len, W) keys; head-first GQA).  [KUNLUN] = "Gemma 4 模型架构解析" §6.5 (K/V are
// read through the block table).
#include <math.h>

#include "attn_common.hpp"

namespace ga {
namespace {

// ---------------------------------------------------------------------------- fp32 -------

// Plain fp32 path (one wavefront per (query, head), one key at a time, fp32 everywhere):
// used for float caches, where the matrix cores would not keep fp32 products exact.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* q, const int32_t* cu,
                                                       const float* kc, const float* vc,
                                                       const int32_t* bt, const int32_t* ctx,
                                                       float* out, int64_t num_blocks,
                                                       int max_blocks, int ring, int batch,
                                                       int Hq,
                                                       int Hkv, int window, int k_eq_v,
                                                       int decode, int total_q, int max_len,
                                                       float scale, float cap, int rope_pairs,
                                                       float rope_theta, float rope_scale,
                                                       const float* kv_kw, const float* kv_vw) {
  constexpr int C = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rq = (int)(wid / Hq), h = (int)(wid - (wid / Hq) * Hq);
  if (rq >= total_q) return;
  int b, i, n;
  if (decode) {
    b = rq; i = 0; n = 1;
  } else {
    int lo = 0, hi = batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= rq) lo = mid; else hi = mid;
    }
    b = lo; i = rq - cu[b]; n = cu[b + 1] - cu[b];
  }
  int L = ctx[b];
  if (decode && L > max_len) {
    debug_flag(kDbgBound);
    L = max_len;
  }
  const int t = L - n + i;
  float* dst = out + ((int64_t)rq * Hq + h) * D + lane * C;
  if (t < 0 || L < 1) {
    debug_flag(kDbgLength);
#pragma unroll
    for (int e = 0; e < C; ++e) dst[e] = 0.f;
    return;
  }
  const int g = h / (Hq / Hkv);
  const int lo = window > 0 ? (t - window + 1 > 0 ? t - window + 1 : 0) : 0;
  float qv[C], o[C];
#pragma unroll
  for (int e = 0; e < C; ++e) {
    qv[e] = q[((int64_t)rq * Hq + h) * D + lane * C + e];
    o[e] = 0.f;
  }
  // exact K=V (k_eq_v = 2): stored keys are unrotated; pair k of this lane's dimensions
  // (lanes 0-31 hold the first halves of the pairs, lanes 32-63 the second) turns by
  // key * omega_k for the scores, in double
  const bool exact = k_eq_v == 2;
  const bool first_half = lane < 32;
  double omega[C];
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const int k = (lane & 31) * C + e;
    omega[e] = (exact && k < rope_pairs)
                   ? pow((double)rope_theta, -2.0 * k / (double)D) / (double)rope_scale
                   : 0.0;
  }
  float m = -INFINITY, l = 0.f;
  for (int key = lo; key <= t; ++key) {
    const int page = key / kPage;
    if (!ring && page >= max_blocks) {
      debug_flag(kDbgBound);
      break;
    }
    const int64_t blk =
        clamp_blk(bt[(int64_t)b * max_blocks + bt_col(page, max_blocks, ring)], num_blocks);
    const int off = key - page * kPage;
    const float* kp = kc + (blk * Hkv + g) * kPage * D;  // K page (k_page_elem layout)
    float kv[C];
#pragma unroll
    for (int e = 0; e < C; ++e) kv[e] = kp[k_page_elem<4>(off, lane * C + e, page)];
    float ks[C];  // the key as the scores see it
#pragma unroll
    for (int e = 0; e < C; ++e) ks[e] = kv[e];
    if (exact && rope_pairs > 0) {
#pragma unroll
      for (int e = 0; e < C; ++e) {
        const float partner = __shfl_xor(kv[e], 32, kWave);
        double sn, cs;
        sincos((double)key * omega[e], &sn, &cs);
        ks[e] = first_half ? (float)((double)kv[e] * cs - (double)partner * sn)
                           : (float)((double)kv[e] * cs + (double)partner * sn);
      }
    }
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < C; ++e) part = fmaf(qv[e], ks[e], part);
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) part += __shfl_xor(part, msk, kWave);
    float sc = part * scale;
    if (cap > 0.f) sc = cap * tanhf(sc / cap);
    const float m_new = fmaxf(m, sc);
    const float alpha = expf(m - m_new);
    const float pw = expf(sc - m_new);
    l = l * alpha + pw;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      const float vv = k_eq_v ? kv[e] : vc[((blk * Hkv + g) * D + lane * C + e) * kPage + off];
      o[e] = o[e] * alpha + pw * vv;
    }
    m = m_new;
  }
#pragma unroll
  for (int e = 0; e < C; ++e) {
    float f = 1.f;  // exact K=V: values are the stored keys times w_v / w_k
    if (kv_vw) f = kv_vw[lane * C + e] / kv_kw[lane * C + e];
    dst[e] = o[e] / l * f;
  }
}

template <int D>
hipError_t launch_f32_t(const AttnLaunch& L, bool decode, hipStream_t s) {
  const int total_q = decode ? L.batch : L.total_q;
  const int64_t waves = (int64_t)total_q * L.Hq;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (const float*)L.q, L.cu_seqlens_q, (const float*)L.k_cache,
                     (const float*)L.v_cache, L.block_table, L.context_lens, (float*)L.out,
                     L.num_blocks, L.max_blocks, L.ring, L.batch, L.Hq, L.Hkv, L.window, L.k_eq_v,
                     decode ? 1 : 0, total_q, L.max_context_len, L.scale, L.softcap,
                     L.rope_theta > 0.f ? L.rope_angles : 0, L.rope_theta, L.rope_scale,
                     L.kv_kw, L.kv_vw);
  return hipGetLastError();
}

}  // namespace

GA_DEBUG_TAKE_DEFINE(debug_take_attention)

AttnArgs make_attn_args(const AttnLaunch& L) {
  AttnArgs a;
  a.q = (const uint16_t*)L.q;
  a.cu = L.cu_seqlens_q;
  a.kc = (const uint16_t*)L.k_cache;
  a.vc = (const uint16_t*)L.v_cache;
  a.bt = L.block_table;
  a.ctx = L.context_lens;
  a.ws_pref = nullptr;
  a.ws_o = nullptr;
  a.ws_ml = nullptr;
  a.out = (uint16_t*)L.out;
  a.num_blocks = L.num_blocks;
  a.max_blocks = L.max_blocks;
  a.ring = L.ring;
  a.batch = L.batch;
  a.max_ctx = L.max_context_len;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.G = L.Hq / L.Hkv;
  a.window = L.window;
  a.nworkers = 0;
  a.max_q_len = L.max_q_len;
  a.total_q = L.total_q;
  a.kv_mode = L.k_eq_v;
  a.rope_pairs = (L.k_eq_v == 2 && L.rope_theta > 0.f) ? L.rope_angles : 0;
  a.rho0 = 1.0 / (2.0 * M_PI * (double)L.rope_scale);
  a.rho_step = a.rope_pairs > 0 ? pow((double)L.rope_theta, -2.0 / (double)L.D) : 1.0;
  a.kv_kw = L.kv_kw;
  a.kv_vw = L.kv_vw;
  if (L.softcap > 0.f) {
    a.sc.c_scale = 0.f;
    a.sc.inv_cap = L.scale / L.softcap;
    a.sc.cap_log2 = L.softcap * kLog2e;
  } else {
    a.sc.c_scale = L.scale * kLog2e;
    a.sc.inv_cap = 0.f;
    a.sc.cap_log2 = 0.f;
  }
  return a;
}

hipError_t launch_attn_f32(const AttnLaunch& L, bool decode, hipStream_t s) {
  switch (L.D) {
    case 128: return launch_f32_t<128>(L, decode, s);
    case 256: return launch_f32_t<256>(L, decode, s);
    case 512: return launch_f32_t<512>(L, decode, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ga
