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

// Plain fp32 path (one workgroup per (query, head), fp32 everywhere): used for float caches,
// where the matrix cores would not keep fp32 products exact.  The 4 waves take turns over the
// steps of kF32Keys keys (wave w the steps w, w + 4, ..) with online softmaxes of their own,
// which are merged at the end through LDS.
constexpr int kF32Keys = 8;  // keys per step of the key loop
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wid = blockIdx.x;
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
  // Keys go U at a time: their loads are issued together, then their scores are reduced and
  // folded into the running softmax at once, so a key costs a fraction of a memory round trip.
  // The block ids of 64 pages at a time sit one per lane and are broadcast with readlane.
  int key_end = t;
  if (!ring && t / kPage >= max_blocks) {
    debug_flag(kDbgBound);
    key_end = max_blocks * kPage - 1;
  }
  const int64_t bt_row = (int64_t)b * max_blocks;
  const int p_last = key_end / kPage;
  auto ids_at = [&](int pw) -> int {  // lane i: block id of page pw + i (clamped)
    const int p = pw + lane < p_last ? pw + lane : p_last;
    return bt[bt_row + bt_col(p, max_blocks, ring)];
  };
  int pw = lo / kPage;
  int ids = ids_at(pw);
  float m = -INFINITY, l = 0.f;
  // steps start at multiples of kF32Keys, so a step's keys lie in one page; keys of a step
  // outside [lo, key_end] are masked (their slots hold written keys, or anything past L)
  static_assert(kPage % kF32Keys == 0, "a step within one page");
  for (int k0 = (lo & ~(kF32Keys - 1)) + wave * kF32Keys; k0 <= key_end; k0 += 4 * kF32Keys) {
    const int page = k0 / kPage, off0 = k0 - page * kPage;
    if (page - pw >= kWave) {  // the step's page leaves the window: move it
      pw = page;
      ids = ids_at(pw);
    }
    const int64_t blk = clamp_blk(__builtin_amdgcn_readlane(ids, page - pw), num_blocks);
    const float* kp = kc + (blk * Hkv + g) * kPage * D;  // K page (k_page_elem layout)
    // every load of the step is issued before any is used
    float kv[kF32Keys][C];
#pragma unroll
    for (int u = 0; u < kF32Keys; ++u)
#pragma unroll
      for (int e = 0; e < C; ++e) kv[u][e] = kp[k_page_elem<4>(off0 + u, lane * C + e, page)];
    // values: dimension d of the step's keys is kF32Keys consecutive floats of the V^T page
    // (with K=V the loads read the K page instead and go unused: no branch between them)
    float4_t vq[C][kF32Keys / 4];
#pragma unroll
    for (int e = 0; e < C; ++e) {
      const float* vp = k_eq_v ? kp + 4 * kF32Keys * e
                               : vc + ((blk * Hkv + g) * D + lane * C + e) * kPage + off0;
#pragma unroll
      for (int w = 0; w < kF32Keys / 4; ++w) vq[e][w] = ((const float4_t*)vp)[w];
    }
    float part[kF32Keys];
#pragma unroll
    for (int u = 0; u < kF32Keys; ++u) {
      float ks[C];  // the key as the scores see it
#pragma unroll
      for (int e = 0; e < C; ++e) ks[e] = kv[u][e];
      if (exact && rope_pairs > 0) {
        const int key = k0 + u;
#pragma unroll
        for (int e = 0; e < C; ++e) {
          const float partner = __shfl_xor(kv[u][e], 32, kWave);
          double sn, cs;
          sincos((double)key * omega[e], &sn, &cs);
          ks[e] = first_half ? (float)((double)kv[u][e] * cs - (double)partner * sn)
                             : (float)((double)kv[u][e] * cs + (double)partner * sn);
        }
      }
      part[u] = 0.f;
#pragma unroll
      for (int e = 0; e < C; ++e) part[u] = fmaf(qv[e], ks[e], part[u]);
    }
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1)
#pragma unroll
      for (int u = 0; u < kF32Keys; ++u) part[u] += __shfl_xor(part[u], msk, kWave);
    float sc[kF32Keys];
    float m_new = m;
#pragma unroll
    for (int u = 0; u < kF32Keys; ++u) {
      float x = part[u] * scale;
      if (cap > 0.f) x = cap * tanhf(x / cap);
      sc[u] = k0 + u >= lo && k0 + u <= key_end ? x : -INFINITY;
      m_new = fmaxf(m_new, sc[u]);
    }
    const float alpha = expf(m - m_new);  // m = -inf on the first step: 0
    l *= alpha;
#pragma unroll
    for (int e = 0; e < C; ++e) o[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kF32Keys; ++u) {
      const bool in = k0 + u >= lo && k0 + u <= key_end;
      const float pw_u = expf(sc[u] - m_new);
      l += pw_u;
      // a masked key's slot may hold anything, NaN included: its value is replaced by 0
#pragma unroll
      for (int e = 0; e < C; ++e) {
        const float vval = k_eq_v ? kv[u][e] : vq[e][u / 4][u % 4];
        o[e] = fmaf(pw_u, in ? vval : 0.f, o[e]);
      }
    }
    m = m_new;
  }
  // merge the 4 waves' softmaxes: out = sum_w o_w e^(m_w - M) / sum_w l_w e^(m_w - M) (a
  // wave without keys has m = -inf and weight 0; wave 0 always has keys)
  __shared__ float red_ml[4][2];
  __shared__ float red_o[4][D];
  if (lane == 0) {
    red_ml[wave][0] = m;
    red_ml[wave][1] = l;
  }
#pragma unroll
  for (int e = 0; e < C; ++e) red_o[wave][lane * C + e] = o[e];
  __syncthreads();
  if (wave != 0) return;
  float M = red_ml[0][0];
#pragma unroll
  for (int w = 1; w < 4; ++w) M = fmaxf(M, red_ml[w][0]);
  float lsum = 0.f, ow[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    ow[w] = expf(red_ml[w][0] - M);
    lsum += ow[w] * red_ml[w][1];
  }
#pragma unroll
  for (int e = 0; e < C; ++e) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += ow[w] * red_o[w][lane * C + e];
    float f = 1.f;  // exact K=V: values are the stored keys times w_v / w_k
    if (kv_vw) f = kv_vw[lane * C + e] / kv_kw[lane * C + e];
    dst[e] = acc / lsum * f;
  }
}

template <int D>
hipError_t launch_f32_t(const AttnLaunch& L, bool decode, hipStream_t s) {
  const int total_q = decode ? L.batch : L.total_q;
  const int64_t blocks = (int64_t)total_q * L.Hq;  // one workgroup per (query, head)
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
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
