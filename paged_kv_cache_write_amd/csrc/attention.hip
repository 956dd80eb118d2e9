// attention.hip -- paged flash attention for gfx950: split-K decode, chunked prefill, combine.
//
// Sources: [INFLM] = "Feat/add gemma3 model" (InfiniLM pull request 581): Gemma-2 §1 (soft cap
// of the scaled scores before mask and softmax), Gemma-3 §3 (band + causal mask, decode reads
// only the last min(len, W) keys, head-first GQA).  [KUNLUN] = "Gemma 4 模型架构解析" §6.5
// (attention reads K/V through the block table).  [MNN] = "MNN 支持 Gemma4 全系列" §6.2 (K=V).
//
// Work decomposition (bf16).  A "row" is one (query position, query head) pair; the 16 rows of
// one matrix-core column block sit on the 16 columns of a 16x16 MFMA tile:
//   S^T[key][row] = K[key][:] . Q[row][:]        (A = K rows from the page, B = Q^T)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]  (A = V^T rows from the transposed V page,
//                                                 B = P^T straight from the S^T registers)
// so every lane's accumulators belong to one row and the softmax rescale is lane-uniform, the
// probabilities never cross lanes, and only the running max needs two cross-lane steps.
// Decode: rows = the G query heads of one kv head (padded to 16); a workgroup of 4 waves walks
// one split of the sequence's visible pages (2 pages = 32 keys per wave step), merges its 4
// waves in LDS and writes an un-normalised partial (m, l, o) that the combine kernel merges.
// Prefill: rows = (position, head) pairs of one kv head, position-major; every wave walks the
// pages its 16 rows can see and writes its normalised output.
// K=V: keys double as values.  The value operand needs the page transposed, so each wave
// stages the page in LDS once and reads the 16x16x16 operand back column-wise.
#include <math.h>

#include "attn_common.hpp"

namespace ga {
namespace {

// Walk pages [p_begin, p_end) of kv head g of sequence b, pages p_begin + first, +stride, ...
// (two at a time for separate K/V, one at a time for K=V).  Rows of this lane's column see
// keys [lo_c, hi_c]; the wave-wide union of visible keys is [vlo, vhi).  Steps whose keys are
// visible to every row of the wave skip all masking.
template <int D, bool CAP, bool KEQV>
__device__ __forceinline__ void walk_pages(Acc<D>& acc, const bf16x8_t (&qf)[D / 32],
                                           const AttnArgs& a, int b, int g, int p_begin,
                                           int p_end, int first, int stride, int lo_c,
                                           int hi_c, int vlo, int vhi, int lo_max, int hi_min,
                                           uint16_t* lds) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, j = lane >> 4;
  const int64_t bt_row = (int64_t)b * a.max_blocks;
  if constexpr (!KEQV) {
    for (int pa = p_begin + first; pa < p_end; pa += stride) {
      const int pb = pa + 1;
      const bool b_ok = pb < p_end;
      const int64_t blkA = clamp_blk(a.bt[bt_row + pa], a.num_blocks);
      const int64_t blkB = b_ok ? clamp_blk(a.bt[bt_row + pb], a.num_blocks) : blkA;
      const uint16_t* kA = a.kc + ((blkA * a.Hkv + g) * kPage + c16) * D + 8 * j;
      const uint16_t* kB = a.kc + ((blkB * a.Hkv + g) * kPage + c16) * D + 8 * j;
      const uint16_t* vA = a.vc + ((blkA * a.Hkv + g) * D + c16) * kPage + 4 * j;
      const uint16_t* vB = a.vc + ((blkB * a.Hkv + g) * D + c16) * kPage + 4 * j;
      const int k0 = pa * kPage;
      const bool full = b_ok && k0 >= lo_max && k0 + 2 * kPage - 1 <= hi_min;
      if (full)
        step_kv2<D, CAP, false>(acc, qf, kA, kB, vA, vB, k0 + 4 * j, k0 + kPage + 4 * j, true,
                                lo_c, hi_c, vlo, vhi, a.sc);
      else
        step_kv2<D, CAP, true>(acc, qf, kA, kB, vA, vB, k0 + 4 * j, k0 + kPage + 4 * j, b_ok,
                               lo_c, hi_c, vlo, vhi, a.sc);
    }
  } else {
    for (int pg = p_begin + first; pg < p_end; pg += stride) {
      const int64_t blk = clamp_blk(a.bt[bt_row + pg], a.num_blocks);
      const uint16_t* kp = a.kc + ((blk * a.Hkv + g) * kPage + c16) * D + 8 * j;
      const int k0 = pg * kPage;
      const bool full = k0 >= lo_max && k0 + kPage - 1 <= hi_min;
      if (full)
        step_keqv1<D, CAP, false>(acc, qf, kp, lds, k0 + 4 * j, lo_c, hi_c, vlo, vhi, a.sc);
      else
        step_keqv1<D, CAP, true>(acc, qf, kp, lds, k0 + 4 * j, lo_c, hi_c, vlo, vhi, a.sc);
    }
  }
}

// ---------------------------------------------------------------------------- prefill ----

// Rows of (sequence b, kv head g) are ordered position-major: row r = i * G + hh.  A workgroup
// owns 64 consecutive rows, each of its waves 16 of them.
template <int D, bool CAP, bool KEQV>
__global__ __launch_bounds__(256) void prefill_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c16 = lane & 15, j = lane >> 4;
  const int G = a.G;
  const int q0 = a.cu[b];
  int n = a.cu[b + 1] - q0;
  n = n > a.max_q_len ? a.max_q_len : n;
  n = n > a.total_q - q0 ? a.total_q - q0 : n;  // never touch rows past the packed queries
  int L = a.ctx[b];
  L = L > a.max_ctx ? a.max_ctx : L;            // never walk past the block table row
  const int past = L - n;
  const int rbase = (blockIdx.x * 4 + wave) * 16;
  if (q0 < 0 || n <= 0 || past < 0 || rbase >= n * G) return;
  const int nrows = (n * G - rbase) < 16 ? (n * G - rbase) : 16;
  // this lane's row
  const bool row_ok = c16 < nrows;
  const int r = rbase + (row_ok ? c16 : 0);
  const int i = r / G, hh = r - (r / G) * G;
  const int t = past + i;
  const int W = a.window;
  const int lo_c = W > 0 ? (t - W + 1 > 0 ? t - W + 1 : 0) : 0;
  // wave-wide bounds: first / last valid row
  const int t_first = past + rbase / G;
  const int t_last = past + (rbase + nrows - 1) / G;
  const int lo_first = W > 0 ? (t_first - W + 1 > 0 ? t_first - W + 1 : 0) : 0;
  const int lo_last = W > 0 ? (t_last - W + 1 > 0 ? t_last - W + 1 : 0) : 0;

  bf16x8_t qf[D / 32];
  load_q<D>(qf, a.q + ((int64_t)(q0 + i) * a.Hq + g * G + hh) * D, row_ok);

  Acc<D> acc;
  acc.init();
  uint16_t* lds = (uint16_t*)smem_raw + (KEQV ? wave * KeqvLds<D>::kElems : 0);
  const int p_begin = lo_first / kPage, p_end = t_last / kPage + 1;
  walk_pages<D, CAP, KEQV>(acc, qf, a, b, g, p_begin, p_end, 0, KEQV ? 1 : 2,
                           row_ok ? lo_c : 1, row_ok ? t : 0, lo_first, t_last + 1, lo_last,
                           t_first, lds);
  acc.l += __shfl_xor(acc.l, 16, kWave);
  acc.l += __shfl_xor(acc.l, 32, kWave);
  if (!row_ok) return;
  const float inv = 1.0f / acc.l;
  uint16_t* dst = a.out + ((int64_t)(q0 + i) * a.Hq + g * G + hh) * D + 4 * j;
#pragma unroll
  for (int nn = 0; nn < D / 16; ++nn)
    *(u32x2_t*)(dst + 16 * nn) = u32x2_t{pack_bf16x2(acc.o[nn][0] * inv, acc.o[nn][1] * inv),
                                         pack_bf16x2(acc.o[nn][2] * inv, acc.o[nn][3] * inv)};
}

// ---------------------------------------------------------------------------- fp32 -------

// Plain fp32 path (one wavefront per (query, head), one key at a time, fp32 everywhere):
// used for float caches, where the matrix cores would not keep fp32 products exact.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* q, const int32_t* cu,
                                                       const float* kc, const float* vc,
                                                       const int32_t* bt, const int32_t* ctx,
                                                       float* out, int64_t num_blocks,
                                                       int max_blocks, int batch, int Hq,
                                                       int Hkv, int window, int k_eq_v,
                                                       int decode, int total_q, int max_len,
                                                       float scale, float cap) {
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
  if (decode && L > max_len) L = max_len;
  const int t = L - n + i;
  float* dst = out + ((int64_t)rq * Hq + h) * D + lane * C;
  if (t < 0 || L < 1) {
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
  float m = -INFINITY, l = 0.f;
  for (int key = lo; key <= t; ++key) {
    const int page = key / kPage;
    if (page >= max_blocks) break;
    const int64_t blk = clamp_blk(bt[(int64_t)b * max_blocks + page], num_blocks);
    const int off = key - page * kPage;
    const float* kr = kc + ((blk * Hkv + g) * kPage + off) * D + lane * C;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < C; ++e) part = fmaf(qv[e], kr[e], part);
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
      const float vv = k_eq_v ? kr[e] : vc[((blk * Hkv + g) * D + lane * C + e) * kPage + off];
      o[e] = o[e] * alpha + pw * vv;
    }
    m = m_new;
  }
#pragma unroll
  for (int e = 0; e < C; ++e) dst[e] = o[e] / l;
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
                     L.num_blocks, L.max_blocks, L.batch, L.Hq, L.Hkv, L.window, L.k_eq_v,
                     decode ? 1 : 0, total_q, L.max_context_len, L.scale, L.softcap);
  return hipGetLastError();
}


template <int D, bool CAP, bool KEQV>
hipError_t launch_prefill_t(const AttnArgs& a, hipStream_t s) {
  const int rows = a.max_q_len * a.G;
  const int wgs = (rows + 63) / 64;
  const size_t lds = KEQV ? (size_t)4 * KeqvLds<D>::kElems * sizeof(uint16_t) : 0;
  hipLaunchKernelGGL((prefill_kernel<D, CAP, KEQV>), dim3(wgs, a.Hkv, a.batch), dim3(256), lds,
                     s, a);
  return hipGetLastError();
}

template <int D>
hipError_t prefill_by_flags(const AttnArgs& a, bool cap, bool keqv, hipStream_t s) {
  if (cap) return keqv ? launch_prefill_t<D, true, true>(a, s) : launch_prefill_t<D, true, false>(a, s);
  return keqv ? launch_prefill_t<D, false, true>(a, s) : launch_prefill_t<D, false, false>(a, s);
}

}  // namespace

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
  a.batch = L.batch;
  a.max_ctx = L.max_context_len;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.G = L.Hq / L.Hkv;
  a.window = L.window;
  a.nworkers = 0;
  a.max_q_len = L.max_q_len;
  a.total_q = L.total_q;
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

hipError_t launch_prefill(const AttnLaunch& L, hipStream_t s) {
  if (L.batch == 0 || L.total_q == 0) return hipSuccess;
  if (!L.dtype_bf16) {
    switch (L.D) {
      case 128: return launch_attn_f32(L, false, s);
      case 256: return launch_attn_f32(L, false, s);
      case 512: return launch_attn_f32(L, false, s);
    }
    return hipErrorInvalidValue;
  }
  AttnArgs a = make_attn_args(L);
  const bool cap = L.softcap > 0.f, keqv = L.k_eq_v != 0;
  switch (L.D) {
    case 128: return prefill_by_flags<128>(a, cap, keqv, s);
    case 256: return prefill_by_flags<256>(a, cap, keqv, s);
    case 512: return prefill_by_flags<512>(a, cap, keqv, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ga
