// kv_write.hip -- fused RMSNorm + rotary embedding + paged scatter (one wavefront per row).
//
// One 64-lane wavefront handles one (token, head) row of q, k or v.  With rotate-half RoPE the
// pair (k, k + D/2) must sit in one lane, so lane l holds the C = D/128 consecutive elements
// starting at l*C of the first half and the matching C of the second half.  The norm's sum of
// squares is a wavefront reduction; the norm and the rotation run in double precision and the
// result is rounded once into the storage type (bf16: round-to-odd to fp32, then to nearest
// even), so the stored cache does not depend on the order of the arithmetic.
//
// Sources: [KUNLUN] = "Gemma 4 模型架构解析" (vLLM-Kunlun adaptation guide), §4.3 (a layer that
// owns its cache norms k, rotates q and k, norms v), §6.3 (slot = page id * 16 + row), §6.4
// (per-token scatter into the cache).  [MNN] = "MNN 支持 Gemma4 全系列", §6.1 (q, k and v norms).
// Layout of the pages: K [blk][g][row][d]; V [blk][g][d][row] (transposed page).
#include "device_common.hpp"
#include "launch.hpp"

namespace ga {
namespace {

struct KvWriteArgs {
  void* q;
  const void* k;
  const void* v;
  const float* wq;
  const float* wk;
  const float* wv;
  const int32_t* cu;
  const int32_t* ctx;
  const int32_t* bt;
  void* kc;
  void* vc;
  int64_t num_blocks;
  int32_t max_blocks, batch, total_tokens;
  int32_t Hq, Hkv, nslots, has_q, k_eq_v;
  double theta, eps;
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ double load(const void* p, int64_t i) {
    return (double)((const float*)p)[i];
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, double x) {
    ((float*)p)[i] = (float)x;  // round to nearest even
  }
};
template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ double load(const void* p, int64_t i) {
    return (double)bf16_to_f32(((const uint16_t*)p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, double x) {
    ((uint16_t*)p)[i] = f64_to_bf16(x);
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a) {
  constexpr int C = D / 128;  // elements per lane in each half
  constexpr int H = D / 2;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t tok = wid / a.nslots;
  const int slot = (int)(wid - tok * a.nslots);
  if (tok >= a.total_tokens) return;

  // sequence that owns this token: the last b with cu[b] <= tok
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu[mid] <= tok) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int64_t n = (int64_t)a.cu[b + 1] - a.cu[b];
  const int64_t t = (int64_t)a.ctx[b] - n + (tok - a.cu[b]);
  const int64_t page = t >> 4;
  if (t < 0 || page >= a.max_blocks) return;  // inconsistent metadata: write nothing
  const int64_t blk = a.bt[(int64_t)b * a.max_blocks + page];
  if (blk < 0 || blk >= a.num_blocks) return;
  const int64_t off = t & 15;

  // which tensor and head this wavefront owns
  int kind, h;  // kind 0 = q, 1 = k, 2 = v
  if (a.has_q && slot < a.Hq) { kind = 0; h = slot; }
  else {
    const int s = slot - (a.has_q ? a.Hq : 0);
    if (s < a.Hkv) { kind = 1; h = s; } else { kind = 2; h = s - a.Hkv; }
  }
  const void* src = kind == 0 ? (const void*)a.q : kind == 1 ? a.k : a.v;
  const float* w = kind == 0 ? a.wq : kind == 1 ? a.wk : a.wv;
  const int heads = kind == 0 ? a.Hq : a.Hkv;
  const int64_t base = (tok * heads + h) * (int64_t)D;

  double x1[C], x2[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    x1[i] = Elem<T>::load(src, base + lane * C + i);
    x2[i] = Elem<T>::load(src, base + H + lane * C + i);
  }
  if (w) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < C; ++i) ss += x1[i] * x1[i] + x2[i] * x2[i];
    ss = wave_sum_f64(ss);
    const double inv = 1.0 / sqrt(ss / D + a.eps);
#pragma unroll
    for (int i = 0; i < C; ++i) {
      x1[i] = x1[i] * inv * (double)w[lane * C + i];
      x2[i] = x2[i] * inv * (double)w[H + lane * C + i];
    }
  }
  if (kind != 2 && a.theta > 0.0) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int kk = lane * C + i;
      const double omega = 1.0 / pow(a.theta, (2.0 * kk) / (double)D);
      double sn, cs;
      sincos((double)t * omega, &sn, &cs);
      const double y1 = x1[i] * cs - x2[i] * sn;
      const double y2 = x2[i] * cs + x1[i] * sn;
      x1[i] = y1;
      x2[i] = y2;
    }
  }
  if (kind == 0) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
      Elem<T>::store(a.q, base + lane * C + i, x1[i]);
      Elem<T>::store(a.q, base + H + lane * C + i, x2[i]);
    }
  } else if (kind == 1) {
    const int64_t row = ((blk * a.Hkv + h) * kPage + off) * D;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      Elem<T>::store(a.kc, row + lane * C + i, x1[i]);
      Elem<T>::store(a.kc, row + H + lane * C + i, x2[i]);
    }
  } else {
    const int64_t pg = (blk * a.Hkv + h) * (int64_t)D * kPage;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      Elem<T>::store(a.vc, pg + (int64_t)(lane * C + i) * kPage + off, x1[i]);
      Elem<T>::store(a.vc, pg + (int64_t)(H + lane * C + i) * kPage + off, x2[i]);
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const KvWriteArgs& a, hipStream_t s) {
  const int64_t waves = (int64_t)a.total_tokens * a.nslots;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((kv_write_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write(const KvWriteLaunch& L, hipStream_t s) {
  KvWriteArgs a;
  a.q = L.q; a.k = L.k; a.v = L.v;
  a.wq = L.wq; a.wk = L.wk; a.wv = L.wv;
  a.cu = L.cu_seqlens; a.ctx = L.context_lens; a.bt = L.block_table;
  a.kc = L.k_cache; a.vc = L.v_cache;
  a.num_blocks = L.num_blocks;
  a.max_blocks = L.max_blocks; a.batch = L.batch; a.total_tokens = L.total_tokens;
  a.Hq = L.Hq; a.Hkv = L.Hkv;
  a.has_q = L.q != nullptr;
  a.k_eq_v = L.k_eq_v;
  a.nslots = (a.has_q ? L.Hq : 0) + L.Hkv + (L.k_eq_v ? 0 : L.Hkv);
  a.theta = (double)L.rope_theta;
  a.eps = (double)L.rms_eps;
  const bool bf = L.dtype_bf16;
  switch (L.D) {
    case 128: return bf ? launch_t<uint16_t, 128>(a, s) : launch_t<float, 128>(a, s);
    case 256: return bf ? launch_t<uint16_t, 256>(a, s) : launch_t<float, 256>(a, s);
    case 512: return bf ? launch_t<uint16_t, 512>(a, s) : launch_t<float, 512>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ga
