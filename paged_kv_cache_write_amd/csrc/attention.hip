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

#include "device_common.hpp"
#include "launch.hpp"

namespace ga {
namespace {

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

// One wave step over two pages A, B (32 keys) with separate K and V caches.
//   kA/kB: K row pointers already offset to (row c16, column 8j); vA/vB: V^T page pointers
//   offset to (d row c16, key 4j); keyA/keyB: absolute key of slot 0 (= page*16 + 4j);
//   [lo_c, hi_c]: keys visible to this lane's row; [vlo, vhi): keys whose V may be read.
template <int D, bool CAP, bool MASKED>
__device__ __forceinline__ void step_kv2(Acc<D>& acc, const bf16x8_t (&qf)[D / 32],
                                         const uint16_t* kA, const uint16_t* kB,
                                         const uint16_t* vA, const uint16_t* vB, int keyA,
                                         int keyB, bool b_ok, int lo_c, int hi_c, int vlo,
                                         int vhi, const ScoreConsts& k) {
  float4_t sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    sA = mfma_16x16x32(as_bf16x8(ld16(kA + 32 * c)), qf[c], sA);
    sB = mfma_16x16x32(as_bf16x8(ld16(kB + 32 * c)), qf[c], sB);
  }
  float x[8], p[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = to_log2<CAP>(sA[r], k);
    x[4 + r] = to_log2<CAP>(sB[r], k);
  }
  uint32_t mA01 = ~0u, mA23 = ~0u, mB01 = ~0u, mB23 = ~0u;
  if constexpr (MASKED) {
    bool va[4], vb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ka = keyA + r, kb = keyB + r;
      if (!(ka >= lo_c && ka <= hi_c)) x[r] = -INFINITY;
      if (!(b_ok && kb >= lo_c && kb <= hi_c)) x[4 + r] = -INFINITY;
      va[r] = ka >= vlo && ka < vhi;
      vb[r] = b_ok && kb >= vlo && kb < vhi;
    }
    mA01 = keep2(va[0], va[1]);
    mA23 = keep2(va[2], va[3]);
    mB01 = keep2(vb[0], vb[1]);
    mB23 = keep2(vb[2], vb[3]);
  }
  softmax_update<D, 8>(acc, x, p);
  const bf16x8_t pf = as_bf16x8(u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                        pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])});
#pragma unroll
  for (int n = 0; n < D / 16; ++n) {
    u32x2_t a = ld8(vA + n * 16 * kPage);
    u32x2_t b = ld8(vB + n * 16 * kPage);
    if constexpr (MASKED) {
      a.x &= mA01; a.y &= mA23;
      b.x &= mB01; b.y &= mB23;
    }
    acc.o[n] = mfma_16x16x32(as_bf16x8(u32x4_t{a.x, a.y, b.x, b.y}), pf, acc.o[n]);
  }
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

// One wave step over one page (16 keys) whose K rows also serve as V (k_eq_v).
template <int D, bool CAP, bool MASKED>
__device__ __forceinline__ void step_keqv1(Acc<D>& acc, const bf16x8_t (&qf)[D / 32],
                                           const uint16_t* kp, uint16_t* lds, int key0,
                                           int lo_c, int hi_c, int vlo, int vhi,
                                           const ScoreConsts& k) {
  constexpr int S = KeqvLds<D>::kStride;
  const int lane = threadIdx.x & 63, c16 = lane & 15, j = lane >> 4;
  float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const u32x4_t kv = ld16(kp + 32 * c);
    *(u32x4_t*)(lds + c16 * S + 32 * c + 8 * j) = kv;
    s = mfma_16x16x32(as_bf16x8(kv), qf[c], s);
  }
  float x[4], p[4];
  bool vk[4] = {true, true, true, true};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = to_log2<CAP>(s[r], k);
    if constexpr (MASKED) {
      const int kk = key0 + r;
      if (!(kk >= lo_c && kk <= hi_c)) x[r] = -INFINITY;
      vk[r] = kk >= vlo && kk < vhi;
    }
  }
  softmax_update<D, 4>(acc, x, p);
  const short4_t pf = as_short4(u32x2_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
  wave_lds_sync();
  const uint16_t* col = lds + (4 * j) * S + c16;
#pragma unroll
  for (int n = 0; n < D / 16; ++n) {
    uint16_t e0 = col[0 * S + 16 * n], e1 = col[1 * S + 16 * n];
    uint16_t e2 = col[2 * S + 16 * n], e3 = col[3 * S + 16 * n];
    if constexpr (MASKED) {
      e0 = vk[0] ? e0 : (uint16_t)0;
      e1 = vk[1] ? e1 : (uint16_t)0;
      e2 = vk[2] ? e2 : (uint16_t)0;
      e3 = vk[3] ? e3 : (uint16_t)0;
    }
    const u32x2_t a = {(uint32_t)e0 | ((uint32_t)e1 << 16), (uint32_t)e2 | ((uint32_t)e3 << 16)};
    acc.o[n] = mfma_16x16x16(as_short4(a), pf, acc.o[n]);
  }
  wave_lds_sync();
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
  float* ws_o;
  float* ws_ml;
  uint16_t* out;
  int64_t num_blocks;
  int32_t max_blocks, batch, max_ctx, Hq, Hkv, G, window;
  int32_t pps, nsplit;  // decode
  int32_t max_q_len, total_q;  // prefill
  ScoreConsts sc;
};

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

// ---------------------------------------------------------------------------- decode -----

template <int D, bool CAP, bool KEQV>
__global__ __launch_bounds__(256) void decode_split_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c16 = lane & 15, j = lane >> 4;
  const int G = a.G;
  int L = a.ctx[b];
  L = L > a.max_ctx ? a.max_ctx : L;
  if (L < 1) return;
  const int lo = a.window > 0 ? (L - a.window > 0 ? L - a.window : 0) : 0;
  const int p0 = lo / kPage, p1 = (L + kPage - 1) / kPage;
  const int ps = p0 + s * a.pps;
  if (ps >= p1) return;
  const int pe = (ps + a.pps < p1) ? ps + a.pps : p1;

  bf16x8_t qf[D / 32];
  const bool head_ok = c16 < G;
  load_q<D>(qf, a.q + ((int64_t)b * a.Hq + g * G + (head_ok ? c16 : 0)) * D, head_ok);

  Acc<D> acc;
  acc.init();
  uint16_t* lds = (uint16_t*)smem_raw + (KEQV ? wave * KeqvLds<D>::kElems : 0);
  walk_pages<D, CAP, KEQV>(acc, qf, a, b, g, ps, pe, KEQV ? wave : 2 * wave, KEQV ? 4 : 8, lo,
                           L - 1, lo, L, lo, L - 1, lds);

  // merge the 4 waves: sum l over lane groups, then through LDS
  acc.l += __shfl_xor(acc.l, 16, kWave);
  acc.l += __shfl_xor(acc.l, 32, kWave);
  if constexpr (KEQV) __syncthreads();  // the page buffers are reused below
  float* so = (float*)smem_raw;               // [4][G][D]
  float* sm = so + 4 * G * D;                 // [4][16] max
  float* sl = sm + 64;                        // [4][16] sum
  if (head_ok) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) so[(wave * G + c16) * D + 16 * n + 4 * j + r] = acc.o[n][r];
    if (j == 0) {
      sm[wave * 16 + c16] = acc.m;
      sl[wave * 16 + c16] = acc.l;
    }
  }
  __syncthreads();
  const int nsplit = a.nsplit;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w * 16 + h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = fast_exp2(sm[w * 16 + h] - M);
      o += e * so[(w * G + h) * D + d];
      l += e * sl[w * 16 + h];
    }
    const int64_t row = ((int64_t)b * a.Hq + g * G + h) * nsplit + s;
    a.ws_o[row * D + d] = o;
    if (d == 0) {
      a.ws_ml[row * 2 + 0] = M;
      a.ws_ml[row * 2 + 1] = l;
    }
  }
}

// Merge the splits of one (sequence, query head): out = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s.
template <int D>
__global__ __launch_bounds__(D / 4) void decode_combine_kernel(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int d = threadIdx.x * 4;
  int L = a.ctx[b];
  L = L > a.max_ctx ? a.max_ctx : L;
  uint16_t* dst = a.out + ((int64_t)b * a.Hq + h) * D + d;
  if (L < 1) {
    *(u32x2_t*)dst = u32x2_t{0u, 0u};
    return;
  }
  const int lo = a.window > 0 ? (L - a.window > 0 ? L - a.window : 0) : 0;
  const int p0 = lo / kPage, p1 = (L + kPage - 1) / kPage;
  int ns = (p1 - p0 + a.pps - 1) / a.pps;
  ns = ns > a.nsplit ? a.nsplit : ns;
  const int64_t row0 = ((int64_t)b * a.Hq + h) * a.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_ml[(row0 + s) * 2]);
  float4_t o = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float e = fast_exp2(a.ws_ml[(row0 + s) * 2] - M);
    l += e * a.ws_ml[(row0 + s) * 2 + 1];
    const float4_t v = *(const float4_t*)(a.ws_o + (row0 + s) * D + d);
    o += e * v;
  }
  const float inv = 1.0f / l;
  *(u32x2_t*)dst = u32x2_t{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
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
hipError_t launch_f32(const AttnLaunch& L, bool decode, hipStream_t s) {
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

AttnArgs make_args(const AttnLaunch& L) {
  AttnArgs a;
  a.q = (const uint16_t*)L.q;
  a.cu = L.cu_seqlens_q;
  a.kc = (const uint16_t*)L.k_cache;
  a.vc = (const uint16_t*)L.v_cache;
  a.bt = L.block_table;
  a.ctx = L.context_lens;
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
  a.pps = 0;
  a.nsplit = 0;
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

template <int D, bool CAP, bool KEQV>
hipError_t launch_decode_t(const AttnArgs& a, hipStream_t s) {
  const size_t combine_bytes = (size_t)(4 * a.G * D + 128) * sizeof(float);
  const size_t page_bytes = KEQV ? (size_t)4 * KeqvLds<D>::kElems * sizeof(uint16_t) : 0;
  const size_t lds = combine_bytes > page_bytes ? combine_bytes : page_bytes;
  hipLaunchKernelGGL((decode_split_kernel<D, CAP, KEQV>), dim3(a.nsplit, a.Hkv, a.batch),
                     dim3(256), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.Hq, a.batch), dim3(D / 4), 0, s, a);
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
hipError_t decode_by_flags(const AttnArgs& a, bool cap, bool keqv, hipStream_t s) {
  if (cap) return keqv ? launch_decode_t<D, true, true>(a, s) : launch_decode_t<D, true, false>(a, s);
  return keqv ? launch_decode_t<D, false, true>(a, s) : launch_decode_t<D, false, false>(a, s);
}

template <int D>
hipError_t prefill_by_flags(const AttnArgs& a, bool cap, bool keqv, hipStream_t s) {
  if (cap) return keqv ? launch_prefill_t<D, true, true>(a, s) : launch_prefill_t<D, true, false>(a, s);
  return keqv ? launch_prefill_t<D, false, true>(a, s) : launch_prefill_t<D, false, false>(a, s);
}

}  // namespace

DecodePlan plan_decode(int D, int Hq, int Hkv, int window, int batch, int max_context_len,
                       bool bf16) {
  DecodePlan p{0, 0, 0};
  if (!bf16) return p;  // the fp32 path needs no workspace
  int64_t pages = (max_context_len + kPage - 1) / kPage;
  if (window > 0) {
    const int64_t wp = (int64_t)window / kPage + 2;  // a window can straddle one extra page
    if (wp < pages) pages = wp;
  }
  if (pages < 1) pages = 1;
  // aim at ~4096 workgroups over the whole batch, each a multiple of 8 pages (4 waves x 2)
  const int64_t units = (int64_t)batch * Hkv * pages;
  int64_t want = (units + 4095) / 4096;
  int pps = 8;
  while (pps < want && pps < 1024) pps *= 2;
  p.pages_per_split = pps;
  p.num_splits = (int)((pages + pps - 1) / pps);
  const int64_t rows = (int64_t)batch * Hq * p.num_splits;
  // [m, l] pairs first, padded to 256 bytes, then the un-normalised partial outputs
  const int64_t ml = (rows * 2 + 63) & ~(int64_t)63;
  p.workspace_bytes = (size_t)(ml + rows * D) * sizeof(float);
  return p;
}

hipError_t launch_decode(const AttnLaunch& L, const DecodePlan& plan, hipStream_t s) {
  if (L.batch == 0) return hipSuccess;
  if (!L.dtype_bf16) {
    switch (L.D) {
      case 128: return launch_f32<128>(L, true, s);
      case 256: return launch_f32<256>(L, true, s);
      case 512: return launch_f32<512>(L, true, s);
    }
    return hipErrorInvalidValue;
  }
  AttnArgs a = make_args(L);
  a.pps = plan.pages_per_split;
  a.nsplit = plan.num_splits;
  const int64_t rows = (int64_t)L.batch * L.Hq * plan.num_splits;
  a.ws_ml = (float*)L.workspace;
  a.ws_o = a.ws_ml + ((rows * 2 + 63) & ~(int64_t)63);
  const bool cap = L.softcap > 0.f, keqv = L.k_eq_v != 0;
  switch (L.D) {
    case 128: return decode_by_flags<128>(a, cap, keqv, s);
    case 256: return decode_by_flags<256>(a, cap, keqv, s);
    case 512: return decode_by_flags<512>(a, cap, keqv, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const AttnLaunch& L, hipStream_t s) {
  if (L.batch == 0 || L.total_q == 0) return hipSuccess;
  if (!L.dtype_bf16) {
    switch (L.D) {
      case 128: return launch_f32<128>(L, false, s);
      case 256: return launch_f32<256>(L, false, s);
      case 512: return launch_f32<512>(L, false, s);
    }
    return hipErrorInvalidValue;
  }
  AttnArgs a = make_args(L);
  const bool cap = L.softcap > 0.f, keqv = L.k_eq_v != 0;
  switch (L.D) {
    case 128: return prefill_by_flags<128>(a, cap, keqv, s);
    case 256: return prefill_by_flags<256>(a, cap, keqv, s);
    case 512: return prefill_by_flags<512>(a, cap, keqv, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ga
