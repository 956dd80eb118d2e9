// kv_write.hip -- fused RMSNorm + rotary embedding + paged scatter.
//
// A workgroup owns one token and a group of its head slots (q heads, then k heads, then v
// heads).  Each wave issues the loads of its first rows before anything else (they depend only
// on the token); then one parallel probe finds the owning sequence and its length, the
// workgroup computes the token's rotation table -- cos and sin of t * omega_k for the D/2
// frequencies, in double precision -- once into LDS, and each of its 4 wavefronts takes one
// (token, head) row at a time.  Large batches give a workgroup all slots of its token;
// small ones (a decode step) split a token's slots over several workgroups so that the launch
// still fills the chip.  Each wave issues the loads of 4 rows before it processes the first.
// With rotate-half RoPE the pair (k, k + D/2) must sit in one lane, so lane l holds the
// C = D/128 consecutive elements starting at l*C of the first half and the matching C of the
// second half.  The norm's sum of squares is a wavefront reduction; the norm and the rotation
// run in double precision and the result is rounded once into the storage type (bf16:
// round-to-odd to fp32, then to nearest even), so the stored cache does not depend on the
// order of the arithmetic.
//
// Sources: [KUNLUN] = "Gemma 4 模型架构解析" (vLLM-Kunlun adaptation guide), §4.3 (a layer that
// owns its cache norms k, rotates q and k, norms v), §6.3 (slot = page id * 16 + row), §6.4
// (per-token scatter into the cache).  [MNN] = "MNN 支持 Gemma4 全系列", §6.1 (q, k and v norms).
// Layout of the pages: K [blk][g] in 16-byte units, chunk-major, rows rotated by 4 on odd
// logical pages and in unit columns with bit 3 set (k_page_elem); V [blk][g][d][row]
// (transposed page).
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
  int32_t slots_per_wg, groups;  // head slots per workgroup; workgroups per token
  double theta, eps, pos_scale;
  double log2_theta;  // log2(theta), formed on the host
  int32_t rope_angles;
  int32_t has_kv;  // 0: q only (a layer that reads another layer's cache)
  int32_t ring;    // block-table rows are rings of max_blocks pages
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ double widen(float x) { return (double)x; }
  static __device__ __forceinline__ void store(void* p, int64_t i, double x) {
    ((float*)p)[i] = (float)x;  // round to nearest even
  }
};
template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ double widen(uint16_t x) { return (double)bf16_to_f32(x); }
  static __device__ __forceinline__ void store(void* p, int64_t i, double x) {
    ((uint16_t*)p)[i] = f64_to_bf16(x);
  }
};

// Store C consecutive elements (index i, a multiple of C, so the run is aligned) with one
// store instruction: a lane's C elements of a half-row are consecutive in q and, inside one
// 16-byte unit, in the K page.
template <typename T, int C>
__device__ __forceinline__ void store_run(void* p, int64_t i, const double (&x)[C]) {
  if constexpr (sizeof(T) == 2 && C == 2) {
    const uint32_t w = (uint32_t)f64_to_bf16(x[0]) | ((uint32_t)f64_to_bf16(x[1]) << 16);
    *(uint32_t*)((uint16_t*)p + i) = w;
  } else if constexpr (sizeof(T) == 2 && C == 4) {
    const uint64_t w = (uint64_t)f64_to_bf16(x[0]) | ((uint64_t)f64_to_bf16(x[1]) << 16) |
                       ((uint64_t)f64_to_bf16(x[2]) << 32) | ((uint64_t)f64_to_bf16(x[3]) << 48);
    *(uint64_t*)((uint16_t*)p + i) = w;
  } else if constexpr (sizeof(T) == 4 && C == 2) {
    *(float2*)((float*)p + i) = make_float2((float)x[0], (float)x[1]);
  } else if constexpr (sizeof(T) == 4 && C == 4) {
    *(float4*)((float*)p + i) = make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
  } else {
#pragma unroll
    for (int e = 0; e < C; ++e) Elem<T>::store(p, i + e, x[e]);
  }
}

constexpr int kRowsInFlight = 4;  // (token, head) rows whose loads one wave keeps in flight

// One (token, head) row of q, k or v as this lane sees it: C elements of each half.
template <typename T, int C>
struct Row {
  bool valid;
  int kind, h;  // kind 0 = q, 1 = k, 2 = v
  const T* src;
  const float* w;
  int64_t base;
  T v1[C], v2[C];
  __device__ __forceinline__ void locate(const KvWriteArgs& a, int slot, int64_t tok, int D) {
    if (a.has_q && slot < a.Hq) { kind = 0; h = slot; }
    else {
      const int s = slot - (a.has_q ? a.Hq : 0);
      if (s < a.Hkv) { kind = 1; h = s; } else { kind = 2; h = s - a.Hkv; }
    }
    src = (const T*)(kind == 0 ? (const void*)a.q : kind == 1 ? a.k : a.v);
    w = kind == 0 ? a.wq : kind == 1 ? a.wk : a.wv;
    const int heads = kind == 0 ? a.Hq : a.Hkv;
    base = (tok * heads + h) * (int64_t)D;
  }
  template <int H>
  __device__ __forceinline__ void load(int lane) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
      v1[i] = src[base + lane * C + i];
      v2[i] = src[base + H + lane * C + i];
    }
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a) {
  constexpr int C = D / 128;  // elements per lane in each half
  constexpr int H = D / 2;
  __shared__ double cos_t[H], sin_t[H];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Workgroup ids are dealt to the 8 XCDs round robin; remap them so that each XCD takes a
  // contiguous range of (token, slot group) items.  Consecutive tokens of a sequence share
  // cache pages (16 rows of every 256-byte K column run and every 32-byte V row), so their
  // partial-line stores then meet in one L2 and leave it as whole lines.  The grid is a
  // multiple of 8, so the remap is a bijection; ids past the work return.
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int64_t tok = item / a.groups;
  const int group = (int)(item - tok * a.groups);
  if (tok >= a.total_tokens) return;

  // this wave's first kRowsInFlight rows are loaded before anything else: they depend only on
  // the token, so their latency overlaps the sequence lookup and the rotation table
  const int s0 = group * a.slots_per_wg;
  const int s1 = s0 + a.slots_per_wg < a.nslots ? s0 + a.slots_per_wg : a.nslots;
  constexpr int U = kRowsInFlight;
  Row<T, C> rows[U];
  auto load_rows = [&](int first) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int slot = first + 4 * u;
      rows[u].valid = slot < s1;
      if (rows[u].valid) rows[u].locate(a, slot, tok, D);
      if (rows[u].valid) rows[u].template load<H>(lane);
    }
  };
  load_rows(s0 + wave);

  // sequence that owns this token: the b with cu[b] <= tok < cu[b + 1] (one parallel probe
  // per sequence instead of a chain of dependent loads; empty sequences never match).  The
  // probe also fetches the owner's context length, so the position is known after one round.
  __shared__ int owner;
  __shared__ int64_t own_t;
  if (threadIdx.x == 0) owner = -1;
  __syncthreads();
  for (int i = threadIdx.x; i < a.batch; i += 256) {
    const int c0 = a.cu[i], c1 = a.cu[i + 1], len = a.ctx[i];
    if (c0 <= tok && tok < c1) {
      owner = i;
      own_t = (int64_t)len - (c1 - c0) + (tok - c0);
    }
  }
  __syncthreads();
  const int b = owner;
  if (b < 0) {  // no sequence owns tok (cu_seqlens inconsistent)
    debug_flag(kDbgOwner);
    return;
  }
  const int64_t t = own_t;
  const int64_t page = t >> 4;
  if (t < 0) {  // inconsistent metadata (n_b > L_b): write nothing
    debug_flag(kDbgLength);
    return;
  }
  int64_t blk = 0;
  if (a.has_kv) {
    if (!a.ring && page >= a.max_blocks) {  // (all the exits are workgroup-uniform)
      debug_flag(kDbgBound);
      return;
    }
    // the block id is checked after the rotation table, which its load latency overlaps
    blk = a.bt[(int64_t)b * a.max_blocks + bt_col((int)page, a.max_blocks, a.ring)];
  }
  const int64_t off = t & 15;

  // rotation table of position t ([KUNLUN] 挑战 5 proportional RoPE; [INFLM] follow-up list,
  // linear scaling): omega_k = theta^(-2k/D) for k < rope_angles, 0 above; angle
  // (t / pos_scale) * omega_k
  const bool rope = a.theta > 0.0;
  if (rope) {
    const double tp = (double)t / a.pos_scale;
    for (int k = threadIdx.x; k < H; k += 256) {
      double sn = 0.0, cs = 1.0;
      if (k < a.rope_angles) {
        // theta^(-2k/D) as exp2 of a product: within a few ulp of the power, like it
        const double omega = exp2(-((2.0 * k) / (double)D) * a.log2_theta);
        sincos(tp * omega, &sn, &cs);
      }
      cos_t[k] = cs;
      sin_t[k] = sn;
    }
  }
  if (a.has_kv && (blk < 0 || blk >= a.num_blocks)) {  // no slot to write: nothing
    debug_flag(kDbgBlockId);
    return;
  }
  __syncthreads();

  // the rows of this wave, kRowsInFlight at a time: all their loads are issued before the
  // first row is processed
  for (int first = s0 + wave; first < s1; first += 4 * U) {
    if (first != s0 + wave) load_rows(first);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!rows[u].valid) continue;
      const Row<T, C>& r = rows[u];
      double x1[C], x2[C];
#pragma unroll
      for (int i = 0; i < C; ++i) {
        x1[i] = Elem<T>::widen(r.v1[i]);
        x2[i] = Elem<T>::widen(r.v2[i]);
      }
      if (r.w) {
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < C; ++i) ss += x1[i] * x1[i] + x2[i] * x2[i];
        ss = wave_sum_f64(ss);
        const double inv = 1.0 / sqrt(ss / D + a.eps);
#pragma unroll
        for (int i = 0; i < C; ++i) {
          x1[i] = x1[i] * inv * (double)r.w[lane * C + i];
          x2[i] = x2[i] * inv * (double)r.w[H + lane * C + i];
        }
      }
      // keys are stored unrotated in the exact K=V form (k_eq_v = 2): the attention kernels
      // rotate them for the scores and read them unrotated as values
      if (rope && (r.kind == 0 || (r.kind == 1 && a.k_eq_v != 2))) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
          const double cs = cos_t[lane * C + i], sn = sin_t[lane * C + i];
          const double y1 = x1[i] * cs - x2[i] * sn;
          const double y2 = x2[i] * cs + x1[i] * sn;
          x1[i] = y1;
          x2[i] = y2;
        }
      }
      if (r.kind == 0) {
        store_run<T, C>(a.q, r.base + lane * C, x1);
        store_run<T, C>(a.q, r.base + H + lane * C, x2);
      } else if (r.kind == 1) {
        const int64_t pg = (blk * a.Hkv + r.h) * (int64_t)D * kPage;
        store_run<T, C>(a.kc, pg + k_page_elem<sizeof(T)>((int)off, lane * C, page), x1);
        store_run<T, C>(a.kc, pg + k_page_elem<sizeof(T)>((int)off, H + lane * C, page), x2);
      } else {
        const int64_t pg = (blk * a.Hkv + r.h) * (int64_t)D * kPage;
#pragma unroll
        for (int i = 0; i < C; ++i) {
          Elem<T>::store(a.vc, pg + (int64_t)(lane * C + i) * kPage + off, x1[i]);
          Elem<T>::store(a.vc, pg + (int64_t)(H + lane * C + i) * kPage + off, x2[i]);
        }
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_t(KvWriteArgs a, hipStream_t s) {
  if (a.total_tokens == 0 || a.nslots == 0) return hipSuccess;
  // Slots per workgroup: all of a token's when there are enough tokens to fill the chip
  // (about 2048 workgroups of 4 waves), otherwise down to one slot per wave.
  const int64_t rows = (int64_t)a.total_tokens * a.nslots;
  int64_t per_wave = (rows + 4 * 2048 - 1) / (4 * 2048);
  const int64_t max_per_wave = (a.nslots + 3) / 4;
  per_wave = per_wave < 1 ? 1 : (per_wave > max_per_wave ? max_per_wave : per_wave);
  a.slots_per_wg = (int)(4 * per_wave);
  a.groups = (a.nslots + a.slots_per_wg - 1) / a.slots_per_wg;
  const int64_t blocks = ((int64_t)a.total_tokens * a.groups + 7) / 8 * 8;  // whole XCD rounds
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kv_write_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

GA_DEBUG_TAKE_DEFINE(debug_take_kv_write)

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
  a.has_kv = L.k != nullptr;
  a.ring = L.ring;
  a.nslots = (a.has_q ? L.Hq : 0) + (a.has_kv ? L.Hkv + (L.k_eq_v ? 0 : L.Hkv) : 0);
  a.theta = (double)L.rope_theta;
  a.log2_theta = a.theta > 0.0 ? log2(a.theta) : 0.0;
  a.rope_angles = L.rope_angles;

  a.pos_scale = (double)L.rope_scale;
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
