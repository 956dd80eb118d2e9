// kv_write.hip -- fused RMSNorm + rotary embedding + paged scatter.
//
// Every access to a row is one 16-byte unit per lane: with rotate-half RoPE the pair
// (k, k + D/2) must meet in one lane, so a lane holds unit u of a row's first half
// (elements uE .. uE+E-1, E = 16 / element size) and unit u of its second half; R = D / (2E)
// lanes cover a row, and one wave instruction covers TT = 64 / R rows (4 at head size 256 in
// bf16): a row group.
//
// For chunks (on average 16 or more new tokens per sequence) a workgroup (4 waves) owns a tile
// of TT consecutive new tokens and a group of head slots (q heads, then k heads, then v heads).
// Row group g of the workgroup is one head slot for the TT tokens of the tile, the tokens side
// by side.  The tokens are then consecutive positions of one sequence, so the lanes holding
// unit u of the TT rows write TT consecutive rows of the same page column: the value elements
// of a transposed V page ([d][16 rows]) merge into one request of 2 TT bytes instead of TT
// requests of 2 bytes, and the K units ([unit column][16 rows]) into 16 TT contiguous bytes.
// Otherwise (a decode step) a workgroup owns one token and a row group holds TT of its head
// slots.  Large batches give a workgroup all slots of its item; small ones split them over
// several workgroups so that the launch still fills the chip.
//
// Values of chunks in bf16 take a pass of their own (kv_write_v_kernel): a workgroup owns 16
// consecutive new tokens and a group of v heads.  Each row is normalised as above, then the
// workgroup stages the head's [d][16 tokens] block in LDS, and 16 consecutive lanes store one
// dimension of the 16 tokens, so the tokens of one page row leave as one contiguous run (two
// when the tile crosses a page).  Measured: a page row written 4 tokens at a time costs about
// as much as all other stores of the chunk together.
//
// Order of work in a workgroup: each wave issues the loads of its first row groups before
// anything else (they depend only on the tile), then every row's R lanes find the sequence
// owning the row's token by an R-ary search of cu_seqlens (one round of loads for up to R
// sequences), which also fetches the owner's length, so the position is known after that
// round; the row's block id load follows.  Meanwhile the workgroup computes the tile's rotation
// table -- cos and sin of t * omega_k for its TT positions and the D/2 frequencies, formed and
// evaluated in double precision -- and stages the norm weights, both in LDS; one barrier
// publishes them.
//
// Precision: bf16 caches take the norm's scale 1/sqrt(mean(x^2) + eps) in fp32 (a relative
// error of a few fp32 ulps, harmless to a bf16 result); the rotated pair x1 c - x2 s,
// x2 c + x1 s is formed in double from the exact products x * w and the double table, because
// when the two terms nearly cancel any fp32 rounding of them would be amplified in the small
// result; the pair is then scaled in fp32 and rounded to bf16 (nearest even).  Every stored
// value is within one ulp of the exact one and almost always equal to its correct rounding.
// fp32 caches keep the whole norm + rotation in double and round once.
//
// Sources: [KUNLUN] = "Gemma 4 模型架构解析" (vLLM-Kunlun adaptation guide), §4.3 (a layer that
// owns its cache norms k, rotates q and k, norms v), §6.3 (slot = page id * 16 + row), §6.4
// (per-token scatter into the cache).  [MNN] = "MNN 支持 Gemma4 全系列", §6.1 (q, k and v norms).
// Layout of the pages: K [blk][g] in 16-byte units, chunk-major, rows rotated by 4 on odd
// logical pages and in unit columns with bit 3 set (k_page_elem); V [blk][g][d][row]
// (transposed page).
#include <type_traits>

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
  int32_t slots_per_wg, groups;  // head slots per workgroup; workgroups per token tile
  double theta, eps, pos_scale;
  double log2_theta;  // log2(theta), formed on the host
  int32_t rope_angles;
  int32_t has_kv;  // 0: q only (a layer that reads another layer's cache)
  int32_t ring;    // block-table rows are rings of max_blocks pages
};

// Geometry of one row in 16-byte units.
template <typename T, int D>
struct Geo {
  static constexpr int E = 16 / (int)sizeof(T);  // elements in one unit
  static constexpr int H = D / 2;
  static constexpr int R = H / E;                // lanes per row
  static constexpr int TT = kWave / R;           // rows (tokens of a tile) per wave instruction
  static_assert(R >= 1 && R <= kWave && kWave % R == 0, "row geometry");
};

// Arithmetic type of the norm's scale: fp32 for bf16 storage, double for fp32.
template <typename T>
using Calc = std::conditional_t<sizeof(T) == 2, float, double>;

constexpr int kRowGroupsInFlight = 4;  // row groups whose loads one wave keeps in flight

// Unpack one 16-byte unit of storage elements into the arithmetic type.
template <typename T>
__device__ __forceinline__ void unpack(const u32x4_t& u, Calc<T> (&x)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = bf16_lo(u[w]);
      x[2 * w + 1] = bf16_hi(u[w]);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) x[w] = (double)__uint_as_float(u[w]);
  }
}

// Round into one 16-byte unit (nearest even, once).
template <typename T>
__device__ __forceinline__ u32x4_t pack(const Calc<T> (&x)[16 / sizeof(T)]) {
  u32x4_t u;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      u[w] = __builtin_bit_cast(uint32_t, cvt_bf16x2(x[2 * w], x[2 * w + 1]));
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) u[w] = __float_as_uint((float)x[w]);
  }
  return u;
}

// Element e of a unit (as stored) for the transposed V page.
template <typename T>
__device__ __forceinline__ void store_elem(void* p, int64_t i, const u32x4_t& u, int e) {
  if constexpr (sizeof(T) == 2) {
    ((uint16_t*)p)[i] = (uint16_t)(u[e >> 1] >> (16 * (e & 1)));
  } else {
    ((uint32_t*)p)[i] = u[e];
  }
}

// The sequence b owning token `tok` (cu[b] <= tok < cu[b + 1]) and the token's position t,
// found by the R lanes of this lane's row (lanes R r .. R r + R - 1 of the wave), each row for
// its own token: an R-ary search of the non-decreasing cu_seqlens in which every lane tests one
// probe and the last probe at or below tok narrows the range R-fold.  The last round (probes
// one apart) also fetches cu[b + 1] and each probe's length, so the position comes with the
// owner.  Empty sequences never own a token: the last b with cu[b] <= tok is the non-empty
// owner.  Returns -1 (for the row) when the metadata has no owner for tok or tok is past the
// tokens of the call.  Every lane of the wave must call it (the rounds are wave-uniform).
template <int R>
__device__ __forceinline__ int find_owner(const KvWriteArgs& a, int64_t tok, int64_t& t) {
  const int lane = threadIdx.x & 63, rl = lane % R, base = lane - rl;
  int lo = 0, hi = tok < a.total_tokens ? a.batch : 0;  // the owner lies in [lo, hi)
  int found = -1;
  int64_t pos = 0;
  // first guess, checked together with the first round's probes: sequence tok * batch / total
  // (exact for one new token per sequence, a decode step, and for equal chunks)
  int gc0 = 0, gc1 = 0, glen = 0, guess = 0;
  if (hi > 0) {
    guess = (int)(tok * a.batch / a.total_tokens);
    gc0 = a.cu[guess];
    gc1 = a.cu[guess + 1];
    glen = a.ctx[guess];
  }
  // rounds: about log_R(batch), the same for every row (the bound depends on batch only)
  for (;;) {
    const bool active = found < 0 && hi - lo >= 1;
    if (__ballot(active) == 0) break;
    const int step = active ? (hi - lo + R - 1) / R : 1;
    const int i = lo + rl * step;
    const bool probe = active && i < hi;
    int c0 = 0, c1 = 0, len = 0;
    if (probe) {
      c0 = a.cu[i];
      if (step == 1) {
        c1 = a.cu[i + 1];
        len = a.ctx[i];
      }
    }
    if (active && gc0 <= tok && tok < gc1) {  // the guess owns tok (its row is done)
      found = guess;
      pos = (int64_t)glen - (gc1 - gc0) + (tok - gc0);
      gc0 = gc1 = 0;  // checked once
      continue;
    }
    gc0 = gc1 = 0;
    const uint64_t all = __ballot(probe && c0 <= tok);
    const uint64_t mine = R == 64 ? all : (all >> base) & ((1ull << (R & 63)) - 1);
    const int last = mine ? 63 - __builtin_clzll(mine) : 0;
    const int c0s = __shfl(c0, base + last, kWave);
    const int c1s = __shfl(c1, base + last, kWave);
    const int lens = __shfl(len, base + last, kWave);
    if (active) {
      if (!mine) {
        hi = lo;  // no probe at or below tok: no owner
      } else if (step == 1) {
        if (tok < c1s) {
          found = lo + last;
          pos = (int64_t)lens - (c1s - c0s) + (tok - c0s);
        } else {
          hi = lo;
        }
      } else {
        lo = lo + last * step;
        hi = lo + step < hi ? lo + step : hi;
      }
    }
  }
  t = pos;
  return found;
}

// TILED: a work item is a tile of TT tokens and a row group one head slot of those tokens
// (chunks); otherwise a work item is one token and a row group TT head slots of it (decode
// steps, where the tokens of a tile would belong to different sequences and gain nothing).
template <typename T, int D, bool TILED>
__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a) {
  using G = Geo<T, D>;
  using C = Calc<T>;
  constexpr int E = G::E, H = G::H, R = G::R, TT = G::TT;
  constexpr int NT = TILED ? TT : 1;  // tokens per work item
  constexpr int U = kRowGroupsInFlight;
  // rotation tables, laid out [token][element e][unit u] (frequency k = uE + e) so that the
  // lanes of a row read consecutive doubles; each token's table is padded by 16 doubles so
  // that the tokens of a row group fall on different halves of the banks
  constexpr int TS = H + 16;
  __shared__ double cos_t[NT * TS], sin_t[NT * TS];
  __shared__ float w_lds[3][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane / R, ul = lane % R;  // row of the group, unit of the half-row
  // Workgroup ids are dealt to the 8 XCDs round robin; remap them so that each XCD takes a
  // contiguous range of (tile, slot group) items: neighbouring tiles share cache pages, so
  // their partial-line stores meet in one L2 and leave it as whole lines.  The grid is a
  // multiple of 8, so the remap is a bijection; ids past the work return.
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int64_t tile = item / a.groups;
  const int group = (int)(item - tile * a.groups);
  const int64_t tok0 = tile * NT;
  if (tok0 >= a.total_tokens) return;
  const int64_t tok = tok0 + (TILED ? rr : 0);  // this lane's token
  const bool tok_ok = tok < a.total_tokens;
  const int s0 = group * a.slots_per_wg;
  const int s1 = s0 + a.slots_per_wg < a.nslots ? s0 + a.slots_per_wg : a.nslots;
  const int ngroups = TILED ? s1 - s0 : (s1 - s0 + TT - 1) / TT;  // row groups of the item

  // this lane's row in row group g: head slot s0 + g of token tok (TILED), or head slot
  // s0 + TT g + rr of the item's token
  struct Row {
    bool valid;
    int kind, h;  // kind 0 = q, 1 = k, 2 = v
    int64_t base;
    u32x4_t u1, u2;
  };
  auto locate = [&](int g, Row& r) {
    const int slot = TILED ? s0 + g : s0 + TT * g + rr;
    r.valid = g < ngroups && tok_ok && slot < s1;
    const int sq = a.has_q ? a.Hq : 0;
    if (slot < sq) { r.kind = 0; r.h = slot; }
    else if (slot - sq < a.Hkv) { r.kind = 1; r.h = slot - sq; }
    else { r.kind = 2; r.h = slot - sq - a.Hkv; }
    const int heads = r.kind == 0 ? a.Hq : a.Hkv;
    r.base = (tok * heads + r.h) * (int64_t)D;
  };
  auto load = [&](Row& r) {
    if (r.valid) {
      const T* src = (const T*)(r.kind == 0 ? (const void*)a.q : r.kind == 1 ? a.k : a.v);
      r.u1 = *(const u32x4_t*)(src + r.base + ul * E);
      r.u2 = *(const u32x4_t*)(src + r.base + H + ul * E);
    }
  };
  // the loads of this wave's first row groups go out before anything else
  Row rows[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    locate(wave + 4 * i, rows[i]);
    load(rows[i]);
  }
  // norm weights, staged in LDS (loaded now, stored after the owner search)
  float wv_reg[3][2];
  const float* wsrc[3] = {a.wq, a.wk, a.wv};
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = threadIdx.x + 256 * i;
      wv_reg[k][i] = (wsrc[k] && d < D) ? wsrc[k][d] : 1.f;
    }

  // the owning sequence, position and block of this lane's token
  int64_t t = 0;
  // (untiled, every lane holds the same token: one 64-ary search)
  const int b = find_owner<TILED ? R : kWave>(a, tok, t);
  const bool pos_ok = b >= 0 && t >= 0;  // the row has a position (q needs nothing more)
  if (tok_ok && b < 0) debug_flag(kDbgOwner);   // cu_seqlens inconsistent: the row is skipped
  if (b >= 0 && t < 0) debug_flag(kDbgLength);  // n_b > L_b: skipped
  const int64_t page = t >> 4, off = t & 15;
  bool slot_ok = pos_ok;  // ... and a cache slot (k and v)
  int64_t blk = 0;
  if (a.has_kv && pos_ok) {
    if (!a.ring && page >= a.max_blocks) {
      debug_flag(kDbgBound);
      slot_ok = false;
    } else {
      // the block id is checked after the rotation table, which its load latency overlaps
      blk = a.bt[(int64_t)b * a.max_blocks + bt_col((int)page, a.max_blocks, a.ring)];
    }
  }

  // rotation tables of the tile's positions ([KUNLUN] 挑战 5 proportional RoPE; [INFLM]
  // follow-up list, linear scaling): omega_k = theta^(-2k/D) for k < rope_angles, 0 above;
  // angle (t / pos_scale) * omega_k, formed and evaluated in double.  Token j's position is
  // held by lane R j of every wave (every wave computes the same owners).
  const bool rope = a.theta > 0.0;
  if (rope) {
    for (int q = threadIdx.x; q < NT * H; q += 256) {
      const int j = q / H, k = q - j * H;
      const int64_t tj = __shfl(t, R * j, kWave);
      double sn = 0.0, cs = 1.0;
      if (k < a.rope_angles) {
        // theta^(-2k/D) as exp2 of a product: within a few ulp of the power, like it
        const double omega = exp2(-((2.0 * k) / (double)D) * a.log2_theta);
        sincos((double)tj / a.pos_scale * omega, &sn, &cs);
      }
      cos_t[j * TS + (k % E) * R + k / E] = cs;
      sin_t[j * TS + (k % E) * R + k / E] = sn;
    }
  }
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = threadIdx.x + 256 * i;
      if (d < D) w_lds[k][d] = wv_reg[k][i];
    }
  if (a.has_kv && slot_ok && (blk < 0 || blk >= a.num_blocks)) {  // no slot: k/v skipped
    debug_flag(kDbgBlockId);
    slot_ok = false;
  }
  __syncthreads();

  auto process = [&](const Row& r) {
    const bool has_w = r.kind == 0 ? a.wq != nullptr : r.kind == 1 ? a.wk != nullptr
                                                                    : a.wv != nullptr;
    // keys are stored unrotated in the exact K=V form (k_eq_v = 2): the attention kernels
    // rotate them for the scores and read them unrotated as values
    const bool rot = rope && (r.kind == 0 || (r.kind == 1 && a.k_eq_v != 2));
    C x1[E], x2[E];
    unpack<T>(r.u1, x1);
    unpack<T>(r.u2, x2);
    // RMSNorm: the row's sum of squares over its R lanes (rows without a weight ignore it)
    C ss = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
#pragma unroll
    for (int m = R / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, kWave);
    C inv = 1;
    if (has_w) {
      if constexpr (sizeof(T) == 2) inv = rsqrtf(ss / (float)D + (float)a.eps);
      else inv = 1.0 / sqrt(ss / D + a.eps);
    }
    const float* w = w_lds[r.kind];  // all ones when the tensor has no weight
    const double* cj = cos_t + (TILED ? rr : 0) * TS + ul;  // element e at cj[e R]
    const double* sj = sin_t + (TILED ? rr : 0) * TS + ul;
    if constexpr (sizeof(T) == 2) {
      if (rot) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const double a1 = (double)x1[e] * (double)w[ul * E + e];  // exact products
          const double a2 = (double)x2[e] * (double)w[H + ul * E + e];
          const double cs = cj[e * R], sn = sj[e * R];
          x1[e] = (float)(a1 * cs - a2 * sn) * inv;
          x2[e] = (float)(a2 * cs + a1 * sn) * inv;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          x1[e] = x1[e] * w[ul * E + e] * inv;
          x2[e] = x2[e] * w[H + ul * E + e] * inv;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        x1[e] = x1[e] * inv * (double)w[ul * E + e];
        x2[e] = x2[e] * inv * (double)w[H + ul * E + e];
      }
      if (rot) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const double cs = cj[e * R], sn = sj[e * R];
          const double y1 = x1[e] * cs - x2[e] * sn;
          const double y2 = x2[e] * cs + x1[e] * sn;
          x1[e] = y1;
          x2[e] = y2;
        }
      }
    }
    const u32x4_t o1 = pack<T>(x1), o2 = pack<T>(x2);
    if (r.kind == 0) {
      *(u32x4_t*)((T*)a.q + r.base + ul * E) = o1;
      *(u32x4_t*)((T*)a.q + r.base + H + ul * E) = o2;
    } else {
      const int64_t pg = (blk * a.Hkv + r.h) * (int64_t)D * kPage;
      if (r.kind == 1) {
        *(u32x4_t*)((T*)a.kc + pg + k_page_elem<sizeof(T)>((int)off, ul * E, page)) = o1;
        *(u32x4_t*)((T*)a.kc + pg + k_page_elem<sizeof(T)>((int)off, H + ul * E, page)) = o2;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          store_elem<T>(a.vc, pg + (int64_t)(ul * E + e) * kPage + off, o1, e);
          store_elem<T>(a.vc, pg + (int64_t)(H + ul * E + e) * kPage + off, o2, e);
        }
      }
    }
  };

  // the row groups of this wave, U at a time: all their loads are issued before the first is
  // processed.  A row is valid for all its R lanes or for none, and the norm's shuffles stay
  // inside a row, so the lanes of a skipped row skip it whole.  q rows need a position only;
  // k and v rows need a cache slot as well.
  for (int first = wave; first < ngroups; first += 4 * U) {
    if (first != wave) {
#pragma unroll
      for (int i = 0; i < U; ++i) {
        locate(first + 4 * i, rows[i]);
        load(rows[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < U; ++i)
      if (rows[i].valid && (rows[i].kind == 0 ? pos_ok : slot_ok)) process(rows[i]);
  }
}

constexpr int kVTile = 16;  // tokens per workgroup of the value pass (one page row)

// The value pass of a bf16 chunk write: v rows of tokens tok0 .. tok0 + 15 for heads
// h0 .. h1 - 1 (RMSNorm with w_v, no rotation), stored into the transposed V pages.
template <int D>
__global__ __launch_bounds__(256) void kv_write_v_kernel(KvWriteArgs a) {
  using T = uint16_t;
  using G = Geo<T, D>;
  constexpr int E = G::E, H = G::H, R = G::R, TT = G::TT;
  constexpr int NQ = kVTile / TT;      // row groups (TT tokens each) of the tile
  constexpr int QW = (NQ + 3) / 4;     // row groups per wave
  constexpr int SD = kVTile + 1;       // staged dimension row, padded (odd): the 16 row lanes
                                       // writing one element index fall on distinct banks
  static_assert(kVTile % TT == 0, "tile of whole row groups");
  __shared__ uint16_t stage[D * SD];
  __shared__ float w_lds[D];
  __shared__ int64_t tok_base[kVTile];  // element offset of (block, slot) of each token, or -1
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane / R, ul = lane % R;
  // XCD-contiguous ranges of (tile, head group) items, as in kv_write_kernel
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int64_t tile = item / a.groups;
  const int group = (int)(item - tile * a.groups);
  const int64_t tok0 = tile * kVTile;
  if (tok0 >= a.total_tokens) return;
  const int h0 = group * a.slots_per_wg;
  const int h1 = h0 + a.slots_per_wg < a.Hkv ? h0 + a.slots_per_wg : a.Hkv;

  // this wave's rows: row group qg = wave + 4 i holds tokens tok0 + TT qg .. + TT - 1
  bool valid[QW];
  int64_t tokr[QW];
  u32x4_t u1[QW], u2[QW];
  auto load = [&](int h) {
#pragma unroll
    for (int i = 0; i < QW; ++i)
      if (valid[i]) {
        const T* src = (const T*)a.v + (tokr[i] * a.Hkv + h) * (int64_t)D;
        u1[i] = *(const u32x4_t*)(src + ul * E);
        u2[i] = *(const u32x4_t*)(src + H + ul * E);
      }
  };
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const int qg = wave + 4 * i;
    tokr[i] = tok0 + TT * qg + rr;
    valid[i] = qg < NQ && tokr[i] < a.total_tokens;
  }
  load(h0);
  if (threadIdx.x < D) w_lds[threadIdx.x] = a.wv ? a.wv[threadIdx.x] : 1.f;
  if (D > 256 && threadIdx.x + 256 < D) w_lds[threadIdx.x + 256] = a.wv ? a.wv[threadIdx.x + 256] : 1.f;
  // owner, position and cache slot of each row's token (every lane of the wave searches)
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    int64_t t = 0;
    const int b = find_owner<R>(a, valid[i] ? tokr[i] : (int64_t)a.total_tokens, t);
    int64_t base = -1;
    if (valid[i]) {
      if (b < 0) debug_flag(kDbgOwner);
      if (b >= 0 && t < 0) debug_flag(kDbgLength);
      if (b >= 0 && t >= 0) {
        const int64_t page = t >> 4;
        if (!a.ring && page >= a.max_blocks) {
          debug_flag(kDbgBound);
        } else {
          const int64_t blk = a.bt[(int64_t)b * a.max_blocks +
                                   bt_col((int)page, a.max_blocks, a.ring)];
          if (blk < 0 || blk >= a.num_blocks) debug_flag(kDbgBlockId);
          else base = blk * a.Hkv * (int64_t)D * kPage + (t & 15);
        }
      }
    }
    if (valid[i] && ul == 0) tok_base[TT * (wave + 4 * i) + rr] = base;
    if (!valid[i] && ul == 0 && wave + 4 * i < NQ) tok_base[TT * (wave + 4 * i) + rr] = -1;
  }
  __syncthreads();
  const int sj = threadIdx.x % kVTile;  // the store phase: token sj, dimensions threadIdx.x / 16 + 16 k
  const int64_t my_base = tok_base[sj];

  for (int h = h0; h < h1; ++h) {
    // normalise this wave's rows of head h into the staging block
#pragma unroll
    for (int i = 0; i < QW; ++i) {
      if (!valid[i]) continue;  // whole rows: the norm's shuffles stay inside a row
      float x1[E], x2[E];
      unpack<T>(u1[i], x1);
      unpack<T>(u2[i], x2);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
#pragma unroll
      for (int m = R / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, kWave);
      const float inv = a.wv ? rsqrtf(ss / (float)D + (float)a.eps) : 1.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        x1[e] = x1[e] * w_lds[ul * E + e] * inv;
        x2[e] = x2[e] * w_lds[H + ul * E + e] * inv;
      }
      const u32x4_t o1 = pack<T>(x1), o2 = pack<T>(x2);
      const int j = TT * (wave + 4 * i) + rr;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        stage[(ul * E + e) * SD + j] = (uint16_t)(o1[e >> 1] >> (16 * (e & 1)));
        stage[(H + ul * E + e) * SD + j] = (uint16_t)(o2[e >> 1] >> (16 * (e & 1)));
      }
    }
    if (h + 1 < h1) load(h + 1);  // the next head's rows, in flight during the stores
    __syncthreads();
    if (my_base >= 0) {
      T* dst = (T*)a.vc + my_base + (int64_t)h * D * kPage;
#pragma unroll 4
      for (int d = threadIdx.x / kVTile; d < D; d += 256 / kVTile)
        dst[(int64_t)d * kPage] = stage[d * SD + sj];
    }
    __syncthreads();
  }
}

template <typename T, int D, bool TILED>
hipError_t launch_tiled(KvWriteArgs a, hipStream_t s) {
  using G = Geo<T, D>;
  constexpr int NT = TILED ? G::TT : 1;        // tokens per work item
  constexpr int SPG = TILED ? 1 : G::TT;       // head slots per row group
  // Slots per workgroup: all of an item's when there are enough items to fill the chip (about
  // 2048 workgroups of 4 waves), otherwise down to one row group per wave.
  const int64_t items = ((int64_t)a.total_tokens + NT - 1) / NT;
  const int64_t rg_per_item = (a.nslots + SPG - 1) / SPG;
  const int64_t rgs = items * rg_per_item;
  int64_t per_wave = (rgs + 4 * 2048 - 1) / (4 * 2048);
  const int64_t max_per_wave = (rg_per_item + 3) / 4;
  per_wave = per_wave < 1 ? 1 : (per_wave > max_per_wave ? max_per_wave : per_wave);
  a.slots_per_wg = (int)(4 * per_wave * SPG);
  a.groups = (a.nslots + a.slots_per_wg - 1) / a.slots_per_wg;
  const int64_t blocks = (items * a.groups + 7) / 8 * 8;  // whole XCD rounds
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kv_write_kernel<T, D, TILED>), dim3((unsigned)blocks), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_values(KvWriteArgs a, hipStream_t s) {
  // heads per workgroup: all of them when the tiles alone fill the chip (about 2048
  // workgroups), fewer otherwise
  const int64_t tiles = ((int64_t)a.total_tokens + kVTile - 1) / kVTile;
  int64_t per_wg = (tiles * a.Hkv + 2047) / 2048;
  per_wg = per_wg < 1 ? 1 : (per_wg > a.Hkv ? a.Hkv : per_wg);
  a.slots_per_wg = (int)per_wg;
  a.groups = (int)((a.Hkv + per_wg - 1) / per_wg);
  const int64_t blocks = (tiles * a.groups + 7) / 8 * 8;  // whole XCD rounds
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kv_write_v_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_t(KvWriteArgs a, hipStream_t s) {
  if (a.total_tokens == 0 || a.nslots == 0) return hipSuccess;
  // token tiles pay off for chunks (on average 16 or more new tokens per sequence)
  if ((int64_t)a.total_tokens < (int64_t)kPage * a.batch) return launch_tiled<T, D, false>(a, s);
  if constexpr (sizeof(T) == 2) {
    if (a.has_kv && !a.k_eq_v) {  // values in a pass of their own
      KvWriteArgs qk = a;
      qk.nslots -= a.Hkv;
      hipError_t e = qk.nslots > 0 ? launch_tiled<T, D, true>(qk, s) : hipSuccess;
      if (e != hipSuccess) return e;
      return launch_values<D>(a, s);
    }
  }
  return launch_tiled<T, D, true>(a, s);
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
