// decode.hip -- streamed flash decoding over the paged cache, then a merge of partial results.
//
// Sources: [INFLM] = "Feat/add gemma3 model" (InfiniLM pull request 581): Gemma-2 §1 (soft cap
// of the scaled scores before the softmax), Gemma-3 §3 (a sliding decode step reads only the
// last min(len, W) keys; head-first GQA).  [KUNLUN] = "Gemma 4 模型架构解析" §6.5 (attention
// reads K/V through the block table).  [MNN] = "MNN 支持 Gemma4 全系列" §6.2 (K=V).
//
// Load balance.  The visible pages of all (sequence, kv head) segments are laid end to end and cut
// into `nworkers` equal runs, one per single-wave worker (as many as the device holds at once for
// this kernel, so the whole grid is resident in one round).  Ragged lengths therefore cost nothing:
// every worker streams the same number of pages.  A worker whose run crosses segment boundaries
// emits one partial (m, l, o) per segment piece; piece (worker w, segment s) is stored at
// index w + s, which is unique, and the pieces of one segment are consecutive, so the merge
// reads a contiguous range.
//
// Pipelining.  A worker keeps one step (two pages; one at head size 512 or with K=V) of K and V
// in registers: the next step's K loads are issued as soon as the current step's QK^T products
// have consumed K, and its V loads as soon as P.V has consumed V, so global loads stay in
// flight while the softmax and matrix-core work of the current step run.  The block ids of a
// piece are fetched 64 at a time into one lane-register each and read back with readlane.
#include <atomic>
#include <mutex>

#include "attn_common.hpp"

namespace ga {
namespace {

constexpr int kMaxWorkers = 2048;

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Inclusive wave scan of one int per lane.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

template <int D, bool KEQV>
struct StepRegs {
  static constexpr int NP = (KEQV || D == 512) ? 1 : 2;  // pages per step
  u32x4_t k[NP][D / 32];
  u32x2_t v[KEQV ? 1 : NP][KEQV ? 1 : D / 16];
};

// One piece: kv head g of sequence b, pages [pbeg, pend) (absolute page indices), visible keys
// [lo, L).  Accumulates into acc.
// EXACT (with KEQV): the stored keys are unrotated; the lane's two units of each of the first
// two chunks (dimensions < 64, the ones exact mode may rotate) and their partners D/2 further
// are rotated for QK^T (rho_x: the frequencies of their first pairs), while the values are
// read unrotated.
template <int D, bool CAP, bool KEQV, bool EXACT>
__device__ __forceinline__ void decode_piece(const AttnArgs& a, const bf16x8_t (&qf)[D / 32],
                                             Acc<D>& acc, int b, int g, int L, int lo,
                                             int pbeg, int pend, uint16_t* lds,
                                             const double (&rho_x)[2]) {
  using R = StepRegs<D, KEQV>;
  constexpr int NP = R::NP, NC = D / 32, ND = D / 16;
  const int lane = threadIdx.x & 63, c16 = lane & 15, j = lane >> 4;
  const int64_t bt_row = (int64_t)b * a.max_blocks;
  const int np = pend - pbeg;
  const int nsteps = (np + NP - 1) / NP;
  const int64_t head_off = (int64_t)g;

  auto load_ids = [&](int chunk) -> int {
    const int i = chunk * 64 + lane;
    return i < np ? (int)clamp_blk(a.bt[bt_row + bt_col(pbeg + i, a.max_blocks, a.ring)],
                                   a.num_blocks)
                  : 0;
  };
  int ids = load_ids(0);
  int ids_next = np > 64 ? load_ids(1) : 0;
  int cur_chunk = 0;
  auto ensure_chunk = [&](int rel) {
    const int c = rel >> 6;
    if (c != cur_chunk) {
      ids = ids_next;
      cur_chunk = c;
      ids_next = (c + 1) * 64 < np ? load_ids(c + 1) : 0;
    }
  };
  auto blk_of = [&](int s, int p) -> int64_t {
    const int rel = s * NP + p;
    const int r = rel < np ? rel : s * NP;  // a missing second page aliases the first (masked)
    return (int64_t)__builtin_amdgcn_readlane(ids, r & 63);
  };

  // page bases are wave-uniform (scalar registers); each lane adds one 32-bit offset
  // K unit (row c16, column 4c + j) of a page of logical parity par: k_page_elem layout, row
  // slot c16 + 4 par + 4 ((c / 2) mod 2), i.e. one of three lane offsets
  const uint32_t koff0 = (uint32_t)(128 * j + 8 * c16);
  const uint32_t koff1 = (uint32_t)(128 * j + 8 * ((c16 + 4) & 15));
  const uint32_t koff2 = (uint32_t)(128 * j + 8 * ((c16 + 8) & 15));
  const uint32_t voff = (uint32_t)(c16 * kPage + 4 * j);
  const int64_t kpage = (int64_t)kPage * D;  // elements per (page, kv head)
  R r;
  auto issue_k = [&](int s) {
    ensure_chunk(s * NP);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint16_t* kp = a.kc + (blk_of(s, p) * a.Hkv + head_off) * kpage;
      const bool odd = ((pbeg + s * NP + p) & 1) != 0;
      const uint32_t kA = odd ? koff1 : koff0, kB = odd ? koff2 : koff1;
#pragma unroll
      for (int c = 0; c < NC; ++c) r.k[p][c] = ld16(kp + (((c >> 1) & 1) ? kB : kA) + 512 * c);
    }
  };
  auto issue_v = [&](int s) {
    if constexpr (!KEQV) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint16_t* vp = a.vc + (blk_of(s, p) * a.Hkv + head_off) * kpage;
#pragma unroll
        for (int n = 0; n < ND; ++n) r.v[p][n] = ld8(vp + voff + n * 16 * kPage);
      }
    }
  };

  if (nsteps > 0) {
    issue_k(0);
    issue_v(0);
  }
  for (int s = 0; s < nsteps; ++s) {
    const int pg0 = pbeg + s * NP;              // first page of the step
    const int k0 = pg0 * kPage;
    const bool full = (s + 1) * NP <= np && k0 >= lo && k0 + NP * kPage <= L;
    // exact K=V: the rotated copies of the rope units of this lane's key (row c16), as
    // hi + lo bf16 terms
    u32x4_t kr[2][2], kl[2][2];
    if constexpr (EXACT) {
      static_assert(KEQV && NP == 1, "exact K=V reads one page per step");
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        kr[c][0] = r.k[0][c];
        kr[c][1] = r.k[0][c + NC / 2];
        kl[c][0] = kl[c][1] = u32x4_t{0u, 0u, 0u, 0u};
      }
      if (a.rope_pairs > 0) {
        const int64_t t = (int64_t)pg0 * kPage + c16;
#pragma unroll
        for (int c = 0; c < 2; ++c)
          rope_units_exact(kr[c][0], kr[c][1], kl[c][0], kl[c][1], 4 * c + j, rho_x[c],
                           a.rho_step, a.rope_pairs, t);
      }
    }
    // S^T = K Q^T for each page of the step
    float4_t sc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      sc[p] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x4_t kop = r.k[p][c];
        if constexpr (EXACT) {
          if (c < 2) {
            kop = kr[c][0];
            sc[p] = mfma_16x16x32(as_bf16x8(kl[c][0]), qf[c], sc[p]);
          }
          if (c >= NC / 2 && c < NC / 2 + 2) {
            kop = kr[c - NC / 2][1];
            sc[p] = mfma_16x16x32(as_bf16x8(kl[c - NC / 2][1]), qf[c], sc[p]);
          }
        }
        sc[p] = mfma_16x16x32(as_bf16x8(kop), qf[c], sc[p]);
      }
    }
    if constexpr (KEQV) {
      // the page goes to this wave's LDS buffer for the transposed value reads
      constexpr int S = KeqvLds<D>::kStride;
#pragma unroll
      for (int c = 0; c < NC; ++c) *(u32x4_t*)(lds + c16 * S + 32 * c + 8 * j) = r.k[0][c];
    }
    if (s + 1 < nsteps) issue_k(s + 1);

    float x[4 * NP], pr[4 * NP];
    bool vk[4 * NP];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[4 * p + i] = to_log2<CAP>(sc[p][i], a.sc);
        vk[4 * p + i] = true;
      }
    if (!full) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + p * kPage + 4 * j + i;
          const bool ok = (s * NP + p < np) && key >= lo && key < L;
          if (!ok) x[4 * p + i] = -INFINITY;
          vk[4 * p + i] = ok;
        }
    }
    softmax_update<D, 4 * NP>(acc, x, pr);

    if constexpr (!KEQV) {
      if constexpr (NP == 2) {
        const bf16x8_t pf =
            as_bf16x8(u32x4_t{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                              pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])});
        const uint32_t mA01 = keep2(vk[0], vk[1]), mA23 = keep2(vk[2], vk[3]);
        const uint32_t mB01 = keep2(vk[4], vk[5]), mB23 = keep2(vk[6], vk[7]);
#pragma unroll
        for (int n = 0; n < ND; ++n) {
          u32x2_t va = r.v[0][n], vb = r.v[1][n];
          if (!full) {
            va.x &= mA01; va.y &= mA23;
            vb.x &= mB01; vb.y &= mB23;
          }
          acc.o[n] = mfma_16x16x32(as_bf16x8(u32x4_t{va.x, va.y, vb.x, vb.y}), pf, acc.o[n]);
        }
      } else {
        const short4_t pf =
            as_short4(u32x2_t{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
        const uint32_t m01 = keep2(vk[0], vk[1]), m23 = keep2(vk[2], vk[3]);
#pragma unroll
        for (int n = 0; n < ND; ++n) {
          u32x2_t va = r.v[0][n];
          if (!full) { va.x &= m01; va.y &= m23; }
          acc.o[n] = mfma_16x16x16(as_short4(va), pf, acc.o[n]);
        }
      }
      if (s + 1 < nsteps) issue_v(s + 1);
    } else {
      constexpr int S = KeqvLds<D>::kStride;
      const short4_t pf = as_short4(u32x2_t{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
      wave_lds_sync();
      // V^T fragment (d = 16 n + c16, keys 4j .. 4j+3) by one transposing read: lane 4e + q
      // of a group points at dimensions 16 n + 4q .. + 3 of key 4j + e
      const uint16_t* col = lds + (4 * j + (c16 >> 2)) * S + 4 * (c16 & 3);
      const uint32_t m01 = keep2(vk[0], vk[1]), m23 = keep2(vk[2], vk[3]);
#pragma unroll
      for (int n = 0; n < ND; ++n) {
        u32x2_t av = lds_read_tr16(col + 16 * n);
        if (!full) {
          av.x &= m01;
          av.y &= m23;
        }
        acc.o[n] = mfma_16x16x16(as_short4(av), pf, acc.o[n]);
      }
      wave_lds_sync();
    }
  }
}

template <int D, bool CAP, bool KEQV, bool EXACT>
__global__ __launch_bounds__(256) void decode_stream_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int lane = threadIdx.x & 63, c16 = lane & 15, j = lane >> 4;
  const int wave = uniform(threadIdx.x >> 6);
  const int worker = blockIdx.x * 4 + wave;
  if (worker >= a.nworkers) return;
  const int G = a.G, Hkv = a.Hkv, B = a.batch;
  uint16_t* lds = (uint16_t*)smem_raw + (KEQV ? wave * KeqvLds<D>::kElems : 0);

  // total visible pages over the batch (and the prefix array, written once by worker 0).  When
  // the batch fits one wave (B <= 64), lane s keeps sequence s's range and inclusive prefix, so
  // the rest of the set-up reads them with readlane instead of loading the lengths again
  const bool one_pass = B <= kWave;
  int rL = 0, rlo = 0, rp0 = 0, rnpg = 0, rincl = 0;
  int64_t total = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    int L = 0, lo = 0, p0 = 0, npg = 0;
    if (c0 + lane < B) decode_range(a, c0 + lane, L, lo, p0, npg);
    const int incl = wave_incl_scan(npg);
    if (worker == 0) {
      if (c0 == 0 && lane == 0) a.ws_pref[0] = 0;
      if (c0 + lane < B) a.ws_pref[c0 + lane + 1] = (int)total + incl;
    }
    if (c0 == 0) {
      rL = L; rlo = lo; rp0 = p0; rnpg = npg; rincl = incl;
    }
    total += __builtin_amdgcn_readlane(incl, 63);
  }
  total *= Hkv;
  if (total == 0) return;
  const int64_t per = (total + a.nworkers - 1) / a.nworkers;
  const int64_t u0 = (int64_t)worker * per;
  const int64_t u1 = u0 + per < total ? u0 + per : total;
  if (u0 >= u1) return;

  // the sequence holding unit u0: first b with Hkv * prefix(b + 1) > u0
  int b = 0;
  int64_t pref = 0;
  if (one_pass) {
    const uint64_t hit = __ballot((int64_t)rincl * Hkv > u0 && lane < B);
    if (!hit) return;  // cannot happen: u0 < total
    b = __builtin_ctzll(hit);
    pref = __builtin_amdgcn_readlane(rincl - rnpg, b);
  } else {
    for (int c0 = 0; c0 < B; c0 += 64) {
      int L, lo, p0, npg = 0;
      if (c0 + lane < B) decode_range(a, c0 + lane, L, lo, p0, npg);
      const int incl = wave_incl_scan(npg);
      const uint64_t hit = __ballot((pref + incl) * Hkv > u0 && c0 + lane < B);
      if (hit) {
        const int f = __builtin_ctzll(hit);
        b = c0 + f;
        pref += __builtin_amdgcn_readlane(incl - npg, f);
        break;
      }
      pref += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  // range of sequence bb (wave-uniform)
  auto seq_range = [&](int bb, int& L, int& lo, int& p0, int& npg) {
    if (one_pass) {
      L = __builtin_amdgcn_readlane(rL, bb);
      lo = __builtin_amdgcn_readlane(rlo, bb);
      p0 = __builtin_amdgcn_readlane(rp0, bb);
      npg = __builtin_amdgcn_readlane(rnpg, bb);
    } else {
      decode_range(a, bb, L, lo, p0, npg);
    }
  };

  double rho_x[2] = {0.0, 0.0};  // exact K=V: frequencies of pairs 8(4c + j), c = 0, 1
  if constexpr (EXACT) {
#pragma unroll
    for (int c = 0; c < 2; ++c) rho_x[c] = rope_rho(a.rho0, a.rho_step, 8 * (4 * c + j));
  }
  bf16x8_t qf[D / 32];
  int64_t u = u0;
  while (u < u1 && b < B) {
    int L, lo, p0, npg;
    seq_range(b, L, lo, p0, npg);
    const int64_t base = pref * Hkv;
    if (npg == 0 || u >= base + (int64_t)npg * Hkv) {
      pref += npg;
      ++b;
      continue;
    }
    const int g = (int)((u - base) / npg);
    const int lp = (int)(u - base - (int64_t)g * npg);
    const int64_t seg_end = base + (int64_t)(g + 1) * npg;
    const int64_t pe_u = u1 < seg_end ? u1 : seg_end;
    const int cnt = (int)(pe_u - u);

    const bool head_ok = c16 < G;
    load_q<D>(qf, a.q + ((int64_t)b * a.Hq + g * G + (head_ok ? c16 : 0)) * D, head_ok);
    Acc<D> acc;
    acc.init();
    decode_piece<D, CAP, KEQV, EXACT>(a, qf, acc, b, g, L, lo, p0 + lp, p0 + lp + cnt, lds,
                                      rho_x);
    acc.l += __shfl_xor(acc.l, 16, kWave);
    acc.l += __shfl_xor(acc.l, 32, kWave);
    const int64_t row = ((int64_t)worker + (int64_t)b * Hkv + g) * G + c16;
    if (head_ok) {
#pragma unroll
      for (int n = 0; n < D / 16; ++n) *(float4_t*)(a.ws_o + row * D + 16 * n + 4 * j) = acc.o[n];
      if (j == 0) *(float2*)(a.ws_ml + row * 2) = make_float2(acc.m, acc.l);
    }
    u = pe_u;
  }
}

// Merge the pieces of one (sequence, query head): out = sum 2^(m_i-M) o_i / sum 2^(m_i-M) l_i.
// The D/4 float4 columns x pieces are split over the 256 threads.  Only the prefix array is
// read before anything else: the (m, l) pairs and the first kPre partial rows of each thread
// are then loaded together (their addresses do not depend on the weights), so the merge waits
// on two round trips to memory, not four.
__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float o = __shfl_xor(v, m, kWave);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(AttnArgs a) {
  constexpr int C4 = D / 4;     // float4 columns
  constexpr int NG = 256 / C4;  // piece groups
  constexpr int kPre = 8;       // partial rows prefetched per thread
  __shared__ float wts[kMaxWorkers + 1];
  __shared__ float red[4];
  __shared__ float4_t part[256];
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int G = a.G, g = h / G, hh = h - g * G;
  uint16_t* dst = a.out + ((int64_t)b * a.Hq + h) * D;
  const int64_t pref_b = a.ws_pref[b];
  const int npg = a.ws_pref[b + 1] - (int)pref_b;
  const int64_t total = (int64_t)a.ws_pref[a.batch] * a.Hkv;
  if (npg <= 0 || total <= 0) {
    if (t < C4) *(u32x2_t*)(dst + 4 * t) = u32x2_t{0u, 0u};
    return;
  }
  const int64_t per = (total + a.nworkers - 1) / a.nworkers;
  const int64_t start = pref_b * a.Hkv + (int64_t)g * npg;
  const int64_t w0 = start / per, w1 = (start + npg - 1) / per;
  const int ns = (int)(w1 - w0 + 1);
  const int64_t row0 = (w0 + (int64_t)b * a.Hkv + g) * G + hh;  // row of piece i: row0 + i*G
  const int c = t % C4, gi = t / C4;
  const float* ocol = a.ws_o + row0 * D + 4 * c;
  const int64_t ostep = (int64_t)G * D;

  float4_t pre[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int i = gi + k * NG;
    pre[k] = i < ns ? *(const float4_t*)(ocol + i * ostep) : float4_t{0.f, 0.f, 0.f, 0.f};
  }
  float2 ml0 = make_float2(-INFINITY, 0.f);
  if (t < ns) ml0 = *(const float2*)(a.ws_ml + (row0 + (int64_t)t * G) * 2);
  float mloc = ml0.x;
  for (int i = t + 256; i < ns; i += 256) mloc = fmaxf(mloc, a.ws_ml[(row0 + (int64_t)i * G) * 2]);
  const float M = block_reduce(mloc, true, red);
  float lloc = 0.f;
  if (t < ns) {
    const float e = fast_exp2(ml0.x - M);
    wts[t] = e;
    lloc = e * ml0.y;
  }
  for (int i = t + 256; i < ns; i += 256) {
    const float2 ml = *(const float2*)(a.ws_ml + (row0 + (int64_t)i * G) * 2);
    const float e = fast_exp2(ml.x - M);
    wts[i] = e;
    lloc += e * ml.y;
  }
  const float Lsum = block_reduce(lloc, false, red);  // its barrier also publishes wts
  const float inv = 1.0f / Lsum;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int i = gi + k * NG;
    if (i < ns) acc += wts[i] * pre[k];
  }
#pragma unroll 4
  for (int i = gi + kPre * NG; i < ns; i += NG)
    acc += wts[i] * *(const float4_t*)(ocol + i * ostep);
  part[t] = acc;
  __syncthreads();
  if (gi == 0) {
#pragma unroll
    for (int g2 = 1; g2 < NG; ++g2) acc += part[g2 * C4 + c];
    float4_t f = {inv, inv, inv, inv};
    if (a.kv_vw) {  // exact K=V: values are the stored keys times w_v / w_k
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] *= a.kv_vw[4 * c + i] / a.kv_kw[4 * c + i];
    }
    *(u32x2_t*)(dst + 4 * c) = u32x2_t{pack_bf16x2(acc[0] * f[0], acc[1] * f[1]),
                                       pack_bf16x2(acc[2] * f[2], acc[3] * f[3])};
  }
}

// Resident single-wave workers the device can hold for one kernel variant: CUs x 4 SIMDs x
// waves per SIMD (from the occupancy of 4-wave workgroups).  The answer depends only on the
// device and the kernel, so it is computed once per (device, variant) and cached.
template <int D, bool CAP, bool KEQV, bool EXACT>
int resident_workers(size_t lds) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 256, blocks = 1;
  if (dev >= 0) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &blocks, reinterpret_cast<const void*>(&decode_stream_kernel<D, CAP, KEQV, EXACT>), 256,
          lds) != hipSuccess || blocks < 1)
    blocks = 1;
  int w = cus * blocks * 4;
  w = w < 1 ? 1 : (w > kMaxWorkers ? kMaxWorkers : w);
  if (dev >= 0) cache[dev].store(w, std::memory_order_relaxed);
  return w;
}

template <int D, bool CAP, bool KEQV, bool EXACT>
hipError_t launch_t(AttnArgs a, int max_workers, hipStream_t s) {
  const size_t lds = KEQV ? (size_t)4 * KeqvLds<D>::kElems * sizeof(uint16_t) : 0;
  const int res = resident_workers<D, CAP, KEQV, EXACT>(lds);
  a.nworkers = res < max_workers ? res : max_workers;
  hipLaunchKernelGGL((decode_stream_kernel<D, CAP, KEQV, EXACT>), dim3((a.nworkers + 3) / 4),
                     dim3(256), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.Hq, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAP>
hipError_t by_kv(const AttnArgs& a, int mw, int kv_mode, hipStream_t s) {
  switch (kv_mode) {
    case 0: return launch_t<D, CAP, false, false>(a, mw, s);
    case 1: return launch_t<D, CAP, true, false>(a, mw, s);
    case 2: return launch_t<D, CAP, true, true>(a, mw, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t by_flags(const AttnArgs& a, int mw, bool cap, int kv_mode, hipStream_t s) {
  return cap ? by_kv<D, true>(a, mw, kv_mode, s) : by_kv<D, false>(a, mw, kv_mode, s);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

GA_DEBUG_TAKE_DEFINE(debug_take_decode)

// Scratch of ga_attn_decode_noalloc: a fixed-size array in device memory, one per device, held
// until the process ends.  In host code `scratch` names a host-side stand-in, not the device
// array, so kernels and copies only ever get the address hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t decode_scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

DecodePlan plan_decode(int D, int Hq, int Hkv, int window, int batch, int max_context_len,
                       bool bf16) {
  DecodePlan p{0, 0, 0, 0, 0, 0};
  if (!bf16) return p;  // the fp32 path needs no workspace
  int64_t pages = (max_context_len + kPage - 1) / kPage;
  if (window > 0) {
    const int64_t wp = (int64_t)window / kPage + 2;  // a window can straddle one extra page
    if (wp < pages) pages = wp;
  }
  if (pages < 1) pages = 1;
  // at most kMaxWorkers single-wave workers (the launch uses as many as are resident), and
  // never more workers than pages
  const int64_t units = (int64_t)batch * Hkv * pages;
  p.nworkers = (int)(units < kMaxWorkers ? units : kMaxWorkers);
  if (p.nworkers < 1) p.nworkers = 1;
  const int G = Hq / Hkv;
  p.npieces = (int64_t)p.nworkers + (int64_t)batch * Hkv;
  p.pref_bytes = align256((size_t)(batch + 1) * sizeof(int32_t));
  p.ml_bytes = align256((size_t)p.npieces * G * 2 * sizeof(float));
  p.o_bytes = align256((size_t)p.npieces * G * D * sizeof(float));
  p.workspace_bytes = p.pref_bytes + p.ml_bytes + p.o_bytes;
  return p;
}

hipError_t launch_decode(const AttnLaunch& L, const DecodePlan& plan, hipStream_t s) {
  if (L.batch == 0) return hipSuccess;
  if (!L.dtype_bf16) return launch_attn_f32(L, true, s);
  AttnArgs a = make_attn_args(L);
  unsigned char* ws = (unsigned char*)L.workspace;
  a.ws_pref = (int32_t*)ws;
  a.ws_ml = (float*)(ws + plan.pref_bytes);
  a.ws_o = (float*)(ws + plan.pref_bytes + plan.ml_bytes);
  const bool cap = L.softcap > 0.f;
  switch (L.D) {
    case 128: return by_flags<128>(a, plan.nworkers, cap, L.k_eq_v, s);
    case 256: return by_flags<256>(a, plan.nworkers, cap, L.k_eq_v, s);
    case 512: return by_flags<512>(a, plan.nworkers, cap, L.k_eq_v, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ga
