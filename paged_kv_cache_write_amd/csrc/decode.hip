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
// Pipelining.  With separate K and V caches a worker keeps one step (two pages; one at head size
// 512) of K and V in registers: the next step's K loads are issued as soon as the current step's
// QK^T products have consumed K, and its V loads as soon as P.V has consumed V, so global loads
// stay in flight while the softmax and matrix-core work of the current step run.  With K=V two
// page buffers alternate, so two pages are always loading.  The softmax reference moves lazily,
// so the accumulators are rescaled only in the rare step where it moves.  The block ids of a
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

// The block ids of pages [pbeg, pbeg + np) of row b of the block table, 64 at a time in one
// lane-register each: ensure(rel) makes page rel's window current (pages are visited in
// increasing order) and prefetches the next window; id(rel) broadcasts page rel's block id.
struct IdWindow {
  const AttnArgs& a;
  int64_t bt_row;
  int pbeg, np, ids, ids_next, cur;
  __device__ __forceinline__ IdWindow(const AttnArgs& a_, int b, int pbeg_, int np_)
      : a(a_), bt_row((int64_t)b * a_.max_blocks), pbeg(pbeg_), np(np_), cur(0) {
    ids = load(0);
    ids_next = load(1);
  }
  // lane i of window c: page 64 c + i, clamped to the piece's last page (np >= 1), so the load
  // needs no branch and no select; the ids are range-checked where they are used.  Together
  // with the scheduling barrier in ensure() this lets the next window load straight into its
  // register, so it is not waited for until its first page
  __device__ __forceinline__ int load(int chunk) const {
    const int i = min(chunk * 64 + (int)(threadIdx.x & 63), np - 1);
    return a.bt[bt_row + bt_col(pbeg + i, a.max_blocks, a.ring)];
  }
  __device__ __forceinline__ void ensure(int rel) {
    const int c = rel >> 6;
    if (c != cur) {
      ids = ids_next;
      cur = c;
      __builtin_amdgcn_sched_barrier(0);
      ids_next = load(c + 1);
    }
  }
  __device__ __forceinline__ int64_t id(int rel) const {
    return clamp_blk(__builtin_amdgcn_readlane(ids, rel & 63), a.num_blocks);
  }
};

// K unit (row c16, column 4c + j) of a page of logical parity par sits at row slot
// c16 + 4 par + 4 ((c / 2) mod 2) of unit column 4c + j (the k_page_elem layout), i.e. at one
// of three lane offsets; page bases are wave-uniform (scalar registers).
struct KOffsets {
  uint32_t o0, o1, o2;
  __device__ __forceinline__ KOffsets() {
    const int lane = threadIdx.x & 63, c16 = lane & 15, j = lane >> 4;
    o0 = (uint32_t)(128 * j + 8 * c16);
    o1 = (uint32_t)(128 * j + 8 * ((c16 + 4) & 15));
    o2 = (uint32_t)(128 * j + 8 * ((c16 + 8) & 15));
  }
  // stride 512 loads the page's units; stride 0 loads the first 1 KiB NC times (a load that
  // only keeps the count of loads in flight the same)
  template <int NC>
  __device__ __forceinline__ void load(u32x4_t (&k)[NC], const uint16_t* kp, bool odd,
                                       uint32_t stride = 512) const {
    const uint32_t kA = odd ? o1 : o0, kB = odd ? o2 : o1;
#pragma unroll
    for (int c = 0; c < NC; ++c) k[c] = ld16(kp + (((c >> 1) & 1) ? kB : kA) + stride * c);
  }
};

// One piece with separate K and V caches: kv head g of sequence b, pages [pbeg, pend)
// (absolute page indices), visible keys [lo, L).  Accumulates into acc.  A step holds two
// pages (one at head size 512) in registers: the next step's K loads are issued as soon as the
// current step's QK^T products have consumed K, and its V loads as soon as P.V has consumed V.
template <int D, bool CAP>
__device__ __forceinline__ void decode_piece_kv(const AttnArgs& a, const bf16x8_t (&qf)[D / 32],
                                                Acc<D>& acc, int b, int g, int L, int lo,
                                                int pbeg, int pend) {
  constexpr int NP = D == 512 ? 1 : 2, NC = D / 32, ND = D / 16;
  const int lane = threadIdx.x & 63, c16 = lane & 15, j = lane >> 4;
  const int np = pend - pbeg;
  const int nsteps = (np + NP - 1) / NP;
  IdWindow win(a, b, pbeg, np);
  auto blk_of = [&](int s, int p) -> int64_t {
    const int rel = s * NP + p;
    return win.id(rel < np ? rel : s * NP);  // a missing second page aliases the first (masked)
  };
  const KOffsets ko;
  const uint32_t voff = (uint32_t)(c16 * kPage + 4 * j);
  const int64_t kpage = (int64_t)kPage * D;  // elements per (page, kv head)
  u32x4_t k[NP][NC];
  u32x2_t v[NP][ND];
  auto issue_k = [&](int s) {
    win.ensure(s * NP);
#pragma unroll
    for (int p = 0; p < NP; ++p)
      ko.load(k[p], a.kc + (blk_of(s, p) * a.Hkv + g) * kpage,
              ((pbeg + s * NP + p) & 1) != 0);
  };
  auto issue_v = [&](int s) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint16_t* vp = a.vc + (blk_of(s, p) * a.Hkv + g) * kpage;
#pragma unroll
      for (int n = 0; n < ND; ++n) v[p][n] = ld8(vp + voff + n * 16 * kPage);
    }
  };

  if (nsteps > 0) {
    issue_k(0);
    issue_v(0);
  }
  for (int s = 0; s < nsteps; ++s) {
    const int k0 = (pbeg + s * NP) * kPage;  // first key of the step
    const bool full = (s + 1) * NP <= np && k0 >= lo && k0 + NP * kPage <= L;
    // S^T = K Q^T for each page of the step
    float4_t sc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      sc[p] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sc[p] = mfma_16x16x32(as_bf16x8(k[p][c]), qf[c], sc[p]);
    }
    if (s + 1 < nsteps) issue_k(s + 1);

    float x[4 * NP];
    uint32_t pw[2 * NP];
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
      // values of keys outside the range may be anything (NaN included): zero them, since a
      // zero weight does not cancel a NaN in the product
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t m01 = keep2(vk[4 * p], vk[4 * p + 1]);
        const uint32_t m23 = keep2(vk[4 * p + 2], vk[4 * p + 3]);
#pragma unroll
        for (int n = 0; n < ND; ++n) {
          v[p][n].x &= m01;
          v[p][n].y &= m23;
        }
      }
    }
    softmax_update<D, 4 * NP>(acc, x, pw);

    if constexpr (NP == 2) {
      const bf16x8_t pf = as_bf16x8(u32x4_t{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
      for (int n = 0; n < ND; ++n)
        acc.o[n] = mfma_16x16x32(
            as_bf16x8(u32x4_t{v[0][n].x, v[0][n].y, v[1][n].x, v[1][n].y}), pf, acc.o[n]);
    } else {
      const short4_t pf = as_short4(u32x2_t{pw[0], pw[1]});
#pragma unroll
      for (int n = 0; n < ND; ++n) acc.o[n] = mfma_16x16x16(as_short4(v[0][n]), pf, acc.o[n]);
    }
    if (s + 1 < nsteps) issue_v(s + 1);
  }
}

// One piece with K=V: the cached page serves as keys and, through this wave's LDS copy, as
// values.  Pages are computed one at a time from two register buffers that alternate, so the
// loads of the page after next are issued as soon as a page's QK^T products and LDS copy have
// consumed its buffer: two pages stay in flight per wave.
// EXACT: the stored keys are unrotated; the lane's two units of each of the first two chunks
// (dimensions < 64, the ones exact mode may rotate) and their partners D/2 further are
// rotated for QK^T (rho_x: the frequencies of their first pairs), while the values are read
// unrotated.
template <int D, bool CAP, bool EXACT>
__device__ __forceinline__ void decode_piece_keqv(const AttnArgs& a,
                                                  const bf16x8_t (&qf)[D / 32], Acc<D>& acc,
                                                  int b, int g, int L, int lo, int pbeg,
                                                  int pend, uint16_t* lds,
                                                  const double (&rho_x)[2]) {
  constexpr int NC = D / 32, ND = D / 16, S = KeqvLds<D>::kStride;
  const int lane = threadIdx.x & 63, c16 = lane & 15, j = lane >> 4;
  const int np = pend - pbeg;
  IdWindow win(a, b, pbeg, np);
  const KOffsets ko;
  const int64_t kpage = (int64_t)kPage * D;  // elements per (page, kv head)
  auto issue = [&](u32x4_t (&k)[NC], int s, bool real) {
    win.ensure(s);
    ko.load(k, a.kc + (win.id(s) * a.Hkv + g) * kpage, ((pbeg + s) & 1) != 0,
            real ? 512u : 0u);
  };
  // this lane writes the units 4c + j of key row c16; the V^T fragment (d = 16 n + c16, keys
  // 4j .. 4j+3) is one transposing read, lane 4e + q of a group pointing at dimensions
  // 16 n + 4q .. + 3 of key 4j + e
  uint16_t* const row_lds = lds + c16 * S + 8 * j;
  const uint16_t* const col = lds + (4 * j + (c16 >> 2)) * S + 4 * (c16 & 3);

  // step s computes page s of the piece from buffer k and then reloads k with page s + 2.  The
  // loads are issued on every step, so the count of loads issued after a buffer's is the same
  // on every path and the wait for a buffer leaves the other one in flight: past the piece's
  // end a step loads the first 1 KiB of its own page NC times (data no step uses unmasked),
  // and a step past the end (s = np, odd np) has every key masked.
  auto step = [&](u32x4_t (&k)[NC], int s) {
    const int k0 = (pbeg + s) * kPage;  // first key of the page
    const bool inside = s < np;
    const bool full = inside && k0 >= lo && k0 + kPage <= L;
    // exact K=V: the rotated copies of the rope units of this lane's key (row c16), as
    // hi + lo bf16 terms
    u32x4_t kr[2][2], kl[2][2];
    if constexpr (EXACT) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        kr[c][0] = k[c];
        kr[c][1] = k[c + NC / 2];
        kl[c][0] = kl[c][1] = u32x4_t{0u, 0u, 0u, 0u};
      }
      if (a.rope_pairs > 0) {
        const int64_t t = (int64_t)k0 + c16;
#pragma unroll
        for (int c = 0; c < 2; ++c)
          rope_units_exact(kr[c][0], kr[c][1], kl[c][0], kl[c][1], 4 * c + j, rho_x[c],
                           a.rho_step, a.rope_pairs, t);
      }
    }
    // S^T = K Q^T
    float4_t sc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4_t kop = k[c];
      if constexpr (EXACT) {
        if (c < 2) {
          kop = kr[c][0];
          sc = mfma_16x16x32(as_bf16x8(kl[c][0]), qf[c], sc);
        }
        if (c >= NC / 2 && c < NC / 2 + 2) {
          kop = kr[c - NC / 2][1];
          sc = mfma_16x16x32(as_bf16x8(kl[c - NC / 2][1]), qf[c], sc);
        }
      }
      sc = mfma_16x16x32(as_bf16x8(kop), qf[c], sc);
    }
    // the page to this wave's LDS buffer (the previous page's value reads have completed);
    // a key outside the range gets a zero row there, since its value may be anything (NaN
    // included) and a zero weight does not cancel a NaN in the product
#pragma unroll
    for (int c = 0; c < NC; ++c) *(u32x4_t*)(row_lds + 32 * c) = k[c];
    if (!full && (!inside || k0 + c16 < lo || k0 + c16 >= L)) {
#pragma unroll
      for (int c = 0; c < NC; ++c) *(u32x4_t*)(row_lds + 32 * c) = u32x4_t{0u, 0u, 0u, 0u};
    }
    issue(k, s + 2 < np ? s + 2 : (s < np ? s : np - 1), s + 2 < np);

    float x[4];
    uint32_t pw[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = to_log2<CAP>(sc[i], a.sc);
    if (!full) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 4 * j + i;
        if (!inside || key < lo || key >= L) x[i] = -INFINITY;
      }
    }
    softmax_update<D, 4>(acc, x, pw);
    const short4_t pf = as_short4(u32x2_t{pw[0], pw[1]});
    wave_lds_sync();
    u32x2_t av[ND];
#pragma unroll
    for (int n = 0; n < ND; ++n) av[n] = lds_read_tr16(col + 16 * n);
#pragma unroll
    for (int n = 0; n < ND; ++n) acc.o[n] = mfma_16x16x16(as_short4(av[n]), pf, acc.o[n]);
    wave_lds_sync();
  };

  if (np <= 0) return;
  u32x4_t kA[NC], kB[NC];
  issue(kA, 0, true);
  issue(kB, np > 1 ? 1 : 0, np > 1);
  for (int s = 0; s < np; s += 2) {
    step(kA, s);
    step(kB, s + 1);
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
    if constexpr (KEQV)
      decode_piece_keqv<D, CAP, EXACT>(a, qf, acc, b, g, L, lo, p0 + lp, p0 + lp + cnt, lds,
                                       rho_x);
    else
      decode_piece_kv<D, CAP>(a, qf, acc, b, g, L, lo, p0 + lp, p0 + lp + cnt);
    acc.l += __shfl_xor(acc.l, 16, kWave);
    acc.l += __shfl_xor(acc.l, 32, kWave);
    if (lp == 0 && cnt == npg) {
      // the worker holds the whole segment, so it writes the output itself (the merge skips
      // the segments of one piece), by the merge's arithmetic for a single piece: o times
      // 1 / l (and, exact K=V, times w_v / w_k)
      if (head_ok) {
        const float inv = 1.0f / acc.l;
        uint16_t* dst = a.out + ((int64_t)b * a.Hq + g * G + c16) * D + 4 * j;
#pragma unroll
        for (int n = 0; n < D / 16; ++n) {
          float f[4] = {inv, inv, inv, inv};
          if constexpr (EXACT) {
            if (a.kv_vw) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                f[i] *= a.kv_vw[16 * n + 4 * j + i] / a.kv_kw[16 * n + 4 * j + i];
            }
          }
          *(u32x2_t*)(dst + 16 * n) =
              u32x2_t{pack_bf16x2(acc.o[n][0] * f[0], acc.o[n][1] * f[1]),
                      pack_bf16x2(acc.o[n][2] * f[2], acc.o[n][3] * f[3])};
        }
      }
    } else if (head_ok) {
      const int64_t row = ((int64_t)worker + (int64_t)b * Hkv + g) * G + c16;
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
  if (ns == 1) return;  // one worker held the whole segment and wrote the output
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
