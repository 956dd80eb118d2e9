// prefill.hip -- chunked-prefill flash attention over the paged cache (bf16, matrix cores).
//
// Sources: [INFLM] = "Feat/add gemma3 model" (InfiniLM pull request 581): Gemma-2 §1 (soft cap
// of the scaled scores before mask and softmax), Gemma-3 §3 (query i of a chunk appended after
// `past` cached tokens sees key j when j <= past + i and, on a sliding layer, past + i - j < W;
// this holds for chunked prefill; head-first GQA) and its follow-up list (only keys inside the
// window need to be visited).  [KUNLUN] = "Gemma 4 模型架构解析" §6.5 (K/V read through the
// block table).  [MNN] = "MNN 支持 Gemma4 全系列" §6.2 (K=V).
//
// Tiling.  A workgroup of 8 waves (two per SIMD, so one wave's softmax and LDS latency hide
// behind the other's matrix-core work) owns 256 rows (128 at head size 512) of one (sequence,
// kv head): rows are (position, query head) pairs ordered position-major, so the G heads of a
// GQA group share every key tile.  Each wave holds 32 rows (two 16-column MFMA blocks; 16 rows
// at head size 512) with Q^T and the O^T accumulators in registers.  Key tiles of 32 keys (two
// pages) are copied from HBM straight into LDS by global_load_lds_dwordx4 (no registers
// involved) through rings of K and V^T tiles (4 stages each, 2 at head size 512); one barrier
// per tile both publishes a tile and frees a stage.  Every copy reads one contiguous 1 KiB
// run (K pages are stored in the order LDS wants them, see below).  A wave's copies for a
// later tile are spread over the matrix-core instructions of the current one (K copies among
// the QK^T products, V copies among the P.V products) instead of queueing behind the barrier.
// Operand fragments are read from LDS kPF fragments ahead of the products that use them: the
// loops are cut into one chunk per fragment by scheduling fences.  Block
// ids are held 64 pages at a time in one register per lane and broadcast with readlane (one
// vector load per 32 tiles); the next tile's page offsets are formed at the end of the
// previous iteration.  Only tiles that intersect the band [past + i - W + 1, past + i] of some row of
// the workgroup are visited, and every wave runs all of them (a tile outside a wave's rows is
// masked whole); tiles whose every key is visible to every row of a wave skip all masking.
// Keys past the context (only in the last tile) are zeroed in LDS once, so no value read
// needs a mask.
//
// Key order inside a tile.  The 16 rows of the first QK^T product of a tile are keys
// {0-3, 8-11} of each of its two pages and the second product's rows are keys {4-7, 12-15},
// so that the four scores lane group j receives from each product are 8 consecutive keys of
// one page (page j/2, keys 8(j%2) .. 8(j%2)+7).  The probabilities then form the P^T operand
// of P.V without moving between lanes, and the matching V^T operand is one 16-byte read.
//
// LDS layouts (per page of 16 keys), chosen so that every operand read is one base register
// plus an immediate offset and is free of bank conflicts; both are the pages' HBM layouts, so
// a tile arrives by plain contiguous copies:
//   K page  chunk-major: the 16-byte chunk x (elements 8x .. 8x+7) of key row r of page p is
//           stored at byte 256 x + 16 ((r + 4p) mod 16), so a QK^T fragment read by 16 lanes
//           (16 distinct rows, one chunk) covers 16 distinct bank groups.  p is the page's
//           place in the tile, which is the parity of its logical index (tiles start at even
//           pages): the cache's K page layout (k_page_elem).  Measured: 1 KiB copies gathered
//           as 16 rows x 64 bytes (what a row-major HBM page needs) move a third of the bytes
//           per clock that contiguous 1 KiB copies move.
//   V^T page [D rows][16 keys] (32 bytes a row), rows in order: the 16 lanes of a lane group
//           read 16 consecutive rows, one half each (measured conflict-free; swapping the halves
//           of every other group of 8 rows makes the read 2-way conflicted).
// The tile loop issues no vector-memory operation other than the tile copies (the Q loads
// are complete before it starts), so the copies' completion is counted exactly.
//
// Order of work: workgroup ids are dealt to the 8 XCDs round robin.  Runs of kRun neighbouring
// row tiles of one (sequence, kv head) go to one XCD (its L2 then serves the key tiles they
// share), the runs of every (sequence, kv head) are spread over all 8 XCDs (so chunks of
// different lengths load the XCDs evenly), and the row tiles with the most keys start first.
#include "prefill_common.hpp"

namespace ga {
namespace {

constexpr int kPF = 3;                // operand fragment reads in flight ahead of their products
constexpr int kRun = 4;               // consecutive row tiles of a group given to one XCD

// Waves per workgroup, two per SIMD on a CU either way (256 registers each): 8 in one
// workgroup per CU at head size 512 and for the exact K=V form, 4 in each of two workgroups per
// CU elsewhere (LDS rings of 64 KiB).  The waves of two workgroups are not held in step by each
// other's barriers, so one workgroup's softmax and its prologue and epilogue run beside the
// other's matrix-core work.
template <int D, bool EXACT>
constexpr int waves_for() { return D <= 256 && !EXACT ? 4 : 8; }

// MFMA column blocks per wave: 2 (32 rows) up to head size 256, 1 (16 rows) at 512, where
// 32 rows of Q^T (128 registers) plus O^T (256) would not fit a wave's 256 registers.
template <int D, int NW>
struct Rows {
  static constexpr int kR = D == 512 ? 1 : 2;
  static constexpr int kPerWave = 16 * kR;
  static constexpr int kPerWg = NW * kPerWave;
};

// LDS: a ring of SK K tiles and a ring of SV V^T tiles (K=V: the K ring only) in 16 KiB per
// wave (measured: a 160 KiB allocation with a deeper K ring at head size 512 runs slower).
// Iteration it reads K(it) and V(it).
template <int D, bool KEQV, int NW>
struct TileLds {
  static constexpr int kPageBytes = kPage * D * 2;  // one page of K (or V^T)
  static constexpr int kTile = 2 * kPageBytes;      // one 32-key tile of K (or of V^T)
  static constexpr int kBudget = NW * 16 * 1024;
  static constexpr int kMaxStages = 4;
  static constexpr int kFit = kBudget / kTile;      // tiles that fit
  static constexpr int SK = KEQV ? (kFit < kMaxStages ? kFit : kMaxStages)
                                 : (kFit >= 2 * kMaxStages ? kMaxStages : (kFit + 1) / 2);
  static constexpr int SV = KEQV ? 0 : (kFit >= 2 * kMaxStages ? kMaxStages : kFit / 2);
  static constexpr int kKRing = 0;
  static constexpr int kVRing = SK * kTile;
  static constexpr int kBytes = (SK + SV) * kTile;
  static constexpr int kChunks = kTile / 1024;          // 1 KiB copies per tile
  static constexpr int kPerWave = kChunks / NW;         // copies per wave per tile
  static_assert(kChunks % NW == 0, "tile copies split evenly over the waves");
  static_assert(SK >= 2 && SK <= kMaxStages && (KEQV ? SK >= 3 : (SV >= 2 && SV <= SK)),
                "ring depths");
  static_assert(kBytes <= kBudget, "LDS budget");
  // exact K=V: the rotated rope units of the two tiles of an iteration, laid out like a K tile
  // of 16 unit columns (the 8 holding dimensions 0-63, then their 8 partners D/2 further)
  static constexpr int kRopePage = 16 * 256;
  static constexpr int kRopeTile = 2 * kRopePage;
  static constexpr int kRopeOff = kBytes;
  static constexpr int kRopeLo = 2 * kRopeTile;  // the lo terms, after the hi terms
  static constexpr int kRopeBytes = 4 * kRopeTile;
};

// Copy i (0 .. kPerWave-1) of this wave for one tile of K (V=false) or of V^T (V=true) into
// `lds_off`: 1 KiB chunk q = wave + NW * i of the tile, from a wave-uniform base plus the
// per-lane offset 16 lane.  offA / offB are the byte offsets of the tile's two pages (the same
// in the K and the V cache).  Both page kinds are copied as they are stored (K pages already
// hold the LDS arrangement: k_page_elem), so every copy reads one contiguous 1 KiB run.
template <int D, bool KEQV, bool V, int NW>
__device__ __forceinline__ void issue_chunk(const AttnArgs& a, uint32_t lds_off, int64_t offA,
                                            int64_t offB, int wave, int i, uint32_t vlane) {
  using T = TileLds<D, KEQV, NW>;
  constexpr int kChunksPerPage = T::kPageBytes / 1024;
  const int q = wave + NW * i;  // 1 KiB chunk of the tile (wave-uniform)
  // the page of chunk q: known at compile time when the waves divide a page's chunks
  // (wave < NW), otherwise a scalar select
  int page;
  if constexpr (kChunksPerPage % NW == 0) page = NW * i / kChunksPerPage;
  else page = q / kChunksPerPage;
  const int qq = q - page * kChunksPerPage;
  const int64_t off = page ? offB : offA;
  const unsigned char* base = (const unsigned char*)(V ? (const void*)a.vc : (const void*)a.kc);
  lds_copy16_sv(base + off + 1024 * qq, vlane, lds_off + q * 1024);
}

// Zero, in one staged tile, the values of key slots nvalid .. 31 (keys past the context):
// the V^T pages (or, K=V, the K pages, which then serve as values).  All threads take part.
template <int D, bool KEQV, int NW>
__device__ __forceinline__ void zero_tail_values(unsigned char* tile, int nvalid) {
  using T = TileLds<D, KEQV, NW>;
  if constexpr (!KEQV) {
    // V^T page [D rows][16 keys]: one row (32 bytes) of one page per step
    for (int q = threadIdx.x; q < 2 * D; q += 64 * NW) {
      const int page = q / D, d = q - page * D;
      unsigned char* row = tile + page * T::kPageBytes + d * 32;
#pragma unroll
      for (int r = 0; r < kPage; ++r)
        if (page * kPage + r >= nvalid)
          *(uint16_t*)(row + 2 * r) = 0;
    }
  } else {
    // chunk-major K page: 16-byte unit (row r, chunk x) at 256 x + 16 k_slot(r, x, page)
    for (int q = threadIdx.x; q < 2 * kPage * (D / 8); q += 64 * NW) {
      const int page = q / (kPage * (D / 8)), u = q - page * (kPage * (D / 8));
      const int x = u >> 4, r = u & 15;
      if (page * kPage + r >= nvalid)
        *(u32x4_t*)(tile + page * T::kPageBytes + 256 * x + 16 * k_slot(r, x, page)) =
            u32x4_t{0u, 0u, 0u, 0u};
    }
  }
}

// K=V value fragment nn: the 16 dimensions of K units x0 = kv_block_unit(nn) and x0 + 8 (units
// whose bit 3 is clear, paired with the unit 8 above: every unit belongs to one fragment).  A
// row i (and output row i of O^T) of the fragment is dimension kv_block_dim(nn, i).
__device__ __forceinline__ constexpr int kv_block_unit(int nn) { return (nn & 7) + 16 * (nn >> 3); }
__device__ __forceinline__ constexpr int kv_block_dim(int nn, int i) {
  return 8 * (kv_block_unit(nn) + 8 * (i >> 3)) + (i & 7);
}

// Exact K=V: the chunk of QK^T fragment f in the rope buffer (chunks 0 and 1, holding
// dimensions 0-63, and their partners NC/2 and NC/2 + 1 become 0 .. 3), -1 for the fragments
// read from the K tile.
template <int NC, int f>
constexpr int rope_chunk_of() {
  constexpr int c = f >> 1;
  return c < 2 ? c : (c >= NC / 2 && c < NC / 2 + 2 ? c - NC / 2 + 2 : -1);
}

// EXACT (with KEQV): keys are stored unrotated.  After each iteration's tiles have landed, the
// workgroup rotates their units holding dimensions 0-63 and the partners of those (one unit
// pair per thread) into a separate LDS buffer that the QK^T fragment reads of those chunks
// use; the values are still read from the unrotated tile.
template <int D, int SM, bool KEQV, bool EXACT>
__global__ __launch_bounds__((64 * waves_for<D, EXACT>()), (8 / waves_for<D, EXACT>())) void
prefill_tiled_kernel(AttnArgs a, int runs_per_bg, int n_groups) {
  constexpr int NW = waves_for<D, EXACT>();
  using T = TileLds<D, KEQV, NW>;
  constexpr int NC = D / 32, ND = D / 16, R = Rows<D, NW>::kR, SK = T::SK, SV = T::SV;
  constexpr int kRowsPerWave = Rows<D, NW>::kPerWave, kRowsPerWg = Rows<D, NW>::kPerWg;
  extern __shared__ __align__(16) unsigned char smem[];
  const uint32_t smem_off =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const int lane = threadIdx.x & 63, c16 = lane & 15, j = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- which (sequence, kv head, row tile) this workgroup owns.  Work items are (group bg,
  // rank r), r = 0 being the group's row tile with the most keys (its last one).  Each group's
  // ranks are cut into runs of kRun consecutive ranks and the runs, group-major, are dealt to
  // the 8 XCDs round robin (workgroup i runs on XCD i mod 8): every XCD gets about an eighth of
  // every group whatever the chunk lengths, while the row tiles running together on one XCD
  // are neighbours that share most of their key tiles in its L2.  Ranks past a group's own
  // row tiles (a shorter chunk than max_q_len) and the padding of the grid return at once.
  const int xcd = blockIdx.x % 8, kq = blockIdx.x / 8;
  const int run = 8 * (kq / kRun) + xcd;
  const int bg = run / runs_per_bg;
  const int rank = (run - bg * runs_per_bg) * kRun + kq % kRun;
  if (bg >= n_groups) return;
  const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
  if (b >= a.batch) return;
  const int G = a.G, W = a.window;
  const int q0 = a.cu[b];
  int n = a.cu[b + 1] - q0;
  if (n > a.max_q_len || n > a.total_q - q0 || n < 0 || q0 < 0) debug_flag(kDbgLength);
  n = n > a.max_q_len ? a.max_q_len : n;
  n = n > a.total_q - q0 ? a.total_q - q0 : n;
  int L = a.ctx[b];
  if (L > a.max_ctx) debug_flag(kDbgBound);
  L = L > a.max_ctx ? a.max_ctx : L;
  const int past = L - n;
  if (past < 0) debug_flag(kDbgLength);
  const int tiles_b = (n * G + kRowsPerWg - 1) / kRowsPerWg;  // row tiles of this group
  if (q0 < 0 || n <= 0 || past < 0 || rank >= tiles_b) return;  // uniform over the workgroup
  const int row0 = (tiles_b - 1 - rank) * kRowsPerWg;

  // ---- key tiles of the workgroup: keys [lo(first row), position(last row)]
  const int nrows_wg = (n * G - row0) < kRowsPerWg ? (n * G - row0) : kRowsPerWg;
  const int t_first_wg = past + row0 / G, t_last_wg = past + (row0 + nrows_wg - 1) / G;
  const int lo_first_wg = W > 0 ? (t_first_wg - W + 1 > 0 ? t_first_wg - W + 1 : 0) : 0;
  const int kt0 = lo_first_wg / kTileKeys, kt1 = t_last_wg / kTileKeys;  // inclusive
  const int ntiles = kt1 - kt0 + 1;

  // ---- this wave's rows
  const int wrow0 = row0 + wave * kRowsPerWave;
  const int wrows = (n * G - wrow0) < kRowsPerWave ? (n * G - wrow0) : kRowsPerWave;
  // Row rb of this lane sees key k iff (unsigned)(k - lo_c[rb]) <= span_c[rb], i.e.
  // lo <= k <= position; padding rows see nothing.
  int lo_c[R];
  uint32_t span_c[R];
  bool ok_c[R];
  int64_t q_off[R];  // element offset of this lane's Q row
  bf16x8_t qf[R][NC];  // loaded after the first tile copies are issued
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    const int rr = 16 * rb + c16;
    ok_c[rb] = rr < wrows;
    const int row = wrow0 + (ok_c[rb] ? rr : 0);
    const int i = row / G, hh = row - (row / G) * G;
    const int t = past + i;
    const int lo = W > 0 ? (t - W + 1 > 0 ? t - W + 1 : 0) : 0;
    lo_c[rb] = ok_c[rb] ? lo : (1 << 30);
    span_c[rb] = ok_c[rb] ? (uint32_t)(t - lo) : 0u;
    q_off[rb] = ((int64_t)(q0 + i) * a.Hq + g * G + hh) * D;
  }
  // wave-uniform bounds: intersection [lo_max, hi_min] of the rows' key ranges (tiles inside it
  // need no mask) and their union [lo_min, hi_max] (tiles outside it are skipped)
  const bool wave_active = wrows > 0;
  const int t_first_w = past + (wave_active ? wrow0 : row0) / G;
  const int t_last_w = past + (wave_active ? wrow0 + wrows - 1 : row0) / G;
  const int lo_max = W > 0 ? (t_last_w - W + 1 > 0 ? t_last_w - W + 1 : 0) : 0;
  const int hi_min = t_first_w;
  const int lo_min = W > 0 ? (t_first_w - W + 1 > 0 ? t_first_w - W + 1 : 0) : 0;
  const int hi_max = wave_active ? t_last_w : -1;

  float m_ref[R], l_run[R];
  float4_t o[R][ND];
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    m_ref[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int nn = 0; nn < ND; ++nn) o[rb][nn] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int64_t bt_row = (int64_t)b * a.max_blocks;
  const int last_page = (L - 1) / kPage;
  // exact K=V: this thread's unit pair in the rotation pass (row, unit column, page, tile of
  // the iteration)

  // Lane offsets inside a tile (bytes); fragment c / column block nn adds an immediate.
  //   K, product m: row qk_row_key(c16, m) of page c16 / 8, chunk 4c + j.
  //   V^T: row d = 16 nn + c16 of page j / 2, the 8 keys 8 (j % 2) .. + 7.
  const int kpage = c16 >> 3;
  // (koff[m][cb]: unit columns 4c + j with bit 3 = cb, i.e. cb = (c / 2) mod 2)
  int koff[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      koff[m][cb] = kpage * T::kPageBytes + 256 * j +
                    16 * ((qk_row_key(c16, m) + 4 * kpage + 4 * cb) & 15);
  const int voff = (j >> 1) * T::kPageBytes + c16 * 32 + (j & 1) * 16;
  // exact K=V: the same lane offsets in the rope buffer (pages of 16 units): koff[m] - rdiff
  const int rdiff = kpage * (T::kPageBytes - T::kRopePage);
  // key of score slot e (product e / 4, register e % 4) of this lane group, minus k0
  const int kslot = (j >> 1) * kPage + 8 * (j & 1);

  // ---- copy schedule.  Group g (iteration g, or the prologue for g < 0) copies tile
  // g - 1 + S into the stages that iteration g - 1 has just released; iteration it reads
  // tile it.
  const int np = ntiles;
  // Byte offsets in the caches of a tile's two pages.  The block ids of the workgroup's pages
  // are held 64 at a time, lane l holding that of page pw0 + l (clamped; on a ring table each
  // page's own column), and broadcast with readlane.  A tile's second page lying past the
  // context aliases its first (its keys are masked and its values zeroed), so nothing past the
  // sequence's last page is read.  A window is loaded every 32 tiles.
  struct TileIds { int64_t a, b; };
  int pw0 = -kWave, pwn = -kWave;  // first pages of the window and of the next one (even;
                                   // wave-uniform)
  int win_bid = 0, win_next = 0;   // this lane's block ids in them
  constexpr int64_t kPageBytesG = (int64_t)kPage * D * 2;
  // pages past the context take the last page's id: the only one read is the second page of
  // the last tile when last_page is even, which aliases the first
  auto win_load = [&](int p0) -> int {
    const int q = p0 + lane < last_page ? p0 + lane : last_page;
    return (int)clamp_blk(a.bt[bt_row + bt_col(q, a.max_blocks, a.ring)], a.num_blocks);
  };
  auto ids_of = [&](int tile) -> TileIds {
    TileIds r{0, 0};
    if (tile < 0 || tile >= ntiles) return r;
    const int page = 2 * (kt0 + tile);  // <= last_page for every tile of the range
    if (page < pw0 || page - pw0 >= kWave) {
      win_bid = page == pwn ? win_next : win_load(page);
      pw0 = page;
    }
    // the next window is loaded a quarter of a window before it is needed, so that its load
    // has landed when the window moves
    if (page - pw0 >= 3 * kWave / 4 && pwn != pw0 + kWave && pw0 + kWave <= last_page) {
      pwn = pw0 + kWave;
      win_next = win_load(pwn);
    }
    const int i = page - pw0;
    const int ba = __builtin_amdgcn_readlane(win_bid, i);
    const int bb = __builtin_amdgcn_readlane(win_bid, i + 1);
    r.a = ((int64_t)ba * a.Hkv + g) * kPageBytesG;
    r.b = ((int64_t)bb * a.Hkv + g) * kPageBytesG;
    return r;
  };
  // Both rings have S stages.  Iteration jj (one barrier) consumes the TB tiles TB*jj ..
  // TB*jj + TB - 1 (two when the ring has four stages, one when it has two) and, in the stages
  // the previous iteration released, copies tiles TB*jj + S - TB .. + TB - 1.  All of those
  // copies are spread over the work on the iteration's first tile (K copies among the QK^T
  // products, V copies among the P.V products), so that at least one tile's work hides the
  // latency of the last of them.  Past the last tile the copies read block 0 into stages no
  // iteration reads any more, so every iteration issues the same number of copies and the
  // count of copies that may stay in flight at a wait is a constant (no branch sits between
  // the matrix-core instructions the copies are spread over).
  static_assert(KEQV || SK == SV, "both rings have the same depth");
  constexpr int S = SK;
  constexpr int TB = S >= 4 ? 2 : 1;
  static_assert(S % TB == 0 && S >= 2 * TB, "ring depth");
  constexpr int kPerTile = T::kPerWave * (KEQV ? 1 : 2);
  constexpr int kWait = (S / TB - 2) * TB * kPerTile;  // copies of later iterations in flight
  const uint32_t vlane = 16u * lane;
  // ring stage of tile t (t >= 0; S a power of two)
  static_assert((S & (S - 1)) == 0, "ring depth a power of two");
  auto stage = [](int t) { return (int)((unsigned)t & (unsigned)(S - 1)); };
  auto k_chunk = [&](int t, const TileIds& ids, int i) {
    issue_chunk<D, KEQV, false, NW>(a, smem_off + T::kKRing + stage(t) * T::kTile, ids.a, ids.b,
                                    wave, i, vlane);
  };
  auto v_chunk = [&](int t, const TileIds& ids, int i) {
    if constexpr (!KEQV)
      issue_chunk<D, KEQV, true, NW>(a, smem_off + T::kVRing + stage(t) * T::kTile, ids.a, ids.b,
                                     wave, i, vlane);
  };
  auto issue_tile = [&](int t, const TileIds& ids) {
#pragma unroll
    for (int i = 0; i < T::kPerWave; ++i) k_chunk(t, ids, i);
#pragma unroll
    for (int i = 0; i < T::kPerWave; ++i) v_chunk(t, ids, i);
  };

  // One tile: S^T, mask, online softmax, O^T; on the way it copies the `ncp` (a compile-time
  // count) tiles ct, ct + 1, .. whose ids are cids[0], cids[1], ..
  auto process_tile = [&](int t, auto ncp, int ct, const TileIds* cids) {
    constexpr int Q = decltype(ncp)::value * T::kPerWave;  // copies of each ring
    const int k0 = (kt0 + t) * kTileKeys;
    const unsigned char* kt = smem + T::kKRing + stage(t) * T::kTile;
    const unsigned char* vt = smem + T::kVRing + stage(t) * T::kTile + voff;
    const unsigned char* rt = smem + T::kRopeOff + ((unsigned)t & 1u) * T::kRopeTile;
    // K fragment f (chunk c = f / 2, product m = f % 2); exact K=V reads the chunks holding
    // dimensions 0-63 and their partners from the rotated copies
    auto kread = [&](auto fc) -> bf16x8_t {
      constexpr int f = decltype(fc)::value, c = f >> 1;
      constexpr int rc = EXACT ? rope_chunk_of<NC, f>() : -1;
      if constexpr (rc >= 0)
        return as_bf16x8(
            *(const u32x4_t*)(rt - rdiff + koff[f & 1][(rc >> 1) & 1] + 1024 * rc));
      else
        return as_bf16x8(*(const u32x4_t*)(kt + koff[f & 1][(c >> 1) & 1] + 1024 * c));
    };

    // ---- S^T = K Q^T: s[m][rb], product m covering the key rows described above.  One
    // chunk per K fragment f (c = f / 2, m = f % 2): its R products, the read of fragment
    // f + kPF and a share of the tile copies; the fences keep the reads kPF fragments ahead of
    // the products that use them.
    float4_t s[2][R];
    bf16x8_t kf[2 * NC];
    sfor<kPF>([&](auto fc) {
      constexpr int f = decltype(fc)::value;
      kf[f] = kread(fc);
    });
    sfor<2 * NC>([&](auto fc) {
      constexpr int f = decltype(fc)::value;
      if constexpr (f + kPF < 2 * NC) kf[f + kPF] = kread(std::integral_constant<int, f + kPF>{});
      sfor<(f + 1) * Q / (2 * NC) - f * Q / (2 * NC)>([&](auto qc) {
        constexpr int q = f * Q / (2 * NC) + decltype(qc)::value;
        k_chunk(ct + q / T::kPerWave, cids[q / T::kPerWave], q % T::kPerWave);
      });
      constexpr int rc = EXACT ? rope_chunk_of<NC, f>() : -1;
      if constexpr (rc >= 0) {  // the lo terms of a rotated fragment
        const bf16x8_t lo = as_bf16x8(*(const u32x4_t*)(rt + T::kRopeLo - rdiff +
                                                         koff[f & 1][(rc >> 1) & 1] + 1024 * rc));
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
          s[f & 1][rb] = mfma_16x16x32(lo, qf[rb][f >> 1],
                                       f < 2 ? float4_t{0.f, 0.f, 0.f, 0.f} : s[f & 1][rb]);
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
          s[f & 1][rb] = mfma_16x16x32(kf[f], qf[rb][f >> 1], s[f & 1][rb]);
      } else {
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
          s[f & 1][rb] = mfma_16x16x32(kf[f], qf[rb][f >> 1],
                                       f < 2 ? float4_t{0.f, 0.f, 0.f, 0.f} : s[f & 1][rb]);
      }
      fence_sched();
    });
    // the first V^T fragments of this tile's P.V, read while the softmax runs
    bf16x8_t vf[ND];
    if constexpr (!KEQV) {
      sfor<kPF>([&](auto nc) {
        constexpr int nn = decltype(nc)::value;
        vf[nn] = as_bf16x8(*(const u32x4_t*)(vt + nn * 512));
      });
    }

    // ---- scores on the log2 scale, band + causal mask (skipped when the whole tile is
    // visible to every row of the wave)
    const bool full = k0 >= lo_max && k0 + kTileKeys - 1 <= hi_min;
    float xs[R][8];
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[rb][e] = score_in<SM>(s[e >> 2][rb][e & 3], a.sc);
    if (!full) {
      const int kk = k0 + kslot;
#pragma unroll
      for (int rb = 0; rb < R; ++rb) {
        const int d0 = kk - lo_c[rb];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          xs[rb][e] = (uint32_t)(d0 + e) <= span_c[rb] ? xs[rb][e] : -INFINITY;
      }
    }
    // ---- online softmax with a lazily moved reference (kLazyLog2), so most tiles skip the
    // rescale of O
    bool need = false;
    float mx[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      const float m = score_max<SM>(max_over_groups_nc(max8_nc(xs[rb])), a.sc);
      mx[rb] = m;
      need |= m > m_ref[rb] + kLazyLog2;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int rb = 0; rb < R; ++rb) {
        const float m_new = mx[rb] > m_ref[rb] + kLazyLog2 ? mx[rb] : m_ref[rb];
        const float alpha = m_ref[rb] == -INFINITY ? 1.f : fast_exp2(m_ref[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int nn = 0; nn < ND; ++nn) o[rb][nn] *= alpha;
        m_ref[rb] = m_new;
      }
    }
    bf16x8_t pf[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      const float mu = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
      bf16x2_t pw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pw[w] = cvt_bf16x2(fast_exp2(score_exp_arg<SM>(xs[rb][2 * w], mu, a.sc)),
                           fast_exp2(score_exp_arg<SM>(xs[rb][2 * w + 1], mu, a.sc)));
        // the row sum uses the same bf16-rounded weights that multiply V
        l_run[rb] = sum_bf16x2(pw[w], l_run[rb]);
      }
      pf[rb] = bf16x8_t{pw[0][0], pw[0][1], pw[1][0], pw[1][1],
                        pw[2][0], pw[2][1], pw[3][0], pw[3][1]};
    }

    // ---- O^T[d][row] += V^T[d][keys] P^T[keys][row], one chunk per V^T fragment
    if constexpr (!KEQV) {
      sfor<ND>([&](auto nc) {
        constexpr int nn = decltype(nc)::value;
        if constexpr (nn + kPF < ND)
          vf[nn + kPF] = as_bf16x8(*(const u32x4_t*)(vt + (nn + kPF) * 512));
        sfor<(nn + 1) * Q / ND - nn * Q / ND>([&](auto qc) {
          constexpr int q = nn * Q / ND + decltype(qc)::value;
          v_chunk(ct + q / T::kPerWave, cids[q / T::kPerWave], q % T::kPerWave);
        });
#pragma unroll
        for (int rb = 0; rb < R; ++rb) o[rb][nn] = mfma_16x16x32(vf[nn], pf[rb], o[rb][nn]);
        fence_sched();
      });
    } else {
      // values are the keys: V^T fragment nn covers the 16 dimensions of units x0(nn) and
      // x0(nn) + 8 (kv_block_unit; A row i is dimension kv_block_dim(nn, i)), keys 8 (j % 2) ..
      // + 7 of page j / 2, by two transposing reads.  Lane 4e + q of a group points at half
      // q % 2 of unit x0 + 8 (q / 2) of key 8 (j % 2) + e (first read) or + 4 + e (second);
      // units x0 and x0 + 8 sit 4 row slots apart, so the reads are free of bank conflicts.
      const int pg = j >> 1, e4 = c16 >> 2, q4 = c16 & 3;
      const int vb = pg * T::kPageBytes + 256 * 8 * (q4 >> 1) + 8 * (q4 & 1);
      const int vr0 = vb + 16 * ((8 * (j & 1) + e4 + 4 * pg + 4 * (q4 >> 1)) & 15);
      const int vr1 = vb + 16 * ((8 * (j & 1) + 4 + e4 + 4 * pg + 4 * (q4 >> 1)) & 15);
#pragma unroll
      for (int nn = 0; nn < ND; ++nn) {
        const u32x2_t lo = lds_read_tr16(kt + vr0 + 256 * kv_block_unit(nn));
        const u32x2_t hi = lds_read_tr16(kt + vr1 + 256 * kv_block_unit(nn));
        const bf16x8_t af = as_bf16x8(u32x4_t{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
        for (int rb = 0; rb < R; ++rb) o[rb][nn] = mfma_16x16x32(af, pf[rb], o[rb][nn]);
      }
    }
  };

  // prologue: tiles 0 .. S - TB - 1, then the Q fragments, so that the latencies of both
  // overlap.  All of them are complete before the loop: left to the compiler, the wait for the
  // Q loads would sit at their first use, inside the tile loop, and drain the in-flight tile
  // copies on every iteration.
  for (int t = 0; t < S - TB; ++t) issue_tile(t, ids_of(t));
#pragma unroll
  for (int rb = 0; rb < R; ++rb) load_q<D>(qf[rb], a.q + q_off[rb], ok_c[rb]);
  wait_vmcnt<0>();
  TileIds cids[TB];
#pragma unroll
  for (int u = 0; u < TB; ++u) cids[u] = ids_of(S - TB + u);

  // Iteration jj starts with the same steps in every wave: the wait for its tiles, the barrier
  // and the cooperative fix-ups of the staged tiles
  auto iteration_begin = [&](int jj) {
    // this iteration's tiles have landed once at most the copies of later iterations remain
    wait_vmcnt<kWait>();
    __syncthreads();
    {
      const int tl = np - 1;  // the last tile holds the keys past the context, if any
      if (tl >= TB * jj && tl < TB * jj + TB && (kt0 + tl) * kTileKeys + kTileKeys > L) {
        // slots of keys >= L may hold anything, NaN included, and a zero weight does not
        // cancel a NaN value: zero the values of those keys once, in LDS
        zero_tail_values<D, KEQV, NW>(smem + (KEQV ? T::kKRing : T::kVRing) + stage(tl) * T::kTile,
                                  L - (kt0 + tl) * kTileKeys);
        __syncthreads();
      }
    }
    if constexpr (EXACT) {
      // the rotated rope units of this iteration's tiles (the previous iteration's readers of
      // the buffer have all passed the barrier above)
      static_assert(TB == 2, "one rope buffer per tile of an iteration");
      // this thread's unit pair (row, unit column, page, tile of the iteration), derived here
      // from an opaque copy of the thread id so that nothing of the pass stays live across
      // the key loop (held there, its values spilled)
      int tid = (int)threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int rp_r = tid & 15, rp_x = (tid >> 4) & 7;
      const int rp_p = (tid >> 7) & 1, rp_u = tid >> 8;
      const int tl = TB * jj + rp_u;
      if (tl < np) {
        // source units rp_x and rp_x + D/16 of the K tile; in the rope buffer they become
        // columns rp_x and 8 + rp_x (row slots by k_slot of those columns)
        const unsigned char* src = smem + T::kKRing + stage(tl) * T::kTile + rp_p * T::kPageBytes;
        u32x4_t ua = *(const u32x4_t*)(src + 256 * rp_x + 16 * k_slot(rp_r, rp_x, rp_p));
        u32x4_t ub = *(const u32x4_t*)(src + 256 * (rp_x + D / 16) +
                                       16 * k_slot(rp_r, rp_x + D / 16, rp_p));
        u32x4_t la = {0u, 0u, 0u, 0u}, lb = {0u, 0u, 0u, 0u};
        const int64_t pos = (int64_t)(kt0 + tl) * kTileKeys + rp_p * kPage + rp_r;
        rope_units_exact(ua, ub, la, lb, rp_x, rope_rho(a.rho0, a.rho_step, 8 * rp_x),
                         a.rho_step, a.rope_pairs, pos);
        unsigned char* dst = smem + T::kRopeOff + rp_u * T::kRopeTile + rp_p * T::kRopePage;
        const int ra = 256 * rp_x + 16 * k_slot(rp_r, rp_x, rp_p);
        const int rb = 256 * (8 + rp_x) + 16 * k_slot(rp_r, 8 + rp_x, rp_p);
        *(u32x4_t*)(dst + ra) = ua;
        *(u32x4_t*)(dst + rb) = ub;
        *(u32x4_t*)(dst + T::kRopeLo + ra) = la;
        *(u32x4_t*)(dst + T::kRopeLo + rb) = lb;
      }
      __syncthreads();
    }
  };
  // ... and ends by fetching the ids of the tiles the next one copies (here, not at the
  // barrier, where every wave of the workgroup would wait for them at the same moment)
  auto iteration_end = [&](int jj) {
#pragma unroll
    for (int u = 0; u < TB; ++u) cids[u] = ids_of(TB * (jj + 1) + S - TB + u);
  };
  // A wave computes only the iterations whose tiles hold a key that one of its rows sees (a
  // sliding window's band is narrower than the workgroup's key range by the workgroup's span of
  // positions, and a wave without rows sees nothing); in the others it only takes its share of
  // the copies.  Three loops rather than a branch per iteration keep the register allocation of
  // the computing loop as it is without them.
  const int nsuper = (np + TB - 1) / TB;
  const int own_lo = lo_min / kTileKeys - kt0, own_hi = hi_max / kTileKeys - kt0;
  const int jj_lo = hi_max < 0 ? nsuper : (own_lo > 0 ? own_lo / TB : 0);
  const int jj_hi = hi_max < 0 ? nsuper : (own_hi / TB + 1 < nsuper ? own_hi / TB + 1 : nsuper);
  auto copies_only = [&](int jj) {
    constexpr int Q = TB * T::kPerWave;
    const int ct = TB * jj + S - TB;
    sfor<Q>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      k_chunk(ct + q / T::kPerWave, cids[q / T::kPerWave], q % T::kPerWave);
    });
    sfor<Q>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      v_chunk(ct + q / T::kPerWave, cids[q / T::kPerWave], q % T::kPerWave);
    });
  };
  for (int jj = 0; jj < jj_lo; ++jj) {
    iteration_begin(jj);
    copies_only(jj);
    iteration_end(jj);
  }
  for (int jj = jj_lo; jj < jj_hi; ++jj) {
    iteration_begin(jj);
    // a tile of the iteration outside the wave's band is masked whole (its weights are
    // exactly 0)
    process_tile(TB * jj, std::integral_constant<int, TB>{}, TB * jj + S - TB, cids);
    if constexpr (TB == 2) {
      if (TB * jj + 1 < np) process_tile(TB * jj + 1, std::integral_constant<int, 0>{}, 0, cids);
    }
    iteration_end(jj);
  }
  for (int jj = jj_hi; jj < nsuper; ++jj) {
    iteration_begin(jj);
    copies_only(jj);
    iteration_end(jj);
  }
  wait_vmcnt<0>();  // no copy may land in LDS after the workgroup has left it

  if (!wave_active) return;
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    float l = l_run[rb];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (!ok_c[rb]) continue;
    const int row = wrow0 + 16 * rb + c16;
    const int i = row / G, hh = row - (row / G) * G;
    const float inv = 1.0f / l;
    uint16_t* dst = a.out + ((int64_t)(q0 + i) * a.Hq + g * G + hh) * D;
#pragma unroll
    for (int nn = 0; nn < ND; ++nn) {
      // output rows 4j .. 4j+3 of fragment nn: dimensions 16 nn + 4j (separate V^T pages) or
      // kv_block_dim(nn, 4j) (values taken from the K tile) onwards
      const int d0 = KEQV ? kv_block_dim(nn, 4 * j) : 16 * nn + 4 * j;
      float f[4] = {inv, inv, inv, inv};
      if constexpr (EXACT) {
        if (a.kv_vw) {  // values are the stored keys times w_v / w_k
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] *= a.kv_vw[d0 + e] / a.kv_kw[d0 + e];
        }
      }
      *(u32x2_t*)(dst + d0) =
          u32x2_t{pack_bf16x2(o[rb][nn][0] * f[0], o[rb][nn][1] * f[1]),
                  pack_bf16x2(o[rb][nn][2] * f[2], o[rb][nn][3] * f[3])};
    }
  }
}

template <int D, int SM, bool KEQV, bool EXACT>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  constexpr int NW = waves_for<D, EXACT>();
  using T = TileLds<D, KEQV, NW>;
  constexpr int kLds = T::kBytes + (EXACT ? T::kRopeBytes : 0);
  constexpr int kRowsPerWg = Rows<D, NW>::kPerWg;
  const int64_t tiles_per_bg = ((int64_t)a.max_q_len * a.G + kRowsPerWg - 1) / kRowsPerWg;
  const int64_t runs_per_bg = (tiles_per_bg + kRun - 1) / kRun;
  const int64_t n_groups = (int64_t)a.Hkv * a.batch;
  const int64_t runs = runs_per_bg * n_groups;
  if (runs == 0) return hipSuccess;
  const int64_t grid = (runs + 7) / 8 * 8 * kRun;  // whole rounds of runs over the 8 XCDs
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  static_assert(kLds <= 160 * 1024, "LDS budget");
  hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&prefill_tiled_kernel<D, SM, KEQV, EXACT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_tiled_kernel<D, SM, KEQV, EXACT>), dim3((unsigned)grid),
                     dim3(64 * NW),
                     kLds, s, a, (int)runs_per_bg, (int)n_groups);
  return hipGetLastError();
}

template <int D, int SM>
hipError_t by_kv(const AttnArgs& a, int kv_mode, hipStream_t s) {
  switch (kv_mode) {
    case 0: return launch_t<D, SM, false, false>(a, s);
    case 1: return launch_t<D, SM, true, false>(a, s);
    case 2: return launch_t<D, SM, true, true>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t by_flags(const AttnArgs& a, bool cap, int kv_mode, hipStream_t s) {
  if (cap) return by_kv<D, kScoreCap>(a, kv_mode, s);
  // a positive scale commutes with the max, so it can be applied inside the exponent
  return a.sc.c_scale > 0.f ? by_kv<D, kScoreFold>(a, kv_mode, s)
                            : by_kv<D, kScorePlain>(a, kv_mode, s);
}

}  // namespace

GA_DEBUG_TAKE_DEFINE(debug_take_prefill)

hipError_t launch_prefill(const AttnLaunch& L, hipStream_t s) {
  if (L.batch == 0 || L.total_q == 0) return hipSuccess;
  if (!L.dtype_bf16) return launch_attn_f32(L, false, s);
  const AttnArgs a = make_attn_args(L);
  const bool cap = L.softcap > 0.f;
  switch (L.D) {
    case 128: return by_flags<128>(a, cap, L.k_eq_v, s);
    case 256: return by_flags<256>(a, cap, L.k_eq_v, s);
    case 512: return by_flags<512>(a, cap, L.k_eq_v, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ga
