/*
 * ga_ref.c -- CPU oracle for paged Gemma-style attention.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the slow, plain, fp64 statement of what the GPU library computes.  Only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header, table or constant with the GPU
 * library: every index formula and every step is written out here on its own.
 *
 * Sources (the web pages this method is taken from), cited below by key:
 *   [KUNLUN] "Gemma 4 模型架构解析" -- Gemma 4 adaptation guide for vLLM-Kunlun
 *            (kenforever1.github.io, llm_cool_docs, gemma4-adaptation-guide).
 *   [MNN]    "MNN 支持 Gemma4 全系列：PLE、KV共享与多模态" (zhaode.wang blog, 2026/gemma4).
 *   [INFLM]  "Feat/add gemma3 model" -- InfiniLM pull request 581, "支持 gemma2 与
 *            gemma3_text 模型推理".
 *
 * What is computed (all arithmetic in double precision, no tiling, no online softmax):
 *   write:     RMSNorm of q, k, v per head ([MNN] §6.1; [INFLM] Gemma-3 §1 QK-norm), then
 *              rotary position embedding of q and k only ([KUNLUN] §4.3 forward listing of the
 *              non-shared layer; [MNN] §6.2), then the scatter of k and v into pages through
 *              the block table ([KUNLUN] §6.3 slot formula, §6.4 write path).
 *   attention: for a query at absolute position t, the visible keys are lo(t) .. t with
 *              lo(t) = max(0, t - W + 1) for a sliding layer and 0 for a global one
 *              ([INFLM] Gemma-3 §3: the band hides a key whose distance from the query's
 *              position reaches W, the causal limit hides later keys, both hold for chunked
 *              prefill, and a sliding decode step reads only the last min(length, W) keys).
 *              Scores are scale * q.k, optionally soft-capped as cap * tanh(s / cap) before
 *              the mask and the softmax ([INFLM] Gemma-2 §1 and the attention-softcap section
 *              of its framework changes), then a plain two-pass softmax and the weighted sum
 *              of V.
 *              GQA: query head h reads kv head h / (Hq / Hkv) ([INFLM] Gemma-3 §3, head-first
 *              regrouping).  K=V: one stored tensor serves as keys and values.
 *
 * Readings where the pages leave a step open (each is listed with its reason in the design
 * notes of the repository):
 *   - RMSNorm: x / sqrt(mean(x^2) + eps) * w, with w the effective weight (NULL: no norm).
 *   - RoPE pairs dimension k with k + D/2 ("rotate half"), frequency theta^(-2k/D) for
 *     k < D/2 ([KUNLUN] 挑战 5 inverse-frequency listing with rope_angles = D/2), angle t*omega
 *     with t the 0-based absolute position.  The pairing convention itself is not stated by
 *     the pages: parity unpinned for the pairing, pinned for the invariants.
 *   - Masked keys are left out of the sums (weight exactly 0).
 *
 * Memory layout of the paged cache (the library's documented format):
 *   K page: k_cache[blk][g][16 rows x D], stored in 16-byte units: unit (row off, x) holds
 *           elements d = x*U .. x*U+U-1 of key row off (U = 8 for bf16, 4 for fp32) and
 *           sits at unit slot 16*x + ((off + 4*(lp % 2) + 4*((x / 8) % 2)) % 16) of the page,
 *           lp = pos / 16 being the page's logical index in its sequence (rows rotated by 4
 *           on odd pages and again in unit columns whose bit 3 is set).
 *   V page: v_cache[blk][g][d][off]   -- d-major, the 16 (block_size) keys of a page contiguous.
 *   With k_eq_v the V operand is read from k_cache.
 * dtype code: 0 = fp32 (float storage), 1 = bf16 (uint16_t storage, round-to-nearest-even).
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_FP32 0
#define REF_BF16 1

/* Threads the parallel loops below will use (1 without OpenMP). */
int ref_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------- number formats --- */

/* bf16 -> double: the 16 stored bits are the top half of an IEEE single. */
static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* double -> bf16 with one rounding, to nearest, ties to even.  bf16 keeps 8 significant
 * bits, the exponent range of IEEE single, and subnormals down to 2^-133. */
uint16_t ref_double_to_bf16(double x) {
  float f;
  uint32_t u;
  if (isnan(x)) return (uint16_t)0x7fc0u;
  if (x == 0.0) {
    f = (float)x; /* keeps the sign of zero */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
  }
  if (isinf(x)) return signbit(x) ? (uint16_t)0xff80u : (uint16_t)0x7f80u;
  {
    int e;
    double m = frexp(fabs(x), &e); /* |x| = m * 2^e, m in [0.5, 1) */
    int q = e - 8;                 /* quantum exponent for 8 significant bits */
    double r;
    if (q < -133) q = -133;        /* subnormal quantum */
    r = nearbyint(ldexp(fabs(x), -q)); /* default rounding mode: to nearest, ties to even */
    r = ldexp(r, q);
    if (r >= ldexp(1.0, 128)) r = INFINITY; /* overflow after rounding */
    f = (float)(signbit(x) ? -r : r);       /* exact: r has at most 8 significant bits */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
  }
}

double ref_bf16_to_double(uint16_t h) { return bf16_bits_to_double(h); }

static double load_elem(const void* base, int dtype, int64_t i) {
  if (dtype == REF_BF16) return bf16_bits_to_double(((const uint16_t*)base)[i]);
  return (double)((const float*)base)[i];
}

static void store_elem(void* base, int dtype, int64_t i, double x) {
  if (dtype == REF_BF16)
    ((uint16_t*)base)[i] = ref_double_to_bf16(x);
  else
    ((float*)base)[i] = (float)x; /* one rounding, to nearest even */
}

/* ---------------------------------------------------------------- paging ----------- */

/* [KUNLUN] §6.3: slot = block_table[req][pos / block_size] * block_size + pos % block_size.
 * ring != 0: the row is a ring of max_blocks entries and logical page pos / block_size sits in
 * entry (pos / block_size) mod max_blocks (a sliding layer's windowed cache, [INFLM] Gemma-3
 * §3, kept in pages).  Returns the slot; *blk and *off receive the page id and the row inside
 * the page. */
int64_t ref_slot(const int32_t* block_table, int32_t max_blocks, int ring, int32_t req,
                 int64_t pos, int32_t block_size, int64_t* blk, int64_t* off) {
  int64_t page = pos / block_size;
  int64_t b = block_table[(int64_t)req * max_blocks + (ring ? page % max_blocks : page)];
  int64_t o = pos % block_size;
  if (blk) *blk = b;
  if (off) *off = o;
  return b * block_size + o;
}

/* Element index of K[g][pos][d] of one sequence inside k_cache: page (blk, g) of bs*D elements,
 * unit layout described at the top (pos % bs == off; the logical page pos / bs fixes the row
 * rotation). */
static int64_t k_index(int64_t blk, int64_t off, int g, int d, int Hkv, int bs, int D, int dtype,
                       int64_t pos) {
  const int64_t U = dtype == 1 ? 8 : 4; /* elements per 16-byte unit */
  const int64_t lp = pos / bs;
  const int64_t x = d / U; /* unit column */
  const int64_t row_slot = (off + 4 * (lp % 2) + 4 * ((x / 8) % 2)) % bs;
  const int64_t unit = x * bs + row_slot;
  return (blk * Hkv + g) * bs * (int64_t)D + unit * U + d % U;
}

/* Element index of V[g][pos][d] inside v_cache ([blk][g][d][off]). */
static int64_t v_index(int64_t blk, int64_t off, int g, int d, int Hkv, int bs, int D) {
  return ((blk * Hkv + g) * (int64_t)D + d) * bs + off;
}

/* ---------------------------------------------------------------- write ------------ */

/* RMSNorm in double: y = x / sqrt(mean(x^2) + eps) * w.  w == NULL: y = x. */
void ref_rms_norm(const double* x, const float* w, int D, double eps, double* y) {
  int d;
  double ss = 0.0, inv;
  if (!w) {
    for (d = 0; d < D; ++d) y[d] = x[d];
    return;
  }
  for (d = 0; d < D; ++d) ss += x[d] * x[d];
  inv = 1.0 / sqrt(ss / D + eps);
  for (d = 0; d < D; ++d) y[d] = x[d] * inv * (double)w[d];
}

/* Rotary embedding at position t, rotate-half pairing (k, k + D/2).
 * [KUNLUN] 挑战 5 (proportional RoPE): the frequency of pair k is 1 / theta^(2k / D) -- the
 * exponent's denominator is the head size -- for the first `angles` pairs, and 0 (no rotation)
 * for the rest; angles = D/2 is the full rotation.  [INFLM] follow-up list (linear RoPE
 * scaling): the position enters as t / pos_scale.  theta <= 0: identity. */
void ref_rope(const double* x, int D, double t, double theta, int angles, double pos_scale,
              double* y) {
  int k, half = D / 2;
  if (theta <= 0.0) {
    for (k = 0; k < D; ++k) y[k] = x[k];
    return;
  }
  for (k = 0; k < half; ++k) {
    double omega = k < angles ? 1.0 / pow(theta, (2.0 * k) / (double)D) : 0.0;
    double a = (t / pos_scale) * omega, c = cos(a), s = sin(a);
    y[k] = x[k] * c - x[k + half] * s;
    y[k + half] = x[k + half] * c + x[k] * s;
  }
}

/* ref_rope applied to n rows x[i*D ..] at positions t[i] (independent rows, in parallel). */
void ref_rope_rows(const double* x, const double* t, int64_t n, int D, double theta, int angles,
                   double pos_scale, double* y) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) ref_rope(x + i * D, D, t[i], theta, angles, pos_scale, y + i * D);
}

/* Norm, rotate and scatter the new tokens of every sequence.
 *   q: [T][Hq][D] raw in, written back normalised and rotated (may be NULL);
 *   k, v: [T][Hkv][D] raw (v NULL iff k_eq_v); k and v both NULL: a layer that shares another
 *   layer's cache ([KUNLUN] §4.3: only q is normed and rotated, nothing is stored);
 *   rope_angles: rotated frequency pairs (0 = all D/2); rope_scale: position divisor (0 = 1);
 *   cu_seqlens[B+1]: offsets of each sequence's new tokens; context_lens[B]: length after the
 *   write, so the new tokens of sequence b sit at positions context_lens[b] - n_b ... */
int ref_kv_cache_write(int dtype, int Hq, int Hkv, int D, int bs, double rope_theta,
                       int rope_angles, double rope_scale, double rms_eps, int k_eq_v, void* q,
                       const void* k, const void* v,
                       const float* wq, const float* wk, const float* wv,
                       const int32_t* cu_seqlens, const int32_t* context_lens,
                       const int32_t* block_table, int32_t max_blocks, int ring,
                       int32_t batch,
                       void* k_cache, void* v_cache) {
  int b;
  const int angles = rope_angles > 0 && rope_angles < D / 2 ? rope_angles : D / 2;
  const double pscale = rope_scale > 0.0 ? rope_scale : 1.0;
  double *x = (double*)malloc(sizeof(double) * D), *y = (double*)malloc(sizeof(double) * D),
         *z = (double*)malloc(sizeof(double) * D);
  if (!x || !y || !z) {
    free(x); free(y); free(z);
    return 1;
  }
  for (b = 0; b < batch; ++b) {
    int n = cu_seqlens[b + 1] - cu_seqlens[b];
    int64_t past = (int64_t)context_lens[b] - n;
    int i, h, d;
    for (i = 0; i < n; ++i) {
      int64_t tok = cu_seqlens[b] + i, t = past + i, blk, off;
      ref_slot(block_table, max_blocks, ring, b, t, bs, &blk, &off);
      if (q) {
        for (h = 0; h < Hq; ++h) {
          int64_t base = (tok * Hq + h) * (int64_t)D;
          for (d = 0; d < D; ++d) x[d] = load_elem(q, dtype, base + d);
          ref_rms_norm(x, wq, D, rms_eps, y);
          ref_rope(y, D, (double)t, rope_theta, angles, pscale, z);
          for (d = 0; d < D; ++d) store_elem(q, dtype, base + d, z[d]);
        }
      }
      for (h = 0; k && h < Hkv; ++h) {
        int64_t base = (tok * Hkv + h) * (int64_t)D;
        for (d = 0; d < D; ++d) x[d] = load_elem(k, dtype, base + d);
        ref_rms_norm(x, wk, D, rms_eps, y);
        ref_rope(y, D, (double)t, rope_theta, angles, pscale, z);
        for (d = 0; d < D; ++d)
          store_elem(k_cache, dtype, k_index(blk, off, h, d, Hkv, bs, D, dtype, t), z[d]);
        if (!k_eq_v) {
          for (d = 0; d < D; ++d) x[d] = load_elem(v, dtype, base + d);
          ref_rms_norm(x, wv, D, rms_eps, y); /* values are not rotated */
          for (d = 0; d < D; ++d) store_elem(v_cache, dtype, v_index(blk, off, h, d, Hkv, bs, D), y[d]);
        }
      }
    }
  }
  free(x); free(y); free(z);
  return 0;
}

/* ---------------------------------------------------------------- attention -------- */

/* Gather keys lo..hi of kv head g of sequence b into K[j-lo][d] and V[j-lo][d] (double). */
static void gather(int dtype, int Hkv, int D, int bs, int k_eq_v, const void* k_cache,
                   const void* v_cache, const int32_t* block_table, int32_t max_blocks,
                   int ring, int b,
                   int g, int64_t lo, int64_t hi, double* K, double* V) {
  int64_t j;
  int d;
  for (j = lo; j <= hi; ++j) {
    int64_t blk, off;
    ref_slot(block_table, max_blocks, ring, b, j, bs, &blk, &off);
    for (d = 0; d < D; ++d) {
      K[(j - lo) * D + d] = load_elem(k_cache, dtype, k_index(blk, off, g, d, Hkv, bs, D, dtype, j));
      V[(j - lo) * D + d] = k_eq_v ? K[(j - lo) * D + d]
                                   : load_elem(v_cache, dtype, v_index(blk, off, g, d, Hkv, bs, D));
    }
  }
}

/* One query vector against n gathered keys: plain softmax attention in double. */
static void attend(const double* qv, const double* K, const double* V, int64_t n, int D,
                   double scale, double cap, double* s, double* out) {
  int64_t j;
  int d;
  double m = -INFINITY, den = 0.0;
  for (j = 0; j < n; ++j) {
    double acc = 0.0;
    for (d = 0; d < D; ++d) acc += qv[d] * K[j * D + d];
    acc *= scale;
    if (cap > 0.0) acc = cap * tanh(acc / cap); /* soft cap before the mask and softmax */
    s[j] = acc;
    if (acc > m) m = acc;
  }
  for (d = 0; d < D; ++d) out[d] = 0.0;
  for (j = 0; j < n; ++j) {
    double p = exp(s[j] - m);
    den += p;
    for (d = 0; d < D; ++d) out[d] += p * V[j * D + d];
  }
  for (d = 0; d < D; ++d) out[d] /= den;
}

/* Attention rows.  Query r (0 <= r < total_q) belongs to sequence b with
 * cu_seqlens_q[b] <= r < cu_seqlens_q[b+1] and sits at absolute position
 * t = context_lens[b] - n_b + (r - cu_seqlens_q[b]).  rows == NULL computes every row;
 * otherwise only rows[0..n_rows-1] (out is still indexed by r).  out: [total_q][Hq][D]. */
int ref_attention(int dtype, int Hq, int Hkv, int D, int bs, int window, double scale,
                  double softcap, int k_eq_v, const void* q, const int32_t* cu_seqlens_q,
                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                  int32_t max_blocks, int ring, const int32_t* context_lens, int32_t batch,
                  int32_t total_q, const int32_t* rows, int32_t n_rows, double* out) {
  int G = Hq / Hkv, nr = rows ? n_rows : total_q, err = 0;
  int64_t maxlen = 0;
  int b, idx;
  for (b = 0; b < batch; ++b)
    if (context_lens[b] > maxlen) maxlen = context_lens[b];
  if (window > 0 && window < maxlen) maxlen = window; /* keys one query can see */
#pragma omp parallel
  {
    double *K = (double*)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1) * D);
    double *V = (double*)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1) * D);
    double *s = (double*)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
    double *qv = (double*)malloc(sizeof(double) * D);
    if (!K || !V || !s || !qv) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (idx = 0; idx < nr; ++idx) {
        int r = rows ? rows[idx] : idx, bb = 0, h, gcur = -1, d;
        int64_t t, lo, past;
        while (bb + 1 < batch && cu_seqlens_q[bb + 1] <= r) ++bb;
        past = (int64_t)context_lens[bb] - (cu_seqlens_q[bb + 1] - cu_seqlens_q[bb]);
        t = past + (r - cu_seqlens_q[bb]);
        lo = (window > 0 && t - window + 1 > 0) ? t - window + 1 : 0;
        for (h = 0; h < Hq; ++h) {
          int g = h / G;
          if (g != gcur) {
            gather(dtype, Hkv, D, bs, k_eq_v, k_cache, v_cache, block_table, max_blocks, ring,
                   bb, g, lo, t, K, V);
            gcur = g;
          }
          for (d = 0; d < D; ++d) qv[d] = load_elem(q, dtype, ((int64_t)r * Hq + h) * D + d);
          attend(qv, K, V, t - lo + 1, D, scale, softcap, s, out + ((int64_t)r * Hq + h) * D);
        }
      }
    }
    free(K); free(V); free(s); free(qv);
  }
  return err;
}

/* Decode: one query per sequence, at position context_lens[b] - 1.  q: [B][Hq][D]. */
int ref_attn_decode(int dtype, int Hq, int Hkv, int D, int bs, int window, double scale,
                    double softcap, int k_eq_v, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_table, int32_t max_blocks,
                    int ring, const int32_t* context_lens, int32_t batch, double* out) {
  int rc, b;
  int32_t* cu = (int32_t*)malloc(sizeof(int32_t) * (batch + 1));
  if (!cu) return 1;
  for (b = 0; b <= batch; ++b) cu[b] = b;
  rc = ref_attention(dtype, Hq, Hkv, D, bs, window, scale, softcap, k_eq_v, q, cu, k_cache,
                     v_cache, block_table, max_blocks, ring, context_lens, batch, batch, NULL, 0,
                     out);
  free(cu);
  return rc;
}
