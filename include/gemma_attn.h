/*
 * gemma_attn.h -- C ABI of the MI355X (gfx950) paged-KV Gemma-style attention library.
 *
 * Three operations make up one attention layer's hot path:
 *   ga_kv_cache_write  RMSNorm of q/k/v, rotary embedding of q/k, scatter of k/v into pages;
 *   ga_attn_decode     one query per sequence against its paged cache (split-K flash decoding);
 *   ga_attn_prefill    a chunk of new queries per sequence against its paged cache (MFMA flash
 *                      attention with the exact band + causal mask).
 *
 * Sources, cited by key:
 *   [KUNLUN] "Gemma 4 模型架构解析" -- the Gemma 4 adaptation guide for vLLM-Kunlun: 挑战 1-3
 *            (per-layer type, head size, k_eq_v), 挑战 5 (RoPE frequencies), §4 (shared KV),
 *            §6.3 (slot formula), §6.4 (write path), §6.5 (paged read path).
 *   [MNN]    "MNN 支持 Gemma4 全系列：PLE、KV共享与多模态": §2.2 (dual RoPE: head size 256 with
 *            theta 1e4 on sliding layers, 512 with 1e6 on global ones), §6.1 (q/k/v norms,
 *            attention scale 1.0), §6.2 (K=V and per-layer-type KV head counts).
 *   [INFLM]  "Feat/add gemma3 model" (InfiniLM pull request 581): Gemma-2 §1 (logit soft cap
 *            after scaling, before mask and softmax; scale from query_pre_attn_scalar),
 *            Gemma-3 §3 (band + causal mask for prefill and chunked prefill, decode reads the
 *            last min(len, W) keys, head-first GQA), and its hardening table (reject bad
 *            configurations loudly, never return silently wrong results).
 *
 * Conventions for every call
 *   - Pointers marked DEVICE are device (HBM) addresses; HOST ones are host addresses.  All
 *     buffers are owned by the caller; the library allocates nothing, frees nothing and keeps
 *     no state between calls, so it is safe to call from several host threads.  The one
 *     exception is ga_attn_decode_noalloc, whose scratch is a fixed device array of the
 *     library (one per device) that its calls share.
 *   - `stream` is a hipStream_t (NULL: the default stream).  Every call only enqueues work on
 *     it and returns; nothing is synchronised.
 *   - Scalar arguments and the params struct are checked on the host before anything is
 *     enqueued; a failing call returns an error and enqueues nothing.  Values that live in
 *     device memory (lengths, block ids) cannot be read by the host without a copy: validate
 *     them with ga_check_metadata_host on host copies.  The kernels clamp every page index and
 *     block id into the buffers they were given, so bad metadata yields wrong numbers but no
 *     out-of-bounds access.  The debug build (libgemma_attn_debug.so) also checks that metadata
 *     in the kernels and reports it through ga_debug_take_error (at the end of this header).
 *   - ga_last_error() returns a thread-local, human-readable reason for the last failure.
 *
 * Paged cache layout (block_size 16, the default page size of vLLM's paged cache; [KUNLUN] §6.3
 * gives the slot arithmetic):
 *   k_cache: [num_blocks][num_kv_heads][16 * head_dim]  one key page per (block, kv head)
 *   v_cache: [num_blocks][num_kv_heads][head_dim][16]   value columns, the 16 keys contiguous
 *   Token position t of sequence b lives in block block_table[b][t / 16], row r = t % 16 of
 *   the page whose logical index in the sequence is lp = t / 16.  With page_ring = 1 (sliding
 *   layers only) the table row is a ring instead: logical page lp lives in block
 *   block_table[b][lp % max_blocks], so a sliding layer holds O(window) pages per sequence
 *   whatever its length ([INFLM] Gemma-3 §3 keeps a windowed cache and reads only the keys
 *   inside the window; follow-up 2 gives the key range a chunk needs, past - W + 1 onwards).
 *   Pages wrap in place: writing position t reuses the block of position t - 16*max_blocks.
 *   A ring row must therefore hold every page a call reads after its write: for decode
 *   max_blocks >= floor((W - 1) / 16) + 2, for a prefill chunk of at most n new tokens
 *   max_blocks >= floor((n + W - 2) / 16) + 3 (the window of the chunk's first query, the
 *   chunk itself, and one page for the 32-key tile alignment of the prefill kernel).  The
 *   attention calls refuse smaller rings; ga_kv_cache_write cannot know the chunk a later call
 *   attends with, so sizing the ring is the caller's part there.
 *   A key page is kept in 16-byte units: unit (row r, x) holds elements x*U .. x*U+U-1 of key
 *   row r (U = 8 for bf16, 4 for fp32) at unit slot 16*x + (r + 4*(lp % 2) + 4*((x/8) % 2)) % 16
 *   of the page, i.e. the 16 rows of one unit column are contiguous (256 bytes) and the rows are
 *   rotated by 4 on pages of odd logical index and again in unit columns whose bit 3 is set.
 *   This is the order in which a 32-key tile (an even page, then an odd one) is read without
 *   LDS bank conflicts by the matrix-core score operands and, in the K=V forms, by the
 *   transposing value reads, so a tile is copied to LDS as whole contiguous 1 KiB runs.
 *   The value page is stored transposed so that the matrix-core operand of P.V reads 16
 *   contiguous bytes per lane; with k_eq_v there is no v_cache and values are read from k_cache.
 */
#ifndef GEMMA_ATTN_H
#define GEMMA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GA_OK = 0,
  GA_ERR_INVALID_ARG = 1, /* a pointer, size or parameter violates this header */
  GA_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (head_dim, group size, dtype) */
  GA_ERR_WORKSPACE = 3,   /* decode workspace missing or smaller than ga_decode_workspace_bytes */
  GA_ERR_HIP = 4          /* the HIP runtime reported an error when enqueuing a kernel */
} ga_status;

typedef enum {
  GA_FP32 = 0, /* q, k, v, caches and out are float */
  GA_BF16 = 1  /* ... are bfloat16 (round-to-nearest-even on every store) */
} ga_dtype;

/* Per-layer constants ([KUNLUN] 挑战 1-2: every layer picks head size, RoPE base and window
 * from its type; [MNN] §2.2, §6.1-6.2). */
typedef struct {
  int32_t dtype;        /* ga_dtype */
  int32_t num_q_heads;  /* Hq >= 1 */
  int32_t num_kv_heads; /* Hkv >= 1, Hq % Hkv == 0; query head h reads kv head h / (Hq/Hkv) */
  int32_t head_dim;     /* D: 128, 256 or 512 */
  int32_t block_size;   /* tokens per page: must be 16 */
  int32_t window;       /* W > 0: sliding layer, a query at position t sees keys t-W+1 .. t;
                           W == 0: global layer (keys 0 .. t); W < 0: GA_ERR_INVALID_ARG */
  float scale;          /* score = scale * q.k (1.0 for Gemma 4; 1/sqrt(query_pre_attn_scalar)
                           for Gemma 2); must be finite */
  float softcap;        /* > 0: score <- softcap * tanh(score / softcap) after scaling and
                           before mask and softmax; 0: off; < 0 or non-finite: invalid */
  int32_t k_eq_v;       /* 0: separate K and V caches.  1: one cache (k_cache) of normalised,
                           rotated keys serves as keys and values.  2: exact K=V ([MNN] §6.2:
                           K is k_norm + RoPE of the shared projection, V its v_norm without
                           RoPE): k_cache holds the normalised keys UNROTATED, the attention
                           kernels rotate them for the scores and read them unrotated, scaled by
                           kv_v_norm_w / kv_k_norm_w (below), as values.  With 1 or 2,
                           v, v_cache and v_norm_w must be NULL */
  float rope_theta;     /* RoPE base (1e4 sliding, 1e6 global); 0: no rotation; < 0 invalid */
  float rms_eps;        /* RMSNorm epsilon, >= 0 (Gemma layers use 1e-6) */
  int32_t rope_angles;  /* rotated frequency pairs n ([KUNLUN] 挑战 5, proportional RoPE): pair k
                           (dimensions k and k + D/2) turns by t * theta^(-2k/D) for k < n and
                           not at all for k >= n; 0 (or D/2) rotates every pair; < 0 or > D/2
                           invalid */
  float rope_scale;     /* linear RoPE scaling ([INFLM] follow-up list: Gemma-3 global layers use
                           a linear factor, e.g. 8): the angle uses t / rope_scale instead of t;
                           0 means 1; < 0 or non-finite invalid */
  int32_t page_ring;    /* 0: block_table[b][lp] holds logical page lp.  1: the table row is a
                           ring of max_blocks pages, lp -> column lp % max_blocks (sliding-window
                           page recycling, see the layout notes above); needs window > 0 and
                           context lengths below 2^30.  Other values invalid */
  const float* kv_k_norm_w; /* k_eq_v = 2 only (NULL otherwise): DEVICE fp32 [head_dim], the
                           layer's k_norm and v_norm weights.  The attention calls take value d of
                           a key as its stored element d times kv_v_norm_w[d] / kv_k_norm_w[d];
                           both NULL: factor 1 (neither norm has a weight).  Weights must be
                           nonzero.  Exact mode supports rope_angles (effective) <= 64 */
  const float* kv_v_norm_w;
} ga_layer_params;

/* Norm + rotate + scatter the new tokens of a batch ([KUNLUN] §4.3 forward of a layer that
 * owns its cache: k_norm, RoPE on q and k, v_norm; §6.3-6.4 slot and write path; [MNN] §6.1).
 *   q            DEVICE [total_tokens][Hq][D]   raw query in; normalised and rotated query out
 *                (in place).  May be NULL (only k/v are written).
 *   k            DEVICE [total_tokens][Hkv][D]  raw keys.  NULL: a layer that reads another
 *                layer's cache ([KUNLUN] §4, YOCO KV sharing: only q is normed and rotated);
 *                q must then be given, v, k_norm_w and v_norm_w must be NULL, and nothing is
 *                stored (block_table, k_cache and v_cache may be NULL and are not read).
 *   v            DEVICE [total_tokens][Hkv][D]  raw values; NULL iff k_eq_v.
 *   q_norm_w,
 *   k_norm_w,
 *   v_norm_w     DEVICE float [D] effective RMSNorm weights, or NULL for "no norm" on that
 *                tensor.  y = x / sqrt(mean(x^2) + eps) * w.  v_norm_w must be NULL if k_eq_v.
 *   cu_seqlens   DEVICE int32 [batch+1]: the new tokens of sequence b are rows
 *                cu_seqlens[b] .. cu_seqlens[b+1]-1; cu_seqlens[batch] == total_tokens.
 *   context_lens DEVICE int32 [batch]: tokens of sequence b after this write; its new tokens
 *                take positions context_lens[b] - n_b .. context_lens[b] - 1.
 *   block_table  DEVICE int32 [batch][max_blocks].
 *   k_cache, v_cache  DEVICE, layouts above; v_cache NULL iff k_eq_v.  num_blocks = pages in each.
 * Rotation: pair (k, k + D/2) turns by angle (t / rope_scale) * theta^(-2k/D) for k <
 * rope_angles (all pairs by default), with the angle formed and the whole norm + rotation
 * evaluated in double precision and rounded once into the storage type.
 * Values are normalised but never rotated. */
ga_status ga_kv_cache_write(const ga_layer_params* p, void* q, const void* k, const void* v,
                            const float* q_norm_w, const float* k_norm_w, const float* v_norm_w,
                            const int32_t* cu_seqlens, const int32_t* context_lens,
                            const int32_t* block_table, int32_t max_blocks, int32_t batch,
                            int32_t total_tokens, void* k_cache, void* v_cache,
                            int64_t num_blocks, void* stream);

/* Bytes of DEVICE scratch that ga_attn_decode needs for this shape (0 if none).  The value
 * depends only on the arguments, never on device data. */
size_t ga_decode_workspace_bytes(const ga_layer_params* p, int32_t batch,
                                 int32_t max_context_len);

/* Decode attention: one query per sequence, at position context_lens[b] - 1 ([INFLM] Gemma-3
 * §3: a sliding layer reads only the last min(len, W) keys; [KUNLUN] §6.5 paged read).
 *   q            DEVICE [batch][Hq][D], already normalised and rotated (ga_kv_cache_write).
 *   k_cache, v_cache  DEVICE (v_cache NULL iff k_eq_v); num_blocks pages each.
 *   block_table  DEVICE int32 [batch][max_blocks].
 *   context_lens DEVICE int32 [batch], each in 1 .. max_context_len (the current token counts).
 *   max_context_len  HOST bound on context_lens, used to size the launch; must satisfy
 *                max_context_len <= max_blocks * 16 (page_ring = 1: max_context_len < 2^30,
 *                and max_blocks >= floor((W - 1) / 16) + 2).
 *   out          DEVICE [batch][Hq][D] in the storage dtype.
 *   workspace    DEVICE scratch of at least ga_decode_workspace_bytes(p, batch,
 *                max_context_len) bytes, 256-byte aligned; contents need no initialisation
 *                and are overwritten.  Concurrent calls must not share it. */
ga_status ga_attn_decode(const ga_layer_params* p, const void* q, const void* k_cache,
                         const void* v_cache, int64_t num_blocks, const int32_t* block_table,
                         int32_t max_blocks, const int32_t* context_lens, int32_t batch,
                         int32_t max_context_len, void* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Decode attention without a caller-supplied workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors as ga_attn_decode, minus `workspace` and
 * `workspace_bytes`: the scratch lives in a fixed array of GA_DECODE_NOALLOC_SCRATCH_BYTES in
 * device memory that the library holds on every device it runs on until the process ends.
 * A shape whose ga_decode_workspace_bytes exceeds that size is refused with GA_ERR_WORKSPACE
 * before anything touches the device.  The call allocates nothing: the array's device address
 * is looked up once per device, on the first call with that device current.  Every call on one
 * device shares the array, so calls that may overlap on one device (several streams, several
 * host threads) race and give wrong results: serialise them, or use ga_attn_decode with a
 * workspace each.  The decode kernels overwrite the scratch before reading it, so nothing left
 * by an earlier call leaks into a later one. */
#define GA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
ga_status ga_attn_decode_noalloc(const ga_layer_params* p, const void* q, const void* k_cache,
                                 const void* v_cache, int64_t num_blocks,
                                 const int32_t* block_table, int32_t max_blocks,
                                 const int32_t* context_lens, int32_t batch,
                                 int32_t max_context_len, void* out, void* stream);

/* Prefill / chunked prefill: the n_b new queries of each sequence, packed, against its cache
 * (the chunk's own keys must already be written).  Query i of sequence b sits at position
 * t = past_b + i with past_b = context_lens[b] - n_b and sees keys max(0, t-W+1) .. t (W = 0:
 * 0 .. t) ([INFLM] Gemma-3 §3: exact band + causal mask, also for chunked prefill).
 *   q            DEVICE [total_q][Hq][D], normalised and rotated.
 *   cu_seqlens_q DEVICE int32 [batch+1], cu_seqlens_q[batch] == total_q.
 *   context_lens DEVICE int32 [batch] = past_b + n_b.
 *   max_q_len    HOST bound on every n_b (sizes the launch); max_q_len <= max_blocks * 16
 *                (page_ring = 1: max_blocks >= floor((max_q_len + W - 2) / 16) + 3, and
 *                context_lens below 2^30).
 *   out          DEVICE [total_q][Hq][D]. */
ga_status ga_attn_prefill(const ga_layer_params* p, const void* q,
                          const int32_t* cu_seqlens_q, const void* k_cache,
                          const void* v_cache, int64_t num_blocks,
                          const int32_t* block_table, int32_t max_blocks,
                          const int32_t* context_lens, int32_t batch, int32_t total_q,
                          int32_t max_q_len, void* out, void* stream);

/* Checks, on HOST copies, the metadata the kernels read from device memory:
 *   cu_seqlens (HOST int32 [batch+1], may be NULL meaning one new token per sequence):
 *     starts at 0, non-decreasing;
 *   context_lens (HOST int32 [batch]): n_b <= context_lens[b] <= max_blocks * 16 (page_ring:
 *     < 2^30), and >= 1 when require_nonempty;
 *   block_table (HOST int32 [batch][max_blocks]): every page a sequence uses holds a block id
 *     in [0, num_blocks), and no two written slots of the call coincide.  page_ring = 1: the
 *     columns of the pages an attention call reads after the write (the window of the first
 *     new query through the last page, from the 32-key tile start when cu_seqlens is given),
 *     as many of them as the ring holds, hold ids in range; that the ring is long enough for
 *     the attention call is checked by that call.
 * Returns GA_OK or GA_ERR_INVALID_ARG (reason in ga_last_error()). */
ga_status ga_check_metadata_host(const ga_layer_params* p, const int32_t* cu_seqlens,
                                 const int32_t* context_lens, const int32_t* block_table,
                                 int32_t batch, int32_t max_blocks, int64_t num_blocks,
                                 int32_t require_nonempty);

/* Static name of a status code. */
const char* ga_status_string(ga_status s);

/* Thread-local reason of the most recent failing call on this thread ("" if none). */
const char* ga_last_error(void);

/* In-kernel metadata checks (the scope table's boundary sketch: a debug build that also checks
 * the device-resident metadata in the kernels and records what it finds in a device word).
 * libgemma_attn_debug.so is built with GA_DEBUG_BOUNDS: its kernels check every block id they
 * read, the lengths against cu_seqlens and the host bounds, and the owner of every new token,
 * and set bits of a per-device word; the results and the clamps that keep every access in
 * bounds are the same as in the regular build.  This call waits for the device, returns the
 * OR of the bits set since the last call into *flags (HOST) and clears them.
 *   GA_DEBUG_BLOCK_ID  a block id the call read lies outside [0, num_blocks) (clamped, or for
 *                      the write: the token is skipped)
 *   GA_DEBUG_LENGTH    lengths inconsistent: L_b < n_b, a decode length < 1, cu_seqlens out of
 *                      order or past total_q / max_q_len
 *   GA_DEBUG_BOUND     a length beyond the host bound (max_context_len; the pages of a
 *                      block-table row)
 *   GA_DEBUG_OWNER     a new token that no sequence of cu_seqlens owns
 * The regular library returns GA_ERR_UNSUPPORTED (and *flags = 0).  GA_ERR_HIP: the word could
 * not be read.  Calls running while this one reads race with its clear. */
#define GA_DEBUG_BLOCK_ID 1u
#define GA_DEBUG_LENGTH 2u
#define GA_DEBUG_BOUND 4u
#define GA_DEBUG_OWNER 8u
ga_status ga_debug_take_error(uint32_t* flags);

#ifdef __cplusplus
}
#endif

#endif /* GEMMA_ATTN_H */
