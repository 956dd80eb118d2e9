// api.cpp -- the C ABI of include/gemma_attn.h: host-side validation, then kernel launches.
//
// Every argument that the host can see is checked before anything is enqueued, in the spirit
// of the hardening table of [INFLM] ("Feat/add gemma3 model", InfiniLM pull request 581):
// unsupported or inconsistent configurations are refused with a reason instead of producing a
// silently wrong result (a negative soft cap, a bad window, a missing tensor, ...).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "gemma_attn.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

ga_status fail(ga_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

ga_status ok() {
  g_err[0] = '\0';
  return GA_OK;
}

constexpr int kPage = 16;
constexpr int kMaxGroupBf16 = 16;  // query heads per kv head held by one MFMA column block
constexpr int kMaxExactAngles = 64;  // pairs the attention kernels rotate in exact K=V mode

ga_status check_params(const ga_layer_params* p) {
  if (!p) return fail(GA_ERR_INVALID_ARG, "params is NULL");
  if (p->dtype != GA_FP32 && p->dtype != GA_BF16)
    return fail(GA_ERR_INVALID_ARG, "dtype %d is not GA_FP32 or GA_BF16", p->dtype);
  if (p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(GA_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", p->num_q_heads,
                p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(GA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", p->num_q_heads,
                p->num_kv_heads);
  if (p->head_dim != 128 && p->head_dim != 256 && p->head_dim != 512)
    return fail(GA_ERR_UNSUPPORTED, "head_dim %d (supported: 128, 256, 512)", p->head_dim);
  if (p->block_size != kPage)
    return fail(GA_ERR_UNSUPPORTED, "block_size %d (only 16 is supported)", p->block_size);
  if (p->window < 0) return fail(GA_ERR_INVALID_ARG, "window %d < 0", p->window);
  if (!isfinite(p->scale)) return fail(GA_ERR_INVALID_ARG, "scale is not finite");
  if (!isfinite(p->softcap) || p->softcap < 0.f)
    return fail(GA_ERR_INVALID_ARG, "softcap %g must be finite and >= 0", (double)p->softcap);
  if (p->k_eq_v < 0 || p->k_eq_v > 2)
    return fail(GA_ERR_INVALID_ARG, "k_eq_v must be 0, 1 or 2");
  if (!isfinite(p->rope_theta) || p->rope_theta < 0.f)
    return fail(GA_ERR_INVALID_ARG, "rope_theta %g must be finite and >= 0",
                (double)p->rope_theta);
  if (!isfinite(p->rms_eps) || p->rms_eps < 0.f)
    return fail(GA_ERR_INVALID_ARG, "rms_eps %g must be finite and >= 0", (double)p->rms_eps);
  if (p->rope_angles < 0 || p->rope_angles > p->head_dim / 2)
    return fail(GA_ERR_INVALID_ARG, "rope_angles %d outside 0 .. head_dim/2", p->rope_angles);
  if (!isfinite(p->rope_scale) || p->rope_scale < 0.f)
    return fail(GA_ERR_INVALID_ARG, "rope_scale %g must be finite and >= 0",
                (double)p->rope_scale);
  if (p->k_eq_v != 2 && (p->kv_k_norm_w || p->kv_v_norm_w))
    return fail(GA_ERR_INVALID_ARG, "kv_k_norm_w / kv_v_norm_w are for k_eq_v = 2 only");
  if (p->k_eq_v == 2 && (p->kv_k_norm_w == nullptr) != (p->kv_v_norm_w == nullptr))
    return fail(GA_ERR_INVALID_ARG, "k_eq_v = 2 needs both kv_k_norm_w and kv_v_norm_w, or "
                "neither (values are the stored keys times v_norm_w / k_norm_w)");
  if (p->k_eq_v == 2 && p->rope_theta > 0.f &&
      (p->rope_angles == 0 ? p->head_dim / 2 : p->rope_angles) > kMaxExactAngles)
    return fail(GA_ERR_UNSUPPORTED, "k_eq_v = 2 rotates at most %d frequency pairs in the "
                "attention kernels (rope_angles %d, head_dim %d)", kMaxExactAngles,
                p->rope_angles, p->head_dim);
  if (p->page_ring != 0 && p->page_ring != 1)
    return fail(GA_ERR_INVALID_ARG, "page_ring %d must be 0 or 1", p->page_ring);
  if (p->page_ring && p->window <= 0)
    return fail(GA_ERR_INVALID_ARG, "page_ring needs a sliding window (window > 0)");
  return GA_OK;
}

ga_status check_attn_params(const ga_layer_params* p) {
  ga_status s = check_params(p);
  if (s != GA_OK) return s;
  if (p->dtype == GA_BF16 && p->num_q_heads / p->num_kv_heads > kMaxGroupBf16)
    return fail(GA_ERR_UNSUPPORTED, "bf16 attention supports up to %d query heads per kv head "
                "(got %d)", kMaxGroupBf16, p->num_q_heads / p->num_kv_heads);
  return GA_OK;
}

ga_status check_table(int32_t max_blocks, int64_t num_blocks, int32_t batch) {
  if (batch < 0) return fail(GA_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (max_blocks < 1) return fail(GA_ERR_INVALID_ARG, "max_blocks %d < 1", max_blocks);
  if ((int64_t)max_blocks * kPage > 0x7fffffffLL)
    return fail(GA_ERR_INVALID_ARG, "max_blocks %d too large", max_blocks);
  if (num_blocks < 1) return fail(GA_ERR_INVALID_ARG, "num_blocks %lld < 1",
                                  (long long)num_blocks);
  return GA_OK;
}

ga_status check_caches(const ga_layer_params* p, const void* k_cache, const void* v_cache) {
  if (!k_cache) return fail(GA_ERR_INVALID_ARG, "k_cache is NULL");
  if (p->k_eq_v && v_cache)
    return fail(GA_ERR_INVALID_ARG, "k_eq_v=%d but v_cache is not NULL", p->k_eq_v);
  if (!p->k_eq_v && !v_cache) return fail(GA_ERR_INVALID_ARG, "v_cache is NULL (k_eq_v=0)");
  return GA_OK;
}

ga_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(GA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Pages a ring row must hold: decode reads the window of its query, [L - W, L) (at most
// floor((W - 1) / 16) + 2 pages); a prefill chunk of n tokens reads from its first query's
// window start, rounded down to a 32-key tile, to its last key (at most
// floor((n + W - 2) / 16) + 3 pages).
int64_t ring_pages_decode(int window) { return (window - 1) / kPage + 2; }
int64_t ring_pages_prefill(int window, int64_t max_q_len) {
  return (max_q_len + window - 2) / kPage + 3;
}
constexpr int64_t kRingMaxLen = int64_t(1) << 30;  // context lengths stay below this

ga::AttnLaunch make_attn(const ga_layer_params* p) {
  ga::AttnLaunch a;
  memset(&a, 0, sizeof a);
  a.dtype_bf16 = p->dtype == GA_BF16;
  a.D = p->head_dim;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.window = p->window;
  a.ring = p->page_ring;
  a.k_eq_v = p->k_eq_v;
  a.rope_theta = p->rope_theta;
  a.rope_angles = p->rope_angles == 0 ? p->head_dim / 2 : p->rope_angles;
  a.rope_scale = p->rope_scale == 0.f ? 1.f : p->rope_scale;
  a.kv_kw = p->kv_k_norm_w;
  a.kv_vw = p->kv_v_norm_w;
  a.scale = p->scale;
  a.softcap = p->softcap;
  return a;
}

}  // namespace

extern "C" {

const char* ga_status_string(ga_status s) {
  switch (s) {
    case GA_OK: return "GA_OK";
    case GA_ERR_INVALID_ARG: return "GA_ERR_INVALID_ARG";
    case GA_ERR_UNSUPPORTED: return "GA_ERR_UNSUPPORTED";
    case GA_ERR_WORKSPACE: return "GA_ERR_WORKSPACE";
    case GA_ERR_HIP: return "GA_ERR_HIP";
  }
  return "GA_UNKNOWN_STATUS";
}

const char* ga_last_error(void) { return g_err; }

ga_status ga_kv_cache_write(const ga_layer_params* p, void* q, const void* k, const void* v,
                            const float* q_norm_w, const float* k_norm_w, const float* v_norm_w,
                            const int32_t* cu_seqlens, const int32_t* context_lens,
                            const int32_t* block_table, int32_t max_blocks, int32_t batch,
                            int32_t total_tokens, void* k_cache, void* v_cache,
                            int64_t num_blocks, void* stream) {
  ga_status s = check_params(p);
  if (s != GA_OK) return s;
  if (total_tokens < 0) return fail(GA_ERR_INVALID_ARG, "total_tokens %d < 0", total_tokens);
  const bool q_only = k == nullptr;  // a layer reading another layer's cache
  if (q_only) {
    if (!q) return fail(GA_ERR_INVALID_ARG, "q and k are both NULL");
    if (v || k_norm_w || v_norm_w)
      return fail(GA_ERR_INVALID_ARG, "k is NULL (q-only write) but v or a k/v norm is given");
    if (batch < 0) return fail(GA_ERR_INVALID_ARG, "batch %d < 0", batch);
    if (!cu_seqlens || !context_lens)
      return fail(GA_ERR_INVALID_ARG, "cu_seqlens and context_lens are required");
  } else {
    if ((s = check_table(max_blocks, num_blocks, batch)) != GA_OK) return s;
    if ((s = check_caches(p, k_cache, v_cache)) != GA_OK) return s;
    if (p->k_eq_v && v)
      return fail(GA_ERR_INVALID_ARG, "k_eq_v=%d but v is not NULL", p->k_eq_v);
    if (!p->k_eq_v && !v) return fail(GA_ERR_INVALID_ARG, "v is NULL (k_eq_v=0)");
    if (p->k_eq_v && v_norm_w)
      return fail(GA_ERR_INVALID_ARG, "k_eq_v=%d but v_norm_w is not NULL", p->k_eq_v);
    if (!cu_seqlens || !context_lens || !block_table)
      return fail(GA_ERR_INVALID_ARG, "cu_seqlens, context_lens and block_table are required");
  }
  if (batch == 0 || total_tokens == 0) return ok();
  ga::KvWriteLaunch a;
  a.dtype_bf16 = p->dtype == GA_BF16;
  a.D = p->head_dim;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.k_eq_v = p->k_eq_v;
  a.rope_theta = p->rope_theta;
  a.rope_angles = p->rope_angles == 0 ? p->head_dim / 2 : p->rope_angles;
  a.rope_scale = p->rope_scale == 0.f ? 1.f : p->rope_scale;
  a.ring = p->page_ring;
  a.rms_eps = p->rms_eps;
  a.q = q;
  a.k = k;
  a.v = v;
  a.wq = q_norm_w;
  a.wk = k_norm_w;
  a.wv = v_norm_w;
  a.cu_seqlens = cu_seqlens;
  a.context_lens = context_lens;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.total_tokens = total_tokens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  return from_hip(ga::launch_kv_write(a, (hipStream_t)stream), "kv_cache_write launch");
}

size_t ga_decode_workspace_bytes(const ga_layer_params* p, int32_t batch,
                                 int32_t max_context_len) {
  if (check_attn_params(p) != GA_OK || batch < 0 || max_context_len < 1) return 0;
  return ga::plan_decode(p->head_dim, p->num_q_heads, p->num_kv_heads, p->window, batch,
                         max_context_len, p->dtype == GA_BF16)
      .workspace_bytes;
}

// Checks shared by both decode entry points; on success *plan holds the launch plan.
static ga_status check_decode(const ga_layer_params* p, const void* q, const void* k_cache,
                              const void* v_cache, int64_t num_blocks,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* context_lens, int32_t batch,
                              int32_t max_context_len, const void* out, ga::DecodePlan* plan) {
  ga_status s = check_attn_params(p);
  if (s != GA_OK) return s;
  if ((s = check_table(max_blocks, num_blocks, batch)) != GA_OK) return s;
  if ((s = check_caches(p, k_cache, v_cache)) != GA_OK) return s;
  if (!q || !out || !block_table || !context_lens)
    return fail(GA_ERR_INVALID_ARG, "q, out, block_table and context_lens are required");
  if (max_context_len < 1)
    return fail(GA_ERR_INVALID_ARG, "max_context_len %d < 1", max_context_len);
  if (p->page_ring) {
    if ((int64_t)max_context_len >= kRingMaxLen)
      return fail(GA_ERR_INVALID_ARG, "max_context_len %d: a ring table needs lengths < 2^30",
                  max_context_len);
    if (max_blocks < ring_pages_decode(p->window))
      return fail(GA_ERR_INVALID_ARG, "ring of %d pages is shorter than the %lld a window of %d "
                  "needs", max_blocks, (long long)ring_pages_decode(p->window), p->window);
  } else if ((int64_t)max_context_len > (int64_t)max_blocks * kPage) {
    return fail(GA_ERR_INVALID_ARG, "max_context_len %d exceeds max_blocks*16 = %lld",
                max_context_len, (long long)max_blocks * kPage);
  }
  {
    int64_t pages = (max_context_len + kPage - 1) / kPage;  // visible pages per sequence
    if (p->window > 0 && pages > p->window / kPage + 2) pages = p->window / kPage + 2;
    if ((int64_t)batch * pages > 0x7fffffffLL)
      return fail(GA_ERR_UNSUPPORTED, "batch x visible pages per sequence exceeds 2^31");
  }
  *plan = ga::plan_decode(p->head_dim, p->num_q_heads, p->num_kv_heads, p->window, batch,
                          max_context_len, p->dtype == GA_BF16);
  return GA_OK;
}

static ga_status launch_decode_checked(const ga_layer_params* p, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       int64_t num_blocks, const int32_t* block_table,
                                       int32_t max_blocks, const int32_t* context_lens,
                                       int32_t batch, int32_t max_context_len, void* out,
                                       void* workspace, const ga::DecodePlan& plan,
                                       void* stream) {
  ga::AttnLaunch a = make_attn(p);
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.context_lens = context_lens;
  a.batch = batch;
  a.max_context_len = max_context_len;
  a.out = out;
  a.workspace = workspace;
  return from_hip(ga::launch_decode(a, plan, (hipStream_t)stream), "attn_decode launch");
}

ga_status ga_attn_decode(const ga_layer_params* p, const void* q, const void* k_cache,
                         const void* v_cache, int64_t num_blocks, const int32_t* block_table,
                         int32_t max_blocks, const int32_t* context_lens, int32_t batch,
                         int32_t max_context_len, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  ga::DecodePlan plan;
  ga_status s = check_decode(p, q, k_cache, v_cache, num_blocks, block_table, max_blocks,
                             context_lens, batch, max_context_len, out, &plan);
  if (s != GA_OK) return s;
  if (plan.workspace_bytes > 0) {
    if (!workspace) return fail(GA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)",
                                plan.workspace_bytes);
    if (workspace_bytes < plan.workspace_bytes)
      return fail(GA_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes,
                  plan.workspace_bytes);
    if (((uintptr_t)workspace & 255) != 0)
      return fail(GA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  if (batch == 0) return ok();
  return launch_decode_checked(p, q, k_cache, v_cache, num_blocks, block_table, max_blocks,
                               context_lens, batch, max_context_len, out, workspace, plan,
                               stream);
}

ga_status ga_attn_decode_noalloc(const ga_layer_params* p, const void* q, const void* k_cache,
                                 const void* v_cache, int64_t num_blocks,
                                 const int32_t* block_table, int32_t max_blocks,
                                 const int32_t* context_lens, int32_t batch,
                                 int32_t max_context_len, void* out, void* stream) {
  static_assert(GA_DECODE_NOALLOC_SCRATCH_BYTES == ga::kNoAllocScratchBytes,
                "scratch size of the header and of the decode kernels");
  ga::DecodePlan plan;
  ga_status s = check_decode(p, q, k_cache, v_cache, num_blocks, block_table, max_blocks,
                             context_lens, batch, max_context_len, out, &plan);
  if (s != GA_OK) return s;
  // the size is checked before the device is touched
  if (plan.workspace_bytes > ga::kNoAllocScratchBytes)
    return fail(GA_ERR_WORKSPACE, "this shape needs %zu bytes of decode scratch; the "
                "allocation-free entry point holds at most %zu (use ga_attn_decode with a "
                "workspace)", plan.workspace_bytes, (size_t)ga::kNoAllocScratchBytes);
  if (batch == 0) return ok();
  void* scratch = nullptr;
  if (plan.workspace_bytes > 0) {
    const hipError_t e = ga::decode_scratch_address(&scratch);
    if (e != hipSuccess) return from_hip(e, "decode scratch address");
  }
  return launch_decode_checked(p, q, k_cache, v_cache, num_blocks, block_table, max_blocks,
                               context_lens, batch, max_context_len, out, scratch, plan, stream);
}

ga_status ga_attn_prefill(const ga_layer_params* p, const void* q,
                          const int32_t* cu_seqlens_q, const void* k_cache,
                          const void* v_cache, int64_t num_blocks,
                          const int32_t* block_table, int32_t max_blocks,
                          const int32_t* context_lens, int32_t batch, int32_t total_q,
                          int32_t max_q_len, void* out, void* stream) {
  ga_status s = check_attn_params(p);
  if (s != GA_OK) return s;
  if ((s = check_table(max_blocks, num_blocks, batch)) != GA_OK) return s;
  if ((s = check_caches(p, k_cache, v_cache)) != GA_OK) return s;
  if (!q || !out || !cu_seqlens_q || !block_table || !context_lens)
    return fail(GA_ERR_INVALID_ARG,
                "q, out, cu_seqlens_q, block_table and context_lens are required");
  if (total_q < 0) return fail(GA_ERR_INVALID_ARG, "total_q %d < 0", total_q);
  if (max_q_len < 0) return fail(GA_ERR_INVALID_ARG, "max_q_len %d < 0", max_q_len);
  if ((int64_t)max_q_len > (int64_t)max_blocks * kPage)
    return fail(GA_ERR_INVALID_ARG, "max_q_len %d exceeds max_blocks*16", max_q_len);
  if (p->page_ring && max_blocks < ring_pages_prefill(p->window, max_q_len))
    return fail(GA_ERR_INVALID_ARG, "ring of %d pages is shorter than the %lld a chunk of %d "
                "with a window of %d needs", max_blocks,
                (long long)ring_pages_prefill(p->window, max_q_len), max_q_len, p->window);
  if (batch == 0 || total_q == 0 || max_q_len == 0) return ok();
  ga::AttnLaunch a = make_attn(p);
  a.q = q;
  a.cu_seqlens_q = cu_seqlens_q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.context_lens = context_lens;
  a.batch = batch;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.max_context_len = p->page_ring ? (int32_t)(kRingMaxLen - 1) : max_blocks * kPage;
  a.out = out;
  return from_hip(ga::launch_prefill(a, (hipStream_t)stream), "attn_prefill launch");
}

ga_status ga_check_metadata_host(const ga_layer_params* p, const int32_t* cu_seqlens,
                                 const int32_t* context_lens, const int32_t* block_table,
                                 int32_t batch, int32_t max_blocks, int64_t num_blocks,
                                 int32_t require_nonempty) {
  ga_status s = check_params(p);
  if (s != GA_OK) return s;
  if ((s = check_table(max_blocks, num_blocks, batch)) != GA_OK) return s;
  if (!context_lens || !block_table)
    return fail(GA_ERR_INVALID_ARG, "context_lens and block_table are required");
  if (cu_seqlens && cu_seqlens[0] != 0)
    return fail(GA_ERR_INVALID_ARG, "cu_seqlens[0] = %d, expected 0", cu_seqlens[0]);
  std::vector<int64_t> written;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = cu_seqlens ? (int64_t)cu_seqlens[b + 1] - cu_seqlens[b] : 1;
    const int64_t L = context_lens[b];
    if (n < 0) return fail(GA_ERR_INVALID_ARG, "cu_seqlens decreases at sequence %d", b);
    if (L < n)
      return fail(GA_ERR_INVALID_ARG, "sequence %d: context_len %lld < new tokens %lld", b,
                  (long long)L, (long long)n);
    if (require_nonempty && L < 1)
      return fail(GA_ERR_INVALID_ARG, "sequence %d: context_len %lld < 1", b, (long long)L);
    const int64_t pages = (L + kPage - 1) / kPage;
    int64_t first = 0;  // first page whose block id must be valid
    if (p->page_ring) {
      if (L >= kRingMaxLen)
        return fail(GA_ERR_INVALID_ARG, "sequence %d: context_len %lld >= 2^30 (ring table)", b,
                    (long long)L);
      // the pages an attention call reads after this write: from the window start of the
      // first new query (prefill: from its 32-key tile) to the last page, as far as the ring
      // holds them (whether it holds them all is checked by the attention calls)
      const int64_t lo = L - n - p->window + 1 > 0 ? L - n - p->window + 1 : 0;
      first = cu_seqlens ? 2 * (lo / (2 * kPage)) : lo / kPage;
      if (pages - first > max_blocks) first = pages - max_blocks;
    } else if (L > (int64_t)max_blocks * kPage) {
      return fail(GA_ERR_INVALID_ARG, "sequence %d: context_len %lld > max_blocks*16", b,
                  (long long)L);
    }
    auto column = [&](int64_t pg) {
      return (int64_t)b * max_blocks + (p->page_ring ? pg % max_blocks : pg);
    };
    for (int64_t pg = first; pg < pages; ++pg) {
      const int64_t blk = block_table[column(pg)];
      if (blk < 0 || blk >= num_blocks)
        return fail(GA_ERR_INVALID_ARG, "sequence %d page %lld: block id %lld outside [0, %lld)",
                    b, (long long)pg, (long long)blk, (long long)num_blocks);
    }
    for (int64_t t = L - n; t < L; ++t)
      written.push_back((int64_t)block_table[column(t / kPage)] * kPage + t % kPage);
  }
  std::sort(written.begin(), written.end());
  if (std::adjacent_find(written.begin(), written.end()) != written.end())
    return fail(GA_ERR_INVALID_ARG, "two new tokens of this call map to the same cache slot");
  return ok();
}

static_assert(ga::kDbgBlockId == GA_DEBUG_BLOCK_ID && ga::kDbgLength == GA_DEBUG_LENGTH &&
                  ga::kDbgBound == GA_DEBUG_BOUND && ga::kDbgOwner == GA_DEBUG_OWNER,
              "check bits of the header and of the kernels");

ga_status ga_debug_take_error(uint32_t* flags) {
  if (!flags) return fail(GA_ERR_INVALID_ARG, "flags is NULL");
  *flags = 0;
#ifdef GA_DEBUG_BOUNDS
  const uint32_t w = ga::debug_take_kv_write() | ga::debug_take_decode() |
                     ga::debug_take_prefill() | ga::debug_take_attention();
  if (w & ga::kDbgReadFailed) return fail(GA_ERR_HIP, "reading the check words failed");
  *flags = w;
  return ok();
#else
  return fail(GA_ERR_UNSUPPORTED, "in-kernel metadata checks are only in the GA_DEBUG_BOUNDS "
                                  "build");
#endif
}

}  // extern "C"
