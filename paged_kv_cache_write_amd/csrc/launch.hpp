// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernel files.
// The host side validates everything before it fills one of these structs; the launchers
// only enqueue kernels and report the HIP status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ga {

struct KvWriteLaunch {
  bool dtype_bf16;
  int D, Hq, Hkv, k_eq_v;
  float rope_theta, rms_eps;
  int rope_angles;   // rotated frequency pairs (1 .. D/2)
  float rope_scale;  // position divisor (> 0)
  void* q;
  const void* k;
  const void* v;
  const float *wq, *wk, *wv;
  const int32_t* cu_seqlens;
  const int32_t* context_lens;
  const int32_t* block_table;
  int32_t max_blocks, batch, total_tokens;
  int ring;  // block-table rows are rings of max_blocks pages
  void* k_cache;
  void* v_cache;
  int64_t num_blocks;
};

// Shared description of an attention call (decode or prefill).
struct AttnLaunch {
  bool dtype_bf16;
  int D, Hq, Hkv, window, k_eq_v;  // k_eq_v: 0 separate V, 1 K=V, 2 exact K=V
  float scale, softcap;
  // exact K=V (k_eq_v = 2): rotation of the stored keys and the value factor w_v / w_k
  float rope_theta, rope_scale;
  int rope_angles;
  const float* kv_kw;
  const float* kv_vw;
  const void* q;
  const int32_t* cu_seqlens_q;  // prefill only
  const void* k_cache;
  const void* v_cache;
  int64_t num_blocks;
  const int32_t* block_table;
  int32_t max_blocks;
  int ring;  // block-table rows are rings of max_blocks pages
  const int32_t* context_lens;
  int32_t batch;
  int32_t max_context_len;  // decode: host bound on context_lens
  int32_t total_q, max_q_len;  // prefill
  void* out;
  void* workspace;
};

// Decode launch plan; a pure function of the host arguments.
struct DecodePlan {
  int nworkers;           // upper bound on the single-wave workers of one launch
  int64_t npieces;        // upper bound on (worker, sequence x kv head) pieces
  size_t pref_bytes, ml_bytes, o_bytes;  // workspace regions (256-byte aligned)
  size_t workspace_bytes;
};

DecodePlan plan_decode(int D, int Hq, int Hkv, int window, int batch, int max_context_len,
                       bool bf16);

// Decode scratch of the allocation-free entry point: a file-scope device array of decode.hip,
// one copy per device, shared by every call on that device.
constexpr size_t kNoAllocScratchBytes = size_t(48) << 20;
// Device address of that array on the current device (looked up once per device).
hipError_t decode_scratch_address(void** ptr);

hipError_t launch_kv_write(const KvWriteLaunch& a, hipStream_t s);
hipError_t launch_decode(const AttnLaunch& a, const DecodePlan& plan, hipStream_t s);
hipError_t launch_prefill(const AttnLaunch& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnLaunch& a, bool decode, hipStream_t s);

// Debug build (GA_DEBUG_BOUNDS): bits of the in-kernel metadata checks.
constexpr uint32_t kDbgBlockId = 1u;  // a block-table entry the call reads is outside [0, nb)
constexpr uint32_t kDbgLength = 2u;   // lengths inconsistent (L_b < n_b, decode L_b < 1, cu out
                                      // of order or past its end)
constexpr uint32_t kDbgBound = 4u;    // a context beyond the host bound (max_context_len, the
                                      // pages of a table row)
constexpr uint32_t kDbgOwner = 8u;    // a new token that no sequence of cu_seqlens owns
constexpr uint32_t kDbgReadFailed = 0x80000000u;  // the word could not be read

// The metadata-check word of each kernel file on the current device, read and cleared (0 in
// the regular build; kDbgReadFailed if a word could not be read).
uint32_t debug_take_kv_write();
uint32_t debug_take_decode();
uint32_t debug_take_prefill();
uint32_t debug_take_attention();

}  // namespace ga
