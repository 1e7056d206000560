// C ABI of libpa: argument validation, plan sizing and kernel launches.
// Every check happens on the host before anything is enqueued.
#include "../../include/pa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>

#include "pa_internal.h"

#ifndef PA_GIT_REV
#define PA_GIT_REV "unknown"
#endif

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The kernels take each row's maximum of the unscaled scores, which is the
// maximum of the scaled ones only for a positive scale.
bool scale_ok(float scale) { return scale > 0.f && scale <= 3.4e38f; }

int check_heads(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  if (head_dim != pa::kHeadDimAbi) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads < 1 || num_kv_heads > 64) return PA_ERR_UNSUPPORTED;
  if (num_q_heads != 6 * num_kv_heads) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int check_cache(const uint16_t* k_cache, const uint16_t* v_cache, int64_t page_stride,
                int32_t block_size, int32_t num_kv_heads) {
  if (!k_cache || !v_cache) return PA_ERR_NULL;
  if (block_size < 1) return PA_ERR_BLOCK_SIZE;
  // Kernels address rows inside a page with 32-bit byte offsets.
  if ((int64_t)block_size * num_kv_heads * pa::kHeadDimAbi * 2 >= ((int64_t)1 << 32)) return PA_ERR_BLOCK_SIZE;
  if (page_stride < (int64_t)block_size * num_kv_heads * pa::kHeadDimAbi) return PA_ERR_STRIDE;
  if (page_stride % 8 != 0) return PA_ERR_ALIGN;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
  return PA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

}  // namespace

extern "C" {

int pa_slot_mapping(int64_t* slot_out, const int64_t* positions, const int32_t* token_seq,
                    int32_t num_tokens, const int32_t* block_table, int32_t bt_stride,
                    int32_t block_size, void* stream) {
  if (!slot_out || !positions || !block_table) return PA_ERR_NULL;
  if (block_size < 1) return PA_ERR_BLOCK_SIZE;
  if (num_tokens < 0 || bt_stride < 1) return PA_ERR_SIZE;
  if (num_tokens == 0) return PA_OK;
  return launch_status(pa::launch_slot_mapping(slot_out, positions, token_seq, num_tokens,
                                               block_table, bt_stride, block_size,
                                               static_cast<hipStream_t>(stream)));
}

static int kv_write_common(uint16_t* k_cache, uint16_t* v_cache, int64_t page_stride,
                           int32_t num_pages, int32_t block_size, int32_t num_kv_heads,
                           int32_t head_dim, const uint16_t* k_new, const uint16_t* v_new,
                           int32_t num_tokens) {
  if (!k_new || !v_new) return PA_ERR_NULL;
  int rc = check_cache(k_cache, v_cache, page_stride, block_size, num_kv_heads);
  if (rc) return rc;
  if (head_dim != pa::kHeadDimAbi || num_kv_heads < 1 || num_kv_heads > 64)
    return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_pages < 1) return PA_ERR_SIZE;
  if (!aligned16(k_new) || !aligned16(v_new)) return PA_ERR_ALIGN;
  return PA_OK;
}

int pa_kv_write(uint16_t* k_cache, uint16_t* v_cache, int64_t page_stride, int32_t num_pages,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                const uint16_t* k_new, const uint16_t* v_new, int32_t num_tokens,
                const int64_t* slot_mapping, void* stream) {
  if (!slot_mapping) return PA_ERR_NULL;
  int rc = kv_write_common(k_cache, v_cache, page_stride, num_pages, block_size, num_kv_heads,
                           head_dim, k_new, v_new, num_tokens);
  if (rc) return rc;
  if (num_tokens == 0) return PA_OK;
  return launch_status(pa::launch_kv_write(k_cache, v_cache, page_stride, num_pages, block_size,
                                           num_kv_heads, k_new, v_new, num_tokens, slot_mapping,
                                           nullptr, nullptr, nullptr, 0, nullptr,
                                           static_cast<hipStream_t>(stream)));
}

int pa_kv_write_fused(uint16_t* k_cache, uint16_t* v_cache, int64_t page_stride,
                      int32_t num_pages, int32_t block_size, int32_t num_kv_heads,
                      int32_t head_dim, const uint16_t* k_new, const uint16_t* v_new,
                      int32_t num_tokens, const int64_t* positions, const int32_t* token_seq,
                      const int32_t* block_table, int32_t bt_stride, int64_t* slot_out,
                      void* stream) {
  if (!positions || !block_table) return PA_ERR_NULL;
  int rc = kv_write_common(k_cache, v_cache, page_stride, num_pages, block_size, num_kv_heads,
                           head_dim, k_new, v_new, num_tokens);
  if (rc) return rc;
  if (bt_stride < 1) return PA_ERR_SIZE;
  if (num_tokens == 0) return PA_OK;
  return launch_status(pa::launch_kv_write(k_cache, v_cache, page_stride, num_pages, block_size,
                                           num_kv_heads, k_new, v_new, num_tokens, nullptr,
                                           positions, token_seq, block_table, bt_stride,
                                           slot_out, static_cast<hipStream_t>(stream)));
}

int pa_decode_workspace_size(int32_t num_seqs, int32_t max_seq_len, int32_t block_size,
                             int32_t num_kv_heads, size_t* bytes_out) {
  if (!bytes_out) return PA_ERR_NULL;
  if (block_size < 1) return PA_ERR_BLOCK_SIZE;
  if (num_kv_heads < 1 || num_kv_heads > 64) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 1 || num_seqs > 65535 || max_seq_len < 1 ||
      (int64_t)max_seq_len + block_size > INT32_MAX)
    return PA_ERR_SIZE;
  const pa::DecodePlan plan = pa::plan_decode(num_seqs, max_seq_len, block_size, num_kv_heads);
  if (plan.steps_ub >= pa::kMaxDecodeSteps) return PA_ERR_SIZE;
  *bytes_out = plan.bytes;
  return PA_OK;
}

static int decode_common(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, int64_t page_stride,
                         const int32_t* block_table, int32_t bt_stride,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                         int32_t block_size, float scale, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, void* workspace,
                         size_t workspace_bytes, const pa::DecodeAppend* append, void* stream,
                         bool validate_only = false) {
  if (!out || !q || !block_table || !seq_lens) return PA_ERR_NULL;
  if (!scale_ok(scale)) return PA_ERR_SCALE;
  int rc = check_cache(k_cache, v_cache, page_stride, block_size, num_kv_heads);
  if (rc) return rc;
  rc = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (rc) return rc;
  if (num_seqs < 1 || num_seqs > 65535 || max_seq_len < 1 ||
      (int64_t)max_seq_len + block_size > INT32_MAX)
    return PA_ERR_SIZE;
  if (bt_stride < 1 || (int64_t)bt_stride * block_size < max_seq_len) return PA_ERR_TABLE;
  if (!aligned16(out) || !aligned16(q)) return PA_ERR_ALIGN;
  const pa::DecodePlan plan = pa::plan_decode(num_seqs, max_seq_len, block_size, num_kv_heads);
  if (plan.steps_ub >= pa::kMaxDecodeSteps) return PA_ERR_SIZE;
  if (validate_only) return PA_OK;
  if (!workspace || workspace_bytes < plan.bytes) return PA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_ALIGN;
  return launch_status(pa::launch_decode(out, q, k_cache, v_cache, page_stride, block_table,
                                         bt_stride, seq_lens, num_seqs, max_seq_len, block_size,
                                         scale, num_kv_heads, plan, workspace, append,
                                         static_cast<hipStream_t>(stream)));
}

int pa_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
              const uint16_t* v_cache, int64_t page_stride, const int32_t* block_table,
              int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
              int32_t max_seq_len, int32_t block_size, float scale, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, void* workspace,
              size_t workspace_bytes, void* stream) {
  return decode_common(out, q, k_cache, v_cache, page_stride, block_table, bt_stride, seq_lens,
                       num_seqs, max_seq_len, block_size, scale, num_q_heads, num_kv_heads,
                       head_dim, workspace, workspace_bytes, nullptr, stream);
}

int pa_decode_noalloc(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                      const uint16_t* v_cache, int64_t page_stride, const int32_t* block_table,
                      int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                      int32_t max_seq_len, int32_t block_size, float scale, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, void* stream) {
  // Size check first (host arithmetic only), then the per-device buffer.
  if (block_size >= 1 && num_kv_heads >= 1 && num_kv_heads <= 64 && num_seqs >= 1 &&
      num_seqs <= 65535 && max_seq_len >= 1 && (int64_t)max_seq_len + block_size <= INT32_MAX) {
    const pa::DecodePlan plan = pa::plan_decode(num_seqs, max_seq_len, block_size, num_kv_heads);
    if (plan.bytes > pa::kDecodeScratchBytes) return PA_ERR_SCRATCH;
  }
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // Argument errors are reported before the device is touched.
  int rc = decode_common(out, q, k_cache, v_cache, page_stride, block_table, bt_stride, seq_lens,
                         num_seqs, max_seq_len, block_size, scale, num_q_heads, num_kv_heads,
                         head_dim, nullptr, 0, nullptr, nullptr, /*validate_only=*/true);
  if (rc) return rc;
  if (pa::decode_scratch_for_current_device(&ws) != hipSuccess) return PA_ERR_LAUNCH;
  ws_bytes = pa::kDecodeScratchBytes;
  return decode_common(out, q, k_cache, v_cache, page_stride, block_table, bt_stride, seq_lens,
                       num_seqs, max_seq_len, block_size, scale, num_q_heads, num_kv_heads,
                       head_dim, ws, ws_bytes, nullptr, stream);
}

int pa_decode_append(uint16_t* out, const uint16_t* q, uint16_t* k_cache, uint16_t* v_cache,
                     int64_t page_stride, const int32_t* block_table, int32_t bt_stride,
                     const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                     int32_t block_size, float scale, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, const uint16_t* k_new,
                     const uint16_t* v_new, int64_t* slot_out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new) return PA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return PA_ERR_ALIGN;
  const pa::DecodeAppend append{k_new, v_new, k_cache, v_cache, slot_out};
  return decode_common(out, q, k_cache, v_cache, page_stride, block_table, bt_stride, seq_lens,
                       num_seqs, max_seq_len, block_size, scale, num_q_heads, num_kv_heads,
                       head_dim, workspace, workspace_bytes, &append, stream);
}

static int check_prefill_shape(int32_t q_len, int32_t start_pos, int32_t block_size,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  if (block_size < 1) return PA_ERR_BLOCK_SIZE;
  const int rc = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (rc) return rc;
  if (q_len < 1 || start_pos < 0 || (int64_t)start_pos + q_len + block_size > INT32_MAX)
    return PA_ERR_SIZE;
  return PA_OK;
}

int pa_prefill_workspace_size(int32_t q_len, int32_t start_pos, int32_t causal, int32_t block_size,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              size_t* bytes_out) {
  if (!bytes_out) return PA_ERR_NULL;
  const int rc = check_prefill_shape(q_len, start_pos, block_size, num_q_heads, num_kv_heads, head_dim);
  if (rc) return rc;
  *bytes_out = pa::plan_prefill(q_len, start_pos, causal ? 1 : 0, block_size, num_kv_heads).bytes;
  return PA_OK;
}

int pa_prefill_chunk(uint16_t* out, const uint16_t* q_chunk, int32_t q_len, int32_t start_pos,
                     int32_t causal, const uint16_t* k_cache, const uint16_t* v_cache,
                     int64_t page_stride, const int32_t* block_table, int32_t num_table_entries,
                     int32_t block_size, float scale, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, void* workspace, size_t workspace_bytes, void* stream) {
  if (!out || !q_chunk || !block_table) return PA_ERR_NULL;
  if (!scale_ok(scale)) return PA_ERR_SCALE;
  int rc = check_cache(k_cache, v_cache, page_stride, block_size, num_kv_heads);
  if (rc) return rc;
  rc = check_prefill_shape(q_len, start_pos, block_size, num_q_heads, num_kv_heads, head_dim);
  if (rc) return rc;
  const int64_t kv_len = (int64_t)start_pos + q_len;
  if (num_table_entries < 1 || (int64_t)num_table_entries * block_size < kv_len)
    return PA_ERR_TABLE;
  if (!aligned16(out) || !aligned16(q_chunk)) return PA_ERR_ALIGN;
  const pa::PrefillPlan plan = pa::plan_prefill(q_len, start_pos, causal ? 1 : 0, block_size, num_kv_heads);
  if (plan.bytes) {
    if (!workspace || workspace_bytes < plan.bytes) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_ALIGN;
  }
  return launch_status(pa::launch_prefill(out, q_chunk, q_len, start_pos, causal, k_cache,
                                          v_cache, page_stride, block_table, block_size, scale,
                                          num_kv_heads, plan, workspace,
                                          static_cast<hipStream_t>(stream)));
}

int pa_prefill_varlen(uint16_t* out, const uint16_t* q, int32_t total_q,
                      const int32_t* cu_seqlens_q, const int32_t* seqused_k, int32_t num_seqs,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t causal,
                      const uint16_t* k_cache, const uint16_t* v_cache, int64_t page_stride,
                      const int32_t* block_table, int32_t bt_stride, int32_t block_size,
                      float scale, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      void* stream) {
  if (!out || !q || !cu_seqlens_q || !seqused_k || !block_table) return PA_ERR_NULL;
  if (!scale_ok(scale)) return PA_ERR_SCALE;
  int rc = check_cache(k_cache, v_cache, page_stride, block_size, num_kv_heads);
  if (rc) return rc;
  rc = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (rc) return rc;
  if (num_seqs < 1 || total_q < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 ||
      (int64_t)max_seqlen_k + block_size > INT32_MAX)
    return PA_ERR_SIZE;
  if (pa::varlen_grid(total_q, num_seqs, num_kv_heads) > INT32_MAX) return PA_ERR_SIZE;
  if (bt_stride < 1 || (int64_t)bt_stride * block_size < max_seqlen_k) return PA_ERR_TABLE;
  if (!aligned16(out) || !aligned16(q)) return PA_ERR_ALIGN;
  return launch_status(pa::launch_prefill_varlen(out, q, total_q, cu_seqlens_q, seqused_k, num_seqs,
                                                 max_seqlen_q, max_seqlen_k, causal, k_cache,
                                                 v_cache, page_stride, block_table, bt_stride,
                                                 block_size, scale, num_kv_heads,
                                                 static_cast<hipStream_t>(stream)));
}

int pa_decode_input_prep(const int64_t* sampled_token_ids, int64_t position, int32_t* input_ids,
                         int64_t* positions, int32_t mrope, int64_t positions_stride,
                         int64_t mrope_delta, int32_t* query_start_loc,
                         int32_t query_start_loc_len, int32_t* seq_lens, int32_t seq_lens_len,
                         uint8_t* discard_request_mask, int32_t discard_len,
                         uint8_t* is_token_ids, int32_t num_kv_groups, const int32_t* block_sizes,
                         const uint64_t* block_table_ptrs, const uint64_t* slot_mapping_ptrs,
                         void* stream) {
  if (!sampled_token_ids || !input_ids || !positions || !query_start_loc || !seq_lens ||
      !discard_request_mask)
    return PA_ERR_NULL;
  if (num_kv_groups < 0 || num_kv_groups > 65535) return PA_ERR_SIZE;
  if (num_kv_groups > 0 && (!block_sizes || !block_table_ptrs || !slot_mapping_ptrs))
    return PA_ERR_NULL;
  if (position < 0 || position >= INT32_MAX) return PA_ERR_SIZE;
  if (query_start_loc_len < 2 || seq_lens_len < 1 || discard_len < 1) return PA_ERR_SIZE;
  if (mrope && positions_stride < 1) return PA_ERR_SIZE;
  pa::InputPrepArgs a;
  a.sampled_token_ids = sampled_token_ids;
  a.position = position;
  a.input_ids = input_ids;
  a.positions = positions;
  a.mrope = mrope ? 1 : 0;
  a.positions_stride = positions_stride;
  a.mrope_delta = mrope_delta;
  a.query_start_loc = query_start_loc;
  a.query_start_loc_len = query_start_loc_len;
  a.seq_lens = seq_lens;
  a.seq_lens_len = seq_lens_len;
  a.discard_request_mask = discard_request_mask;
  a.discard_len = discard_len;
  a.is_token_ids = is_token_ids;
  a.num_kv_groups = num_kv_groups;
  a.block_sizes = block_sizes;
  a.block_table_ptrs = block_table_ptrs;
  a.slot_mapping_ptrs = slot_mapping_ptrs;
  return launch_status(pa::launch_decode_input_prep(a, static_cast<hipStream_t>(stream)));
}

int pa_page_size_for_hybrid(int64_t mamba_page_bytes, int64_t attn_page_bytes_per_token,
                            int32_t alignment_tokens, int32_t* block_size_out) {
  if (!block_size_out) return PA_ERR_NULL;
  if (mamba_page_bytes <= 0 || attn_page_bytes_per_token <= 0 || alignment_tokens <= 0)
    return PA_ERR_SIZE;
  // bytes of one alignment group of attention tokens; quotient rounded up
  if (attn_page_bytes_per_token > INT64_MAX / alignment_tokens) return PA_ERR_SIZE;
  const int64_t group_bytes = attn_page_bytes_per_token * alignment_tokens;
  const int64_t groups = mamba_page_bytes / group_bytes + (mamba_page_bytes % group_bytes != 0);
  if (groups > INT32_MAX / alignment_tokens) return PA_ERR_SIZE;
  *block_size_out = (int32_t)(groups * alignment_tokens);
  return PA_OK;
}

int pa_gemv_bf16(void* y, int32_t y_f32, const void* W, const void* x, int32_t N, int32_t K,
                 int64_t ldw, void* stream) {
  if (N < 0 || K < 0 || (K & 7) || ldw < K || (ldw & 7)) return PA_ERR_SIZE;
  if (N == 0) return PA_OK;
  if (!y || (K > 0 && (!W || !x))) return PA_ERR_NULL;
  const uintptr_t ya = reinterpret_cast<uintptr_t>(y);
  if ((K > 0 && (!aligned16(W) || !aligned16(x))) || (ya & (y_f32 ? 3u : 1u))) return PA_ERR_ALIGN;
  return launch_status(pa::launch_gemv(y, y_f32 != 0, static_cast<const uint16_t*>(W),
                                       static_cast<const uint16_t*>(x), N, K, ldw,
                                       static_cast<hipStream_t>(stream)));
}

const char* pa_strerror(int code) {
  switch (code) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_BLOCK_SIZE: return "block_size must be >= 1 and one page of one cache below 4 GiB";
    case PA_ERR_UNSUPPORTED: return "unsupported shape: need head_dim 256, num_q_heads = 6 * num_kv_heads, 1 <= num_kv_heads <= 64";
    case PA_ERR_SIZE: return "a count or position is out of range";
    case PA_ERR_WORKSPACE: return "workspace is NULL or smaller than pa_decode_workspace_size() / pa_prefill_workspace_size()";
    case PA_ERR_TABLE: return "the block table has fewer entries than the lengths need";
    case PA_ERR_STRIDE: return "page_stride is smaller than one page";
    case PA_ERR_ALIGN: return "a tensor is not aligned (bf16 tensors: 16 bytes, workspace: 256 bytes)";
    case PA_ERR_SCALE: return "scale must be a positive finite number";
    case PA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case PA_ERR_SCRATCH: return "the batch needs more decode scratch than the library's static buffer holds (16 MiB): use pa_decode with a workspace";
    default: return "unknown error code";
  }
}

const char* pa_build_info(void) {
  static const std::string info = std::string("libpa rev=") + PA_GIT_REV +
                                 " target=gfx950 " + pa::kDecodeVariant + " " +
                                 pa::kPrefillVariant + " kv_write-v1(one-wg-per-token) " +
                                 pa::gemv_variant();
  return info.c_str();
}

}  // extern "C"
