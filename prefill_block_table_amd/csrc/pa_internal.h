// Internal launcher declarations of libpa (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kHeadDimAbi = 256;  // the only head size the kernels are built for

hipError_t launch_slot_mapping(int64_t* slot_out, const int64_t* positions,
                               const int32_t* token_seq, int32_t num_tokens,
                               const int32_t* block_table, int32_t bt_stride,
                               int32_t block_size, hipStream_t stream);

hipError_t launch_kv_write(uint16_t* k_cache, uint16_t* v_cache, int64_t page_stride,
                           int32_t num_pages, int32_t block_size, int32_t num_kv_heads,
                           const uint16_t* k_new, const uint16_t* v_new, int32_t num_tokens,
                           const int64_t* slot_mapping, const int64_t* positions,
                           const int32_t* token_seq, const int32_t* block_table,
                           int32_t bt_stride, int64_t* slot_out, hipStream_t stream);

// Decode split plan.  A step is 16 tokens of one page for `heads_per_wg`
// KV heads (16 * 4 / heads_per_wg tokens when a workgroup's four waves share
// fewer heads).  The batch's steps are cut into `num_wgs` near-equal ranges.
#ifndef PA_DECODE_WGS
#define PA_DECODE_WGS 256
#endif
constexpr int kDecodeWorkgroups = PA_DECODE_WGS;   // one per MI355X CU

struct DecodePlan {
  int32_t heads_per_wg;
  int32_t step_tokens;
  int32_t steps_per_page;
  int32_t num_wgs;
  int64_t steps_ub;      // upper bound of the batch's steps (must stay below 2^31)
  size_t meta_off, p_ml_off, p_acc_off, bytes;
};
constexpr int64_t kMaxDecodeSteps = (int64_t)1 << 31;

DecodePlan plan_decode(int32_t num_seqs, int32_t max_seq_len, int32_t block_size,
                       int32_t num_kv_heads);

// Token appended by the decode launch itself (pa_decode_append): row [s]
// of k_new / v_new ([num_seqs][num_kv_heads][256]) is the token at position
// seq_lens[s] - 1; k_cache / v_cache are the same caches the decode reads.
struct DecodeAppend {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int64_t* slot_out;   // NULL = do not store the slots
};

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, int64_t page_stride,
                         const int32_t* block_table, int32_t bt_stride,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                         int32_t block_size, float scale, int32_t num_kv_heads,
                         const DecodePlan& plan, void* workspace, const DecodeAppend* append,
                         hipStream_t stream);

// Allocation-free decode (pa_decode_noalloc): the same kernels with the
// workspace in a file-scope device buffer of kDecodeScratchBytes (one copy
// per GPU, alive until the process ends).  Its device address is looked up
// once per device (hipGetSymbolAddress with that device current) and kept.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch_for_current_device(void** ptr);

// Chunked prefill work plan: how many items (query head x 128-row tile) run
// whole, and how the rest are cut along their key groups.
constexpr int kPrefillSlots = 256;      // workgroups per round: one per MI355X CU
constexpr int kPrefillMaxSplit = 16;
struct PrefillPlan {
  int64_t num_items;
  int64_t num_full;      // items 0 .. num_full-1 (heavy first) run whole
  int64_t split_items;   // the remaining items, each cut into `split` parts
  int32_t split;
  size_t part_o_off, part_ml_off, bytes;   // workspace layout (bytes = 0: none needed)
};

PrefillPlan plan_prefill(int32_t q_len, int32_t start_pos, int32_t causal, int32_t block_size,
                         int32_t num_kv_heads);

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, int32_t q_len, int32_t start_pos,
                          int32_t causal, const uint16_t* k_cache, const uint16_t* v_cache,
                          int64_t page_stride, const int32_t* block_table, int32_t block_size,
                          float scale, int32_t num_kv_heads, const PrefillPlan& plan,
                          void* workspace, hipStream_t stream);

// Single-token decode input preparation (pa_decode_input_prep).
struct InputPrepArgs {
  const int64_t* sampled_token_ids;
  int64_t position;
  int32_t* input_ids;
  int64_t* positions;
  int32_t mrope;
  int64_t positions_stride;
  int64_t mrope_delta;
  int32_t* query_start_loc;
  int32_t query_start_loc_len;
  int32_t* seq_lens;
  int32_t seq_lens_len;
  uint8_t* discard_request_mask;
  int32_t discard_len;
  uint8_t* is_token_ids;           // NULL: not written
  int32_t num_kv_groups;
  const int32_t* block_sizes;
  const uint64_t* block_table_ptrs;
  const uint64_t* slot_mapping_ptrs;
};

hipError_t launch_decode_input_prep(const InputPrepArgs& a, hipStream_t stream);

// Workgroups of a several-sequence prefill launch: total_q / 128 + num_seqs
// tile slots (each sequence's rows and at most one spare slot), each one
// workgroup per query head (6 per KV head).
inline int64_t varlen_grid(int32_t total_q, int32_t num_seqs, int32_t num_kv_heads) {
  return ((int64_t)total_q / 128 + num_seqs) * num_kv_heads * 6;
}

hipError_t launch_prefill_varlen(uint16_t* out, const uint16_t* q, int32_t total_q,
                                 const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                                 int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int32_t causal, const uint16_t* k_cache, const uint16_t* v_cache,
                                 int64_t page_stride, const int32_t* block_table, int32_t bt_stride,
                                 int32_t block_size, float scale, int32_t num_kv_heads,
                                 hipStream_t stream);

extern const char* const kDecodeVariant;
extern const char* const kPrefillVariant;

// bf16 M=1 GEMV y = W x (gemv.hip); y is bf16 or fp32.
hipError_t launch_gemv(void* y, bool y_f32, const uint16_t* W, const uint16_t* x, int32_t N,
                       int32_t K, int64_t ldw, hipStream_t stream);
const char* gemv_variant();

}  // namespace pa
