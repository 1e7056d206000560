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

// Split-K plan of a decode batch: a "unit" is one 64-token group of one page
// (a page of B tokens has ceil(B / 64) units, the last one a tail when B is
// not a multiple of 64); a split is `groups_per_split` consecutive units.
struct DecodePlan {
  int32_t units_per_page;
  int32_t groups_per_split;
  int32_t max_splits;       // splits of the longest sequence (grid x)
  int32_t cluster;          // splits merged together at the first merge level
  int32_t max_clusters;     // clusters of the longest sequence
  size_t cnt1_off, cnt2_off, p1_ml_off, p2_ml_off, p1_acc_off, p2_acc_off, bytes;
};

DecodePlan plan_decode(int32_t num_seqs, int32_t max_seq_len, int32_t block_size,
                       int32_t num_kv_heads);

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, int64_t page_stride,
                         const int32_t* block_table, int32_t bt_stride,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                         int32_t block_size, float scale, int32_t num_kv_heads,
                         const DecodePlan& plan, void* workspace, hipStream_t stream);

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, int32_t q_len, int32_t start_pos,
                          int32_t causal, const uint16_t* k_cache, const uint16_t* v_cache,
                          int64_t page_stride, const int32_t* block_table, int32_t block_size,
                          float scale, int32_t num_kv_heads, hipStream_t stream);

extern const char* const kDecodeVariant;
extern const char* const kPrefillVariant;

}  // namespace pa
