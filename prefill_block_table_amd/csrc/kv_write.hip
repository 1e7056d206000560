// Slot mapping and KV-cache write kernels (gfx950).
//
// Slot of a token ([PREP] §3.2, §5): slot = block_table[seq][pos / B] * B +
// pos % B.  The write copies the token's K and V rows (num_kv_heads * 256
// bf16 each) to row slot % B of page slot / B.  Both are integer / bit work:
// one workgroup per token, 16-byte vector loads and stores.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

__device__ __forceinline__ int64_t compute_slot(int64_t pos, int32_t seq, const int32_t* bt,
                                                int32_t bt_stride, int32_t block_size) {
  if (pos < 0) return -1;
  const int64_t logical = pos / block_size;
  if (logical >= bt_stride) return -1;
  const int64_t page = bt[(int64_t)seq * bt_stride + logical];
  return page * block_size + (pos - logical * block_size);
}

__global__ void __launch_bounds__(256) slot_mapping_kernel(
    int64_t* __restrict__ slot_out, const int64_t* __restrict__ positions,
    const int32_t* __restrict__ token_seq, int32_t num_tokens,
    const int32_t* __restrict__ block_table, int32_t bt_stride, int32_t block_size) {
  const int32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i >= num_tokens) return;
  const int32_t seq = token_seq ? token_seq[i] : 0;
  slot_out[i] = compute_slot(positions[i], seq, block_table, bt_stride, block_size);
}

// One workgroup of 256 threads per token.  The K row and the V row are each
// row_vecs 16-byte vectors (row_vecs = num_kv_heads * 256 * 2 / 16); thread t
// copies vectors t, t + 256, ... of the concatenated [K row | V row].
__global__ void __launch_bounds__(256) kv_write_kernel(
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, int64_t page_stride,
    int64_t num_slots, int32_t block_size, int32_t row_elems,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, const int64_t* __restrict__ positions,
    const int32_t* __restrict__ token_seq, const int32_t* __restrict__ block_table,
    int32_t bt_stride, int64_t* __restrict__ slot_out) {
  const int32_t i = blockIdx.x;
  const int64_t src = (int64_t)i * row_elems;
  const int32_t row_vecs = row_elems / 8;
  // The new rows do not depend on the slot: load them first so their latency
  // overlaps the positions -> block table -> slot chain.
  u32x4 vec[4];
  int nvec = 0;
  for (int32_t v = threadIdx.x; v < 2 * row_vecs && nvec < 4; v += 256, ++nvec) {
    const bool is_v = v >= row_vecs;
    const int32_t e = (is_v ? v - row_vecs : v) * 8;
    vec[nvec] = *reinterpret_cast<const u32x4*>((is_v ? v_new : k_new) + src + e);
  }
  int64_t slot;
  if (slot_mapping) {
    slot = slot_mapping[i];
  } else {
    const int32_t seq = token_seq ? token_seq[i] : 0;
    slot = compute_slot(positions[i], seq, block_table, bt_stride, block_size);
    if (slot_out && threadIdx.x == 0) slot_out[i] = slot;
  }
  if (slot < 0 || slot >= num_slots) return;
  const int64_t page = slot / block_size;
  const int64_t row = slot - page * block_size;
  const int64_t dst = page * page_stride + row * row_elems;
  int k = 0;
  for (int32_t v = threadIdx.x; v < 2 * row_vecs; v += 256, ++k) {
    const bool is_v = v >= row_vecs;
    const int32_t e = (is_v ? v - row_vecs : v) * 8;
    u32x4 x;
    if (k < 4) {
      x = vec[k];
    } else {   // rows longer than 4 x 256 vectors (more than 32 KV heads)
      x = *reinterpret_cast<const u32x4*>((is_v ? v_new : k_new) + src + e);
    }
    *reinterpret_cast<u32x4*>((is_v ? v_cache : k_cache) + dst + e) = x;
  }
}

}  // namespace

hipError_t launch_slot_mapping(int64_t* slot_out, const int64_t* positions,
                               const int32_t* token_seq, int32_t num_tokens,
                               const int32_t* block_table, int32_t bt_stride,
                               int32_t block_size, hipStream_t stream) {
  const int32_t blocks = (num_tokens + 255) / 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks), dim3(256), 0, stream, slot_out,
                     positions, token_seq, num_tokens, block_table, bt_stride, block_size);
  return hipGetLastError();
}

hipError_t launch_kv_write(uint16_t* k_cache, uint16_t* v_cache, int64_t page_stride,
                           int32_t num_pages, int32_t block_size, int32_t num_kv_heads,
                           const uint16_t* k_new, const uint16_t* v_new, int32_t num_tokens,
                           const int64_t* slot_mapping, const int64_t* positions,
                           const int32_t* token_seq, const int32_t* block_table,
                           int32_t bt_stride, int64_t* slot_out, hipStream_t stream) {
  const int64_t num_slots = (int64_t)num_pages * block_size;
  hipLaunchKernelGGL(kv_write_kernel, dim3(num_tokens), dim3(256), 0, stream, k_cache,
                     v_cache, page_stride, num_slots, block_size, num_kv_heads * kHeadDim,
                     k_new, v_new, slot_mapping, positions, token_seq, block_table, bt_stride,
                     slot_out);
  return hipGetLastError();
}

}  // namespace pa
