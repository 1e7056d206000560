// Single-request, single-token decode input preparation in one launch
// (gfx950).
//
// What it writes ([PREP] §2, §4, §5): when exactly one request advances by
// exactly one token, every model input and attention-metadata entry of the
// step is a closed form of the previous step's sampled token (already in
// device memory) and the token's position:
//   input_ids[0]        = sampled_token_ids[0]
//   positions           = position (M-RoPE: the same in all three rows, plus
//                         the request's M-RoPE offset)
//   query_start_loc     = [0, 1, 1, ...]          (whole buffer)
//   seq_lens            = [position + 1, 0, 0, ...] (whole buffer)
//   discard mask        = all false                (whole buffer)
//   is_token_ids[0]     = true (when the buffer is given)
// and, for every KV-cache group g with its own page size B_g, block-table
// row and slot-mapping buffer (reached through device arrays of 64-bit
// addresses, so one launch serves any number of groups):
//   slot_g = block_table_g[position / B_g] * B_g + position % B_g ([PREP]
//   §3.2).
// Workgroup g computes group g's slot; workgroup 0 also writes the shared
// entries.  Integer work only.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

__global__ void __launch_bounds__(64) decode_input_prep_kernel(InputPrepArgs a) {
  const int g = blockIdx.x;
  const int t = threadIdx.x;
  if (g < a.num_kv_groups) {
    const int32_t B = a.block_sizes[g];
    const int32_t* bt = reinterpret_cast<const int32_t*>(a.block_table_ptrs[g]);
    int64_t* sm = reinterpret_cast<int64_t*>(a.slot_mapping_ptrs[g]);
    if (t == 0) {
      const int64_t logical = B > 0 ? a.position / B : 0;
      sm[0] = B > 0 ? (int64_t)bt[logical] * B + (a.position - logical * B) : -1;
    }
  }
  if (g != 0) return;
  if (t == 0) {
    a.input_ids[0] = (int32_t)a.sampled_token_ids[0];
    if (a.mrope) {
      const int64_t p = a.position + a.mrope_delta;
      a.positions[0] = p;
      a.positions[a.positions_stride] = p;
      a.positions[2 * a.positions_stride] = p;
    } else {
      a.positions[0] = a.position;
    }
    if (a.is_token_ids) a.is_token_ids[0] = 1;
  }
  for (int32_t i = t; i < a.query_start_loc_len; i += 64) a.query_start_loc[i] = i == 0 ? 0 : 1;
  for (int32_t i = t; i < a.seq_lens_len; i += 64) a.seq_lens[i] = i == 0 ? (int32_t)(a.position + 1) : 0;
  for (int32_t i = t; i < a.discard_len; i += 64) a.discard_request_mask[i] = 0;
}

}  // namespace

hipError_t launch_decode_input_prep(const InputPrepArgs& a, hipStream_t stream) {
  const int grid = a.num_kv_groups > 0 ? a.num_kv_groups : 1;
  hipLaunchKernelGGL(decode_input_prep_kernel, dim3(grid), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
