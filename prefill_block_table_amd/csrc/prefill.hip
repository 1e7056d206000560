// Chunked-prefill paged GQA attention for gfx950 (bf16 MFMA, fp32 accumulate).
//
// What it computes ([ALIGN] §6): for the q_len query tokens of one chunk at
// positions start_pos + i, complete causal attention over the paged K/V of
// the first start_pos + q_len tokens; no key skipped that the causal mask
// allows, none added that it forbids ([ALIGN] §5, §9).
//
// Work decomposition (ours): a workgroup of 4 wave64s owns a 128-row query
// tile of one query head; wave w owns 32 rows.  Keys stream through LDS one
// 64-token group of one page at a time (the page's tail group is masked when
// the page size is not a multiple of 64).  Per group:
//   S^T[64 keys x 32 rows] = K[64 x 256] Q^T     (32 MFMA 32x32x16 per wave)
//   online softmax on S^T: each lane holds one query row, so the row max and
//   sum need one cross-lane exchange (lane ^ 32) only
//   O^T[256 x 32 rows] += V^T[256 x 64] P^T     (32 MFMA 32x32x16 per wave)
// The transposed orientation makes P^T's MFMA operand a register-local
// reinterpretation of S^T's accumulator (no shuffles); V is transposed once
// while it is staged into LDS.  Groups entirely above the causal diagonal of
// the tile are never visited; the mask is evaluated only on groups that
// cross the diagonal or end a page early.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

const char* const kPrefillVariant = "prefill-v1(bm128,bn64,mfma32x32x16,st-orient,lds-vt,heavy-first)";

namespace {

constexpr int kBM = 128;
constexpr int kKStride = kHeadDim + 8;  // bf16 elements per K row in LDS (16 B pad)
constexpr int kVtStride = kGroup + 4;   // bf16 elements per V^T row in LDS (8 B pad)

struct PrefillArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int64_t page_stride;
  const int32_t* block_table;
  int32_t q_len;
  int32_t start_pos;
  int32_t causal;
  int32_t block_size;
  float scale_log2;
  int32_t num_kv_heads;
  int32_t num_q_tiles;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ void __launch_bounds__(256, 1) prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kGroup * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kHeadDim * kVtStride];

  const int head = blockIdx.x;
  const int tile = a.num_q_tiles - 1 - (int)blockIdx.y;   // heaviest (latest) rows first
  const int g = head / kGqa;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hh = lane >> 5;
  const int col = lane & 31;
  const int Hq = a.num_kv_heads * kGqa;
  const int64_t row_stride = (int64_t)a.num_kv_heads * kHeadDim;
  const int64_t q_stride = (int64_t)Hq * kHeadDim;
  const int B = a.block_size;

  const int q0 = tile * kBM;
  const int my_row = q0 + 32 * w + col;
  const bool row_ok = my_row < a.q_len;
  const int my_pos = a.start_pos + my_row;
  const int wave_first_pos = a.start_pos + q0 + 32 * w;

  // Q^T as the B operand of S^T = K Q^T: lane supplies column n = col (its
  // query row) and k = 8*hh + i of each 16-wide step ds -> d = 16*ds + 8*hh + i.
  bf16x8 qb[16];
  {
    const uint16_t* qp = a.q + (int64_t)(row_ok ? my_row : 0) * q_stride + head * kHeadDim + 8 * hh;
#pragma unroll
    for (int ds = 0; ds < 16; ++ds) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = load16(qp + 16 * ds);
      qb[ds] = as_bf16x8(v);
    }
  }

  const int kv_len = a.start_pos + a.q_len;
  const int tile_last = min(q0 + kBM, a.q_len) - 1;
  const int kv_end = a.causal ? a.start_pos + tile_last + 1 : kv_len;
  const int upp = (B + kGroup - 1) / kGroup;
  const int last_page = (kv_end - 1) / B;
  const int units = last_page * upp + (kv_end - last_page * B + kGroup - 1) / kGroup;

  f32x16 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  for (int u = 0; u < units; ++u) {
    const int page = u / upp;
    const int grp = u - page * upp;
    const int key0 = page * B + grp * kGroup;                 // absolute position of key 0
    const int n = min(kGroup, min(B - grp * kGroup, kv_end - key0));
    const int64_t phys = a.block_table[page];
    const int64_t off = phys * a.page_stride + (int64_t)grp * kGroup * row_stride + (int64_t)g * kHeadDim;
    const uint16_t* kg = a.k_cache + off;
    const uint16_t* vg = a.v_cache + off;

    __syncthreads();   // all waves are done reading the previous group
    // K rows -> LDS (64 rows x 32 vectors of 16 B).
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c = it * 256 + tid;
      const int row = c >> 5;
      const int ch = c & 31;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < n) v = load16(kg + (int64_t)row * row_stride + 8 * ch);
      *reinterpret_cast<u32x4*>(&k_lds[row * kKStride + 8 * ch]) = v;
    }
    // V rows -> V^T in LDS: each thread takes 4 keys x 8 dims and writes 8
    // rows of V^T, 4 keys (8 B) each.
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = it * 256 + tid;
      const int kq = c >> 5;          // key quad 0..15
      const int dc = c & 31;          // 8-dim chunk 0..31
      u32x4 r4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * kq + i;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < n) v = load16(vg + (int64_t)row * row_stride + 8 * dc);
        r4[i] = v;
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int wd = dd >> 1;
        const int sh = (dd & 1) * 16;
        const uint32_t e0 = (r4[0][wd] >> sh) & 0xffffu;
        const uint32_t e1 = (r4[1][wd] >> sh) & 0xffffu;
        const uint32_t e2 = (r4[2][wd] >> sh) & 0xffffu;
        const uint32_t e3 = (r4[3][wd] >> sh) & 0xffffu;
        u32x2 pk = {e0 | (e1 << 16), e2 | (e3 << 16)};
        *reinterpret_cast<u32x2*>(&vt_lds[(8 * dc + dd) * kVtStride + 4 * kq]) = pk;
      }
    }
    __syncthreads();

    // S^T = K Q^T for keys 0..31 (st0) and 32..63 (st1).
    f32x16 st0, st1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { st0[r] = 0.f; st1[r] = 0.f; }
#pragma unroll
    for (int ds = 0; ds < 16; ++ds) {
      const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(&k_lds[col * kKStride + 16 * ds + 8 * hh]);
      const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(&k_lds[(32 + col) * kKStride + 16 * ds + 8 * hh]);
      st0 = mfma32(ka0, qb[ds], st0);
      st1 = mfma32(ka1, qb[ds], st1);
    }
    // Accumulator register r of st{kh} holds key 32*kh + 8*(r/4) + 4*hh + r%4
    // for query row `col` of this wave.
    float sv[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) { sv[r] = st0[r] * a.scale_log2; sv[16 + r] = st1[r] * a.scale_log2; }
    const bool need_mask = (n < kGroup) || (a.causal && key0 + kGroup - 1 > wave_first_pos);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int key = (r >> 4) * 32 + 8 * ((r & 15) >> 2) + 4 * hh + (r & 3);
        if (key >= n || (a.causal && key0 + key > my_pos)) sv[r] = -INFINITY;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int r = 1; r < 32; ++r) mx = fmaxf(mx, sv[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
    uint32_t pk[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = fast_exp2(sv[2 * i] - m_use);
      const float p1 = fast_exp2(sv[2 * i + 1] - m_use);
      rs += p0 + p1;
      pk[i] = pack_bf16x2(p0, p1);
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    // O^T += V^T P^T over 4 steps of 16 keys.  MFMA k = 8*hh + 4*jj + i maps
    // to key 16*ks + 8*jj + 4*hh + i on both operands.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kh = ks >> 1;
      const int j0 = 2 * (ks & 1);
      const u32x4 pb = {pk[8 * kh + 2 * j0], pk[8 * kh + 2 * j0 + 1],
                        pk[8 * kh + 2 * j0 + 2], pk[8 * kh + 2 * j0 + 3]};
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint16_t* vrow = &vt_lds[(32 * db + col) * kVtStride + 16 * ks + 4 * hh];
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(vrow + 8);
        const u32x4 va = {a0[0], a0[1], a1[0], a1[1]};
        o[db] = mfma32(as_bf16x8(va), as_bf16x8(pb), o[db]);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (row_ok) {
    uint16_t* op = a.out + (int64_t)my_row * q_stride + head * kHeadDim;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * hh;
        u32x2 v = {pack_bf16x2(o[db][4 * j] * inv, o[db][4 * j + 1] * inv),
                   pack_bf16x2(o[db][4 * j + 2] * inv, o[db][4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = v;
      }
  }
}

}  // namespace

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, int32_t q_len, int32_t start_pos,
                          int32_t causal, const uint16_t* k_cache, const uint16_t* v_cache,
                          int64_t page_stride, const int32_t* block_table, int32_t block_size,
                          float scale, int32_t num_kv_heads, hipStream_t stream) {
  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_stride = page_stride;
  a.block_table = block_table;
  a.q_len = q_len;
  a.start_pos = start_pos;
  a.causal = causal ? 1 : 0;
  a.block_size = block_size;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_kv_heads = num_kv_heads;
  a.num_q_tiles = (q_len + kBM - 1) / kBM;
  hipLaunchKernelGGL(prefill_kernel, dim3(num_kv_heads * kGqa, a.num_q_tiles), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pa
