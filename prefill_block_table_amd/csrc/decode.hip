// Single-token paged GQA decode for gfx950 (split-K / flash-decoding).
//
// What it computes ([ALIGN] §7): for each sequence and query head, softmax
// attention of the one query over all seq_len keys, walking the pages of the
// sequence in order, one block-table lookup per page, token groups inside
// each page, online softmax.  The last group of a page is masked when the
// page size is not a multiple of the group ([ALIGN] §2, §5).
//
// Two kernels (ours):
// 1. decode_split_kernel.  The work of the batch is a list of items (one per
//    sequence and group of 4 KV heads), each a run of steps; a step is 16
//    tokens of one page for the item's 4 KV heads (wave w takes KV head w, so
//    a step is 32 KB of consecutive cache rows for K and for V; with fewer
//    KV heads, waves of one head take consecutive 16-token slices).  The
//    flattened step list is cut into one near-equal contiguous range per
//    workgroup, about one workgroup per CU, so short and long sequences of a
//    batch are balanced.  Per wave and step:
//    - K and V rows go from HBM into wave-private LDS with the direct-to-LDS
//      load (no VGPRs; 16-byte chunks XOR-swizzled by row so the operand reads
//      below are bank-conflict free), two steps in flight;
//    - the 6 query heads of the KV head share every K/V byte read (GQA 6):
//      S^T[16 keys x 16] = K Q^T is eight 16x16x32 bf16 MFMAs; in this
//      orientation each lane holds one query head, so the online-softmax max
//      and sum take two cross-lane shuffles and P^T is already laid out as
//      the next MFMA's operand;
//    - V^T operands come out of LDS with the gfx950 transposing read, and
//      O^T[256 x 16] += V^T P^T is sixteen 16x16x16 bf16 MFMAs;
//    - O^T is re-based to a new running max only when a score exceeds the
//      current reference by more than 2^8 (exact; keeps the accumulator out
//      of the VALU on almost every step).
//    Each (item, workgroup) pair that shares work leaves one partial (m, l,
//    unnormalised O) per KV head; an item done by a single workgroup writes
//    bf16 output directly.
// 2. decode_merge_kernel.  One workgroup per (sequence, query head, 16-dim
//    slice); its 256 threads take 16 partials at a time, so all loads of a
//    workgroup are in flight together.  Merge order is fixed: results are
//    bitwise repeatable, no atomics anywhere.
// Nothing is read past a page's or a sequence's last live row (such rows are
// replaced by the page's first row, whose weight is exactly 0), so poisoned
// rows never reach the output.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

const char* const kDecodeVariant =
    "decode-v6(split+merge,balanced-steps,4heads-per-wg,16tok-steps,kv-lds-dma,2stage,"
    "mfma16x16x32-qk,tr16-vt,mfma16x16x16-pv,lazy-rescale)";

namespace {

constexpr int kWaves = 4;
constexpr int kStages = 2;
constexpr int kRowBytes = kHeadDim * 2;            // one KV head's row: 512 B
constexpr int kTileBytes = 16 * kRowBytes;         // 16 K (or V) rows of one wave step: 8 KB
constexpr int kStageBytes = 2 * kTileBytes;        // K tile then V tile
constexpr int kSmemBytes = kWaves * kStages * kStageBytes;   // 128 KB
constexpr float kRescaleSlack = 8.f;               // log2 headroom before re-basing O
constexpr int kMergeSlices = 16;                   // partials merged in parallel per dim
constexpr int kMergeDims = 16;                     // dims per merge workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define PA_LDS __attribute__((address_space(3)))

// Waits on this wave's outstanding memory operations.  Inline asm with a
// memory clobber, so the compiler cannot move LDS reads of direct-to-LDS
// data above the wait.  Vector memory operations retire in issue order.
#define PA_WAIT_VMCNT(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")
#define PA_WAIT_LGKMCNT0() asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory")

struct DecodeArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int64_t page_stride;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  int32_t num_seqs;
  int32_t max_seq_len;
  int32_t block_size;
  float scale_log2;        // scale * log2(e): scores live in the exp2 domain
  int32_t num_kv_heads;
  int32_t heads_per_wg;    // KV heads of one item (4, 2 or 1)
  int32_t step_tokens;     // 16 * (4 / heads_per_wg)
  int32_t steps_per_page;
  int32_t num_wgs;         // split workgroups (grid of the split kernel)
  float* p_acc;            // [slot][heads_per_wg][6][256], slot = item + workgroup
  float* p_ml;             // [slot][heads_per_wg][6][2]
  int32_t* meta;           // [item][2]: first workgroup, number of partials
};

__device__ __forceinline__ int clamp_len(int L, int max_len) {
  return L < 0 ? 0 : (L > max_len ? max_len : L);
}

// Live steps of a sequence of L tokens (0 for L == 0).
__device__ __forceinline__ int live_steps(int L, int B, int spp, int step_tokens) {
  if (L <= 0) return 0;
  const int last_page = (L - 1) / B;
  const int rem = L - last_page * B;
  return last_page * spp + (rem + step_tokens - 1) / step_tokens;
}

// Workgroup ranges: workgroup w owns flattened steps [bnd(w), bnd(w + 1)),
// bnd(w) = floor(w * T / N); the workgroup owning step x is
// floor(((x + 1) * N - 1) / T).
__device__ __forceinline__ int64_t wg_bound(int64_t w, int64_t T, int64_t N) { return w * T / N; }
__device__ __forceinline__ int64_t wg_of(int64_t x, int64_t T, int64_t N) {
  return ((x + 1) * N - 1) / T;
}

// Pair reductions across lanes l and l ^ 16 (or l ^ 32) with the gfx950
// lane-swap instructions: with both operands x, the two results hold x of
// the even and of the odd 16-lane row (32-lane half) of each pair, at every
// lane; combining them is a plain VALU op (no LDS round trip) and gives both
// lanes of a pair the same bits.
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// K rows: 16-byte chunk c of row r sits at position c ^ (r & 7), so the 8
// rows of an MFMA-operand read hit 8 different bank quads.  V rows: chunk c
// at c ^ ((r & 3) << 1), so the 4 rows of a transposing read hit 4 different
// 32-byte bank groups.
__device__ __forceinline__ int kswz(int r) { return r & 7; }
__device__ __forceinline__ int vswz(int r) { return (r & 3) << 1; }

// Read-only metadata (block tables) read at a wave-uniform address: through
// the constant address space, so it is a scalar load whose wait does not
// drain this wave's in-flight vector loads.
__device__ __forceinline__ int32_t load_const_i32(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// 32-bit LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const PA_LDS char*)p;
}
// LDS operand reads the compiler does not track (see compute() below).
#define PA_DS_READ_B128(dst, addr, off) \
  asm volatile("ds_read_b128 %0, %1 offset:" #off : "=v"(dst) : "v"(addr))
#define PA_DS_READ_TR16(dst, addr, off) \
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:" #off : "=v"(dst) : "v"(addr))

// Sum over 256 threads (all threads get the result).
__device__ __forceinline__ int64_t block_sum(int64_t v, int64_t* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__global__ void __launch_bounds__(256, 1) decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  __shared__ int64_t red[4];
  __shared__ int64_t scan_lds[kWaves];

  const int wgi = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * kGqa;
  const int B = a.block_size;
  const int hpw = a.heads_per_wg;
  const int ng = Hkv / hpw;               // items per sequence
  const int ksl = kWaves / hpw;
  const int jw = w % hpw;                 // this wave's KV head within the item
  const int ks = w / hpw;                 // this wave's 16-token slice of a step
  const int spp = a.steps_per_page;
  const int stok = a.step_tokens;
  const int c16 = lane & 15;
  const int kq = lane >> 4;

  // Total steps T of the batch, this workgroup's range [x0, x1) and the
  // sequence holding step x0.  One pass over seq_lens when the batch has at
  // most 256 sequences (a second pass locates x0 in larger batches).
  int64_t T = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 256) {
    const int s = c0 + tid;
    const int64_t v = s < a.num_seqs
        ? (int64_t)live_steps(clamp_len(a.seq_lens[s], a.max_seq_len), B, spp, stok) * ng : 0;
    T += block_sum(v, red);
  }
  if (T == 0) return;
  // Effective workgroup count min(launched, T): every workgroup below it owns
  // at least one step, so the workgroups sharing an item are consecutive and
  // its partials occupy consecutive slots.
  const int64_t N = T < a.num_wgs ? T : a.num_wgs;
  if (wgi >= N) return;
  const int64_t x0 = wg_bound(wgi, T, N);
  const int64_t x1 = wg_bound(wgi + 1, T, N);
  if (x0 >= x1) return;
  int s_cur = 0;
  int64_t seq_start = 0;    // flattened index of the first step of s_cur
  for (int c0 = 0; c0 < a.num_seqs; c0 += 256) {
    const int s = c0 + tid;
    const int64_t v = s < a.num_seqs
        ? (int64_t)live_steps(clamp_len(a.seq_lens[s], a.max_seq_len), B, spp, stok) * ng : 0;
    // exclusive prefix of v over the block: wave scan, then wave totals
    int64_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    __syncthreads();
    if (lane == 63) scan_lds[w] = incl;
    __syncthreads();
    int64_t before = 0, total = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      before += ww < w ? scan_lds[ww] : 0;
      total += scan_lds[ww];
    }
    const int64_t lo = seq_start + before + incl - v;
    const int64_t hi = seq_start + before + incl;
    const bool found = x0 < seq_start + total;
    if (found) {
      if (s < a.num_seqs && lo <= x0 && x0 < hi) { red[0] = s; red[1] = lo; }
      __syncthreads();
      // wave-uniform from here on (scalar registers, scalar block-table loads)
      s_cur = __builtin_amdgcn_readfirstlane((int)red[0]);
      seq_start = ((int64_t)__builtin_amdgcn_readfirstlane((int)(red[1] >> 32)) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)(red[1] & 0xffffffff));
      break;
    }
    seq_start += total;
  }

  const int64_t row_stride = (int64_t)Hkv * kHeadDim;   // elements per cache row (token)
  char* vbase = smem + w * (kStages * kStageBytes);

  // Walk the items (s, hg) overlapping [x0, x1).
  int64_t x = x0;
  while (x < x1) {
    const int s = __builtin_amdgcn_readfirstlane(s_cur);
    const int L = clamp_len(a.seq_lens[s], a.max_seq_len);
    const int steps = live_steps(L, B, spp, stok);
    if (steps == 0) { ++s_cur; continue; }
    const int hg = (int)((x - seq_start) / steps);
    const int64_t item_start = seq_start + (int64_t)hg * steps;
    const int64_t item_end = item_start + steps;
    const int la = (int)(x - item_start);
    const int lb = (int)((x1 < item_end ? x1 : item_end) - item_start);
    const int item = s * ng + hg;
    const int g = hg * hpw + jw;
    const int64_t first_wg = wg_of(item_start, T, N);
    const int64_t last_wg = wg_of(item_end - 1, T, N);
    const int nparts = (int)(last_wg - first_wg + 1);

    const int32_t* bt = a.block_table + (int64_t)s * a.bt_stride;
    // Q^T as the B operand of S^T = K Q^T (16x16x32): lane supplies column
    // n = c16 (query head; columns 6..15 are zero) and k = 8*kq + i of
    // operand step t, mapped to d = 32*t + 8*kq + i (K's A operand uses the
    // same map).
    bf16x8 qb[8];
    {
      const uint16_t* qp = a.q + ((int64_t)s * Hq + g * kGqa + (c16 < kGqa ? c16 : 0)) * kHeadDim + 8 * kq;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c16 < kGqa) v = load16(qp + 32 * t);
        qb[t] = as_bf16x8(v);
      }
    }
    // Softmax state of query head c16.  O^T and l are kept relative to the
    // reference m_run, which is re-based only when a score exceeds it by more
    // than kRescaleSlack (so weights stay <= 2^8); the final O / l is the same.
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[16];                            // O^T: head c16, d = 16*db + 4*kq + r
#pragma unroll
    for (int db = 0; db < 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t* kbase_g = a.k_cache + (int64_t)g * kHeadDim;
    const uint16_t* vbase_g = a.v_cache + (int64_t)g * kHeadDim;
    // Row geometry of local step u: first row kb (of this wave's 16) and the
    // page's live rows.
    auto geom = [&](int u, int& kb, int& page_len) {
      const int page = u / spp;
      page_len = min(B, L - page * B);
      kb = (u - page * spp) * stok + 16 * ks;
      return page;
    };
    // Issue one step: 8 + 8 direct-to-LDS loads of two rows (1 KB) each.
    // Rows past the page's live end reload the page's first row (finite;
    // masked out of the softmax).
    // Block-table entry of the page being loaded, re-read only when the
    // page changes (a scalar load).
    int cached_page = -1;
    int64_t cached_poff = 0;
    auto issue = [&](int u, char* st) {
      int kb, page_len;
      const int page = geom(u, kb, page_len);
      if (page != cached_page) {
        cached_page = page;
        cached_poff = (int64_t)load_const_i32(bt + page) * a.page_stride;
      }
      // Wave-uniform page bases and 32-bit per-lane byte offsets (a page of
      // one KV head's rows spans < 2^31 bytes).
      const int64_t poff = cached_poff;
      const char* kpage = reinterpret_cast<const char*>(kbase_g + poff);
      const char* vpage = reinterpret_cast<const char*>(vbase_g + poff);
      const uint32_t rs_bytes = (uint32_t)(row_stride * 2);
      const int pos = lane & 31;
      const int half = lane >> 5;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 2 * j + half;
        const int key = kb + row;
        const uint32_t roff = (uint32_t)(key < page_len ? key : 0) * rs_bytes;
        __builtin_amdgcn_global_load_lds(kpage + roff + ((pos ^ kswz(row)) << 4),
                                         (PA_LDS void*)(st + j * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vpage + roff + ((pos ^ vswz(row)) << 4),
                                         (PA_LDS void*)(st + kTileBytes + j * 1024), 16, 0, 0);
      }
    };
    auto compute = [&](int u, const char* st) {
      int kb, page_len;
      geom(u, kb, page_len);
      // Operand reads from LDS, written as inline asm: the compiler's wait
      // insertion cannot tell which direct-to-LDS load wrote which bytes and
      // would otherwise drain every in-flight load (the prefetched step too)
      // before each read.  The explicit vmcnt wait before compute() orders
      // these reads after this step's loads; one lgkmcnt wait below, which
      // takes every result as an operand, orders their uses after the reads.
      const uint32_t st_lds = lds_addr(st);
      // K A-operand: row c16 (key), 16-byte chunk 4*t + kq at position
      // (4*t + kq) ^ (c16 & 7) = 8*(t >> 1) + (4*((t & 1) ^ (c16 >> 2 & 1)) + (kq ^ (c16 & 3))).
      const uint32_t kr = st_lds + c16 * kRowBytes;
      const uint32_t k_even = kr + ((((c16 >> 2) & 1) * 4 + (kq ^ (c16 & 3))) << 4);
      const uint32_t k_odd = kr + (((((c16 >> 2) & 1) ^ 1) * 4 + (kq ^ (c16 & 3))) << 4);
      u32x4 kv[8];
      PA_DS_READ_B128(kv[0], k_even, 0);
      PA_DS_READ_B128(kv[1], k_odd, 0);
      PA_DS_READ_B128(kv[2], k_even, 128);
      PA_DS_READ_B128(kv[3], k_odd, 128);
      PA_DS_READ_B128(kv[4], k_even, 256);
      PA_DS_READ_B128(kv[5], k_odd, 256);
      PA_DS_READ_B128(kv[6], k_even, 384);
      PA_DS_READ_B128(kv[7], k_odd, 384);
      // V^T operands.  Transposing read: lane (kq, c16) points at
      // V[4*kq + c16/4][16*db + 4*(c16%4)] and receives V[4*kq + e][16*db + c16],
      // e = 0..3: the A operand of V^T.  With the row swizzle the byte offset
      // is 32*((db & 3) ^ (vrow & 3)) + 128*(db >> 2) + 16*h1 + 8*h0.
      const int vrow = 4 * kq + (c16 >> 2);
      const uint32_t vr = st_lds + kTileBytes + vrow * kRowBytes + (((c16 & 3) >> 1) << 4) + (c16 & 1) * 8;
      const uint32_t v0 = vr + ((0 ^ (vrow & 3)) << 5);
      const uint32_t v1 = vr + ((1 ^ (vrow & 3)) << 5);
      const uint32_t v2 = vr + ((2 ^ (vrow & 3)) << 5);
      const uint32_t v3 = vr + ((3 ^ (vrow & 3)) << 5);
      u32x2 va[16];
      PA_DS_READ_TR16(va[0], v0, 0);    PA_DS_READ_TR16(va[1], v1, 0);
      PA_DS_READ_TR16(va[2], v2, 0);    PA_DS_READ_TR16(va[3], v3, 0);
      PA_DS_READ_TR16(va[4], v0, 128);  PA_DS_READ_TR16(va[5], v1, 128);
      PA_DS_READ_TR16(va[6], v2, 128);  PA_DS_READ_TR16(va[7], v3, 128);
      PA_DS_READ_TR16(va[8], v0, 256);  PA_DS_READ_TR16(va[9], v1, 256);
      PA_DS_READ_TR16(va[10], v2, 256); PA_DS_READ_TR16(va[11], v3, 256);
      PA_DS_READ_TR16(va[12], v0, 384); PA_DS_READ_TR16(va[13], v1, 384);
      PA_DS_READ_TR16(va[14], v2, 384); PA_DS_READ_TR16(va[15], v3, 384);
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(kv[0]), "+v"(kv[1]), "+v"(kv[2]), "+v"(kv[3]), "+v"(kv[4]), "+v"(kv[5]),
                     "+v"(kv[6]), "+v"(kv[7]), "+v"(va[0]), "+v"(va[1]), "+v"(va[2]), "+v"(va[3]),
                     "+v"(va[4]), "+v"(va[5]), "+v"(va[6]), "+v"(va[7]), "+v"(va[8]), "+v"(va[9]),
                     "+v"(va[10]), "+v"(va[11]), "+v"(va[12]), "+v"(va[13]), "+v"(va[14]),
                     "+v"(va[15]));
      // S^T = K Q^T as two independent MFMA chains over d.
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv[t]), qb[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv[t + 4]), qb[t + 4], s1, 0, 0, 0);
      }
      // lane: query head c16, keys kb + 4*kq + q4
      float sv[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        sv[q4] = (kb + 4 * kq + q4 < page_len) ? (s0[q4] + s1[q4]) * a.scale_log2 : -INFINITY;
      const float mx = pair32_max(pair16_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]))));
      if (__any(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
        for (int db = 0; db < 16; ++db) o[db] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float pr[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) pr[q4] = fast_exp2(sv[q4] - m_use);
      l_run += pair32_sum(pair16_sum((pr[0] + pr[1]) + (pr[2] + pr[3])));
      const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
#pragma unroll
      for (int db = 0; db < 16; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, va[db]), pb, o[db], 0, 0, 0);
    };

    // Two-stage pipeline, unrolled by two so stage addresses are static.
    char* stA = vbase;
    char* stB = vbase + kStageBytes;
    issue(la, stA);
    for (int u = la; u < lb; u += 2) {
      if (u + 1 < lb) {
        issue(u + 1, stB);
        PA_WAIT_VMCNT(16);   // step u has landed; step u + 1 may be in flight
      } else {
        PA_WAIT_VMCNT(0);
      }
      compute(u, stA);
        if (u + 1 >= lb) break;
      if (u + 2 < lb) {
        issue(u + 2, stA);
        PA_WAIT_VMCNT(16);
      } else {
        PA_WAIT_VMCNT(0);
      }
      compute(u + 1, stB);
    }

    // With fewer than 4 KV heads per item, waves of one head merge through
    // LDS (the stages are free now).
    if (ksl > 1) {
      __syncthreads();
      float* macc = reinterpret_cast<float*>(smem);                 // [4][6][256]
      float* mml = macc + kWaves * kGqa * kHeadDim;                 // [4][6][2]
      if (c16 < kGqa) {
#pragma unroll
        for (int db = 0; db < 16; ++db)
          *reinterpret_cast<f32x4*>(&macc[(w * kGqa + c16) * kHeadDim + 16 * db + 4 * kq]) = o[db];
        if (kq == 0) { mml[(w * kGqa + c16) * 2] = m_run; mml[(w * kGqa + c16) * 2 + 1] = l_run; }
      }
      __syncthreads();
      if (ks == 0 && c16 < kGqa) {
        float M = -INFINITY;
        for (int k2_ = 0; k2_ < ksl; ++k2_) M = fmaxf(M, mml[((w + k2_ * hpw) * kGqa + c16) * 2]);
        const float mu = M == -INFINITY ? 0.f : M;
        float Ls = 0.f;
#pragma unroll
        for (int db = 0; db < 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k2_ = 0; k2_ < ksl; ++k2_) {
          const int ww = w + k2_ * hpw;
          const float f = fast_exp2(mml[(ww * kGqa + c16) * 2] - mu);
          Ls += f * mml[(ww * kGqa + c16) * 2 + 1];
#pragma unroll
          for (int db = 0; db < 16; ++db)
            o[db] += f * *reinterpret_cast<const f32x4*>(&macc[(ww * kGqa + c16) * kHeadDim + 16 * db + 4 * kq]);
        }
        m_run = M;
        l_run = Ls;
      }
      __syncthreads();   // LDS is reused as stages by the next item
    }

    if (ks == 0 && c16 < kGqa) {
      if (nparts == 1) {
        const float inv = 1.f / l_run;
        uint16_t* op = a.out + ((int64_t)s * Hq + g * kGqa + c16) * kHeadDim + 4 * kq;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          const u32x2 v = {pack_bf16x2(o[db][0] * inv, o[db][1] * inv), pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
          *reinterpret_cast<u32x2*>(op + 16 * db) = v;
        }
      } else {
        const int64_t slot = (int64_t)item + wgi;
        float* pacc = a.p_acc + (slot * hpw + jw) * (kGqa * kHeadDim) + c16 * kHeadDim + 4 * kq;
#pragma unroll
        for (int db = 0; db < 16; ++db) *reinterpret_cast<f32x4*>(pacc + 16 * db) = o[db];
        if (kq == 0) {
          a.p_ml[(slot * hpw + jw) * (kGqa * 2) + 2 * c16] = m_run;
          a.p_ml[(slot * hpw + jw) * (kGqa * 2) + 2 * c16 + 1] = l_run;
        }
      }
    }
    if (tid == 0 && first_wg == wgi) {
      a.meta[2 * item] = (int32_t)first_wg;
      a.meta[2 * item + 1] = nparts;
    }
    x = item_start + lb;
    if (x == item_end && hg == ng - 1) { ++s_cur; seq_start = x; }
  }
}

// Merge of the partials: workgroup (query head h, 16-dim slice, sequence).
// Thread t: slice z = t / 16 takes partials z, z + 16, ...; dim d = t % 16.
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeArgs a) {
  __shared__ float red_o[kMergeSlices][kMergeDims];
  __shared__ float red_m[kMergeSlices];
  __shared__ float red_l[kMergeSlices];
  const int h = blockIdx.x / (kHeadDim / kMergeDims);
  const int dc = blockIdx.x % (kHeadDim / kMergeDims);
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  const int z = tid / kMergeDims;
  const int dd = tid % kMergeDims;
  const int d = dc * kMergeDims + dd;
  const int Hkv = a.num_kv_heads;
  const int hpw = a.heads_per_wg;
  const int g = h / kGqa;
  const int hh = h % kGqa;
  const int item = s * (Hkv / hpw) + g / hpw;
  const int jw = g % hpw;
  uint16_t* outp = a.out + ((int64_t)s * Hkv * kGqa + h) * kHeadDim + d;
  const int L = clamp_len(a.seq_lens[s], a.max_seq_len);
  if (L == 0) {
    if (z == 0) *outp = 0;
    return;
  }
  const int nparts = a.meta[2 * item + 1];
  if (nparts <= 1) return;                 // the split kernel wrote the output
  const int64_t slot0 = (int64_t)item + a.meta[2 * item];
  const float* ml = a.p_ml + (slot0 * hpw + jw) * (kGqa * 2) + 2 * hh;
  const float* acc = a.p_acc + (slot0 * hpw + jw) * (kGqa * kHeadDim) + hh * kHeadDim + d;
  const int64_t pstride = (int64_t)hpw;    // consecutive slots

  // One pass: each slice keeps its own running max.
  float M = -INFINITY, O = 0.f, Ls = 0.f;
#ifndef PA_MERGE_UNROLL
#define PA_MERGE_UNROLL 8
#endif
  constexpr int kUnroll = PA_MERGE_UNROLL;
  for (int p0 = z; p0 < nparts; p0 += kMergeSlices * kUnroll) {
    float mv[kUnroll], lv[kUnroll], av[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int p = p0 + k * kMergeSlices;
      const bool ok = p < nparts;
      mv[k] = ok ? ml[p * pstride * (kGqa * 2)] : -INFINITY;
      lv[k] = ok ? ml[p * pstride * (kGqa * 2) + 1] : 0.f;
      av[k] = ok ? acc[p * pstride * (kGqa * kHeadDim)] : 0.f;
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) mb = fmaxf(mb, mv[k]);
    const float mu = mb == -INFINITY ? 0.f : mb;
    const float r = fast_exp2(M - mu);
    O *= r;
    Ls *= r;
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const float f = fast_exp2(mv[k] - mu);
      Ls += f * lv[k];
      O += f * av[k];
    }
    M = mb;
  }
  red_o[z][dd] = O;
  if (dd == 0) { red_m[z] = M; red_l[z] = Ls; }
  __syncthreads();
  if (z == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int zz = 0; zz < kMergeSlices; ++zz) Mt = fmaxf(Mt, red_m[zz]);
    float Ot = 0.f, Lt = 0.f;
#pragma unroll
    for (int zz = 0; zz < kMergeSlices; ++zz) {
      const float f = fast_exp2(red_m[zz] - Mt);
      Ot += f * red_o[zz][dd];
      Lt += f * red_l[zz];
    }
    *outp = (uint16_t)f32_to_bf16_rne(Ot / Lt);
  }
}

int64_t live_steps_host(int64_t L, int32_t B, int32_t spp, int32_t step_tokens) {
  const int64_t last_page = (L - 1) / B;
  const int64_t rem = L - last_page * B;
  return last_page * spp + (rem + step_tokens - 1) / step_tokens;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

DecodePlan plan_decode(int32_t num_seqs, int32_t max_seq_len, int32_t block_size,
                       int32_t num_kv_heads) {
  DecodePlan p{};
#ifdef PA_DECODE_HPW
  p.heads_per_wg = PA_DECODE_HPW;
#else
  p.heads_per_wg = num_kv_heads % 4 == 0 ? 4 : (num_kv_heads % 2 == 0 ? 2 : 1);
#endif
  p.step_tokens = 16 * (kWaves / p.heads_per_wg);
  p.steps_per_page = (block_size + p.step_tokens - 1) / p.step_tokens;
  const int64_t items = (int64_t)num_seqs * (num_kv_heads / p.heads_per_wg);
  const int64_t steps_ub = items * live_steps_host(max_seq_len, block_size, p.steps_per_page,
                                                   p.step_tokens);
  // One split workgroup per CU (each holds 128 KB of LDS), never more
  // workgroups than steps.
  int64_t n = kDecodeWorkgroups;
  if (n > steps_ub) n = steps_ub;
  p.num_wgs = (int32_t)n;
  const size_t slots = (size_t)(items + n);
  size_t off = 0;
  p.meta_off = off;  off += align256((size_t)items * 2 * sizeof(int32_t));
  p.p_ml_off = off;  off += align256(slots * p.heads_per_wg * kGqa * 2 * sizeof(float));
  p.p_acc_off = off; off += align256(slots * p.heads_per_wg * kGqa * kHeadDim * sizeof(float));
  p.bytes = off;
  return p;
}

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, int64_t page_stride,
                         const int32_t* block_table, int32_t bt_stride,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                         int32_t block_size, float scale, int32_t num_kv_heads,
                         const DecodePlan& plan, void* workspace, hipStream_t stream) {
  DecodeArgs a;
  char* ws = static_cast<char*>(workspace);
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_stride = page_stride;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.max_seq_len = max_seq_len;
  a.block_size = block_size;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_kv_heads = num_kv_heads;
  a.heads_per_wg = plan.heads_per_wg;
  a.step_tokens = plan.step_tokens;
  a.steps_per_page = plan.steps_per_page;
  a.num_wgs = plan.num_wgs;
  a.meta = reinterpret_cast<int32_t*>(ws + plan.meta_off);
  a.p_ml = reinterpret_cast<float*>(ws + plan.p_ml_off);
  a.p_acc = reinterpret_cast<float*>(ws + plan.p_acc_off);
  hipLaunchKernelGGL(decode_split_kernel, dim3(plan.num_wgs), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(num_kv_heads * kGqa * (kHeadDim / kMergeDims), num_seqs),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
