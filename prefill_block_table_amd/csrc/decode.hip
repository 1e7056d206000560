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
//    - K and V rows go from HBM into registers with 16-byte loads (V's with
//      the streaming hint: each V load covers whole 128-byte lines read
//      once), three steps in flight per wave: each lane's K loads are exactly its
//      MFMA A operand (row = key, 8 consecutive dims), so K never touches
//      LDS; V rows pass through a wave-private LDS tile (16-byte chunks
//      XOR-swizzled by row, so the transposing reads below are bank-conflict
//      free).  Every load in flight is a register load, so the compiler's
//      waits on them are exact;
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
//    Each (item, workgroup) pair that shares work leaves one partial per KV
//    head: the running max m and sum l in fp32 and the normalised O / l in
//    bf16 (half the bytes of fp32 on both sides of the kernel boundary; one
//    more bf16 rounding than the single-workgroup path, whose O / l is the
//    output itself); an item done by a single workgroup writes bf16 output
//    directly.
// 2. decode_merge_kernel.  One workgroup per (sequence, query head, 32-dim
//    slice of a partial); its 256 threads load all (at most 256) partials of
//    the slice in one round, so every load of a workgroup is in flight at
//    once, then combine them with cross-lane shuffles.  The two slices that
//    share a 128-byte line run on one XCD, so each line is fetched once.  Merge order is fixed: results are bitwise repeatable, no
//    atomics anywhere.
// Nothing is read past a page's or a sequence's last live row (such rows are
// replaced by the page's first row, whose weight is exactly 0), so poisoned
// rows never reach the output.
#include <math.h>

#include <mutex>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

const char* const kDecodeVariant =
    "decode-v8(split+merge,balanced-steps,4heads-per-wg,16tok-steps,kv-in-registers,3-steps-in-flight,nt-v,bf16-partials,"
    "mfma16x16x32-qk,v-lds-transpose,tr16-vt,mfma16x16x16-pv,lazy-rescale,append)";

namespace {

constexpr int kWaves = 4;
constexpr int kStages = 3;                         // steps in flight per wave
constexpr int kRowBytes = kHeadDim * 2;            // one KV head's row: 512 B
constexpr int kTileBytes = 16 * kRowBytes;         // 16 V rows of one wave step: 8 KB
// LDS: one V tile per wave (the transpose buffer); the in-workgroup merge
// of waves sharing a KV head reuses it.
constexpr int kMergeLds = kWaves * kGqa * (kHeadDim + 2) * 4;
constexpr int kSmemBytes = kWaves * kTileBytes > kMergeLds ? kWaves * kTileBytes : kMergeLds;
constexpr float kRescaleSlack = 8.f;               // log2 headroom before re-basing O
#ifndef PA_MERGE_DIMS
#define PA_MERGE_DIMS 32
#endif
constexpr int kMergeDims = PA_MERGE_DIMS;          // dims per merge workgroup (32: 64 contiguous bytes of a bf16 partial)
constexpr int kMergeSlices = 1024 / kMergeDims;    // partials merged in parallel per dim
constexpr int kLineSlices = kMergeDims >= 64 ? 1 : 64 / kMergeDims;   // merge slices per 128 B line
constexpr int kMergeParts = 256 / kMergeSlices;    // partials per merge thread
static_assert(kDecodeWorkgroups <= kMergeSlices * kMergeParts, "one merge round covers all partials");

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define PA_LDS __attribute__((address_space(3)))


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
  uint16_t* p_acc;         // [slot][heads_per_wg][6][256] bf16 O / l, slot = item + workgroup
  float* p_ml;             // [slot][heads_per_wg][6][2]
  int32_t* meta;           // [item][2]: first workgroup, number of partials
  // Appended token (NULL k_new: plain decode).  Row [s][g] of k_new / v_new
  // is the token at position seq_lens[s] - 1; it is stored to that slot of
  // k_dst / v_dst (the same caches) and attended from the new rows.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_dst;
  uint16_t* v_dst;
  int64_t* slot_out;       // [num_seqs] or NULL
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
// bnd(w) = floor(w * T / N).  With T = q N + r, bnd(w) = w q + floor(w r / N);
// w, r <= N <= 256 and T < 2^31 (checked on the host), so this is 32-bit
// arithmetic.  The workgroup owning step x is floor(((x + 1) N - 1) / T).
__device__ __forceinline__ int wg_bound(int w, int q, int r, int N) { return w * q + (w * r) / N; }
__device__ __forceinline__ int wg_of(int x, int T, int N) {
  return (int)(((int64_t)(x + 1) * N - 1) / T);
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

// V rows in the LDS tile: chunk c at c ^ ((r & 3) << 1), so the 4 rows of a
// transposing read hit 4 different 32-byte bank groups.
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

template <int HPW>
__global__ void __launch_bounds__(256, 1) decode_split_kernel(DecodeArgs a) {
  constexpr int KSL = kWaves / HPW;      // waves sharing one KV head
  constexpr int STOK = 16 * KSL;         // tokens per step
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  __shared__ int red[2];
  __shared__ int scan_lds[2][kWaves];
  __shared__ int excl_lds[256];
  __shared__ int lens_lds[256];

  const int wgi = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index: uniform per wave, so head / slice indices and the cache page
  // bases derived from them live in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * kGqa;
  const int B = a.block_size;
  const int ng = Hkv / HPW;               // items per sequence
  const int jw = w % HPW;                 // this wave's KV head within the item
  const int ks = w / HPW;                 // this wave's 16-token slice of a step
  const int spp = a.steps_per_page;
  const int c16 = lane & 15;
  const int kq = lane >> 4;

  // Total steps T of the batch, this workgroup's range [x0, x1) and the
  // sequence holding step x0.  One sequence: one scalar load.  Otherwise one
  // read of seq_lens (thread t takes sequences t, t + 256, ...) and a block
  // scan give every sequence's first step; the lengths of the first 256
  // sequences stay in LDS for the item loop.
  int T = 0;
  int s_cur = 0;
  int seq_start = 0;    // flattened index of the first step of s_cur
  const bool single = a.num_seqs == 1;
  int L_single = 0, raw_single = 0;
  if (single) {
    raw_single = load_const_i32(a.seq_lens);
    L_single = clamp_len(raw_single, a.max_seq_len);
    T = live_steps(L_single, B, spp, STOK) * ng;
  } else {
    for (int c0 = 0; c0 < a.num_seqs; c0 += 256) {
      const int s = c0 + tid;
      const int L = s < a.num_seqs ? clamp_len(a.seq_lens[s], a.max_seq_len) : 0;
      if (c0 == 0) lens_lds[tid] = L;
      const int v = live_steps(L, B, spp, STOK) * ng;
      int incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      if (lane == 63) scan_lds[(c0 >> 8) & 1][w] = incl;
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const int t = scan_lds[(c0 >> 8) & 1][ww];
        before += ww < w ? t : 0;
        total += t;
      }
      excl_lds[tid] = T + before + incl - v;    // first step of sequence s
      T += total;
      if (c0 + 256 < a.num_seqs) __syncthreads();
    }
  }
  if (T == 0) return;
  // Effective workgroup count min(launched, T): every workgroup below it owns
  // at least one step, so the workgroups sharing an item are consecutive and
  // its partials occupy consecutive slots.
  const int N = T < a.num_wgs ? T : a.num_wgs;
  if (wgi >= N) return;
  const int tq = T / N, tr = T - tq * N;
  const int x0 = wg_bound(wgi, tq, tr, N);
  const int x1 = wg_bound(wgi + 1, tq, tr, N);
  if (x0 >= x1) return;
  if (single) {
    // s_cur = 0, seq_start = 0
  } else if (a.num_seqs <= 256) {
    // sequence s holds x0 iff excl[s] <= x0 < excl[s] + steps(s) (exactly
    // one s: empty sequences have empty ranges)
    __syncthreads();
    const int s = tid;
    const int lo = excl_lds[s];
    const int hi = lo + live_steps(lens_lds[s], B, spp, STOK) * ng;
    if (s < a.num_seqs && lo <= x0 && x0 < hi) { red[0] = s; red[1] = lo; }
    __syncthreads();
    s_cur = __builtin_amdgcn_readfirstlane(red[0]);
    seq_start = __builtin_amdgcn_readfirstlane(red[1]);
  } else {
    // larger batches: a second pass locates x0
    for (int c0 = 0; c0 < a.num_seqs; c0 += 256) {
      const int s = c0 + tid;
      const int v = s < a.num_seqs
          ? live_steps(clamp_len(a.seq_lens[s], a.max_seq_len), B, spp, STOK) * ng : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      __syncthreads();
      if (lane == 63) scan_lds[0][w] = incl;
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        before += ww < w ? scan_lds[0][ww] : 0;
        total += scan_lds[0][ww];
      }
      const int lo = seq_start + before + incl - v;
      const int hi = seq_start + before + incl;
      const bool found = x0 < seq_start + total;
      if (found) {
        if (s < a.num_seqs && lo <= x0 && x0 < hi) { red[0] = s; red[1] = lo; }
        __syncthreads();
        s_cur = __builtin_amdgcn_readfirstlane(red[0]);
        seq_start = __builtin_amdgcn_readfirstlane(red[1]);
        break;
      }
      seq_start += total;
    }
  }

  // ---- per-lane constants, computed once ----
  const uint32_t rs_bytes = (uint32_t)Hkv * kRowBytes;   // bytes per cache row (token)
  const int64_t page_bytes = a.page_stride * 2;
  // Direct-to-LDS load j of a step moves rows 2j (lanes 0..31) and 2j + 1
  // (lanes 32..63) of this wave's 16; lane offset from the step's first row.
  // K rows: 16-byte chunk c of row r lands at position c ^ (r & 7); V rows at
  // c ^ ((r & 3) << 1) (bank-conflict-free operand reads, see compute).
  const int pos = lane & 31;
  const int half = lane >> 5;
  // V rows 2*jj + half, chunk pos: source offset within the step (plus
  // 2*jj rows), and LDS position of the chunk (row-swizzled, see vswz).
  const uint32_t v_lane_src = (uint32_t)half * rs_bytes + 16u * pos;
  // This wave's V tile (LDS transpose buffer).
  char* vt0 = smem + w * kTileBytes;
  // K A-operand of operand step t: row c16 (key) of the step, 16-byte chunk
  // 4*t + kq (d = 32*t + 8*kq .. +7): loaded from HBM straight into the
  // registers that feed the MFMA.
  const uint32_t k_lane = (uint32_t)c16 * rs_bytes + 16u * kq;
  // V^T operands.  Transposing read: lane (kq, c16) points at
  // V[4*kq + c16/4][16*db + 4*(c16%4)] and receives V[4*kq + e][16*db + c16],
  // e = 0..3: the A operand of V^T.  With the row swizzle the byte offset
  // is 32*((db & 3) ^ (vrow & 3)) + 128*(db >> 2) + 16*h1 + 8*h0.
  const int vrow = 4 * kq + (c16 >> 2);
  const uint32_t vr = lds_addr(vt0) + vrow * kRowBytes + (((c16 & 3) >> 1) << 4) + (c16 & 1) * 8;
  const uint32_t v0 = vr + ((0 ^ (vrow & 3)) << 5);
  const uint32_t v1 = vr + ((1 ^ (vrow & 3)) << 5);
  const uint32_t v2 = vr + ((2 ^ (vrow & 3)) << 5);
  const uint32_t v3 = vr + ((3 ^ (vrow & 3)) << 5);
  // Query head of this lane's S^T column: lanes 6..15 of each 16 repeat
  // heads 0..3 / 0..5 (valid data, results discarded), so no lane is masked.
  const int qh = c16 % kGqa;

  // Walk the items (s, hg) overlapping [x0, x1).
  int x = x0;
  while (x < x1) {
    const int s = __builtin_amdgcn_readfirstlane(s_cur);
    const int L = single ? L_single : __builtin_amdgcn_readfirstlane(
        s < 256 ? lens_lds[s] : clamp_len(a.seq_lens[s], a.max_seq_len));
    const int steps = live_steps(L, B, spp, STOK);
    if (steps == 0) { ++s_cur; continue; }
    const int hg = ng == 1 ? 0 : (x - seq_start) / steps;
    const int item_start = seq_start + hg * steps;
    const int item_end = item_start + steps;
    const int la = x - item_start;
    const int lb = (x1 < item_end ? x1 : item_end) - item_start;
    const int item = s * ng + hg;
    const int g = hg * HPW + jw;
    const int32_t* bt = a.block_table + (int64_t)s * a.bt_stride;
    const int last_page = (L - 1) / B;
    const char* kcache = reinterpret_cast<const char*>(a.k_cache + (int64_t)g * kHeadDim);
    const char* vcache = reinterpret_cast<const char*>(a.v_cache + (int64_t)g * kHeadDim);
    // Appending (pa_decode_append): the step holding the new token takes its
    // K/V rows straight from k_new / v_new (see issue); the workgroup that
    // owns the item's last step also stores them to the cache (after its
    // loop).  Nothing else in the launch reads that cache row.  A sequence
    // whose length is above max_seq_len attends its first max_seq_len cached
    // rows as they are (no fresh row among them) and stores the new token at
    // position seq_lens - 1, past every row the launch reads, as the
    // separate slot-mapping write would.
    const bool append = a.k_new != nullptr;
    const int raw = !append ? L : (single ? raw_single : __builtin_amdgcn_readfirstlane(load_const_i32(a.seq_lens + s)));
    const bool fresh_ok = append && raw <= a.max_seq_len;
    const char* knew = append ? reinterpret_cast<const char*>(a.k_new + ((int64_t)s * Hkv + g) * kHeadDim) : nullptr;
    const char* vnew = append ? reinterpret_cast<const char*>(a.v_new + ((int64_t)s * Hkv + g) * kHeadDim) : nullptr;
    const bool append_store = append && lb == steps && ks == 0;

    // Q^T as the B operand of S^T = K Q^T (16x16x32): lane supplies column
    // n = c16 and k = 8*kq + i of operand step t, mapped to d = 32*t + 8*kq + i
    // (K's A operand uses the same map).
    bf16x8 qb[8];
    {
      const uint16_t* qp = a.q + ((int64_t)s * Hq + g * kGqa + qh) * kHeadDim + 8 * kq;
#pragma unroll
      for (int t = 0; t < 8; ++t) qb[t] = as_bf16x8(load16(qp + 32 * t));
    }
    u32x2 knew_v = {0u, 0u}, vnew_v = {0u, 0u};
    if (append_store) {
      knew_v = *reinterpret_cast<const u32x2*>(knew + 8 * lane);
      vnew_v = *reinterpret_cast<const u32x2*>(vnew + 8 * lane);
    }

    // Issue cursor: logical page ip and step isp inside it; the block-table
    // entry is read (a scalar load) when a step of a new page is issued.
    const int page0 = la / spp;
    int ip = page0;
    int isp = la - page0 * spp;
    int ip_loaded = -1;
    int64_t ip_base = 0;
    // K and V of the steps in flight: kreg[slot][t] / vreg[slot][jj], slot =
    // step % kStages (relative to la).  All of them are plain loads into
    // registers, so the compiler's own waits on them are exact.
    u32x4 kreg[kStages][8];
    u32x4 vreg[kStages][8];
    // Step issue into slot j: the 16 K rows of this wave go to kreg[j] (lane
    // (kq, c16) takes 16 bytes of row c16 per operand step: the MFMA A
    // operand as it is); the 16 V rows to vreg[j] (lane (half, pos) takes
    // 16-byte chunk pos of rows 2*jj + half).  V is read with streaming
    // (non-temporal) loads, whole 512-byte rows per instruction; K with plain
    // loads, since each K load covers only half of a 128-byte line and the
    // next operand step reads the other half from L2 (streaming K loads were
    // measured slower at 8K).
    auto issue = [&](const int j) __attribute__((always_inline)) {
      if (ip != ip_loaded) {
        ip_loaded = ip;
        ip_base = (int64_t)load_const_i32(bt + ip) * page_bytes;
      }
      const int kb = isp * STOK + 16 * ks;          // first row of this wave's 16
      const int page_len = min(B, L - ip * B);      // live rows of the page
      // rows up to lim - 1 come from the cache as they are; the rest are
      // masked rows (or, when appending, the new token's row and after)
      const int lim = (fresh_ok && ip == last_page) ? page_len - 1 : page_len;
      if (kb + 16 <= lim) {
        const char* kp = kcache + ip_base + (uint32_t)kb * rs_bytes + k_lane;
        const char* vp = vcache + ip_base + (uint32_t)kb * rs_bytes + v_lane_src;
#pragma unroll
        for (int t = 0; t < 8; ++t) kreg[j][t] = *reinterpret_cast<const u32x4*>(kp + 64 * t);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) vreg[j][jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + 2 * jj * rs_bytes));
      } else {
        // Tail step: rows at or past lim reload the page's first row
        // (finite; masked out of the softmax) or, when appending, take
        // k_new / v_new.
        {
          const int key = kb + c16;
          const bool fresh = key >= lim && fresh_ok && ip == last_page;
          const char* kp = fresh ? knew + 16 * kq
                                 : kcache + ip_base + (uint32_t)(key < lim ? key : 0) * rs_bytes + 16 * kq;
#pragma unroll
          for (int t = 0; t < 8; ++t) kreg[j][t] = *reinterpret_cast<const u32x4*>(kp + 64 * t);
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int key = kb + 2 * jj + half;
          const bool fresh = key >= lim && fresh_ok && ip == last_page;
          const char* vp = fresh ? vnew + 16 * pos
                                 : vcache + ip_base + (uint32_t)(key < lim ? key : 0) * rs_bytes + 16 * pos;
          vreg[j][jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp));
        }
      }
      if (++isp == spp) { isp = 0; ++ip; }
    };
    const int nsteps = lb - la;
    // With at least 2 * kStages steps the first kStages go out
    // unconditionally on the path that leads to the steady loop, so the
    // compiler's count of memory operations issued after each K load is
    // the same on entry and around the loop (no full drain per round).
    const bool deep = nsteps >= 2 * kStages;

    // Softmax state of query head c16.  O^T and l are kept relative to the
    // reference m_run, which is re-based only when a score exceeds it by more
    // than kRescaleSlack (so weights stay <= 2^8); the final O / l is the same.
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[16];                            // O^T: head c16, d = 16*db + 4*kq + r
#pragma unroll
    for (int db = 0; db < 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Compute cursor (same walk as the issue cursor, one or two steps behind).
    int cp = page0;
    int csp = la - page0 * spp;
    auto compute = [&](const int j) __attribute__((always_inline)) {
      const int kb = csp * STOK + 16 * ks;
      // V rows into this wave's LDS tile, chunk c of row r at c ^ vswz(r).
      // The previous step's reads of the tile have completed (lgkmcnt(0)
      // below), and one wave's LDS operations run in order.
      {
        const int ln = __lane_id(), ps = ln & 31, hf = ln >> 5;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int row = 2 * jj + hf;
          *reinterpret_cast<u32x4*>(vt0 + row * kRowBytes + ((ps ^ vswz(row)) << 4)) = vreg[j][jj];
        }
        // the writes land before the transposing reads below (which the
        // compiler does not see as memory accesses)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      const int page_len = min(B, L - cp * B);
      if (++csp == spp) { csp = 0; ++cp; }
      // V^T operand reads (transposing) as inline asm; one lgkmcnt wait
      // below, which takes every result as an operand, orders their uses
      // after the reads.
      const uint32_t w0 = v0, w1 = v1, w2 = v2, w3 = v3;
      u32x2 va[16];
      PA_DS_READ_TR16(va[0], w0, 0);    PA_DS_READ_TR16(va[1], w1, 0);
      PA_DS_READ_TR16(va[2], w2, 0);    PA_DS_READ_TR16(va[3], w3, 0);
      PA_DS_READ_TR16(va[4], w0, 128);  PA_DS_READ_TR16(va[5], w1, 128);
      PA_DS_READ_TR16(va[6], w2, 128);  PA_DS_READ_TR16(va[7], w3, 128);
      PA_DS_READ_TR16(va[8], w0, 256);  PA_DS_READ_TR16(va[9], w1, 256);
      PA_DS_READ_TR16(va[10], w2, 256); PA_DS_READ_TR16(va[11], w3, 256);
      PA_DS_READ_TR16(va[12], w0, 384); PA_DS_READ_TR16(va[13], w1, 384);
      PA_DS_READ_TR16(va[14], w2, 384); PA_DS_READ_TR16(va[15], w3, 384);
      // (memory clobber: the next step's writes to the tile stay after the reads)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(va[0]), "+v"(va[1]), "+v"(va[2]), "+v"(va[3]), "+v"(va[4]), "+v"(va[5]),
                     "+v"(va[6]), "+v"(va[7]), "+v"(va[8]), "+v"(va[9]), "+v"(va[10]), "+v"(va[11]),
                     "+v"(va[12]), "+v"(va[13]), "+v"(va[14]), "+v"(va[15])
                   :
                   : "memory");
      const u32x4* kv = kreg[j];
      // S^T = K Q^T as two independent MFMA chains over d.
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv[t]), qb[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv[t + 4]), qb[t + 4], s1, 0, 0, 0);
      }
      // lane: query head c16, keys kb + 4*kq + q4; rows past the page's live
      // end (only in a page's last step) are masked
      float sv[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) sv[q4] = (s0[q4] + s1[q4]) * a.scale_log2;
      if (kb + 16 > page_len) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          if (kb + 4 * kq + q4 >= page_len) sv[q4] = -INFINITY;
      }
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

    // kStages-deep pipeline.  Before step i (relative to la) is computed,
    // steps up to i + kStages - 1 have been issued; after it, step
    // i + kStages goes into the slot it frees.  The steady loop always has
    // kStages steps in flight (its issue is unconditional); the remaining
    // steps are computed after it.  The waits for each step's registers are
    // the compiler's (exact: every load in flight is a plain register load).
    int i0 = 0;
    if (deep) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) issue(j);
      for (; i0 + 2 * kStages <= nsteps; i0 += kStages) {
#pragma unroll
        for (int j = 0; j < kStages; ++j) {
          compute(j);
          issue(j);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kStages; ++j)
        if (j < nsteps) issue(j);
    }
#pragma unroll
    for (int j = 0; j < 2 * kStages - 1; ++j) {
      const int i = i0 + j;
      if (i >= nsteps) break;
      compute(j % kStages);
      if (i + kStages < nsteps) issue(j % kStages);
    }
    if (append_store) {
      // position of the new token and its logical page; a page past the
      // table row gives slot -1 and no store (as the slot mapping defines)
      const int64_t pos_new = (int64_t)(fresh_ok ? L : raw) - 1;
      const int64_t lp = pos_new / B;
      if (lp < a.bt_stride) {
        const int64_t page_id = load_const_i32(bt + lp);
        const int64_t off = pos_new - lp * B;
        const int64_t dst = page_id * a.page_stride + off * Hkv * kHeadDim + (int64_t)g * kHeadDim + 4 * lane;
        *reinterpret_cast<u32x2*>(a.k_dst + dst) = knew_v;
        *reinterpret_cast<u32x2*>(a.v_dst + dst) = vnew_v;
        if (a.slot_out && jw == 0 && lane == 0) a.slot_out[s] = page_id * B + off;
      } else if (a.slot_out && jw == 0 && lane == 0) {
        a.slot_out[s] = -1;
      }
    }
    // Partial slots of this item: its workgroups are consecutive; only the
    // workgroup's first item can have started in an earlier workgroup and
    // only its last can continue in a later one.
    const int first_wg = item_start >= x0 ? wgi : (item_start == 0 ? 0 : wg_of(item_start, T, N));
    const int last_wg = item_end <= x1 ? wgi : (item_end == T ? N - 1 : wg_of(item_end - 1, T, N));
    const int nparts = last_wg - first_wg + 1;

    // With fewer than 4 KV heads per item, waves of one head merge through
    // LDS (the stages are free now).
    if (KSL > 1) {
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
#pragma unroll
        for (int k2 = 0; k2 < KSL; ++k2) M = fmaxf(M, mml[((w + k2 * HPW) * kGqa + c16) * 2]);
        const float mu = M == -INFINITY ? 0.f : M;
        float Ls = 0.f;
#pragma unroll
        for (int db = 0; db < 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k2 = 0; k2 < KSL; ++k2) {
          const int ww = w + k2 * HPW;
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
        const float inv = 1.f / l_run;
        uint16_t* pacc = a.p_acc + (slot * HPW + jw) * (kGqa * kHeadDim) + c16 * kHeadDim + 4 * kq;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          const u32x2 v = {pack_bf16x2(o[db][0] * inv, o[db][1] * inv), pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
          *reinterpret_cast<u32x2*>(pacc + 16 * db) = v;
        }
        if (kq == 0)
          *reinterpret_cast<f32x2*>(a.p_ml + (slot * HPW + jw) * (kGqa * 2) + 2 * c16) = f32x2{m_run, l_run};
      }
    }
    if (tid == 0 && first_wg == wgi) {
      a.meta[2 * item] = first_wg;
      a.meta[2 * item + 1] = nparts;
    }
    x = item_start + lb;
    if (x == item_end && hg == ng - 1) { ++s_cur; seq_start = x; }
  }
}

// Merge of the partials: workgroup (query head h, kMergeDims-dim slice,
// sequence).  Thread t: slice z = t / (kMergeDims / 4) takes partials z,
// z + kMergeSlices, ...; it reads dims 4*(t % (kMergeDims / 4)) .. +3 of the
// slice, so with 32 dims eight threads read one partial slice (64 bytes of bf16).
// (Measured: 32 dims per workgroup beats 16 and 8.)
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float red_o[4][kMergeDims];
  __shared__ float red_m[4];
  __shared__ float red_l[4];
  // One workgroup per slice dc0 of query head h (kNdc = 1 slice each).
  // Workgroups go round-robin to the 8 XCDs (id % 8) and each XCD has its own
  // L2, so the kLineSlices slices that share a 128-byte line of a partial are
  // given ids with the same id % 8: each line is then fetched by one L2.
  // gridDim.x = Hq * kHeadDim / kMergeDims is a multiple of 8 * kLineSlices.
  constexpr int kNdc = 1;
  int h, dc0;
  {
    const int xcd = blockIdx.x % 8;
    const int q8 = blockIdx.x / 8;
    const int slice = (q8 / kLineSlices * 8 + xcd) * kLineSlices + q8 % kLineSlices;
    h = slice / (kHeadDim / kMergeDims);
    dc0 = slice % (kHeadDim / kMergeDims);
  }
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  const int z = tid / (kMergeDims / 4);
  const int dg = tid % (kMergeDims / 4);
  const int Hkv = a.num_kv_heads;
  const int hpw = a.heads_per_wg;
  const int g = h / kGqa;
  const int hh = h % kGqa;
  const int item = s * (Hkv / hpw) + g / hpw;
  const int jw = g % hpw;
  uint16_t* outh = a.out + ((int64_t)s * Hkv * kGqa + h) * kHeadDim + 4 * dg;
  // A workgroup leaves at most one partial per item and there are at most
  // kDecodeWorkgroups of them, so one round of kMergeParts loads per thread
  // covers every partial.  The partials of item i sit at slots
  // i + first .. i + first + nparts - 1, where (first, nparts) come from the
  // split kernel's meta; first is 0 for the batch's first item (every item of
  // a single-sequence batch with <= 4 KV heads), so for one sequence those
  // loads are issued together with the meta load, assuming first = 0, and
  // re-issued only when meta says otherwise.  Every slot below items +
  // num_wgs is allocated, so the guessed loads stay in bounds.  (Batches of
  // several sequences go to decode_merge_wide_kernel; should one come here,
  // meta is read first.)
  constexpr int kParts = kMergeParts;
  const int64_t pml = (int64_t)hpw * (kGqa * 2);          // stride between consecutive slots
  const int64_t pacc = (int64_t)hpw * (kGqa * kHeadDim);
  f32x2 mlv[kParts];
  u32x2 av[kParts];
  auto load_parts = [&](int64_t slot0, int count, int d) {
    const float* ml = a.p_ml + (slot0 * hpw + jw) * (kGqa * 2) + 2 * hh;
    const uint16_t* acc = a.p_acc + (slot0 * hpw + jw) * (kGqa * kHeadDim) + hh * kHeadDim + d;
#pragma unroll
    for (int k = 0; k < kParts; ++k) {
      const int p = z + k * kMergeSlices;
      const bool ok = p < count;
      mlv[k] = ok ? *reinterpret_cast<const f32x2*>(ml + p * pml) : f32x2{-INFINITY, 0.f};
      av[k] = ok ? *reinterpret_cast<const u32x2*>(acc + p * pacc) : u32x2{0u, 0u};
    }
  };
  const bool guess = a.num_seqs == 1;
  if (guess) load_parts(item, a.num_wgs, dc0 * kMergeDims + 4 * dg);
  // meta of an empty sequence is stale and unused
  const int first = a.meta[2 * item];
  const int nparts = a.meta[2 * item + 1];
  const int L = clamp_len(a.seq_lens[s], a.max_seq_len);
  if (L == 0) {
    if (z == 0)
      for (int i = 0; i < kNdc; ++i) *reinterpret_cast<u32x2*>(outh + (dc0 + i) * kMergeDims) = u32x2{0u, 0u};
    return;
  }
  if (nparts <= 1) return;                 // the split kernel wrote the output
#pragma unroll 1
  for (int i = 0; i < kNdc; ++i) {
  const int dc = dc0 + i;
  uint16_t* outp = outh + dc * kMergeDims;
  if (!guess || first != 0 || dc != dc0) load_parts((int64_t)item + first, nparts, dc * kMergeDims + 4 * dg);
#pragma unroll
  for (int k = 0; k < kParts; ++k) {
    if (z + k * kMergeSlices >= nparts) { mlv[k] = f32x2{-INFINITY, 0.f}; av[k] = u32x2{0u, 0u}; }
  }
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kParts; ++k) M = fmaxf(M, mlv[k][0]);
  const float mu = M == -INFINITY ? 0.f : M;
  float Ls = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kParts; ++k) {
    const float f = fast_exp2(mlv[k][0] - mu) * mlv[k][1];
    Ls += f;
    O += f * f32x4{bf16_lo(av[k][0]), bf16_hi(av[k][0]), bf16_lo(av[k][1]), bf16_hi(av[k][1])};
  }
  // Combine the kMergeSlices slices: within a wave over the lane bits above
  // the dim group, then the four waves' results through LDS.
  auto combine = [&](float M2, float L2, f32x4 O2) {
    const float Mn = fmaxf(M, M2);
    const float mu = Mn == -INFINITY ? 0.f : Mn;
    const float f1 = fast_exp2(M - mu), f2 = fast_exp2(M2 - mu);
    Ls = f1 * Ls + f2 * L2;
    O = f1 * O + f2 * O2;
    M = Mn;
  };
#pragma unroll
  for (int off = kMergeDims / 4; off < 64; off <<= 1) {
    f32x4 O2;
#pragma unroll
    for (int r = 0; r < 4; ++r) O2[r] = __shfl_xor(O[r], off);
    const float M2 = __shfl_xor(M, off);
    const float L2 = __shfl_xor(Ls, off);
    combine(M2, L2, O2);
  }
  const int wv = tid >> 6;
  if ((tid & 63) < kMergeDims / 4) {
    *reinterpret_cast<f32x4*>(&red_o[wv][4 * dg]) = O;
    if (dg == 0) { red_m[wv] = M; red_l[wv] = Ls; }
  }
  __syncthreads();
  if (tid < kMergeDims / 4) {
#pragma unroll
    for (int ww = 1; ww < 4; ++ww)
      combine(red_m[ww], red_l[ww], *reinterpret_cast<const f32x4*>(&red_o[ww][4 * dg]));
    const float inv = 1.f / Ls;
    *reinterpret_cast<u32x2*>(outp) = u32x2{pack_bf16x2(O[0] * inv, O[1] * inv),
                                             pack_bf16x2(O[2] * inv, O[3] * inv)};
  }
  if (i + 1 < kNdc) __syncthreads();   // red_o is rewritten by the next slice
  }
}

// Merge for batches of several sequences: one workgroup per (query head,
// sequence) covers all 256 dims at once (lane l: dims 4l .. 4l+3), and wave w
// takes partials w, w + 4, ... of the item, four at a time, with an online
// re-basing of its running max.  Most items of a batch have one partial (the
// split kernel wrote their output) or a few, so a workgroup reads the item's
// meta and then needs at most one round of loads per wave; the per-slice
// kernel would give each of those items 8 workgroups with a round trip each.
// The four waves combine through LDS in a fixed order (bitwise repeatable).
__global__ void __launch_bounds__(256) decode_merge_wide_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float red_o[4][kHeadDim];
  __shared__ float red_m[4];
  __shared__ float red_l[4];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int Hkv = a.num_kv_heads;
  const int hpw = a.heads_per_wg;
  const int g = h / kGqa;
  const int hh = h % kGqa;
  const int item = s * (Hkv / hpw) + g / hpw;
  const int jw = g % hpw;
  const int d = 4 * lane;
  uint16_t* outp = a.out + ((int64_t)s * Hkv * kGqa + h) * kHeadDim + d;
  // meta of an empty sequence is stale and unused
  const int first = a.meta[2 * item];
  const int nparts = a.meta[2 * item + 1];
  const int L = clamp_len(a.seq_lens[s], a.max_seq_len);
  if (L == 0) {
    if (w == 0) *reinterpret_cast<u32x2*>(outp) = u32x2{0u, 0u};
    return;
  }
  if (nparts <= 1) return;                 // the split kernel wrote the output
  const int64_t slot0 = (int64_t)item + first;
  const int64_t pml = (int64_t)hpw * (kGqa * 2);          // stride between consecutive slots
  const int64_t pacc = (int64_t)hpw * (kGqa * kHeadDim);
  const float* ml = a.p_ml + (slot0 * hpw + jw) * (kGqa * 2) + 2 * hh;
  const uint16_t* acc = a.p_acc + (slot0 * hpw + jw) * (kGqa * kHeadDim) + hh * kHeadDim + d;
  float M = -INFINITY;
  float Ls = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = w; p0 < nparts; p0 += 16) {
    f32x2 mlv[4];
    u32x2 av[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = p0 + 4 * k;
      const bool ok = p < nparts;
      mlv[k] = ok ? *reinterpret_cast<const f32x2*>(ml + p * pml) : f32x2{-INFINITY, 0.f};
      av[k] = ok ? *reinterpret_cast<const u32x2*>(acc + p * pacc) : u32x2{0u, 0u};
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < 4; ++k) Mn = fmaxf(Mn, mlv[k][0]);
    const float base = Mn == -INFINITY ? 0.f : Mn;
    const float c = fast_exp2(M - base);   // 0 while nothing was added
    Ls *= c;
    O *= c;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float f = fast_exp2(mlv[k][0] - base) * mlv[k][1];
      Ls += f;
      O += f * f32x4{bf16_lo(av[k][0]), bf16_hi(av[k][0]), bf16_lo(av[k][1]), bf16_hi(av[k][1])};
    }
    M = Mn;
  }
  *reinterpret_cast<f32x4*>(&red_o[w][d]) = O;
  if (lane == 0) { red_m[w] = M; red_l[w] = Ls; }
  __syncthreads();
  if (w == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) Mt = fmaxf(Mt, red_m[ww]);
    const float mt = Mt == -INFINITY ? 0.f : Mt;
    float Lt = 0.f;
    f32x4 Ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = fast_exp2(red_m[ww] - mt);
      Lt += f * red_l[ww];
      Ot += f * *reinterpret_cast<const f32x4*>(&red_o[ww][d]);
    }
    const float inv = 1.f / Lt;
    *reinterpret_cast<u32x2*>(outp) = u32x2{pack_bf16x2(Ot[0] * inv, Ot[1] * inv),
                                             pack_bf16x2(Ot[2] * inv, Ot[3] * inv)};
  }
}

int64_t live_steps_host(int64_t L, int32_t B, int32_t spp, int32_t step_tokens) {
  const int64_t last_page = (L - 1) / B;
  const int64_t rem = L - last_page * B;
  return last_page * spp + (rem + step_tokens - 1) / step_tokens;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Workspace of pa_decode_noalloc, for callers that cannot allocate (code
// under HIP graph capture, serving loops that forbid hipMalloc).  In host
// code `scratch` names a host-side stand-in, not the device buffer: kernels
// only ever receive the address hipGetSymbolAddress returns for it.  Every
// call on one GPU shares the buffer; nothing in it needs to start at zero
// (each launch writes what it later reads).
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t decode_scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidValue;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

DecodePlan plan_decode(int32_t num_seqs, int32_t max_seq_len, int32_t block_size,
                       int32_t num_kv_heads) {
  DecodePlan p{};
  p.heads_per_wg = num_kv_heads % 4 == 0 ? 4 : (num_kv_heads % 2 == 0 ? 2 : 1);
  p.step_tokens = 16 * (kWaves / p.heads_per_wg);
  p.steps_per_page = (block_size + p.step_tokens - 1) / p.step_tokens;
  const int64_t items = (int64_t)num_seqs * (num_kv_heads / p.heads_per_wg);
  const int64_t steps_ub = items * live_steps_host(max_seq_len, block_size, p.steps_per_page,
                                                   p.step_tokens);
  // One split workgroup per CU (its four waves take ~450 registers each, one
  // wave per SIMD), never more workgroups than steps.
  int64_t n = kDecodeWorkgroups;
  if (n > steps_ub) n = steps_ub;
  p.num_wgs = (int32_t)n;
  p.steps_ub = steps_ub;
  const size_t slots = (size_t)(items + n);
  size_t off = 0;
  p.meta_off = off;  off += align256((size_t)items * 2 * sizeof(int32_t));
  p.p_ml_off = off;  off += align256(slots * p.heads_per_wg * kGqa * 2 * sizeof(float));
  p.p_acc_off = off; off += align256(slots * p.heads_per_wg * kGqa * kHeadDim * sizeof(uint16_t));
  p.bytes = off;
  return p;
}

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, int64_t page_stride,
                         const int32_t* block_table, int32_t bt_stride,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                         int32_t block_size, float scale, int32_t num_kv_heads,
                         const DecodePlan& plan, void* workspace, const DecodeAppend* append,
                         hipStream_t stream) {
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
  a.p_acc = reinterpret_cast<uint16_t*>(ws + plan.p_acc_off);
  a.k_new = append ? append->k_new : nullptr;
  a.v_new = append ? append->v_new : nullptr;
  a.k_dst = append ? append->k_cache : nullptr;
  a.v_dst = append ? append->v_cache : nullptr;
  a.slot_out = append ? append->slot_out : nullptr;
  switch (plan.heads_per_wg) {
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, dim3(plan.num_wgs), dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, dim3(plan.num_wgs), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(decode_split_kernel<1>, dim3(plan.num_wgs), dim3(256), 0, stream, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (num_seqs == 1)
    hipLaunchKernelGGL(decode_merge_kernel, dim3(num_kv_heads * kGqa * (kHeadDim / kMergeDims)), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(decode_merge_wide_kernel, dim3(num_kv_heads * kGqa, num_seqs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
