// Chunked-prefill paged GQA attention for gfx950 (bf16 MFMA, fp32 accumulate).
//
// What it computes ([ALIGN] §6): for the q_len query tokens of one chunk at
// positions start_pos + i, complete causal attention over the paged K/V of
// the first start_pos + q_len tokens; no key skipped that the causal mask
// allows, none added that it forbids ([ALIGN] §5, §9).
//
// Work decomposition (ours): a workgroup of 8 wave64s owns a 128-row query
// tile of one query head.  Waves w and w ^ 1 own the same 32 query rows; in
// every 64-token key group one takes keys 0..31 and the other keys 32..63,
// each with its own online soft-max, and the two halves are merged once at
// the end.  Each K or V operand read from LDS so feeds two MFMAs (two 16-row
// blocks), half the LDS traffic per flop of a 16-row wave.  Waves w and
// w + 4 share a SIMD; waves 4..7 run each group's PV one iteration late, so
// on every SIMD one wave's soft-max meets the other wave's MFMAs.  Keys
// stream through LDS in groups of 64 consecutive logical tokens, gathered
// through the block table row by row: a group lies in one page or, when the
// page size is not a multiple of 64 ([ALIGN] §2: 784 = 12 x 64 + 16), spans
// two, so only the context's last group is short (the pages' kernels mask a
// tail group in every such page instead; pages under 64 tokens make groups
// of one page).  Per group and wave, for row blocks rb = 0, 1:
//   S^T[32 keys x 16 rows] = K[32 x 256] Q_rb^T    (16 MFMA 16x16x32)
//   online softmax on S^T: each lane holds 8 scores of one query row, so
//   the row max and sum take two cross-lane swaps; the accumulator is
//   re-based only when the max grows by more than 2^8
//   O_rb^T[256 x 16 rows] += V^T[256 x 32] P_rb^T  (16 MFMA 16x16x32)
// The transposed orientation makes P^T's MFMA operand a register-local
// reinterpretation of S^T's accumulator (keys in the order the accumulator
// holds them; V^T's operand reads use the same order).  K and V rows go from
// HBM straight into LDS with the direct-to-LDS load (two K tiles and three V
// tiles: the next group is in flight while this one is computed), 16-byte chunks
// XOR-swizzled by row so operand reads are bank-conflict free; V^T operands
// come out of LDS with the gfx950 transposing read.  Groups entirely above
// the causal diagonal of the tile are never visited, a wave skips a key half
// that lies wholly above its rows, and the mask is evaluated only on groups
// that cross the diagonal or end the context.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

const char* const kPrefillVariant =
    "prefill-v11(bm128,8waves,pairs-32rows-keyhalves,adjacent-pairs,lean-softmax,bn64-logical-groups-span-pages,mfma16x16x32,st-orient,lds-dma-kv,2k3v-tiles,"
    "late-pv-on-waves4-7,prio-mfma-phases,"
    "tr16-vt,lazy-rescale,heavy-first,xcd-kvhead-map,hw-bf16-pack)";

namespace {

constexpr int kWavesPf = 8;
constexpr int kRowsPerWave = 32;                    // two 16-row MFMA blocks
constexpr int kBM = (kWavesPf / 2) * kRowsPerWave;  // 128 query rows per workgroup
constexpr int kHalfKeys = kGroup / 2;               // keys per wave per group
constexpr int kRowBytes = kHeadDim * 2;             // one KV head's row: 512 B
constexpr int kTileBytes = kGroup * kRowBytes;      // 64 rows: 32 KB
constexpr int kLoopBytes = 5 * kTileBytes;          // two K tiles, three V tiles: 160 KB
// End merge: every wave hands its partner the half of O^T the partner
// finishes (2 row blocks x 8 d-blocks x 64 lanes x 16 B) plus (m, l).
constexpr int kXoWaveBytes = 2 * 8 * 64 * 16;
constexpr int kMlOff = kWavesPf * kXoWaveBytes;
constexpr int kSmemBytes = kMlOff + kWavesPf * 2 * 64 * 8 > kLoopBytes ? kMlOff + kWavesPf * 2 * 64 * 8
                                                                       : kLoopBytes;
constexpr float kRescaleSlack = 8.f;
constexpr float kMinusHuge = -1e30f;

#define PA_LDS __attribute__((address_space(3)))
#define PA_WAIT_VMCNT(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")
// Workgroup barrier without a memory fence.  Every wave orders its own
// direct-to-LDS loads (vmcnt) and LDS operand reads (lgkmcnt) with explicit
// waits before it arrives; a fenced barrier would in addition wait for the
// next group's loads, which may be in flight, and so serialize the prefetch
// with the compute it is meant to overlap.
#define PA_BARRIER() __builtin_amdgcn_s_barrier()

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
  float scale_log2;        // scale * log2(e) (> 0)
  float inv_scale_log2;    // its reciprocal
  int32_t num_kv_heads;
  int32_t num_q_tiles;
  // Work split (see plan_prefill): items 0 .. num_full-1 (heavy first) get
  // one workgroup each; each later item is cut into `split` contiguous key
  // ranges whose partial results go to part_o / part_ml.
  int32_t num_full;
  int32_t split;
  uint16_t* part_o;        // [slot][128 rows][256] bf16 O / l, slot = (item - num_full) * split + part
  float* part_ml;          // [slot][128 rows][2]: row max (log2 units), row sum
  // Several sequences (pa_prefill_varlen; NULL cu_seqlens_q: one sequence,
  // q_len / start_pos / block_table above): sequence s has query rows
  // cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 and seqused_k[s] keys, its block-table
  // row at block_table + s * bt_stride.  Each tile slot is 6 * num_kv_heads
  // workgroups; the grid covers total_q / 128 + num_seqs slots, so its size
  // follows the rows actually batched rather than num_seqs times the longest
  // sequence.  Batches of up to 64 sequences give the slots to the sequences
  // heaviest (most keys) first; larger ones in input order (see the kernel's
  // prologue).
  const int32_t* cu_seqlens_q;
  const int32_t* seqused_k;
  int32_t num_seqs;
  int32_t bt_stride;
  int32_t total_q;         // rows of q / out
  int32_t max_q;           // host bounds the device lengths are clamped to
  int32_t max_k;
};

// Item (a query head's 128-row tile) of index J, heaviest (latest rows)
// first.  Consecutive workgroup ids go to the 8 XCDs in turn; when the KV
// heads divide the XCDs evenly, every XCD serves one KV head (8 / G XCDs per
// head, taking alternate entries of that head's heavy-first list), so the K/V
// a workgroup streams are the ones its XCD's L2 already holds for its
// neighbours.
__device__ __forceinline__ void map_item(int J, int G, int T, int& g, int& head, int& tile) {
  if (8 % G == 0 && (kGqa * G * T) % 8 == 0) {
    const int x = J & 7, slot = J >> 3;
    g = x % G;
    const int k = slot * (8 / G) + x / G;        // 0 .. 6T-1 within KV head g
    tile = T - 1 - k / kGqa;
    head = g * kGqa + k % kGqa;
  } else {
    const int Hq = G * kGqa;
    tile = T - 1 - J / Hq;
    head = J % Hq;
    g = head / kGqa;
  }
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const PA_LDS char*)p;
}

__device__ __forceinline__ int32_t load_const_i32(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Pair reductions across lanes l and l ^ 16 (or l ^ 32) with the gfx950
// lane-swap instructions (both lanes of a pair get the same bits).
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

// Plain v_max_f32 / v_max3_f32.  The scores are never NaN, so the operand
// quieting that fmaxf adds under IEEE mode (one extra instruction per
// input) is not needed.
// x.lo + x.hi (two bf16) + acc in fp32.
__device__ __forceinline__ float dot2_ones(uint32_t x, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), one, acc, false);
}
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// LDS rows are 512 bytes, so every row starts at the same bank.  16-byte
// chunk c of K row r sits at position c ^ (r & 15): the 16 rows one pass of
// an operand read touches (16 lanes x 16 B) land on 16 different 16-byte
// bank groups.  V row r: chunk c at c ^ ((r & 7) << 1): the 8 rows one pass
// of a transposing read touches (32 lanes, 8 rows x 32 B) land on 8
// different 32-byte bank groups.
__device__ __forceinline__ int kswz(int r) { return r & 15; }
__device__ __forceinline__ int vswz(int r) { return (r & 7) << 1; }

// Lane index read afresh at the point of use: values derived from it are
// recomputed (a few VALU ops) instead of being held in registers.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// LDS operand reads the compiler does not track (it cannot tell which
// direct-to-LDS load wrote which bytes and would drain the prefetched group
// before every read); callers order them with explicit waits.
#define PA_DS_READ_B128(dst, addr, off) \
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(off))
#define PA_DS_READ_TR16(dst, addr, off) \
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(off))

__global__ void __launch_bounds__(kWavesPf * 64, 1) prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];

  // Workgroup -> item (query head, query tile) and, for a split item, the
  // part of its key groups this workgroup takes.
  const int L = blockIdx.x;
  int item = L, part = -1;
  int32_t q_len = a.q_len, start_pos = a.start_pos;
  int T = a.num_q_tiles;                             // tiles of this workgroup's sequence
  const int32_t* bt = a.block_table;
  int64_t row0 = 0;                                  // first q / out row of the sequence
  if (a.cu_seqlens_q) {
    // Device offsets are clamped to [0, total_q] and lengths to the
    // host-checked bounds, so no load leaves q, out or a sequence's
    // block-table row.
    const int Hqs = a.num_kv_heads * kGqa;
    const int t = L / Hqs;                           // this workgroup's tile slot
    const int ln = threadIdx.x & 63;
    int sq = -1, p0 = 0;
    if (a.num_seqs <= 64) {
      // Up to 64 sequences: the slots go to the sequences in decreasing order
      // of their key count (the cost of their heaviest tile; ties by index),
      // each sequence's tiles together and heaviest first, so the last
      // workgroups dispatched hold the lightest tiles of the batch.  Lane i
      // takes sequence i; its rank and the slots of the sequences before it
      // are counted over the other lanes.
      int tl = 0, key = -1;
      if (ln < a.num_seqs) {
        const int c0 = min(max(a.cu_seqlens_q[ln], 0), a.total_q);
        const int c1 = min(max(a.cu_seqlens_q[ln + 1], 0), a.total_q);
        const int ql = min(c1 - c0, a.max_q);
        const int kvl = min(a.seqused_k[ln], a.max_k);
        if (ql > 0 && kvl - ql >= 0) { tl = (ql + kBM - 1) / kBM; key = kvl; }
      }
      int before = 0;                                // slots of the sequences ranked ahead
      for (int j = 0; j < a.num_seqs; ++j) {
        const int kj = __builtin_amdgcn_readlane(key, j);
        const int tj = __builtin_amdgcn_readlane(tl, j);
        if (kj > key || (kj == key && j < ln)) before += tj;
      }
      const uint64_t mine = __ballot(tl > 0 && t >= before && t < before + tl);
      if (mine == 0) return;                         // past the batch's last tile
      sq = __builtin_amdgcn_readfirstlane(__builtin_ctzll(mine));
      p0 = __builtin_amdgcn_readlane(before, sq);
    } else {
      // More sequences: input order.  Sequence s owns the slots from
      // P(s) = cu_seqlens_q[s] / 128 + s; the sequence of slot t is the
      // largest s with P(s) <= t, found as the count of such s in 0 ..
      // num_seqs (P is nondecreasing) with one vector load per 64 entries and
      // a ballot.  Offsets that decrease give slots that match no sequence,
      // and those workgroups leave.
      int cnt = 0;
      for (int base = 0; base <= a.num_seqs; base += 64) {
        const int i = base + ln;
        bool le = false;
        if (i <= a.num_seqs) {
          const int c = min(max(a.cu_seqlens_q[i], 0), a.total_q);
          le = c / kBM + i <= t;
        }
        cnt += __popcll(__ballot(le));
      }
      sq = __builtin_amdgcn_readfirstlane(cnt) - 1;
      if (sq < 0 || sq >= a.num_seqs) return;
    }
    const int c0 = min(max(load_const_i32(a.cu_seqlens_q + sq), 0), a.total_q);
    const int c1 = min(max(load_const_i32(a.cu_seqlens_q + sq + 1), 0), a.total_q);
    if (a.num_seqs > 64) {
      p0 = c0 / kBM + sq;
      if (t >= c1 / kBM + sq + 1) return;
    }
    q_len = min(c1 - c0, a.max_q);
    const int kv = min(load_const_i32(a.seqused_k + sq), a.max_k);
    start_pos = kv - q_len;                          // the chunk's rows end at the last key
    if (q_len <= 0 || start_pos < 0) return;
    T = (q_len + kBM - 1) / kBM;
    item = L - Hqs * p0;
    if (item >= Hqs * T) return;                     // the sequence's spare slot
    row0 = c0;
    bt = a.block_table + (int64_t)sq * a.bt_stride;
  } else if (L >= a.num_full) {
    const int qq = L - a.num_full;
    item = a.num_full + qq / a.split;
    part = qq % a.split;
  }
  int g, head, tile;
  map_item(item, a.num_kv_heads, T, g, head, tile);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index, uniform per wave: LDS destinations and row bases stay scalar
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = w & 1;         // key half of every group this wave takes
  const int c16 = lane & 15;     // this lane's query row within a 16-row block
  const int kq = lane >> 4;      // lane group: keys 4*kq .. 4*kq+3 of each 16-key block
  const int Hq = a.num_kv_heads * kGqa;
  const int64_t row_stride = (int64_t)a.num_kv_heads * kHeadDim;
  const int64_t q_stride = (int64_t)Hq * kHeadDim;
  const int B = a.block_size;
  const uint16_t* qbase = a.q + row0 * q_stride;
  uint16_t* obase = a.out + row0 * q_stride;

  const int q0 = tile * kBM;
  const int wrow0 = q0 + kRowsPerWave * (w >> 1);            // first query row of this wave
  const int wave_rows = max(0, min(kRowsPerWave, q_len - wrow0));
  const int wave_first_pos = start_pos + wrow0;
  const int wave_last_pos = wave_first_pos + wave_rows - 1;
  int my_row[2];
  bool row_ok[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    my_row[rb] = wrow0 + 16 * rb + c16;
    row_ok[rb] = my_row[rb] < q_len;
  }

  // Q^T as the B operand of S^T = K Q^T (16x16x32): lane supplies column
  // n = c16 (its query row) and k = 8*kq + i of d-step ds -> d = 32*ds + 8*kq + i.
  u32x4 qb[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const uint16_t* qp = qbase + (int64_t)(row_ok[rb] ? my_row[rb] : 0) * q_stride + head * kHeadDim + 8 * kq;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok[rb]) v = load16(qp + 32 * ds);
      qb[rb][ds] = v;
    }
  }

  const int kv_len = start_pos + q_len;
  const int tile_last = min(q0 + kBM, q_len) - 1;
  const int kv_end = a.causal ? start_pos + tile_last + 1 : kv_len;
  // Key groups are runs of GK = min(B, 64) consecutive logical keys: group u
  // holds keys GK*u .. GK*u + GK - 1 (the last one cut at kv_end).  With
  // pages of 64 tokens or more a group lies in one page or spans two (a page
  // of 784 = 12 x 64 + 16 tokens hands its last 16 rows and the next page's
  // first 48 to one group), so no group is a masked page tail.
  const int GK = B < kGroup ? B : kGroup;
  const int units = (kv_end + GK - 1) / GK;
  // this workgroup's key groups [ga, gb) of the tile
  const int ga = part < 0 ? 0 : (int)((int64_t)units * part / a.split);
  const int gb = part < 0 ? units : (int)((int64_t)units * (part + 1) / a.split);

  // O^T accumulators: row block rb, d-block db (16 d), register r -> d =
  // 16*db + 4*kq + r of query row 16*rb + c16.
  f32x4 o[16][2];
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Reference the accumulator is scaled to (log2 units).  It starts at a
  // finite sentinel far below any score, so -m_run is always a usable
  // exponent offset: the first live score re-bases it, and masked scores
  // (-inf) give exp2(-inf) = 0 whatever it is.
  float m_run[2] = {kMinusHuge, kMinusHuge};
  float l_run[2] = {0.f, 0.f};               // this lane's partial row sums (8 keys per group)

  const char* kbase_g = reinterpret_cast<const char*>(a.k_cache + (int64_t)g * kHeadDim);
  const char* vbase_g = reinterpret_cast<const char*>(a.v_cache + (int64_t)g * kHeadDim);
  const uint32_t rs_bytes = (uint32_t)(row_stride * 2);
  const int64_t page_bytes = a.page_stride * 2;
  // Per-lane parts of the load source offsets.  Lane (half, pos) loads
  // 16-byte chunk pos of row 8w + 2j + half; the K swizzle (row & 15) is
  // 8*(w & 1) | 2j | half and the V swizzle ((row & 7) << 1) is 4j | 2*half,
  // so chunk positions are a per-lane base XOR a per-j constant.  Row
  // strides are multiples of 512 bytes, clear of the chunk bits.
  // (All per-lane values here are derived from a fresh lane index inside
  // issue() so that none is held in a register across the loop.)

  // Issue cursor: group iu.  The block-table entries of the (at most two)
  // pages a group touches are scalar loads, kept for the next group (whose
  // first page is this group's last).
  int iu = ga;
  int pa_idx = -1, pb_idx = -1;
  int64_t pa_base = 0, pb_base = 0;
  // Position of group iu: page ipg, row ioff there (advanced by GK per group;
  // GK <= B, so a step crosses at most one page boundary).
  int ipg = (ga * GK) / B;
  int ioff = ga * GK - ipg * B;
  // This wave's share of the next group: rows 8w .. 8w+7 of K (into K tile
  // kst) and of V (into V tile vst), four direct-to-LDS loads each (rows
  // 8w + 2j on lanes 0..31, 8w + 2j + 1 on lanes 32..63).  Rows past the
  // group's live end reload its first row (finite; masked out of the softmax).
  auto issue = [&](char* kst, char* vst) {
    const int key0 = iu * GK;
    const int live = min(GK, kv_end - key0);
    const int pg = ipg;                            // first page of the group
    const int off = ioff;                          // its first row there
    const int na = min(live, B - off);             // rows in that page; the rest in page pg + 1
    ioff += GK;
    if (ioff >= B) { ioff -= B; ++ipg; }
    if (pg != pa_idx) {
      if (pg == pb_idx) {
        pa_base = pb_base;
      } else {
        pa_base = (int64_t)load_const_i32(bt + pg) * page_bytes;
      }
      pa_idx = pg;
    }
    if (na < live && pb_idx != pg + 1) {
      pb_base = (int64_t)load_const_i32(bt + pg + 1) * page_bytes;
      pb_idx = pg + 1;
    }
    ++iu;
    const uint32_t gofs = (uint32_t)off * rs_bytes;
    const char* kp = kbase_g + pa_base;
    const char* vp = vbase_g + pa_base;
    const int ln = lane_here(), pos = ln & 31, half = ln >> 5;
    if (na == kGroup) {
      const uint32_t k_src = (uint32_t)half * rs_bytes + ((uint32_t)(pos ^ (8 * (w & 1) + half)) << 4);
      const uint32_t v_src = (uint32_t)half * rs_bytes + ((uint32_t)(pos ^ (2 * half)) << 4);
      // whole group: every row is live; row offsets are scalar
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t rowofs = gofs + (uint32_t)(8 * w + 2 * j) * rs_bytes;
        const int ro = (8 * w + 2 * j) * kRowBytes;
        __builtin_amdgcn_global_load_lds(kp + rowofs + (k_src ^ (32u * j)), (PA_LDS void*)(kst + ro), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp + rowofs + (v_src ^ (64u * j)), (PA_LDS void*)(vst + ro), 16, 0, 0);
      }
    } else {
      // a short group (the context's last, or one of a page smaller than
      // 64), or one that continues in the next page
      const int64_t db = pb_base - pa_base;        // second page, relative to the first
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 8 * w + 2 * j + half;
        const bool in_b = row >= na && row < live;
        const uint32_t rb = row < na ? gofs + (uint32_t)row * rs_bytes
                                     : (in_b ? (uint32_t)(row - na) * rs_bytes : gofs);
        const int64_t pbase = in_b ? db : 0;
        const int ro = (8 * w + 2 * j) * kRowBytes;
        __builtin_amdgcn_global_load_lds(kp + pbase + (rb + ((uint32_t)(pos ^ kswz(row)) << 4)),
                                         (PA_LDS void*)(kst + ro), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp + pbase + (rb + ((uint32_t)(pos ^ vswz(row)) << 4)),
                                         (PA_LDS void*)(vst + ro), 16, 0, 0);
      }
    }
  };

  // Per-lane operand read offsets within a K or V tile (this wave's key half
  // is rows 32*kh .. 32*kh+31 of the tile).  Tile bases are multiples of
  // 32 KB, so the swizzled bits of an operand address are XORed onto one
  // per-lane base.
  // K A-operand (16x16x32) of key block kb and d-step ds: row 32*kh + 16*kb
  // + c16, 16-byte chunk 4*ds + kq, stored at (4*ds + kq) ^ c16
  // = 16*(ds >> 2) + 4*((ds & 3) ^ (c16 >> 2)) + (kq ^ (c16 & 3)):
  // address k_lane ^ ((ds & 3) << 6), immediate 8192*kb + 256*(ds >> 2).
  const uint32_t k_lane = kh * (kHalfKeys * kRowBytes) + c16 * kRowBytes +
                          ((4 * (c16 >> 2) + (kq ^ (c16 & 3))) << 4);
  // V^T A-operand of d-block db: transposing reads, lane (kq, j = c16)
  // pointing at V[k0 + (j >> 2)][16*db + 4*(j & 3)] with k0 = 32*kh + 4*kq
  // (first read, k = 0..3 of the operand) and k0 + 16 (second read, k =
  // 4..7).  Row r = k0 + (j >> 2) has r & 7 = 4*(kq & 1) + (j >> 2) =: m,
  // so chunk 2*db + ((j & 3) >> 1) sits at 2*(8*(db >> 3) + ((db & 7) ^ m))
  // + ((j & 3) >> 1): address v_lane ^ ((db & 7) << 5), immediate
  // 256*(db >> 3) (+ 16 rows).
  const int vm = 4 * (kq & 1) + (c16 >> 2);
  const uint32_t v_lane = (uint32_t)(kHalfKeys * kh + 4 * kq + (c16 >> 2)) * kRowBytes +
                          (vm << 5) + (((c16 & 3) >> 1) << 4) + (c16 & 1) * 8;

  // LDS: K tiles at 0 and 32 KB (group u: tile (u - ga) % 2), V tiles at 64,
  // 96 and 128 KB (group u: tile (u - ga) % 3).  V has a third tile because
  // waves 4..7 run the PV of a group one iteration later (see below).
  auto ktile = [&](int r) { return smem + (r & 1) * kTileBytes; };
  auto vtile = [&](int r) { return smem + (2 + r % 3) * kTileBytes; };
  if (ga < gb) issue(ktile(0), vtile(0));

  // P and V tile of the group whose PV comes next.
  bool pv_go = false;
  u32x4 pcur[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  uint32_t pv_vbase = 0;

  // O^T += V^T P^T for the group whose P is pbv and whose V tile starts at vbase
  // (this wave's key half): V^T operands come from transposing LDS reads one
  // batch of two d-blocks ahead of the MFMAs.
  auto pv = [&](const u32x4 (&pbv)[2], const uint32_t vbase) {
    __builtin_amdgcn_s_setprio(1);
    u32x2 va[2][2][2];
    // batch b: d-blocks 2*b, 2*b + 1
    auto vread = [&](int b, u32x2 (&d)[2][2]) {
      switch (b) {
#define PA_VR(BB)                                                                        \
  case BB: {                                                                             \
    constexpr int db0 = 2 * (BB), db1 = 2 * (BB) + 1;                                    \
    const uint32_t a0 = vbase ^ ((db0 & 7) << 5), a1 = vbase ^ ((db1 & 7) << 5);         \
    PA_DS_READ_TR16(d[0][0], a0, 256 * (db0 >> 3));                                      \
    PA_DS_READ_TR16(d[0][1], a0, 256 * (db0 >> 3) + 16 * kRowBytes);                     \
    PA_DS_READ_TR16(d[1][0], a1, 256 * (db1 >> 3));                                      \
    PA_DS_READ_TR16(d[1][1], a1, 256 * (db1 >> 3) + 16 * kRowBytes);                     \
  } break;
        PA_VR(0) PA_VR(1) PA_VR(2) PA_VR(3) PA_VR(4) PA_VR(5) PA_VR(6) PA_VR(7)
#undef PA_VR
      }
    };
    vread(0, va[0]);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int cur = b & 1;
      if (b < 7) {
        vread(b + 1, va[cur ^ 1]);
        asm volatile("s_waitcnt lgkmcnt(4)"
                     : "+v"(va[cur][0][0]), "+v"(va[cur][0][1]), "+v"(va[cur][1][0]), "+v"(va[cur][1][1]));
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(va[cur][0][0]), "+v"(va[cur][0][1]), "+v"(va[cur][1][0]), "+v"(va[cur][1][1]));
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 av = {va[cur][t][0][0], va[cur][t][0][1], va[cur][t][1][0], va[cur][t][1][1]};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) o[2 * b + t][rb] = mfma16(av, pbv[rb], o[2 * b + t][rb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  int cu = ga;                              // compute cursor (group)
  // One barrier per group.  Waves w and w + 4 share a SIMD.  Waves 0..3 run
  // each group as scores, softmax, PV; waves 4..7 run the PV of a group at
  // the start of the next iteration, before that one's scores, so on every
  // SIMD one wave's softmax (VALU) meets the other wave's MFMAs instead of
  // both waves idling the matrix unit in the softmax together.  Entering
  // iteration u every wave waits for its own loads of group u; the barrier
  // makes all of group u visible and guarantees every wave has finished
  // iteration u - 1, after which K tile (u + 1) % 2 (group u - 1) and V tile
  // (u + 1) % 3 (group u - 2; waves 4..7 read it in iteration u - 1) are
  // free for group u + 1's loads.  Waves 0..3 issue their part right away,
  // waves 4..7 after their deferred PV.
  for (int u = ga; u < gb; ++u) {
    const int r = u - ga;
    char* const kt = ktile(r);
    char* const vt = vtile(r);
    PA_WAIT_VMCNT(0);
    PA_BARRIER();
    const bool more = u + 1 < gb;

    auto qksm = [&]() {
      const int key0 = cu * GK;
      const int n = min(GK, kv_end - key0);
      ++cu;
      const int hk0 = key0 + kHalfKeys * kh;   // first key of this wave's half
      // The half holds no live key, or (causal) every key of it lies after
      // the wave's last row: nothing to add.
      const bool active = wave_rows > 0 && kHalfKeys * kh < n && !(a.causal && hk0 > wave_last_pos);
      if (!active) return false;
    // S^T = K Q^T: key block kb (16 keys), row block rb in s[kb][rb].  LDS
    // reads run one d-step ahead of the MFMAs; each read feeds two MFMAs.
    f32x4 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_setprio(1);
    {
      const uint32_t kbase = lds_addr(kt) + k_lane;
      u32x4 kv[2][2];
      // d-step ds: address kbase ^ ((ds & 3) << 6), immediate kb * 8192 + (ds >> 2) * 256
      auto kread = [&](int ds, u32x4 (&d)[2]) {
        switch (ds) {
#define PA_KR(DS)                                                                  \
  case DS: {                                                                       \
    const uint32_t ad = kbase ^ (((DS) & 3) << 6);                                 \
    PA_DS_READ_B128(d[0], ad, 0 * 8192 + ((DS) >> 2) * 256);                       \
    PA_DS_READ_B128(d[1], ad, 1 * 8192 + ((DS) >> 2) * 256);                       \
  } break;
          PA_KR(0) PA_KR(1) PA_KR(2) PA_KR(3) PA_KR(4) PA_KR(5) PA_KR(6) PA_KR(7)
#undef PA_KR
        }
      };
      kread(0, kv[0]);
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        const int cur = ds & 1;
        if (ds < 7) {
          kread(ds + 1, kv[cur ^ 1]);
          asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(kv[cur][0]), "+v"(kv[cur][1]));
        } else {
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kv[cur][0]), "+v"(kv[cur][1]));
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) s[kb][rb] = mfma16(kv[cur][kb], qb[rb][ds], s[kb][rb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // Soft-max.  s[kb][rb][r] is key hk0 + 16*kb + 4*kq + r of query row
    // 16*rb + c16; scores stay unscaled until the exponent (one fma).
    const bool need_mask = (kHalfKeys * kh + kHalfKeys > n) || (a.causal && hk0 + kHalfKeys - 1 > wave_first_pos);
    if (need_mask) {
      // key hk0 + 16*kb + 4*kq + r is allowed iff it is below the group's
      // live rows and (causal) at most the row's position
      const int ln = lane_here();
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row_pos = wave_first_pos + 16 * rb + (ln & 15);
        const int lim = a.causal ? min(n, row_pos - key0 + 1) : n;
        const int lim_lane = lim - kHalfKeys * kh - 4 * (ln >> 4);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + r >= lim_lane) s[kb][rb][r] = -INFINITY;
      }
    }
    // Lane maxima; only when one exceeds its row's threshold are the row
    // maxima formed (two lane swaps) and the accumulators re-based.
    float lm[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      lm[rb] = vmax(vmax3(vmax3(s[0][rb][0], s[0][rb][1], s[0][rb][2]), s[0][rb][3], s[1][rb][0]),
                    vmax3(s[1][rb][1], s[1][rb][2], s[1][rb][3]));
    // A raw score above (m_run + slack) / (scale log2 e) needs re-basing.
    const float thr0 = fmaf(m_run[0], a.inv_scale_log2, kRescaleSlack * a.inv_scale_log2);
    const float thr1 = fmaf(m_run[1], a.inv_scale_log2, kRescaleSlack * a.inv_scale_log2);
    if (__any(lm[0] > thr0 || lm[1] > thr1)) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float mx = pair32_max(pair16_max(lm[rb])) * a.scale_log2;
        const float m_new = fmaxf(m_run[rb], mx);
        const float alpha = fast_exp2(m_run[rb] - m_new);
#pragma unroll
        for (int db = 0; db < 16; ++db) o[db][rb] *= alpha;
        l_run[rb] *= alpha;
        m_run[rb] = m_new;
      }
    }
    u32x4 (&pb)[2] = pcur;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      // P^T operand: k = 0..3 <- key block 0, k = 4..7 <- key block 1
      // (registers r = 0..3), packed to bf16
      float p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(fmaf(s[0][rb][r], a.scale_log2, -m_run[rb]));
        p[4 + r] = fast_exp2(fmaf(s[1][rb][r], a.scale_log2, -m_run[rb]));
      }
      pb[rb] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                     pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      // row sum of the rounded P (the values PV multiplies), two at a time
#pragma unroll
      for (int j = 0; j < 4; ++j) l_run[rb] = dot2_ones(pb[rb][j], l_run[rb]);
    }

      return true;
    };
    if (w < 4) {
      if (more) issue(ktile(r + 1), vtile(r + 1));
      pv_go = qksm();
      pv_vbase = lds_addr(vt) + v_lane;
    }
    if (pv_go) pv(pcur, pv_vbase);
    if (w >= 4) {
      if (more) issue(ktile(r + 1), vtile(r + 1));
      pv_go = qksm();
      pv_vbase = lds_addr(vt) + v_lane;
    }
  }
  if (w >= 4 && pv_go) {
    pv(pcur, pv_vbase);
  }

  // Merge the two key halves of every row, then normalize and store (or, for
  // a part of a split item, store the unnormalised partial with its row max
  // and sum).  Lane (kq, c16) holds d = 16*db + 4*kq + r of query row 16*rb +
  // c16; wave w finishes d-blocks 8*kh .. 8*kh+7 and hands its partner
  // (w ^ 1) the other eight.  Lane-derived values are recomputed here rather than kept
  // in registers across the loop.
  const int lane_e = __lane_id();
  float l_tot[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) l_tot[rb] = pair32_sum(pair16_sum(l_run[rb]));
  __syncthreads();   // every wave is done with the stages
  f32x4* xo_mine = reinterpret_cast<f32x4*>(smem + w * kXoWaveBytes);
  const f32x4* xo_peer = reinterpret_cast<const f32x4*>(smem + (w ^ 1) * kXoWaveBytes);
  float* ml_mine = reinterpret_cast<float*>(smem + kMlOff + w * (2 * 64 * 8));
  const float* ml_peer = reinterpret_cast<const float*>(smem + kMlOff + (w ^ 1) * (2 * 64 * 8));
  // d-blocks 8*mine .. 8*mine+7 are this wave's; the half index is a
  // template constant so the accumulator stays in registers.
  auto hand_off = [&](auto half_tag) {
    constexpr int other = 1 - decltype(half_tag)::value;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int j = 0; j < 8; ++j) xo_mine[(rb * 8 + j) * 64 + lane_e] = o[8 * other + j][rb];
      ml_mine[(rb * 64 + lane_e) * 2] = m_run[rb];
      ml_mine[(rb * 64 + lane_e) * 2 + 1] = l_tot[rb];
    }
  };
  auto finish = [&](auto half_tag) {
    constexpr int mine = decltype(half_tag)::value;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float mp = ml_peer[(rb * 64 + lane_e) * 2];
      const float lp = ml_peer[(rb * 64 + lane_e) * 2 + 1];
      const float M = fmaxf(m_run[rb], mp);
      const float f = fast_exp2(m_run[rb] - M);
      const float fp = fast_exp2(mp - M);
      const float lsum = f * l_tot[rb] + fp * lp;
      const int row = wrow0 + 16 * rb + (lane_e & 15);
      if (part >= 0) {
        if (row < q_len) {
          const int64_t slot = (int64_t)(item - a.num_full) * a.split + part;
          const int trow = row - q0;
          // The part's O / l in bf16 (zero for a row with no key in the
          // part: l = 0 there, and the merge gives it weight 0).
          const float pinv = lsum > 0.f ? 1.f / lsum : 0.f;
          const float wa = f * pinv, wb = fp * pinv;
          uint16_t* po = a.part_o + (slot * kBM + trow) * kHeadDim + 4 * (lane_e >> 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const f32x4 x = o[8 * mine + j][rb];
            const f32x4 y = xo_peer[(rb * 8 + j) * 64 + lane_e];
            *reinterpret_cast<u32x2*>(po + 16 * (8 * mine + j)) =
                u32x2{pack_bf16x2(x[0] * wa + y[0] * wb, x[1] * wa + y[1] * wb),
                      pack_bf16x2(x[2] * wa + y[2] * wb, x[3] * wa + y[3] * wb)};
          }
          if (mine == 0 && (lane_e >> 4) == 0)
            *reinterpret_cast<f32x2*>(a.part_ml + (slot * kBM + trow) * 2) = f32x2{M, lsum};
        }
        continue;
      }
      const float inv = 1.f / lsum;
      const float fa = f * inv, fb = fp * inv;
      if (row < q_len) {
        uint16_t* op = obase + (int64_t)row * q_stride + head * kHeadDim + 4 * (lane_e >> 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f32x4 x = o[8 * mine + j][rb];
          const f32x4 y = xo_peer[(rb * 8 + j) * 64 + lane_e];
          const u32x2 v = {pack_bf16x2(x[0] * fa + y[0] * fb, x[1] * fa + y[1] * fb),
                           pack_bf16x2(x[2] * fa + y[2] * fb, x[3] * fa + y[3] * fb)};
          *reinterpret_cast<u32x2*>(op + 16 * (8 * mine + j)) = v;
        }
      }
    }
  };
  if (kh == 0) hand_off(std::integral_constant<int, 0>{});
  else hand_off(std::integral_constant<int, 1>{});
  __syncthreads();
  if (kh == 0) finish(std::integral_constant<int, 0>{});
  else finish(std::integral_constant<int, 1>{});
}

// Combine the parts of the split items: workgroup (split item, 4-row block),
// thread (row, 4 dims); parts in order, so results are bitwise repeatable.
__global__ void __launch_bounds__(256) prefill_merge_kernel(PrefillArgs a) {
  const int item_idx = blockIdx.x / (kBM / 4);
  const int trow = 4 * (blockIdx.x % (kBM / 4)) + (threadIdx.x >> 6);
  const int d = 4 * (threadIdx.x & 63);
  int g, head, tile;
  map_item(a.num_full + item_idx, a.num_kv_heads, a.num_q_tiles, g, head, tile);
  const int row = tile * kBM + trow;
  if (row >= a.q_len) return;
  float M = kMinusHuge;
  for (int k = 0; k < a.split; ++k) {
    const int64_t slot = (int64_t)item_idx * a.split + k;
    M = fmaxf(M, a.part_ml[(slot * kBM + trow) * 2]);
  }
  float lsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < a.split; ++k) {
    const int64_t slot = (int64_t)item_idx * a.split + k;
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.part_ml + (slot * kBM + trow) * 2);
    const float f = fast_exp2(ml[0] - M) * ml[1];   // weight of the part's O / l
    lsum += f;
    const u32x2 v = *reinterpret_cast<const u32x2*>(a.part_o + (slot * kBM + trow) * kHeadDim + d);
    acc += f * f32x4{bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1])};
  }
  const float inv = 1.f / lsum;
  const int64_t q_stride = (int64_t)a.num_kv_heads * kGqa * kHeadDim;
  *reinterpret_cast<u32x2*>(a.out + (int64_t)row * q_stride + head * kHeadDim + d) =
      u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
}

int tile_units(int32_t q_len, int32_t start_pos, int32_t causal, int32_t block_size, int tile) {
  const int64_t kv_end = causal ? (int64_t)start_pos + std::min<int64_t>((int64_t)(tile + 1) * kBM, q_len)
                                : (int64_t)start_pos + q_len;
  const int64_t gk = block_size < kGroup ? block_size : kGroup;   // keys per group
  return (int)((kv_end + gk - 1) / gk);
}

}  // namespace

PrefillPlan plan_prefill(int32_t q_len, int32_t start_pos, int32_t causal, int32_t block_size,
                         int32_t num_kv_heads) {
  // One workgroup per CU (160 KB of LDS each).  Items fill whole rounds of
  // kPrefillSlots workgroups heaviest first; the r items of an incomplete last
  // round (or all items, when there are fewer than the slots) are cut into
  // `split` parts so that round fills the CUs.  The lightest tile bounds the
  // split so no part is empty.
  PrefillPlan p{};
  const int T = (q_len + kBM - 1) / kBM;
  const int64_t U = (int64_t)num_kv_heads * kGqa * T;
  int64_t r = U <= kPrefillSlots ? U : U % kPrefillSlots;
  int64_t S = r > 0 ? kPrefillSlots / r : 1;
  const int min_units = tile_units(q_len, start_pos, causal, block_size, 0);
  if (S > kPrefillMaxSplit) S = kPrefillMaxSplit;
  if (S > min_units) S = min_units;
  if (S < 2) { S = 1; r = 0; }
  p.num_items = U;
  p.num_full = U - r;
  p.split = (int32_t)S;
  p.split_items = r;
  const size_t slots = (size_t)(r * (S > 1 ? S : 0));
  p.part_o_off = 0;
  p.part_ml_off = (slots * kBM * kHeadDim * sizeof(uint16_t) + 255) & ~(size_t)255;
  p.bytes = slots ? p.part_ml_off + ((slots * kBM * 2 * sizeof(float) + 255) & ~(size_t)255) : 0;
  return p;
}

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, int32_t q_len, int32_t start_pos,
                          int32_t causal, const uint16_t* k_cache, const uint16_t* v_cache,
                          int64_t page_stride, const int32_t* block_table, int32_t block_size,
                          float scale, int32_t num_kv_heads, const PrefillPlan& plan,
                          void* workspace, hipStream_t stream) {
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
  a.inv_scale_log2 = 1.f / a.scale_log2;
  a.num_kv_heads = num_kv_heads;
  a.num_q_tiles = (q_len + kBM - 1) / kBM;
  a.num_full = (int32_t)plan.num_full;
  a.split = plan.split;
  a.cu_seqlens_q = nullptr;
  a.seqused_k = nullptr;
  a.num_seqs = 1;
  a.bt_stride = 0;
  a.total_q = q_len;
  a.max_q = q_len;
  a.max_k = start_pos + q_len;
  char* ws = static_cast<char*>(workspace);
  a.part_o = plan.bytes ? reinterpret_cast<uint16_t*>(ws + plan.part_o_off) : nullptr;
  a.part_ml = plan.bytes ? reinterpret_cast<float*>(ws + plan.part_ml_off) : nullptr;
  const int64_t grid = plan.num_full + plan.split_items * plan.split;
  hipLaunchKernelGGL(prefill_kernel, dim3((uint32_t)grid), dim3(kWavesPf * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.split_items == 0) return e;
  hipLaunchKernelGGL(prefill_merge_kernel, dim3((uint32_t)(plan.split_items * (kBM / 4))), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_varlen(uint16_t* out, const uint16_t* q, int32_t total_q,
                                 const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                                 int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int32_t causal, const uint16_t* k_cache, const uint16_t* v_cache,
                                 int64_t page_stride, const int32_t* block_table, int32_t bt_stride,
                                 int32_t block_size, float scale, int32_t num_kv_heads,
                                 hipStream_t stream) {
  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_stride = page_stride;
  a.block_table = block_table;
  a.q_len = 0;
  a.start_pos = 0;
  a.causal = causal ? 1 : 0;
  a.block_size = block_size;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.inv_scale_log2 = 1.f / a.scale_log2;
  a.num_kv_heads = num_kv_heads;
  a.num_q_tiles = (max_seqlen_q + kBM - 1) / kBM;
  a.num_full = INT32_MAX;          // no split
  a.split = 1;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.cu_seqlens_q = cu_seqlens_q;
  a.seqused_k = seqused_k;
  a.num_seqs = num_seqs;
  a.bt_stride = bt_stride;
  a.total_q = total_q;
  a.max_q = max_seqlen_q;
  a.max_k = max_seqlen_k;
  const int64_t grid = varlen_grid(total_q, num_seqs, num_kv_heads);
  hipLaunchKernelGGL(prefill_kernel, dim3((uint32_t)grid), dim3(kWavesPf * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
