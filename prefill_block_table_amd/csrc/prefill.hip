// Chunked-prefill paged GQA attention for gfx950 (bf16 MFMA, fp32 accumulate).
//
// What it computes ([ALIGN] §6): for the q_len query tokens of one chunk at
// positions start_pos + i, complete causal attention over the paged K/V of
// the first start_pos + q_len tokens; no key skipped that the causal mask
// allows, none added that it forbids ([ALIGN] §5, §9).
//
// Work decomposition (ours): a workgroup of 8 wave64s owns a 128-row query
// tile of one query head; wave w owns 16 rows, and two waves share each SIMD
// so that one wave's LDS reads, soft-max and barrier waits overlap the other
// wave's MFMAs.  Keys stream through LDS one 64-token group of one page at a
// time (the page's tail group is masked when the page size is not a multiple
// of 64).  Per group and wave:
//   S^T[64 keys x 16 rows] = K[64 x 256] Q^T     (32 MFMA 16x16x32)
//   online softmax on S^T: each lane holds 16 scores of one query row, so
//   the row max and sum take two cross-lane swaps; the accumulator is
//   re-based only when the max grows by more than 2^8
//   O^T[256 x 16 rows] += V^T[256 x 64] P^T      (32 MFMA 16x16x32)
// The transposed orientation makes P^T's MFMA operand a register-local
// reinterpretation of S^T's accumulator (keys in the order the accumulator
// holds them; V^T's operand reads use the same order).  K and V rows go from
// HBM straight into LDS with the direct-to-LDS load, double-buffered (the
// next group is in flight while this one is computed), 16-byte chunks
// XOR-swizzled by row so operand reads are bank-conflict free; V^T operands
// come out of LDS with the gfx950 transposing read.  Groups entirely above
// the causal diagonal of the tile are never visited; the mask is evaluated
// only on groups that cross the diagonal or end a page early.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

const char* const kPrefillVariant =
    "prefill-v5(bm128,8waves-16rows,2waves-per-simd,bn64,mfma16x16x32,st-orient,lds-dma-kv,2stage,"
    "tr16-vt,lazy-rescale,heavy-first,xcd-kvhead-map,hw-bf16-pack)";

namespace {

constexpr int kWavesPf = 8;
constexpr int kRowsPerWave = 16;
constexpr int kBM = kWavesPf * kRowsPerWave;        // 128 query rows per workgroup
constexpr int kRowBytes = kHeadDim * 2;             // one KV head's row: 512 B
constexpr int kTileBytes = kGroup * kRowBytes;      // 64 rows: 32 KB
constexpr int kStageBytes = 2 * kTileBytes;         // K tile then V tile
constexpr int kSmemBytes = 2 * kStageBytes;         // two stages: 128 KB
constexpr float kRescaleSlack = 8.f;

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
  float scale_log2;
  int32_t num_kv_heads;
  int32_t num_q_tiles;
};

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

// LDS rows are 512 bytes, so every row starts at the same bank.  16-byte
// chunk c of K row r sits at position c ^ (r & 15): the 16 rows one pass of
// an operand read touches (16 lanes x 16 B) land on 16 different 16-byte
// bank groups.  V row r: chunk c at c ^ ((r & 7) << 1): the 8 rows one pass
// of a transposing read touches (32 lanes, 8 rows x 32 B) land on 8
// different 32-byte bank groups.
__device__ __forceinline__ int kswz(int r) { return r & 15; }
__device__ __forceinline__ int vswz(int r) { return (r & 7) << 1; }

// LDS operand reads the compiler does not track (it cannot tell which
// direct-to-LDS load wrote which bytes and would drain the prefetched group
// before every read); callers order them with explicit waits.
#define PA_DS_READ_B128(dst, addr, off) \
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(off))
#define PA_DS_READ_TR16(dst, addr, off) \
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(off))

__global__ void __launch_bounds__(kWavesPf * 64, 1) prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];

  // Workgroup -> (query head, query tile).  Tiles run heaviest (latest
  // rows) first.  Consecutive workgroup ids go to the 8 XCDs in turn; when
  // the KV heads divide the XCDs evenly, every XCD serves one KV head (8 / G
  // XCDs per head, taking alternate entries of that head's heavy-first
  // list), so the K/V a workgroup streams are the ones its XCD's L2 already
  // holds for its neighbours.
  const int G = a.num_kv_heads;
  const int T = a.num_q_tiles;
  const int L = blockIdx.x;
  int g, head, tile;
  if (8 % G == 0 && (kGqa * G * T) % 8 == 0) {
    const int x = L & 7, slot = L >> 3;
    g = x % G;
    const int k = slot * (8 / G) + x / G;        // 0 .. 6T-1 within KV head g
    tile = T - 1 - k / kGqa;
    head = g * kGqa + k % kGqa;
  } else {
    const int Hq_ = G * kGqa;
    tile = T - 1 - L / Hq_;
    head = L % Hq_;
    g = head / kGqa;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index, uniform per wave: LDS destinations and row bases stay scalar
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;     // this lane's query row within the wave (S^T / O^T column)
  const int kq = lane >> 4;      // lane group: keys 4*kq .. 4*kq+3 of each 16-key block
  const int Hq = a.num_kv_heads * kGqa;
  const int64_t row_stride = (int64_t)a.num_kv_heads * kHeadDim;
  const int64_t q_stride = (int64_t)Hq * kHeadDim;
  const int B = a.block_size;

  const int q0 = tile * kBM;
  const int my_row = q0 + kRowsPerWave * w + c16;
  const bool row_ok = my_row < a.q_len;
  const int my_pos = a.start_pos + my_row;
  const int wave_first_pos = a.start_pos + q0 + kRowsPerWave * w;

  // Q^T as the B operand of S^T = K Q^T (16x16x32): lane supplies column
  // n = c16 (its query row) and k = 8*kq + i of d-step ds -> d = 32*ds + 8*kq + i.
  u32x4 qb[8];
  {
    const uint16_t* qp = a.q + (int64_t)(row_ok ? my_row : 0) * q_stride + head * kHeadDim + 8 * kq;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = load16(qp + 32 * ds);
      qb[ds] = v;
    }
  }

  const int kv_len = a.start_pos + a.q_len;
  const int tile_last = min(q0 + kBM, a.q_len) - 1;
  const int kv_end = a.causal ? a.start_pos + tile_last + 1 : kv_len;
  const int upp = (B + kGroup - 1) / kGroup;
  const int last_page = (kv_end - 1) / B;
  const int units = last_page * upp + (kv_end - last_page * B + kGroup - 1) / kGroup;

  // O^T accumulator: d-block db (16 d), register r -> d = 16*db + 4*kq + r of
  // query row c16.
  f32x4 o[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;    // reference the accumulator is scaled to
  float l_run = 0.f;          // this lane's partial row sum (its 16 keys per group)

  const char* kbase_g = reinterpret_cast<const char*>(a.k_cache + (int64_t)g * kHeadDim);
  const char* vbase_g = reinterpret_cast<const char*>(a.v_cache + (int64_t)g * kHeadDim);
  const uint32_t rs_bytes = (uint32_t)(row_stride * 2);
  const int64_t page_bytes = a.page_stride * 2;
  const int pos = lane & 31;
  const int half = lane >> 5;

  // Issue cursor: logical page ip, group ig inside it; the block-table entry
  // is read (a scalar load) when the first group of a new page is issued.
  int ip = 0, ig = 0, ip_loaded = -1;
  int64_t ip_base = 0;
  // This wave's share of the next group: rows 8w .. 8w+7 of K and of V, four
  // direct-to-LDS loads each (rows 8w + 2j on lanes 0..31, 8w + 2j + 1 on
  // lanes 32..63).  Rows past the group's live end reload the page's first
  // row (finite; masked out of the softmax).
  auto issue = [&](char* st) {
    if (ip != ip_loaded) {
      ip_loaded = ip;
      ip_base = (int64_t)load_const_i32(a.block_table + ip) * page_bytes;
    }
    const int live = min(kGroup, min(B - ig * kGroup, kv_end - (ip * B + ig * kGroup)));
    const uint32_t gofs = (uint32_t)(ig * kGroup) * rs_bytes;
    const char* kp = kbase_g + ip_base;
    const char* vp = vbase_g + ip_base;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 8 * w + 2 * j + half;
      const uint32_t rb = row < live ? gofs + (uint32_t)row * rs_bytes : 0u;
      char* dst = st + (8 * w + 2 * j) * kRowBytes;
      __builtin_amdgcn_global_load_lds(kp + (rb + ((uint32_t)(pos ^ kswz(row)) << 4)),
                                       (PA_LDS void*)dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vp + (rb + ((uint32_t)(pos ^ vswz(row)) << 4)),
                                       (PA_LDS void*)(dst + kTileBytes), 16, 0, 0);
    }
    if (++ig == upp) { ig = 0; ++ip; }
  };

  // Per-lane operand read offsets within a stage.
  // K A-operand (16x16x32) of key block kb and d-step ds: row 16*kb + c16,
  // 16-byte chunk 4*ds + kq, stored at (4*ds + kq) ^ c16
  // = 16*(ds >> 2) + 4*((ds & 3) ^ (c16 >> 2)) + (kq ^ (c16 & 3)):
  // base k_t[ds & 3], immediate 8192*kb + 256*(ds >> 2).
  uint32_t k_t[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    k_t[t] = c16 * kRowBytes + ((4 * (t ^ (c16 >> 2)) + (kq ^ (c16 & 3))) << 4);
  // V^T A-operand of d-block db and key step ks (keys 32*ks ..): transposing
  // reads, lane (kq, j = c16) pointing at V[k0 + (j >> 2)][16*db + 4*(j & 3)]
  // with k0 = 32*ks + 4*kq (first read, k = 0..3 of the operand) and
  // k0 + 16 (second read, k = 4..7).  Row r = k0 + (j >> 2) has r & 7 =
  // 4*(kq & 1) + (j >> 2) =: m, so chunk 2*db + ((j & 3) >> 1) sits at
  // 2*(8*(db >> 3) + ((db & 7) ^ m)) + ((j & 3) >> 1): base v_t[db & 7],
  // immediate 256*(db >> 3) + 512*k0's multiple of 16.
  const int vm = 4 * (kq & 1) + (c16 >> 2);
  const uint32_t vrow = (uint32_t)(4 * kq + (c16 >> 2)) * kRowBytes + (((c16 & 3) >> 1) << 4) + (c16 & 1) * 8;
  uint32_t v_t[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) v_t[t] = kTileBytes + vrow + ((t ^ vm) << 5);

  char* st0 = smem;
  char* st1 = smem + kStageBytes;
  issue(st0);

  int cp = 0, cg = 0;        // compute cursor (page, group)
  // One barrier per group: entering iteration u every wave waits for its own
  // loads of group u, then the barrier makes all of group u visible and
  // guarantees every wave has finished group u - 1, whose stage the loads of
  // group u + 1 then overwrite.  Waves 0..3 issue their part of those loads
  // right away, waves 4..7 (the other wave of each SIMD) after their scores,
  // so the two waves of a SIMD do not wait for the CU's load path together.
  for (int u = 0; u < units; ++u) {
    char* st = (u & 1) ? st1 : st0;
    char* nst = (u & 1) ? st0 : st1;
    PA_WAIT_VMCNT(0);
    PA_BARRIER();
    const bool more = u + 1 < units;
    if (more && w < 4) issue(nst);

    const int key0 = cp * B + cg * kGroup;
    const int n = min(kGroup, min(B - cg * kGroup, kv_end - key0));
    if (++cg == upp) { cg = 0; ++cp; }
    const uint32_t sbase = lds_addr(st);

    // S^T = K Q^T: key block kb (16 keys) in s[kb].  LDS reads run one
    // d-step ahead of the MFMAs.
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const uint32_t k0a = sbase + k_t[0], k1a = sbase + k_t[1], k2a = sbase + k_t[2], k3a = sbase + k_t[3];
      u32x4 kv[2][4];
      // d-step ds: base k_t[ds & 3], immediate kb * 8192 + (ds >> 2) * 256
      auto kread = [&](int ds, u32x4 (&d)[4]) {
        switch (ds) {
#define PA_KB(DS) (((DS) & 3) == 0 ? k0a : ((DS) & 3) == 1 ? k1a : ((DS) & 3) == 2 ? k2a : k3a)
#define PA_KR(DS)                                                                  \
  case DS:                                                                         \
    PA_DS_READ_B128(d[0], PA_KB(DS), 0 * 8192 + ((DS) >> 2) * 256);                \
    PA_DS_READ_B128(d[1], PA_KB(DS), 1 * 8192 + ((DS) >> 2) * 256);                \
    PA_DS_READ_B128(d[2], PA_KB(DS), 2 * 8192 + ((DS) >> 2) * 256);                \
    PA_DS_READ_B128(d[3], PA_KB(DS), 3 * 8192 + ((DS) >> 2) * 256);                \
    break;
          PA_KR(0) PA_KR(1) PA_KR(2) PA_KR(3) PA_KR(4) PA_KR(5) PA_KR(6) PA_KR(7)
#undef PA_KR
#undef PA_KB
        }
      };
      kread(0, kv[0]);
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        const int cur = ds & 1;
        if (ds < 7) {
          kread(ds + 1, kv[cur ^ 1]);
          asm volatile("s_waitcnt lgkmcnt(4)"
                       : "+v"(kv[cur][0]), "+v"(kv[cur][1]), "+v"(kv[cur][2]), "+v"(kv[cur][3]));
        } else {
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(kv[cur][0]), "+v"(kv[cur][1]), "+v"(kv[cur][2]), "+v"(kv[cur][3]));
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[kb] = mfma16(kv[cur][kb], qb[ds], s[kb]);
      }
    }
    if (more && w >= 4) issue(nst);

    // Soft-max.  s[kb][r] is key key0 + 16*kb + 4*kq + r of query row c16.
    float sv[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[kb][r] = s[kb][r] * a.scale_log2;
    const bool need_mask = (n < kGroup) || (a.causal && key0 + kGroup - 1 > wave_first_pos);
    if (need_mask) {
      // key key0 + 16*kb + 4*kq + r is allowed iff it is below the group's
      // live rows and (causal) at most my_pos
      const int lim = a.causal ? min(n, my_pos - key0 + 1) : n;
      const int lim_lane = lim - 4 * kq;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kb + r >= lim_lane) sv[kb][r] = -INFINITY;
    }
    float mx = sv[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sv[kb][r]);
    mx = pair32_max(pair16_max(mx));
    if (__any(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int db = 0; db < 16; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    // P^T operand of key step ks: k = 0..3 <- block 2*ks, k = 4..7 <- block
    // 2*ks + 1 (registers r = 0..3), packed to bf16
    u32x4 pb[2];
    float rs = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(sv[2 * ks][r] - m_use);
        p[4 + r] = fast_exp2(sv[2 * ks + 1][r] - m_use);
      }
      rs += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      pb[ks] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                     pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    }
    l_run += rs;

    // O^T += V^T P^T: d-block db, key step ks.  The reads of a batch (four
    // d-blocks, one key step) run one batch ahead of its MFMAs.
    {
      uint32_t wv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) wv[t] = sbase + v_t[t];
      u32x2 va[2][4][2];
      // batch b = 2*dg + ks: d-blocks 4*dg .. 4*dg+3 (bases v_t[4*(dg & 1) + t],
      // immediate 256*(dg >> 1)), keys 32*ks + 4*kq (immediate 32*ks*512) and
      // + 16 (another 16*512)
      auto vread = [&](int b, u32x2 (&d)[4][2]) {
        switch (b) {
#define PA_VR(BB)                                                                        \
  case BB: {                                                                             \
    constexpr int dg = (BB) >> 1;                                                        \
    constexpr int off0 = 256 * (dg >> 1) + 32 * ((BB) & 1) * kRowBytes;                  \
    constexpr int off1 = off0 + 16 * kRowBytes;                                          \
    constexpr int tb = 4 * (dg & 1);                                                     \
    PA_DS_READ_TR16(d[0][0], wv[tb + 0], off0); PA_DS_READ_TR16(d[0][1], wv[tb + 0], off1); \
    PA_DS_READ_TR16(d[1][0], wv[tb + 1], off0); PA_DS_READ_TR16(d[1][1], wv[tb + 1], off1); \
    PA_DS_READ_TR16(d[2][0], wv[tb + 2], off0); PA_DS_READ_TR16(d[2][1], wv[tb + 2], off1); \
    PA_DS_READ_TR16(d[3][0], wv[tb + 3], off0); PA_DS_READ_TR16(d[3][1], wv[tb + 3], off1); \
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
          asm volatile("s_waitcnt lgkmcnt(8)"
                       : "+v"(va[cur][0][0]), "+v"(va[cur][0][1]), "+v"(va[cur][1][0]), "+v"(va[cur][1][1]),
                         "+v"(va[cur][2][0]), "+v"(va[cur][2][1]), "+v"(va[cur][3][0]), "+v"(va[cur][3][1]));
        } else {
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(va[cur][0][0]), "+v"(va[cur][0][1]), "+v"(va[cur][1][0]), "+v"(va[cur][1][1]),
                         "+v"(va[cur][2][0]), "+v"(va[cur][2][1]), "+v"(va[cur][3][0]), "+v"(va[cur][3][1]));
        }
        const int dg = b >> 1, ks = b & 1;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // d-block 4*dg + t
          const u32x4 av = {va[cur][t][0][0], va[cur][t][0][1], va[cur][t][1][0], va[cur][t][1][1]};
          o[4 * dg + t] = mfma16(av, pb[ks], o[4 * dg + t]);
        }
      }
    }
  }

  // Row sum over the four lanes of the row, then normalize and store:
  // lane (kq, c16) holds d = 16*db + 4*kq + r of query row c16.
  const float l_tot = pair32_sum(pair16_sum(l_run));
  const float inv = 1.f / l_tot;
  if (row_ok) {
    uint16_t* op = a.out + (int64_t)my_row * q_stride + head * kHeadDim + 4 * kq;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const u32x2 v = {pack_bf16x2(o[db][0] * inv, o[db][1] * inv), pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
      *reinterpret_cast<u32x2*>(op + 16 * db) = v;
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
  hipLaunchKernelGGL(prefill_kernel, dim3(num_kv_heads * kGqa * a.num_q_tiles), dim3(kWavesPf * 64),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
