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
//   online softmax on S^T: each lane holds one query row, so the row max
//   needs one cross-lane exchange (lane ^ 32); the accumulator is re-based
//   only when the max grows by more than 2^8
//   O^T[256 x 32 rows] += V^T[256 x 64] P^T     (32 MFMA 32x32x16 per wave)
// The transposed orientation makes P^T's MFMA operand a register-local
// reinterpretation of S^T's accumulator.  K and V rows go from HBM straight
// into LDS with the direct-to-LDS load, double-buffered (the next group is in
// flight while this one is computed), 16-byte chunks XOR-swizzled by row so
// operand reads are bank-conflict free; V^T operands come out of LDS with the
// gfx950 transposing read.  Groups entirely above the causal diagonal of the
// tile are never visited; the mask is evaluated only on groups that cross the
// diagonal or end a page early.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

const char* const kPrefillVariant =
    "prefill-v3(bm128,bn64,mfma32x32x16,st-orient,lds-dma-kv,2stage,tr16-vt,lazy-rescale,heavy-first,"
    "xcd-kvhead-map,hw-bf16-pack)";

namespace {

constexpr int kBM = 128;
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
// next group's loads, which were issued just before, and so serialize the
// prefetch with the compute it is meant to overlap.
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

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const PA_LDS char*)p;
}

__device__ __forceinline__ int32_t load_const_i32(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 16-byte chunk c of K row r at position c ^ (r & 15): the 16 rows one
// operand read touches at a time hit 16 different bank quads.  V row r: chunk
// c at c ^ ((r & 7) << 2): the 8 rows x 64 bytes of one transposing read are
// spread over the banks.
__device__ __forceinline__ int kswz(int r) { return r & 15; }
__device__ __forceinline__ int vswz(int r) { return (r & 7) << 2; }

// LDS reads the compiler does not track (it cannot tell which direct-to-LDS
// load wrote which bytes and would drain the prefetched group before every
// read); callers order them with explicit waits.
#define PA_DS_READ_B128(dst, addr) asm volatile("ds_read_b128 %0, %1" : "=v"(dst) : "v"(addr))
#define PA_DS_READ_TR16(dst, addr) asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(dst) : "v"(addr))

__global__ void __launch_bounds__(256, 1) prefill_kernel(PrefillArgs a) {
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
  float m_run = -INFINITY;    // reference the accumulator is scaled to
  float l_run = 0.f;          // this lane's partial row sum (its 32 keys per group)

  const char* kbase_g = reinterpret_cast<const char*>(a.k_cache + (int64_t)g * kHeadDim);
  const char* vbase_g = reinterpret_cast<const char*>(a.v_cache + (int64_t)g * kHeadDim);
  const uint32_t rs_bytes = (uint32_t)(row_stride * 2);
  const int64_t page_bytes = a.page_stride * 2;

  // Wave w loads rows 16w .. 16w+15 of each group's K and V tiles: direct-to-
  // LDS load j moves rows 16w + 2j (lanes 0..31) and 16w + 2j + 1 (lanes
  // 32..63).  Per-lane byte offsets from the group's first row, with the
  // chunk swizzle of the destination row, are computed once.
  const int pos = lane & 31;
  const int half = lane >> 5;
  uint32_t koff[8], voff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 16 * w + 2 * j + half;
    koff[j] = (uint32_t)row * rs_bytes + ((uint32_t)(pos ^ kswz(row)) << 4);
    voff[j] = (uint32_t)row * rs_bytes + ((uint32_t)(pos ^ vswz(row)) << 4);
  }
  // Issue cursor: logical page ip, group ig inside it; the block-table entry
  // is read (a scalar load) when the first group of a new page is prepared.
  int ip = 0, ig = 0, ip_loaded = -1;
  int64_t ip_base = 0;
  // Loads of the group being issued: uniform page bases and row offset, and
  // whether every row is live.
  const char* ikp = nullptr;
  const char* ivp = nullptr;
  uint32_t igofs = 0;
  int in_live = kGroup;
  auto prepare = [&]() {
    if (ip != ip_loaded) {
      ip_loaded = ip;
      ip_base = (int64_t)load_const_i32(a.block_table + ip) * page_bytes;
    }
    const int key0 = ip * B + ig * kGroup;
    in_live = min(kGroup, min(B - ig * kGroup, kv_end - key0));
    ikp = kbase_g + ip_base;
    ivp = vbase_g + ip_base;
    igofs = (uint32_t)(ig * kGroup) * rs_bytes;
    if (++ig == upp) { ig = 0; ++ip; }
  };
  // Direct-to-LDS loads j (rows 16w + 2j and 16w + 2j + 1 of K and of V) of
  // the prepared group into stage st.  Rows past the group's live end reload
  // the page's first row (finite; masked out).
  auto row_base = [&](int j) {
    uint32_t rb = igofs;
    if (in_live < kGroup) {
      const int row = 16 * w + 2 * j + half;
      if (row >= in_live) rb = (uint32_t)(-row) * rs_bytes;      // -> page row 0
    }
    return rb;
  };
  auto issue_k = [&](int j, char* st) {
    __builtin_amdgcn_global_load_lds(ikp + (row_base(j) + koff[j]),
                                     (PA_LDS void*)(st + (16 * w + 2 * j) * kRowBytes), 16, 0, 0);
  };
  auto issue_v = [&](int j, char* st) {
    __builtin_amdgcn_global_load_lds(ivp + (row_base(j) + voff[j]),
                                     (PA_LDS void*)(st + kTileBytes + (16 * w + 2 * j) * kRowBytes), 16, 0, 0);
  };
  auto issue_all = [&](char* st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) { issue_k(j, st); issue_v(j, st); }
  };

  char* st0 = smem;
  char* st1 = smem + kStageBytes;
  prepare();
  issue_all(st0);
  int cp = 0, cg = 0;      // compute cursor (page, group)

  // One barrier per group: entering iteration u every wave waits for its own
  // loads of group u, then the barrier makes all of group u visible and
  // guarantees every wave has finished group u - 1, whose stage the loads of
  // group u + 1 then overwrite.
  for (int u = 0; u < units; ++u) {
    char* st = (u & 1) ? st1 : st0;
    char* nst = (u & 1) ? st0 : st1;
    PA_WAIT_VMCNT(0);         // this wave's part of group u has landed
    PA_BARRIER();             // every wave's part of group u has landed
    const bool more = u + 1 < units;
    if (more) prepare();

    const int key0 = cp * B + cg * kGroup;
    const int n = min(kGroup, min(B - cg * kGroup, kv_end - key0));
    if (++cg == upp) { cg = 0; ++cp; }
    const uint32_t kt = lds_addr(st);
    const uint32_t vt = kt + kTileBytes;

    // S^T = K Q^T for keys 0..31 (s0) and 32..63 (s1).  A operand: key row
    // 32*kh + col, 16-byte chunk 2*ds + hh.  LDS reads run one batch (two
    // d-steps) ahead of the MFMAs (lgkmcnt(4) keeps the newer batch in flight).
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
    {
      const uint32_t ka0 = kt + col * kRowBytes;
      const uint32_t ka1 = kt + (32 + col) * kRowBytes;
      const int sw = kswz(col);      // (32 + col) & 15 == col & 15
      u32x4 kb[2][4];
      auto kread = [&](int ds, u32x4& d0, u32x4& d1) {
        PA_DS_READ_B128(d0, ka0 + (((2 * ds + hh) ^ sw) << 4));
        PA_DS_READ_B128(d1, ka1 + (((2 * ds + hh) ^ sw) << 4));
      };
      kread(0, kb[0][0], kb[0][1]);
      kread(1, kb[0][2], kb[0][3]);
#pragma unroll
      for (int bt = 0; bt < 8; ++bt) {
        const int cur = bt & 1;
        // wave w's loads of the next group go out at its own point of the
        // group's work (waves 0 and 1 during S^T, 2 and 3 during PV): the
        // CU's load path then serves one wave at a time, and a wave waiting
        // for it leaves the other three computing
        if (more && bt == 4 * w) issue_all(nst);
        if (bt < 7) {
          kread(2 * bt + 2, kb[cur ^ 1][0], kb[cur ^ 1][1]);
          kread(2 * bt + 3, kb[cur ^ 1][2], kb[cur ^ 1][3]);
          asm volatile("s_waitcnt lgkmcnt(4)"
                       : "+v"(kb[cur][0]), "+v"(kb[cur][1]), "+v"(kb[cur][2]), "+v"(kb[cur][3]));
        } else {
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(kb[cur][0]), "+v"(kb[cur][1]), "+v"(kb[cur][2]), "+v"(kb[cur][3]));
        }
        s0 = mfma32(as_bf16x8(kb[cur][0]), qb[2 * bt], s0);
        s1 = mfma32(as_bf16x8(kb[cur][1]), qb[2 * bt], s1);
        s0 = mfma32(as_bf16x8(kb[cur][2]), qb[2 * bt + 1], s0);
        s1 = mfma32(as_bf16x8(kb[cur][3]), qb[2 * bt + 1], s1);
      }
    }

    // Accumulator register r of s{kh} holds key 32*kh + 8*(r/4) + 4*hh + r%4
    // for query row `col` of this wave.  Scaled in place.
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] *= a.scale_log2; s1[r] *= a.scale_log2; }
    const bool need_mask = (n < kGroup) || (a.causal && key0 + kGroup - 1 > wave_first_pos);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key_lo = 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key_lo >= n || (a.causal && key0 + key_lo > my_pos)) s0[r] = -INFINITY;
        if (key_lo + 32 >= n || (a.causal && key0 + key_lo + 32 > my_pos)) s1[r] = -INFINITY;
      }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = pair32_max(mx);
    if (__any(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    // pk[i] packs the weights of accumulator registers 2i, 2i+1 (s0: i < 8, s1: i >= 8)
    uint32_t pk[16];
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = fast_exp2(s0[2 * i] - m_use);
      const float p1 = fast_exp2(s0[2 * i + 1] - m_use);
      const float p2 = fast_exp2(s1[2 * i] - m_use);
      const float p3 = fast_exp2(s1[2 * i + 1] - m_use);
      rs += (p0 + p1) + (p2 + p3);
      pk[i] = pack_bf16x2(p0, p1);
      pk[8 + i] = pack_bf16x2(p2, p3);
    }
    l_run += rs;

    // O^T += V^T P^T over 4 steps of 16 keys.  MFMA k = 8*hh + 4*jj + e maps
    // to key 16*ks + 8*jj + 4*hh + e on both operands.  V^T operand: two
    // transposing reads, lane group (hh, dsub = lane/16 & 1) pointing at
    // V[key0 + (j >> 2)][d0 + 4*(j & 3)], key0 = 16*ks + 8*jj + 4*hh,
    // d0 = 32*db + 16*dsub (j = lane % 16).
    {
      const int j16 = lane & 15;
      const int dsub = (lane >> 4) & 1;
      const int vrow_lo = 4 * hh + (j16 >> 2);          // + 16*ks + 8*jj
      const uint32_t dofs = (uint32_t)(16 * dsub + 4 * (j16 & 3)) * 2;   // bytes within 32-d block
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kh = ks >> 1;
        const int j0 = 2 * (ks & 1);
        const u32x4 pb = {pk[8 * kh + 2 * j0], pk[8 * kh + 2 * j0 + 1],
                          pk[8 * kh + 2 * j0 + 2], pk[8 * kh + 2 * j0 + 3]};
        const int r0 = 16 * ks + vrow_lo;       // jj = 0
        const int r1 = r0 + 8;                  // jj = 1
        const uint32_t v0 = vt + r0 * kRowBytes;
        const uint32_t v1 = vt + r1 * kRowBytes;
        const int sw0 = vswz(r0), sw1 = vswz(r1);
        u32x2 va[2][4][2];
        auto vread = [&](int db, u32x2 (&dst)[2]) {
          const uint32_t byte = (uint32_t)db * 64 + dofs;   // 32 d = 64 bytes per block
          const uint32_t ch = byte >> 4, lo = byte & 15;
          PA_DS_READ_TR16(dst[0], v0 + ((ch ^ sw0) << 4) + lo);
          PA_DS_READ_TR16(dst[1], v1 + ((ch ^ sw1) << 4) + lo);
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) vread(i, va[0][i]);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          if (more && half == 0 && 2 * ks == 4 * (w - 2)) issue_all(nst);
          if (half == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) vread(4 + i, va[1][i]);
            asm volatile("s_waitcnt lgkmcnt(8)"
                         : "+v"(va[0][0][0]), "+v"(va[0][0][1]), "+v"(va[0][1][0]), "+v"(va[0][1][1]),
                           "+v"(va[0][2][0]), "+v"(va[0][2][1]), "+v"(va[0][3][0]), "+v"(va[0][3][1]));
          } else {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(va[1][0][0]), "+v"(va[1][0][1]), "+v"(va[1][1][0]), "+v"(va[1][1][1]),
                           "+v"(va[1][2][0]), "+v"(va[1][2][1]), "+v"(va[1][3][0]), "+v"(va[1][3][1]));
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int db = 4 * half + i;
            const u32x4 av = {va[half][i][0][0], va[half][i][0][1], va[half][i][1][0], va[half][i][1][1]};
            o[db] = mfma32(as_bf16x8(av), as_bf16x8(pb), o[db]);
          }
        }
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
  hipLaunchKernelGGL(prefill_kernel, dim3(num_kv_heads * kGqa * a.num_q_tiles), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pa
