// Single-token paged GQA decode for gfx950 (split-K / flash-decoding).
//
// What it computes ([ALIGN] §7): for each sequence and query head, softmax
// attention of the one query over all seq_len keys, walking the pages of the
// sequence in order, one block-table lookup per page, 64-token groups inside
// each page, online softmax.  Pages whose size is not a multiple of 64 end in
// a tail group that is masked ([ALIGN] §2, §5).
//
// Work decomposition (ours): a unit is one 64-token group of one page of one
// KV head; a workgroup (4 wave64s) takes `groups_per_split` consecutive units
// of one (sequence, KV head).  In each unit, wave w owns keys 16w .. 16w+15
// and keeps its own online-softmax state, so the unit loop has no workgroup
// barrier:
//  - the 6 query heads of the KV head share every K/V byte read (GQA 6);
//  - S^T[16 keys x 16] = K Q^T is one chain of eight 16x16x32 bf16 MFMAs, K
//    taken straight from 16-byte global loads (each byte is used once, by one
//    wave, so K is not staged in LDS).  In this orientation each lane holds
//    one query head, so the max and sum of the online softmax need two
//    cross-lane shuffles and P^T is already laid out as the next MFMA's
//    operand;
//  - V is transposed in registers and written to a wave-private LDS tile;
//    O^T[256 x 16] += V^T P^T is sixteen 16x16x16 bf16 MFMAs.
// The workgroup then merges its 4 waves through LDS into one split-K partial
// (m, l, unnormalised acc).  Partials are merged in two levels: the last
// workgroup of a cluster of splits to arrive merges the cluster, and the last
// cluster to arrive merges the clusters and writes bf16 output.  Merge order
// is fixed by split index (bitwise repeatable, no float atomics).  Nothing is
// read past a page's or a sequence's last live row, so poisoned rows there
// never reach the output.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_DECODE_TARGET_WGS
#define PA_DECODE_TARGET_WGS 1024
#endif

namespace pa {

const char* const kDecodeVariant =
    "decode-v2(splitk,wave16keys,st-orient,mfma16x16x32-qk,mfma16x16x16-pv,lds-vt,2level-merge)";

namespace {

constexpr int kWaves = 4;
constexpr int kVtStride = 16 + 4;      // bf16 per V^T row in LDS: 16 keys + 8 B pad
constexpr int kMaxFan = 64;            // partials merged by one workgroup at either level

typedef short s16x4 __attribute__((ext_vector_type(4)));

struct DecodeArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int64_t page_stride;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t block_size;
  float scale_log2;        // scale * log2(e): scores live in the exp2 domain
  int32_t num_kv_heads;
  int32_t units_per_page;
  int32_t groups_per_split;
  int32_t max_splits;
  int32_t cluster;         // splits merged together at the first level
  int32_t max_clusters;
  float* p1_acc;           // [S][Hkv][max_splits][6][256]   split partials
  float* p1_ml;            // [S][Hkv][max_splits][6][2]
  float* p2_acc;           // [S][Hkv][max_clusters][6][256] cluster partials
  float* p2_ml;            // [S][Hkv][max_clusters][6][2]
  uint32_t* cnt1;          // [S][Hkv][max_clusters]
  uint32_t* cnt2;          // [S][Hkv]
};

// Number of live units of a sequence of L >= 1 tokens.
__device__ __forceinline__ int live_units(int L, int B, int upp) {
  const int last_page = (L - 1) / B;
  const int rem = L - last_page * B;
  return last_page * upp + (rem + kGroup - 1) / kGroup;
}

// Orders this wave's LDS writes before its later LDS reads (wave-private data;
// LDS accesses of one wave complete in issue order once lgkmcnt drains).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Device-coherent accesses to split-K partials (written by workgroups that
// may run on another XCD, whose L2 is not coherent with ours).
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge n partials (acc [n][6][256], ml [n][6][2]) for dim d = threadIdx.x.
__device__ void merge_partials(int n, const float* __restrict__ acc, const float* __restrict__ ml,
                               float* ml_lds, float O[kGqa], float M[kGqa], float Ls[kGqa]) {
  const int d = threadIdx.x;
  for (int e = d; e < n * kGqa * 2; e += 256) ml_lds[e] = coherent_load(ml + e);
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kGqa; ++h) { M[h] = -INFINITY; Ls[h] = 0.f; O[h] = 0.f; }
  for (int sp = 0; sp < n; ++sp)
#pragma unroll
    for (int h = 0; h < kGqa; ++h) M[h] = fmaxf(M[h], ml_lds[sp * kGqa * 2 + 2 * h]);
  for (int sp0 = 0; sp0 < n; sp0 += 8) {
    float v[8][kGqa];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int h = 0; h < kGqa; ++h)
        v[k][h] = (sp0 + k < n) ? coherent_load(acc + (int64_t)(sp0 + k) * (kGqa * kHeadDim) + h * kHeadDim + d) : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (sp0 + k < n) {
#pragma unroll
        for (int h = 0; h < kGqa; ++h) {
          const float f = fast_exp2(ml_lds[(sp0 + k) * kGqa * 2 + 2 * h] - M[h]);
          Ls[h] += f * ml_lds[(sp0 + k) * kGqa * 2 + 2 * h + 1];
          O[h] += f * v[k][h];
        }
      }
    }
  }
}

__device__ __forceinline__ void store_partial(float* acc, float* ml, const float O[kGqa],
                                              const float M[kGqa], const float Ls[kGqa]) {
  const int d = threadIdx.x;
#pragma unroll
  for (int h = 0; h < kGqa; ++h) coherent_store(acc + h * kHeadDim + d, O[h]);
  if (d < kGqa) {
#pragma unroll
    for (int h = 0; h < kGqa; ++h)
      if (h == d) { coherent_store(ml + 2 * h, M[h]); coherent_store(ml + 2 * h + 1, Ls[h]); }
  }
}

__device__ __forceinline__ void store_output(uint16_t* out_sg, const float O[kGqa],
                                             const float Ls[kGqa]) {
  const int d = threadIdx.x;
#pragma unroll
  for (int h = 0; h < kGqa; ++h) out_sg[h * kHeadDim + d] = (uint16_t)f32_to_bf16_rne(O[h] / Ls[h]);
}

// Count this workgroup's arrival; true for the last one.  Partials are
// written and read with device-coherent (agent-scope) accesses, so ordering
// only needs every store of the workgroup to have completed (vmcnt drained)
// before the counter update; the workgroup barriers keep the compiler from
// moving memory accesses across it.  No cache-wide writeback or invalidate.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, unsigned expected, int* flag_lds) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    *flag_lds = (__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 expected - 1) ? 1 : 0;
  __syncthreads();
  return *flag_lds != 0;
}

constexpr int kVtBytes = kWaves * kHeadDim * kVtStride * 2;                  // 40960
constexpr int kMergeBytes = kWaves * kGqa * kHeadDim * 4 + kWaves * kGqa * 2 * 4;
constexpr int kSmemBytes = kVtBytes > kMergeBytes ? kVtBytes : kMergeBytes;

__global__ void __launch_bounds__(256, 2) decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  __shared__ int flag_lds;

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * kGqa;
  const int B = a.block_size;
  const int upp = a.units_per_page;
  const int G = a.groups_per_split;

  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  uint16_t* out_sg = a.out + ((int64_t)s * Hq + (int64_t)g * kGqa) * kHeadDim;
  if (L == 0) {
    if (split == 0)
      for (int e = tid; e < kGqa * kHeadDim; e += 256) out_sg[e] = 0;
    return;
  }
  const int units = live_units(L, B, upp);
  const int u0 = split * G;
  if (u0 >= units) return;                       // beyond this sequence: no work
  const int u1 = min(u0 + G, units);
  const int nsplit = (units + G - 1) / G;

  const int64_t row_stride = (int64_t)Hkv * kHeadDim;  // elements per cache row (token)
  const int32_t* bt = a.block_table + (int64_t)s * a.bt_stride;
  const int c16 = lane & 15;
  const int kq = lane >> 4;

  // Q^T as the B operand of S^T = K Q^T (16x16x32): lane supplies column
  // n = c16 (query head; columns 6..15 are zero) and k = 8*kq + i of step st,
  // mapped to d = 32*st + 8*kq + i (the same map as K's A operand below).
  bf16x8 qb[8];
  {
    const uint16_t* qp = a.q + ((int64_t)s * Hq + g * kGqa + (c16 < kGqa ? c16 : 0)) * kHeadDim + 8 * kq;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c16 < kGqa) v = load16(qp + 32 * st);
      qb[st] = as_bf16x8(v);
    }
  }

  // Online-softmax state of query head c16 (identical in the 4 lanes of it).
  float m_run = -INFINITY, l_run = 0.f;
  // O^T accumulator: lane holds head c16, d = 16*db + 4*kq + r.
  f32x4 o[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + w * (kHeadDim * kVtStride);

  for (int u = u0; u < u1; ++u) {
    const int page = u / upp;
    const int grp = u - page * upp;
    const int page_len = min(B, L - page * B);            // live rows of this page
    const int64_t phys = bt[page];
    const int kb = grp * kGroup + 16 * w;                 // this wave's first row in the page
    const uint16_t* kpage = a.k_cache + phys * a.page_stride + (int64_t)g * kHeadDim;
    const uint16_t* vpage = a.v_cache + phys * a.page_stride + (int64_t)g * kHeadDim;

    // K as the A operand: row m = key kb + c16, d = 32*st + 8*kq + i.
    const int kr = kb + c16;
    u32x4 kreg[8];
    {
      const bool ok = kr < page_len;
      const uint16_t* kp = kpage + (int64_t)(ok ? kr : 0) * row_stride + 8 * kq;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = load16(kp + 32 * st);
        kreg[st] = v;
      }
    }
    // V: keys kb + 4*kq + i (i = 0..3), dims 16*c16 .. +15 (two 16-byte loads).
    u32x4 vreg[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vr = kb + 4 * kq + i;
      const bool ok = vr < page_len;
      const uint16_t* vp = vpage + (int64_t)(ok ? vr : 0) * row_stride + 16 * c16;
      u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
      if (ok) { v0 = load16(vp); v1 = load16(vp + 8); }
      vreg[i][0] = v0;
      vreg[i][1] = v1;
    }

    // S^T = K Q^T: lane holds head c16, keys kb + 4*kq + r.
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 8; ++st)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kreg[st]), qb[st], sacc, 0, 0, 0);

    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sv[r] = (kb + 4 * kq + r < page_len) ? sacc[r] * a.scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(sv[r] - m_use);
    float ps = (p[0] + p[1]) + (p[2] + p[3]);
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;

    // V^T into this wave's LDS region: row d = 16*c16 + dd gets keys 4*kq .. +3.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w0 = vreg[0][j >> 2][j & 3];
      const uint32_t w1 = vreg[1][j >> 2][j & 3];
      const uint32_t w2 = vreg[2][j >> 2][j & 3];
      const uint32_t w3 = vreg[3][j >> 2][j & 3];
      const u32x2 lo = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
      const u32x2 hi = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
      *reinterpret_cast<u32x2*>(&vt[(16 * c16 + 2 * j) * kVtStride + 4 * kq]) = lo;
      *reinterpret_cast<u32x2*>(&vt[(16 * c16 + 2 * j + 1) * kVtStride + 4 * kq]) = hi;
    }
    wave_lds_sync();

    // O^T = alpha * O^T + V^T P^T (16x16x16): A = V^T rows d = 16*db + c16,
    // keys 4*kq .. +3; B = P^T column head c16, the same 4 keys.
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 16; ++db) o[db] *= alpha;
    }
    const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const s16x4 va = *reinterpret_cast<const s16x4*>(&vt[(16 * db + c16) * kVtStride + 4 * kq]);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[db], 0, 0, 0);
    }
    wave_lds_sync();   // reads of vt done before the next unit overwrites it
  }

  // Merge the four waves of the workgroup (LDS reused from the V^T regions).
  __syncthreads();
  float* merge_acc = reinterpret_cast<float*>(smem);                  // [4][6][256]
  float* merge_ml = merge_acc + kWaves * kGqa * kHeadDim;            // [4][6][2]
  if (c16 < kGqa) {
#pragma unroll
    for (int db = 0; db < 16; ++db)
      *reinterpret_cast<f32x4*>(&merge_acc[(w * kGqa + c16) * kHeadDim + 16 * db + 4 * kq]) = o[db];
    if (kq == 0) {
      merge_ml[(w * kGqa + c16) * 2] = m_run;
      merge_ml[(w * kGqa + c16) * 2 + 1] = l_run;
    }
  }
  __syncthreads();

  const int d = tid;  // 256 threads <-> 256 dims
  float Mh[kGqa], Lh[kGqa], Oh[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, merge_ml[(ww * kGqa + h) * 2]);
    const float mu = M == -INFINITY ? 0.f : M;
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(merge_ml[(ww * kGqa + h) * 2] - mu);
      Ls += f * merge_ml[(ww * kGqa + h) * 2 + 1];
      O += f * merge_acc[(ww * kGqa + h) * kHeadDim + d];
    }
    Mh[h] = M; Lh[h] = Ls; Oh[h] = O;
  }

  if (nsplit == 1) {
    store_output(out_sg, Oh, Lh);
    return;
  }

  // Level 1: splits of a cluster; the last arrival merges them.
  const int64_t sg = (int64_t)s * Hkv + g;
  constexpr int kPart = kGqa * kHeadDim;
  store_partial(a.p1_acc + (sg * a.max_splits + split) * kPart,
                a.p1_ml + (sg * a.max_splits + split) * (kGqa * 2), Oh, Mh, Lh);
  const int C = a.cluster;
  const int cl = split / C;
  const int ncl = (nsplit + C - 1) / C;
  const int members = min(C, nsplit - cl * C);
  uint32_t* c1 = a.cnt1 + sg * a.max_clusters + cl;
  if (!arrive_last(c1, (unsigned)members, &flag_lds)) return;
  float* ml_lds = reinterpret_cast<float*>(smem);
  merge_partials(members, a.p1_acc + (sg * a.max_splits + (int64_t)cl * C) * kPart,
                 a.p1_ml + (sg * a.max_splits + (int64_t)cl * C) * (kGqa * 2), ml_lds, Oh, Mh, Lh);
  if (tid == 0) __hip_atomic_store(c1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (ncl == 1) {
    store_output(out_sg, Oh, Lh);
    return;
  }

  // Level 2: clusters of the (sequence, KV head); the last arrival writes out.
  store_partial(a.p2_acc + (sg * a.max_clusters + cl) * kPart,
                a.p2_ml + (sg * a.max_clusters + cl) * (kGqa * 2), Oh, Mh, Lh);
  uint32_t* c2 = a.cnt2 + sg;
  if (!arrive_last(c2, (unsigned)ncl, &flag_lds)) return;
  __syncthreads();   // every thread is done with ml_lds from level 1
  merge_partials(ncl, a.p2_acc + sg * a.max_clusters * kPart,
                 a.p2_ml + sg * a.max_clusters * (kGqa * 2), ml_lds, Oh, Mh, Lh);
  store_output(out_sg, Oh, Lh);
  if (tid == 0) __hip_atomic_store(c2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int32_t live_units_host(int64_t L, int32_t B, int32_t upp) {
  const int64_t last_page = (L - 1) / B;
  const int64_t rem = L - last_page * B;
  return (int32_t)(last_page * upp + (rem + kGroup - 1) / kGroup);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

DecodePlan plan_decode(int32_t num_seqs, int32_t max_seq_len, int32_t block_size,
                       int32_t num_kv_heads) {
  DecodePlan p{};
  p.units_per_page = (block_size + kGroup - 1) / kGroup;
  const int32_t units = live_units_host(max_seq_len, block_size, p.units_per_page);
  // Enough workgroups to cover the chip several times over, as few partials
  // as that allows; at most kMaxFan^2 splits per sequence so that both merge
  // levels fan in at most kMaxFan partials.
  const int64_t total = (int64_t)num_seqs * num_kv_heads * units;
  int64_t G = total / PA_DECODE_TARGET_WGS;
  if (G < 1) G = 1;
  const int64_t min_g = (units + kMaxFan * kMaxFan - 1) / (kMaxFan * kMaxFan);
  if (G < min_g) G = min_g;
  if (G > units) G = units;
  p.groups_per_split = (int32_t)G;
  p.max_splits = (int32_t)((units + G - 1) / G);
  if (p.max_splits <= 16) {
    p.cluster = p.max_splits;
  } else {
    int32_t c = 1;
    while (c * c < p.max_splits) ++c;
    p.cluster = c;
  }
  p.max_clusters = (p.max_splits + p.cluster - 1) / p.cluster;
  const size_t sg = (size_t)num_seqs * num_kv_heads;
  const size_t part = (size_t)kGqa * kHeadDim * sizeof(float);
  const size_t ml = (size_t)kGqa * 2 * sizeof(float);
  size_t off = 0;
  p.cnt1_off = off;  off += align256(sg * p.max_clusters * sizeof(uint32_t));
  p.cnt2_off = off;  off += align256(sg * sizeof(uint32_t));
  p.p1_ml_off = off; off += align256(sg * p.max_splits * ml);
  p.p2_ml_off = off; off += align256(sg * p.max_clusters * ml);
  p.p1_acc_off = off; off += align256(sg * p.max_splits * part);
  p.p2_acc_off = off; off += align256(sg * p.max_clusters * part);
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
  a.max_seq_len = max_seq_len;
  a.block_size = block_size;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_kv_heads = num_kv_heads;
  a.units_per_page = plan.units_per_page;
  a.groups_per_split = plan.groups_per_split;
  a.max_splits = plan.max_splits;
  a.cluster = plan.cluster;
  a.max_clusters = plan.max_clusters;
  a.cnt1 = reinterpret_cast<uint32_t*>(ws + plan.cnt1_off);
  a.cnt2 = reinterpret_cast<uint32_t*>(ws + plan.cnt2_off);
  a.p1_ml = reinterpret_cast<float*>(ws + plan.p1_ml_off);
  a.p2_ml = reinterpret_cast<float*>(ws + plan.p2_ml_off);
  a.p1_acc = reinterpret_cast<float*>(ws + plan.p1_acc_off);
  a.p2_acc = reinterpret_cast<float*>(ws + plan.p2_acc_off);
  hipLaunchKernelGGL(decode_kernel, dim3(plan.max_splits, num_kv_heads, num_seqs), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pa
