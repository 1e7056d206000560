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
// of one (sequence, KV head).  In each unit, wave w owns keys 16w .. 16w+15:
//  - the 6 query heads of the KV head share every K/V byte read (GQA 6):
//    S[6 x 16] = Q[6 x 256] K^T is one chain of eight 16x16x32 bf16 MFMAs with
//    K taken straight from the 16-byte global loads (no LDS staging: each byte
//    is used by exactly one wave, once);
//  - the online-softmax max and sum are wavefront shuffles across the 16 lanes
//    that hold one head's 16 scores;
//  - P V runs on the VALU in fp32 from V rows loaded 512 bytes per key.
// The workgroup then merges its 4 waves through LDS and writes one split-K
// partial (m, l, unnormalised acc); the last workgroup of the (sequence, KV
// head) to arrive merges all partials in split order (deterministic, no float
// atomics) and writes bf16 output.  Nothing is ever read past a page's or a
// sequence's last live row, so poisoned rows there never reach the output.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_DECODE_TARGET_WGS
#define PA_DECODE_TARGET_WGS 1024
#endif

namespace pa {

const char* const kDecodeVariant = "decode-v1(splitk,wave16keys,mfma16x16x32-qk,valu-pv,fused-combine)";

namespace {

constexpr int kWaves = 4;
constexpr int kMaxSplits = 512;   // partial (m, l) of every split fit the combine's LDS

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
  float* part_acc;         // [S][Hkv][max_splits][6][256]
  float* part_ml;          // [S][Hkv][max_splits][6][2]
  uint32_t* counters;      // [S][Hkv]
};

// Number of live units of a sequence of L >= 1 tokens.
__device__ __forceinline__ int live_units(int L, int B, int upp) {
  const int last_page = (L - 1) / B;
  const int rem = L - last_page * B;
  return last_page * upp + (rem + kGroup - 1) / kGroup;
}

__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float p_lds[kWaves][16][8];
  __shared__ float alpha_lds[kWaves][8];
  __shared__ __attribute__((aligned(16))) float merge_acc[kWaves][kGqa][kHeadDim];
  __shared__ float merge_ml[kWaves][kGqa][2];
  __shared__ int is_last_lds;

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

  // Q as the A operand of S = Q K^T (16x16x32): lane supplies row m = lane & 15
  // (query head within the group; rows 6..15 are zero) and k = 8*(lane>>4)+i of
  // each 32-wide step st, which we map to d = 32*st + 8*(lane>>4) + i.
  const int qh = lane & 15;
  const int kq = lane >> 4;
  bf16x8 qa[8];
  {
    const uint16_t* qp = a.q + ((int64_t)s * Hq + g * kGqa + (qh < kGqa ? qh : 0)) * kHeadDim + 8 * kq;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qh < kGqa) v = load16(qp + 32 * st);
      qa[st] = as_bf16x8(v);
    }
  }

  // Softmax state in the MFMA output layout: lane holds heads 4*kq + r.
  float m_r[4], l_r[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_r[r] = -INFINITY; l_r[r] = 0.f; }
  // P V accumulator: lane holds d = 8*(lane & 31) .. +7 of all 6 heads, for the
  // keys of parity lane >> 5.
  float acc[kGqa][8];
#pragma unroll
  for (int h = 0; h < kGqa; ++h)
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) acc[h][dd] = 0.f;

  const int vpar = lane >> 5;
  const int vd = 8 * (lane & 31);

  for (int u = u0; u < u1; ++u) {
    const int page = u / upp;
    const int grp = u - page * upp;
    const int page_len = min(B, L - page * B);            // live rows of this page
    const int64_t phys = bt[page];
    const int kb = grp * kGroup + 16 * w;                 // this wave's first row in the page
    const uint16_t* kpage = a.k_cache + phys * a.page_stride + (int64_t)g * kHeadDim;
    const uint16_t* vpage = a.v_cache + phys * a.page_stride + (int64_t)g * kHeadDim;

    // K: lane's key row kb + (lane & 15), 8 x 16 B at d = 32*st + 8*kq.
    const int kr = kb + qh;
    const bool kvalid = kr < page_len;
    u32x4 kreg[8];
    {
      const uint16_t* kp = kpage + (int64_t)(kvalid ? kr : 0) * row_stride + 8 * kq;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (kvalid) v = load16(kp + 32 * st);
        kreg[st] = v;
      }
    }
    // V: keys kb + 2i + vpar, d = vd .. vd+7 (512 contiguous bytes per key).
    u32x4 vreg[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int vr = kb + 2 * i + vpar;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (vr < page_len) v = load16(vpage + (int64_t)vr * row_stride + vd);
      vreg[i] = v;
    }

    // S = Q K^T: output lane holds key n = lane & 15, heads m = 4*kq + r.
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 8; ++st)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st], as_bf16x8(kreg[st]), sacc, 0, 0, 0);

    float p[4], alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sv = kvalid ? sacc[r] * a.scale_log2 : -INFINITY;
      float mx = sv;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m_r[r], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[r] = fast_exp2(m_r[r] - m_use);
      p[r] = fast_exp2(sv - m_use);
      float ps = p[r];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ps += __shfl_xor(ps, off);
      l_r[r] = l_r[r] * alpha[r] + ps;
      m_r[r] = m_new;
    }
    if (lane < 32) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * kq + r;
        if (h < kGqa) {
          p_lds[w][qh][h] = p[r];
          if (qh == 0) alpha_lds[w][h] = alpha[r];
        }
      }
    }
    __syncthreads();

    float al[kGqa];
#pragma unroll
    for (int h = 0; h < kGqa; ++h) al[h] = alpha_lds[w][h];
#pragma unroll
    for (int h = 0; h < kGqa; ++h)
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) acc[h][dd] *= al[h];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 2 * i + vpar;
      const f32x4 pa = *reinterpret_cast<const f32x4*>(&p_lds[w][key][0]);
      const f32x4 pb = *reinterpret_cast<const f32x4*>(&p_lds[w][key][4]);
      const float ph[kGqa] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1]};
      const u32x4 vv = vreg[i];
      const float vf[8] = {bf16_lo(vv[0]), bf16_hi(vv[0]), bf16_lo(vv[1]), bf16_hi(vv[1]),
                           bf16_lo(vv[2]), bf16_hi(vv[2]), bf16_lo(vv[3]), bf16_hi(vv[3])};
#pragma unroll
      for (int h = 0; h < kGqa; ++h)
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) acc[h][dd] = fmaf(ph[h], vf[dd], acc[h][dd]);
    }
    __syncthreads();
  }

  // Merge the two key parities of the wave (same softmax state), then the
  // four waves of the workgroup.
#pragma unroll
  for (int h = 0; h < kGqa; ++h)
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) acc[h][dd] += __shfl_xor(acc[h][dd], 32);
  if (lane < 32) {
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      f32x4* dst = reinterpret_cast<f32x4*>(&merge_acc[w][h][vd]);
      dst[0] = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
      dst[1] = f32x4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
    }
  }
  if (lane == 0 || lane == 16) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * kq + r;
      if (h < kGqa) { merge_ml[w][h][0] = m_r[r]; merge_ml[w][h][1] = l_r[r]; }
    }
  }
  __syncthreads();

  const int d = tid;  // 256 threads <-> 256 dims
  float Mh[kGqa], Lh[kGqa], Oh[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, merge_ml[ww][h][0]);
    const float mu = M == -INFINITY ? 0.f : M;
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(merge_ml[ww][h][0] - mu);
      Ls += f * merge_ml[ww][h][1];
      O += f * merge_acc[ww][h][d];
    }
    Mh[h] = M; Lh[h] = Ls; Oh[h] = O;
  }

  if (nsplit == 1) {
#pragma unroll
    for (int h = 0; h < kGqa; ++h) out_sg[h * kHeadDim + d] = (uint16_t)f32_to_bf16_rne(Oh[h] / Lh[h]);
    return;
  }

  const int64_t sg = (int64_t)s * Hkv + g;
  float* pacc = a.part_acc + (sg * a.max_splits + split) * (kGqa * kHeadDim);
  float* pml = a.part_ml + sg * a.max_splits * (kGqa * 2);
#pragma unroll
  for (int h = 0; h < kGqa; ++h) pacc[h * kHeadDim + d] = Oh[h];
  if (tid < kGqa) {
    pml[split * (kGqa * 2) + 2 * tid] = Mh[tid];
    pml[split * (kGqa * 2) + 2 * tid + 1] = Lh[tid];
  }
  // Release our partial, count arrivals; the last arrival merges.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&a.counters[sg], 1u);
    is_last_lds = (prev == (unsigned)(nsplit - 1));
  }
  __syncthreads();
  if (!is_last_lds) return;
  __threadfence();

  float* mls = &merge_acc[0][0][0];   // reuse: nsplit * 12 floats <= 6144
  for (int e = tid; e < nsplit * kGqa * 2; e += 256) mls[e] = pml[e];
  __syncthreads();
  float M[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) M[h] = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp)
#pragma unroll
    for (int h = 0; h < kGqa; ++h) M[h] = fmaxf(M[h], mls[sp * kGqa * 2 + 2 * h]);
  float Ls[kGqa], O[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) { Ls[h] = 0.f; O[h] = 0.f; }
  const float* pacc0 = a.part_acc + sg * a.max_splits * (kGqa * kHeadDim);
  for (int sp = 0; sp < nsplit; ++sp) {
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      const float f = fast_exp2(mls[sp * kGqa * 2 + 2 * h] - M[h]);
      Ls[h] += f * mls[sp * kGqa * 2 + 2 * h + 1];
      O[h] += f * pacc0[(int64_t)sp * (kGqa * kHeadDim) + h * kHeadDim + d];
    }
  }
#pragma unroll
  for (int h = 0; h < kGqa; ++h) out_sg[h * kHeadDim + d] = (uint16_t)f32_to_bf16_rne(O[h] / Ls[h]);
  if (tid == 0) atomicExch(&a.counters[sg], 0u);
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
  // as that allows; never more than kMaxSplits splits per sequence.
  const int64_t total = (int64_t)num_seqs * num_kv_heads * units;
  int64_t G = total / PA_DECODE_TARGET_WGS;
  if (G < 1) G = 1;
  const int64_t min_g = (units + kMaxSplits - 1) / kMaxSplits;
  if (G < min_g) G = min_g;
  if (G > units) G = units;
  p.groups_per_split = (int32_t)G;
  p.max_splits = (int32_t)((units + G - 1) / G);
  const size_t sg = (size_t)num_seqs * num_kv_heads;
  p.counters_off = 0;
  p.ml_off = align256(sg * sizeof(uint32_t));
  p.acc_off = p.ml_off + align256(sg * p.max_splits * kGqa * 2 * sizeof(float));
  p.bytes = p.acc_off + align256(sg * p.max_splits * kGqa * kHeadDim * sizeof(float));
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
  a.counters = reinterpret_cast<uint32_t*>(ws + plan.counters_off);
  a.part_ml = reinterpret_cast<float*>(ws + plan.ml_off);
  a.part_acc = reinterpret_cast<float*>(ws + plan.acc_off);
  hipLaunchKernelGGL(decode_kernel, dim3(plan.max_splits, num_kv_heads, num_seqs), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pa
