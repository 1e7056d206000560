// bf16 M=1 GEMM (GEMV), y = W x, for the decode-time linear layers (gfx950).
//
// What it computes ([MEAS] §4: y[j] = sum_k x[k] * W[j, k] with bf16 weights
// and input and fp32 accumulation; §5: the 14336 / 16384 / 34816 x 5120
// weight shapes, outputs bitwise identical across row blockings).  One output
// column, so no MFMA: the kernel streams W from HBM once.
//
// Fixed summation order, the same for every blocking and pass size (so any
// two launch shapes give bitwise identical results, and the oracle can
// reproduce them): the wave that owns row j splits the row into 16-byte
// chunks of 8 elements; lane l takes chunks l, l + 64, l + 128, ... in that
// order and, inside a chunk, the elements in index order (each dword is a
// pair: low half, then high half), adding x[k] * W[j][k] to one fp32 sum with
// a fused multiply-add.  A bf16 x bf16 product is exact in fp32, so each step
// rounds once, exactly like an fp32 add of the exact product.  The 64 lane
// sums are then combined by an xor butterfly (lane distances 32, 16, 8, 4, 2,
// 1; every lane ends with the same value) and written as fp32 or rounded to
// bf16 (nearest even).
//
// Layout: W row-major [N, K] with a row stride of ldw elements, x [K], y [N];
// K, ldw multiples of 8 and W, x 16-byte aligned (checked by the caller).
#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_GEMV_RPW
#define PA_GEMV_RPW 1   // output rows per wave
#endif
#ifndef PA_GEMV_WPG
#define PA_GEMV_WPG 8   // waves per workgroup
#endif

namespace pa {
namespace {

constexpr int kRpw = PA_GEMV_RPW;
constexpr int kWpg = PA_GEMV_WPG;

__device__ __forceinline__ float chunk_fma(u32x4 w, u32x4 x, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_fmaf(bf16_lo(x[i]), bf16_lo(w[i]), acc);
    acc = __builtin_fmaf(bf16_hi(x[i]), bf16_hi(w[i]), acc);
  }
  return acc;
}

// NCH: chunks per lane held in registers at once (a pass covers 64 * NCH
// chunks); every load of a pass is issued before its first product.
template <int NCH, bool F32OUT>
__global__ void __launch_bounds__(kWpg * 64) gemv_kernel(void* __restrict__ y,
                                                         const uint16_t* __restrict__ W,
                                                         const uint16_t* __restrict__ x,
                                                         int32_t N, int32_t K, int64_t ldw) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * kWpg + wave) * kRpw;
  const int nchunks = K >> 3;
  float acc[kRpw];
#pragma unroll
  for (int r = 0; r < kRpw; ++r) acc[r] = 0.f;
  for (int c0 = 0; c0 < nchunks; c0 += 64 * NCH) {
    u32x4 xv[NCH];
    u32x4 wv[kRpw][NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = c0 + lane + 64 * i;
      const bool ok = c < nchunks;
      xv[i] = ok ? load16(x + 8 * (int64_t)c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < kRpw; ++r) {
        const int64_t row = row0 + r;
        wv[r][i] = (ok && row < N)
                       ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + row * ldw + 8 * (int64_t)c))
                       : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (c0 + lane + 64 * i >= nchunks) break;
#pragma unroll
      for (int r = 0; r < kRpw; ++r) acc[r] = chunk_fma(wv[r][i], xv[i], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < kRpw; ++r) {
    float v = acc[r];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off);
    const int64_t row = row0 + r;
    if (lane == 0 && row < N) {
      if constexpr (F32OUT) {
        static_cast<float*>(y)[row] = v;
      } else {
        static_cast<uint16_t*>(y)[row] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
      }
    }
  }
}

template <bool F32OUT>
hipError_t launch_nch(int nch, dim3 grid, hipStream_t stream, void* y, const uint16_t* W,
                      const uint16_t* x, int32_t N, int32_t K, int64_t ldw) {
  const dim3 block(kWpg * 64);
  switch (nch) {
    case 1: hipLaunchKernelGGL((gemv_kernel<1, F32OUT>), grid, block, 0, stream, y, W, x, N, K, ldw); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<2, F32OUT>), grid, block, 0, stream, y, W, x, N, K, ldw); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<4, F32OUT>), grid, block, 0, stream, y, W, x, N, K, ldw); break;
    case 8: hipLaunchKernelGGL((gemv_kernel<8, F32OUT>), grid, block, 0, stream, y, W, x, N, K, ldw); break;
    case 10: hipLaunchKernelGGL((gemv_kernel<10, F32OUT>), grid, block, 0, stream, y, W, x, N, K, ldw); break;
    default: hipLaunchKernelGGL((gemv_kernel<16, F32OUT>), grid, block, 0, stream, y, W, x, N, K, ldw); break;
  }
  return hipGetLastError();
}

}  // namespace

#define PA_STR2(x) #x
#define PA_STR(x) PA_STR2(x)
const char* gemv_variant() {
  return "gemv-v1(rows/wave=" PA_STR(PA_GEMV_RPW) ",waves/wg=" PA_STR(PA_GEMV_WPG) ")";
}

hipError_t launch_gemv(void* y, bool y_f32, const uint16_t* W, const uint16_t* x, int32_t N,
                       int32_t K, int64_t ldw, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const int64_t rows_per_wg = (int64_t)kWpg * kRpw;
  const dim3 grid((uint32_t)((N + rows_per_wg - 1) / rows_per_wg));
  // smallest register pass that covers the row in one go, else passes of 16
  const int per_lane = ((K >> 3) + 63) / 64;
  int nch = 16;
  for (int c : {1, 2, 4, 8, 10, 16}) {
    if (c >= per_lane) { nch = c; break; }
  }
  return y_f32 ? launch_nch<true>(nch, grid, stream, y, W, x, N, K, ldw)
               : launch_nch<false>(nch, grid, stream, y, W, x, N, K, ldw);
}

}  // namespace pa
