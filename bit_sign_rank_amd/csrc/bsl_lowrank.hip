// Kernels of the equal-size vanilla-SVD baseline (the "w/o AVD" ablation of the
// paper-review page's Figure 5 caption): y = sum_i (x V'_i) U'_i^T for up to 8 tokens.
//
// Both phases stream their factor once from HBM and are bound by its bandwidth:
//  * phase 1 (lowrank_xv_kernel): one wave per rank row of V'^T, contiguous 1 KiB loads
//    along d, the tokens' x read through L1/L2 beside it, one wave reduction per token;
//  * phase 2 (lowrank_tu_kernel): one workgroup per 64 output rows, one row per lane, so
//    each wave load of U' is one contiguous 1 KiB (8 ranks x 64 rows) and no lane
//    reduction is needed; the 8 waves split the rank columns and add their partial
//    sums through LDS in a fixed order.  t is read with scalar loads (uniform).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsl_internal.h"

namespace bsl {

namespace {

typedef _Float16 lr_half2 __attribute__((ext_vector_type(2)));
typedef uint32_t lr_u32x4 __attribute__((ext_vector_type(4)));

// By value: this compiler's __builtin_bit_cast of an ext-vector element (v[j]) reads
// element 0 whatever j is, so elements are copied out first.
__device__ __forceinline__ lr_half2 lr_as_half2(uint32_t v) { return __builtin_bit_cast(lr_half2, v); }

__device__ __forceinline__ float dot8(const lr_u32x4& a, const lr_u32x4& b, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_fdot2(lr_as_half2(a[j]), lr_as_half2(b[j]), acc, false);
  return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Index of the weight whose range [begin, next begin) holds `pos` (uniform).
template <typename F>
__device__ __forceinline__ int find_lr_weight(const LrArgs& a, int pos, F begin_of) {
  int wi = 0;
  while (wi + 1 < a.count && pos >= begin_of(a.w[wi + 1])) ++wi;
  return wi;
}

// Tokens past a.T compute on copies of the last token's x (phase 1) or on the spare
// rows of the t workspace (phase 2) and are never stored: the loops carry no branch.
template <int TT>
__global__ __launch_bounds__(256) void lowrank_xv_kernel(LrArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= a.total_rows) return;
  const int wi = find_lr_weight(a, row, [](const LrWeight& w) { return w.row_begin; });
  const int r = row - a.w[wi].row_begin;
  const int d = a.w[wi].d, d_pad = a.w[wi].d_pad, ld = a.w[wi].ld, T = a.T;
  const uint16_t* vrow = a.w[wi].vt + (size_t)r * d_pad + 8 * lane;
  const uint16_t* xr[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) xr[t] = a.w[wi].x + (size_t)(t < T ? t : T - 1) * d + 8 * lane;
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
  const int steps = d_pad / kLrColAlign;
  // columns past d (only in the last 512-column step) hold zeros in V'^T; x is not read there
  const int full = d / kLrColAlign;  // steps whose 512 columns are all below d
  int s = 0;
  for (; s + 4 <= full; s += 4) {  // four 1 KiB loads of the row in flight
    lr_u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const lr_u32x4*>(vrow + (s + j) * kLrColAlign);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < TT; ++t)
        acc[t] = dot8(v[j], *reinterpret_cast<const lr_u32x4*>(xr[t] + (s + j) * kLrColAlign), acc[t]);
  }
  for (; s < steps; ++s) {
    const lr_u32x4 v = *reinterpret_cast<const lr_u32x4*>(vrow + s * kLrColAlign);
    if (s * kLrColAlign + 8 * lane < d) {
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[t] = dot8(v, *reinterpret_cast<const lr_u32x4*>(xr[t] + s * kLrColAlign), acc[t]);
    }
  }
  float* tout = a.w[wi].t + r;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float sum = wave_sum(acc[t]);
    if (lane == 0 && t < T) tout[(size_t)t * ld] = sum;
  }
}

template <int TT>
__global__ __launch_bounds__(512) void lowrank_tu_kernel(LrArgs a) {
  __shared__ float part[kLrPhase2Waves][TT][kLrRowGroup];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x;
  const int wi = find_lr_weight(a, g, [](const LrWeight& w) { return w.rg_begin; });
  const int rg = g - a.w[wi].rg_begin;
  const int used = a.w[wi].kcat / 8;  // loaded column groups
  const int ld = a.w[wi].ld, m = a.w[wi].m, T = a.T;
  const float* tbase = a.w[wi].t;
  const uint16_t* base = a.w[wi].ut + (size_t)rg * (ld / 8) * 512 + 8 * lane;
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
  auto apply = [&](const lr_u32x4& u, int q) {
    float uf[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const lr_half2 h = lr_as_half2(u[j]);
      uf[2 * j] = (float)h[0];
      uf[2 * j + 1] = (float)h[1];
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float* tv = tbase + (size_t)t * ld + 8 * q;  // uniform: scalar loads
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[t] = __builtin_fmaf(uf[j], tv[j], acc[t]);
    }
  };
  constexpr int kUnroll = 8;  // 1 KiB loads in flight per wave
  int q = wave;
  for (; q + (kUnroll - 1) * kLrPhase2Waves < used; q += kUnroll * kLrPhase2Waves) {
    lr_u32x4 u[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) u[j] = *reinterpret_cast<const lr_u32x4*>(base + (size_t)(q + j * kLrPhase2Waves) * 512);
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) apply(u[j], q + j * kLrPhase2Waves);
  }
  for (; q < used; q += kLrPhase2Waves) apply(*reinterpret_cast<const lr_u32x4*>(base + (size_t)q * 512), q);
#pragma unroll
  for (int t = 0; t < TT; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  // wave t adds token t's partial sums in wave order and stores its row
  if (wave < T) {
    const int t = wave;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kLrPhase2Waves; ++w) sum += part[w][t][lane];
    const int row = rg * kLrRowGroup + lane;
    if (row < m) {
      if (a.y_fp32) static_cast<float*>(a.w[wi].y)[(size_t)t * m + row] = sum;
      else static_cast<_Float16*>(a.w[wi].y)[(size_t)t * m + row] = (_Float16)sum;
    }
  }
}

template <int TT>
int launch_lowrank_t(const LrArgs& a, hipStream_t st) {
  if (a.total_rows > 0) {
    hipLaunchKernelGGL(lowrank_xv_kernel<TT>, dim3((a.total_rows + 3) / 4), dim3(256), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  hipLaunchKernelGGL(lowrank_tu_kernel<TT>, dim3(a.total_rgs), dim3(64 * kLrPhase2Waves), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace

int launch_lowrank(const LrArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.T <= 1) return launch_lowrank_t<1>(a, st);
  if (a.T <= 2) return launch_lowrank_t<2>(a, st);
  if (a.T <= 4) return launch_lowrank_t<4>(a, st);
  return launch_lowrank_t<8>(a, st);
}

}  // namespace bsl
