// Measured peaks of one MI355X (gfx950) for the roofline fractions of the benchmark:
// HBM streaming rates (read only, and read + write) and the sustained issue rate of the
// matrix-core instructions the layer's kernels use, each alone and the sparse one beside
// an HBM stream.  Nothing here is part of the layer; libbsl_peaks.so is built beside the
// library and only the benchmark loads it.
//
// Every kernel writes a value that depends on all of its work, so none of it can be
// removed by the compiler, and records the shader clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) at its start and end, from which the host
// derives the clock the chip held.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

#define PK_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const PK_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(p)));
}

// clocks[4 * block + 0..3] = memtime start, memtime end, realtime start, realtime end
__device__ __forceinline__ void stamp(uint64_t* clocks, int slot, uint64_t t, uint64_t rt) {
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + slot] = t;
    clocks[4 * blockIdx.x + 2 + slot] = rt;
  }
}

// Read-only stream: each thread reads 16-byte words at a grid stride, 8 loads in flight.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* src, uint64_t n16, uint32_t* out, uint64_t* clocks) {
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load_nt(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= load_nt(src + i);
  out[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __syncthreads();
  stamp(clocks, 1, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime());
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 2] = r0;
  }
}

// Copy: read and write the same number of bytes.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* src, u32x4* dst, uint64_t n16, uint64_t* clocks) {
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = load_nt(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(v[k], reinterpret_cast<PK_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(dst + i + k * stride)));
  }
  for (; i < n16; i += stride) dst[i] = src[i];
  __syncthreads();
  stamp(clocks, 1, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime());
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 2] = r0;
  }
}

// Matrix-core loops: 16 independent accumulator chains per wave, `iters` rounds of 16
// instructions.  KIND 0: v_mfma_f32_16x16x32_f16 (dense, 16384 flop); KIND 1:
// v_smfmac_f32_16x16x64_f16 (2:4 sparse A, 16384 multiply-adds of nonzeros, i.e. the
// same 16384 useful flop per instruction in the way the layer uses it); KIND 2:
// v_mfma_f32_32x32x16_f16 (dense, 32768 flop, 4 chains).  With STREAM, every round also
// issues one 16-byte non-temporal load per lane of `src` (1 KiB per wave per 16
// instructions, the sign-stream to matrix-core ratio of the single-token kernel), consumed
// four rounds later; src holds a power-of-two number of 16-byte words (n16), wrapped over.
// iters is a multiple of 4.
template <int KIND, bool STREAM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void mfma_kernel(int iters, float* out, uint64_t* clocks, const u32x4* src, uint64_t n16) {
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const int lane = threadIdx.x & 63;
  half8 a;
  half16 b;
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = (_Float16)(0.001f * (lane + k));
#pragma unroll
  for (int k = 0; k < 16; ++k) b[k] = (_Float16)(0.001f * (lane - k));
  int idx = 0x44444444;  // every group picks its slots 0 and 1
  asm volatile("" : "+v"(a), "+v"(b), "+v"(idx));
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t li = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 pend[4] = {};
  u32x4 sacc = {0u, 0u, 0u, 0u};
  float total = 0.f;
  if constexpr (KIND == 2) {
    float16v c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = (float16v){};
    const half8 b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, 6, 7);
    for (int it = 0; it < iters; it += 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b8, c[k], 0, 0, 0);
      if constexpr (STREAM) {
        sacc ^= pend[q];
        pend[q] = load_nt(src + (li & (n16 - 1)));
        li += stride;
      }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int v = 0; v < 16; ++v) total += c[k][v];
  } else {
    float4v c[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) c[k] = (float4v){0.f, 0.f, 0.f, 0.f};
    const half8 b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, 6, 7);
    for (int it = 0; it < iters; it += 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        if constexpr (KIND == 0) {
          c[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b8, c[k], 0, 0, 0);
          c[k + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b8, c[k + 1], 0, 0, 0);
        } else {
          c[k] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c[k], idx, 0, 0);
          c[k + 1] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c[k + 1], idx, 0, 1);
        }
      }
      if constexpr (STREAM) {
        sacc ^= pend[q];
        pend[q] = load_nt(src + (li & (n16 - 1)));
        li += stride;
      }
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) total += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) sacc ^= pend[k];
  out[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = total + (float)(sacc[0] ^ sacc[1] ^ sacc[2] ^ sacc[3]) * 1e-30f;
  __syncthreads();
  stamp(clocks, 1, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime());
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 2] = r0;
  }
}

// LDS read rate: every wave reads 16-byte words of a 32 KiB array (64 consecutive words
// per instruction, no bank conflicts), `iters` rounds of 16 reads.
__global__ __launch_bounds__(256) void lds_kernel(int iters, uint32_t* out, uint64_t* clocks) {
  __shared__ u32x4 buf[2048];
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int k = threadIdx.x; k < 2048; k += 256) buf[k] = (u32x4){(uint32_t)k, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int base = 64 * wave;
  asm volatile("" : "+v"(base));
  for (int it = 0; it < iters; ++it) {
    u32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = buf[((base + 128 * k) & 2047) + lane];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc ^= v[k];
    base += 64;
  }
  out[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __syncthreads();
  stamp(clocks, 1, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime());
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 2] = r0;
  }
}

// The single-token kernel's inner pattern: 16 planes per round; per plane every wave
// reads that plane's 32-byte B operand per lane from LDS (two 16-byte reads, shared by
// the workgroup) and runs R sparse MFMAs with it (R independent accumulators, an index
// per accumulator).  R = 4, 8 or 16.  MODE 0: A = 1.0, B near 1.0 (few mantissa bits);
// MODE 1: A = 1.0, B pseudo-random fp16 of magnitude 2^-8..2^-2 (the shared-operand
// decode: A all ones, B = +-V x); MODE 2: A and B pseudo-random (the wave-private decode:
// A = x, B = +-V).  With src non-null every wave also streams one 16-byte non-temporal
// load per lane per 16 MFMAs (the decode's sign bytes per MFMA), each consumed four
// loads later.
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
// fp16 pair with random sign and mantissa, exponent 2^-8..2^-2
__device__ __forceinline__ uint32_t rand_half2(uint32_t h) {
  const uint32_t e0 = 7u + (h & 7u), e1 = 7u + ((h >> 3) & 7u);
  const uint32_t lo = ((h >> 6) & 0x83FFu) | (e0 << 10), hi = ((h >> 16) & 0x83FFu) | (e1 << 10);
  return lo | (hi << 16);
}

template <int R, int MODE, bool STREAM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void mfma_lds_kernel(int iters, float* out, uint64_t* clocks, const u32x4* src, uint64_t n16) {
  __shared__ u32x4 zs[16][2][64];
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const int lane = threadIdx.x & 63;
  for (int k = threadIdx.x; k < 16 * 2 * 64; k += 256) {
    u32x4 v;
    for (int q = 0; q < 4; ++q) v[q] = MODE == 0 ? (q == 0 ? 0x3c003c00u ^ (uint32_t)k : 0x3c003c00u) : rand_half2(hash32(4 * k + q));
    (&zs[0][0][0])[k] = v;
  }
  __syncthreads();
  typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
  u32x4 araw;
  for (int q = 0; q < 4; ++q) araw[q] = MODE == 2 ? rand_half2(hash32(0x9e3779b9u * (threadIdx.x + 1) + q)) : 0x3c003c00u;
  half8 a = __builtin_bit_cast(half8, araw);
  constexpr int NI = R < 8 ? R : 8;  // distinct sparse indices
  int idx[NI];
#pragma unroll
  for (int t = 0; t < NI; ++t) idx[t] = (int)(0x44444444u | (hash32(t * 64 + lane) & 0xAAAAAAAAu));
  asm volatile("" : "+v"(a));
  float4v c[R];
#pragma unroll
  for (int t = 0; t < R; ++t) c[t] = (float4v){0.f, 0.f, 0.f, 0.f};
  auto read_b = [&](int b) {
    const u32x4 lo = zs[b][0][lane], hi = zs[b][1][lane];
    return __builtin_bit_cast(half16, (u32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t li = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 pend[4] = {};
  u32x4 sacc = {0u, 0u, 0u, 0u};
  constexpr int PLANES_PER_LOAD = 16 / R;  // planes per 16 MFMAs
  half16 cur = read_b(0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (STREAM) {
        if (b % PLANES_PER_LOAD == 0) {
          const int slot = (b / PLANES_PER_LOAD) & 3;
          sacc ^= pend[slot];
          pend[slot] = load_nt(src + (li & (n16 - 1)));
          li += stride;
        }
      }
      const half16 nxt = read_b((b + 1) & 15);  // the next plane's operand, read while this one runs
#pragma unroll
      for (int t = 0; t < R; ++t) {
        if (b & 1) c[t] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, cur, c[t], idx[t % NI], 0, 1);
        else c[t] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, cur, c[t], idx[t % NI], 0, 0);
      }
      cur = nxt;
    }
  }
  float total = 0.f;
#pragma unroll
  for (int t = 0; t < R; ++t) total += c[t][0] + c[t][1] + c[t][2] + c[t][3];
#pragma unroll
  for (int k = 0; k < 4; ++k) sacc ^= pend[k];
  out[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = total + (float)(sacc[0] ^ sacc[1] ^ sacc[2] ^ sacc[3]) * 1e-30f;
  __syncthreads();
  stamp(clocks, 1, __builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime());
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 2] = r0;
  }
}

}  // namespace

extern "C" {

// All pointers are device memory of the current device; `stream` is a hipStream_t.
// out / clocks must hold grid * 256 words / 4 * grid 64-bit values.  Return hipError_t.
int bslp_read(const void* src, uint64_t bytes, uint32_t* out, uint64_t* clocks, int grid, void* stream) {
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, out, clocks);
  return (int)hipGetLastError();
}

int bslp_copy(const void* src, void* dst, uint64_t bytes, uint64_t* clocks, int grid, void* stream) {
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16, clocks);
  return (int)hipGetLastError();
}

// kind: 0 dense 16x16x32 f16, 1 sparse 16x16x64 f16, 2 dense 32x32x16 f16.  With src
// non-null (and bytes > 0) the loop also streams src (see mfma_kernel).  Each workgroup
// has 4 waves; `grid` workgroups.
int bslp_mfma(int kind, int iters, float* out, uint64_t* clocks, const void* src, uint64_t bytes, int grid,
              void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* s = static_cast<const u32x4*>(src);
  const uint64_t n16 = bytes / 16;
  const bool str = s != nullptr && n16 > 0;
  if (kind == 0 && !str) hipLaunchKernelGGL((mfma_kernel<0, false>), dim3(grid), dim3(256), 0, st, iters, out, clocks, s, n16);
  else if (kind == 1 && !str) hipLaunchKernelGGL((mfma_kernel<1, false>), dim3(grid), dim3(256), 0, st, iters, out, clocks, s, n16);
  else if (kind == 2 && !str) hipLaunchKernelGGL((mfma_kernel<2, false>), dim3(grid), dim3(256), 0, st, iters, out, clocks, s, n16);
  else if (kind == 0) hipLaunchKernelGGL((mfma_kernel<0, true>), dim3(grid), dim3(256), 0, st, iters, out, clocks, s, n16);
  else if (kind == 1) hipLaunchKernelGGL((mfma_kernel<1, true>), dim3(grid), dim3(256), 0, st, iters, out, clocks, s, n16);
  else if (kind == 2) hipLaunchKernelGGL((mfma_kernel<2, true>), dim3(grid), dim3(256), 0, st, iters, out, clocks, s, n16);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// LDS read rate: grid workgroups of 4 waves, `iters` rounds of 16 reads of 1 KiB per wave.
int bslp_lds(int iters, uint32_t* out, uint64_t* clocks, int grid, void* stream) {
  hipLaunchKernelGGL(lds_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), iters, out, clocks);
  return (int)hipGetLastError();
}

// Sparse MFMAs fed from LDS: r = 4, 8 or 16 MFMAs per 2 KiB B operand read per wave;
// mode 0, 1, 2 (operand values, see mfma_lds_kernel); src / bytes: the optional stream
// (bytes a power of two times 16).
int bslp_mfma_lds(int r, int mode, int iters, float* out, uint64_t* clocks, const void* src, uint64_t bytes, int grid,
                  void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* s = static_cast<const u32x4*>(src);
  const uint64_t n16 = bytes / 16;
  const bool str = s != nullptr && n16 > 0;
#define BSLP_CASE(RR, MM)                                                                                           \
  if (r == RR && mode == MM) {                                                                                      \
    if (str) hipLaunchKernelGGL((mfma_lds_kernel<RR, MM, true>), dim3(grid), dim3(256), 0, st, iters, out, clocks, s, n16); \
    else hipLaunchKernelGGL((mfma_lds_kernel<RR, MM, false>), dim3(grid), dim3(256), 0, st, iters, out, clocks, s, n16);   \
    return (int)hipGetLastError();                                                                                  \
  }
  BSLP_CASE(4, 0) BSLP_CASE(4, 1) BSLP_CASE(4, 2) BSLP_CASE(8, 0) BSLP_CASE(8, 1) BSLP_CASE(8, 2)
  BSLP_CASE(16, 0) BSLP_CASE(16, 1) BSLP_CASE(16, 2)
#undef BSLP_CASE
  return (int)hipErrorInvalidValue;
}

}  // extern "C"
