// HIP kernels of libbitstack_linear for gfx950 (MI355X).
//
// The layer (BitStack OpenReview discussion, weight-restoration reply; paper-review
// page, Figure 3 caption) is y = x W_hat^T with W_hat = sum_i S_i * (U_i V_i^T).  By
// linearity,
//     y[t, j] = sum_i sum_r U_i[j, r] * P_i[j, (t, r)],   P_i = S_i Z_i,
//     Z_i[c, (t, r)] = V_i[c, r] * x[t, c],
// so each block costs one dense contraction of the sign matrix with Z_i (width 16 M)
// on the matrix cores (v_mfma_f32_16x16x32_f16: fp16 inputs, fp32 accumulation), a
// Hadamard product with U_i and a sum over r that is done once for all blocks.
//
// Sign tiles (16 rows x 512 columns, 1 KiB) are read with one 16-byte load per lane
// and turned into MFMA A fragments in registers; nothing is staged through LDS on the
// single-token path, where the unpack and the MFMA issue share each SIMD and any LDS
// round trip would cost more than the HBM read it serves.
//
// Two sign encodings share the stored layout:
//  * single-token kernel (M = 1): "bit planes".  Plane b of a lane's four words keeps
//    bits (pos, pos + 16) after one optional shift, so the A fragment is one AND per
//    dword.  The fp16 element is then bit * 2^(pos - 24) (exact subnormal or normal
//    powers of two, honoured exactly by the MFMA), i.e. a 0/1 encoding of the sign.
//    The power of two and the factor -2 of S = 1 - 2 bit are folded exactly into the
//    activations of that plane, and the missing "sum of Z over the chunk" term is put
//    into the accumulator's initial value, so
//        acc = 2^-17 * (sum_c Z_c - 2 sum_c bit_c Z_c) = 2^-17 * P.
//  * multi-token kernel (M >= 2): "+-1".  Shift the plane's bits to positions 15/31
//    and OR in 1.0, giving exact +-1 fp16 elements (unpack cost is amortised over the
//    token tile there).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "bsl_internal.h"

namespace bsl {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Accumulators of the bit-plane path hold 2^-17 times the layer's partial sums.
constexpr float kPlaneAccScale = 1.0f / 131072.0f;
constexpr float kPlaneOutScale = 131072.0f;

// Bit position (within each 16-bit half) that plane b occupies after its shift:
// planes 0-5 come from (w << 6), planes 6-11 from w, planes 12-15 from (w >> 6).
__host__ __device__ constexpr int plane_pos(int b) { return b < 6 ? b + 6 : (b < 12 ? b : b - 6); }

// fp16 bit pattern of the exact factor -2^(8 - pos) applied to the plane's activations.
// The A element is 2^(pos - 24) for a set bit, so A * x * factor = -2 * bit * x * 2^-17.
__host__ __device__ constexpr uint16_t plane_x_factor_bits(int b) {
  // -2^(8 - pos): pos = 6..11 -> -4, -2, -1, -0.5, -0.25, -0.125
  return (uint16_t)(0x8000u | (uint16_t)((15 + 8 - plane_pos(b)) << 10));
}
// fp16 bit pattern of 1 / factor = -2^(pos - 8) (to recover Z from the scaled products).
__host__ __device__ constexpr uint16_t plane_inv_factor_bits(int b) {
  return (uint16_t)(0x8000u | (uint16_t)((15 + plane_pos(b) - 8) << 10));
}

// Order in which the single-token kernel visits the planes: 6-11 straight from the
// loaded words, 12-15 after rotating them right by 6, 0-5 after rotating by 20 more.
__host__ __device__ constexpr int plane_order(int s) { return s < 10 ? s + 6 : s - 10; }

// Same factors for a plane index that is only known at run time (wave-uniform).
__device__ __forceinline__ uint32_t plane_x_factor_bits_dyn(int b) {
  const int pos = b < 6 ? b + 6 : (b < 12 ? b : b - 6);
  return 0x8000u | (uint32_t)((23 - pos) << 10);
}
__device__ __forceinline__ uint32_t plane_inv_factor_bits_dyn(int b) {
  const int pos = b < 6 ? b + 6 : (b < 12 ? b : b - 6);
  return 0x8000u | (uint32_t)((7 + pos) << 10);
}

__device__ __forceinline__ half8 as_half8(u32x4 v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ half2v as_half2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

// Loads through the global address space.  Pointers read from the block table are
// generic; without the cast the compiler emits flat loads, which also count against
// the LDS wait counter, so every LDS wait would stall on outstanding HBM reads.
#define BSL_GLOBAL __attribute__((address_space(1)))
#define BSL_CONST __attribute__((address_space(4)))
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const BSL_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(p));
}
// Data read exactly once (sign tiles): non-temporal, so it does not evict reused lines.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const BSL_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ u32x2 load8(const void* p) {
  return *reinterpret_cast<const BSL_GLOBAL u32x2*>(reinterpret_cast<uintptr_t>(p));
}
// A wave-uniform 64-bit pointer held in vector registers, moved to scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ BlockPtrs uniform_block(const BlockPtrs& b) {
  BlockPtrs r;
  r.signs = uniform_ptr(b.signs);
  r.u = uniform_ptr(b.u);
  r.v = uniform_ptr(b.v);
  return r;
}

// Block table entries are read with scalar loads (the table does not change while a
// kernel runs and the index is uniform).
__device__ __forceinline__ BlockPtrs load_block(const BlockPtrs* table, int i) {
  const BSL_CONST BlockPtrs* t = reinterpret_cast<const BSL_CONST BlockPtrs*>(reinterpret_cast<uintptr_t>(table)) + i;
  BlockPtrs b;
  b.signs = t->signs;
  b.u = t->u;
  b.v = t->v;
  return b;
}

// A fragment of plane b (bit-plane encoding) from a lane's four raw words.
template <int B>
__device__ __forceinline__ u32x4 plane_fragment(const u32x4& w, const u32x4& lo, const u32x4& hi) {
  constexpr uint32_t mask = 0x00010001u << plane_pos(B);
  const u32x4& src = B < 6 ? lo : (B < 12 ? w : hi);
  return src & mask;
}

// A fragment of plane b (+-1 encoding).
__device__ __forceinline__ u32x4 pm1_fragment(const u32x4& w, int b) {
  const int s = 15 - b;
  u32x4 a;
#pragma unroll
  for (int q = 0; q < 4; ++q) a[q] = ((w[q] << s) & 0x80008000u) | 0x3C003C00u;
  return a;
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowRor8 = 0x128;        // lane i <- lane (i + 8) mod 16 of its row
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7 - i of its 8-lane half
constexpr int kDppQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]

// Sum a C fragment (lane L holds rows 4 (L/16) + v, v = 0..3, of column L % 16) over
// the 16 columns, in registers (DPP).  Returns, in every lane, the sum for row
// 4 (L/16) + vsel(L) with vsel(L) = 2 ((L >> 3) & 1) + ((L >> 2) & 1); lanes with
// L % 4 == 0 hold distinct rows.  Round 1 pairs lanes L, L^8 and keeps rows {0,1} or
// {2,3}; round 2 pairs L with 7 - L (other half of its bit-2 group) and keeps one row;
// rounds 3-4 add over the quad.
__device__ __forceinline__ float reduce_columns(float4v a, int lane) {
  const bool hi8 = lane & 8, hi4 = lane & 4;
  const float keep0 = hi8 ? a[2] : a[0], keep1 = hi8 ? a[3] : a[1];
  const float send0 = hi8 ? a[0] : a[2], send1 = hi8 ? a[1] : a[3];
  const float k0 = keep0 + dpp_mov<kDppRowRor8>(send0);
  const float k1 = keep1 + dpp_mov<kDppRowRor8>(send1);
  const float keep = hi4 ? k1 : k0, send = hi4 ? k0 : k1;
  float r = keep + dpp_mov<kDppRowHalfMirror>(send);
  r += dpp_mov<kDppQuadSwap2>(r);
  r += dpp_mov<kDppQuadSwap1>(r);
  return r;
}

// Sum over the four 16-lane groups (lanes L, L^16, L^32, L^48).
__device__ __forceinline__ float sum_over_lane_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ int reduced_row(int lane) { return 4 * (lane >> 4) + 2 * ((lane >> 3) & 1) + ((lane >> 2) & 1); }

__device__ __forceinline__ void store_y(void* y, size_t idx, float v, int fp32) {
  if (fp32) reinterpret_cast<float*>(y)[idx] = v;
  else reinterpret_cast<_Float16*>(y)[idx] = (_Float16)v;
}

// Workgroup barrier that orders LDS accesses only.  Unlike __syncthreads() it does not
// wait for this wave's outstanding global loads, so prefetches stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Pick the descriptor of the weight that owns `item` (uniform across the wave).
__device__ __forceinline__ WeightDesc find_weight(const GroupArgs& args, int item) {
  WeightDesc W = args.w[0];
#pragma unroll
  for (int j = 1; j < kMaxGroup; ++j)
    if (j < args.count && item >= args.w[j].item_begin) W = args.w[j];
  return W;
}

// ============================================================ single-token kernel
// Persistent workgroups of NW waves.  The work is a list of units (weight, row group of
// NW R = 64 row tiles, block, 512-column chunk) in that order; with U units and G
// workgroups, workgroup L walks units [L U / G, (L + 1) U / G).
//
// For every unit the workgroup builds the chunk's Z tile once, in LDS (double buffered;
// wave w builds planes PP w .. PP w + PP - 1) and each wave runs its R row tiles against
// it, accumulating the raw products over the chunks of a block in registers.  After a
// block's last chunk (or the end of the range) the products get the block's column-sum
// term and are weighted by U (the r-sum is linear, so a block split over two workgroups
// is fine); after a row group's last unit (or the end of the range) each wave sums its
// tiles over r and stores the workgroup's 1024-row "piece" of the row group.  At the end
// of its range the workgroup counts itself in for every row group it touched; the last
// workgroup to arrive at a row group adds its pieces in workgroup order and writes y.
//
// Sign tiles are fetched one unit ahead, V fragments and activations two units ahead and
// U fragments one unit ahead, across block, row-group and weight boundaries, so the HBM
// stream never waits on compute; fetches past the end of the range read a page of zeros.
// Sign tiles are read once, so they are loaded non-temporally and leave the L2 to the V
// and U fragments that other workgroups re-read.  Nothing waits on outstanding loads
// before the end of the range.
struct DecodeCursor {
  int32_t j, rg, i, ch;  // weight slot in the launch, row group, block, chunk
  uint32_t u;            // unit index
  bool valid;            // false past the end of the workgroup's range
  // fields of weight j, kept in scalar registers (reloaded only when j changes)
  int32_t nb, nch, groups, mt, d;
  uint32_t rg_begin;
  const uint16_t* x;
};

// Units [start(o), start(o + 1)) belong to workgroup o.
__device__ __forceinline__ uint32_t range_start(uint32_t o, uint32_t units, int lg) {
  return (uint32_t)(((uint64_t)o * units) >> lg);
}

template <int NW, int R, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void decode_m1_kernel(GroupArgs args) {
  static_assert(NW * R == kDecodeGroupTiles && kPlanes % NW == 0 && R == 4, "decode tiling");
  constexpr int PP = kPlanes / NW;       // Z planes each wave builds
  __shared__ u32x4 zs[2][kPlanes][64];   // Z fragments of two units (32 KiB)
  __shared__ float csum[2][NW][16];      // per-wave column sums of Z over a block's chunks
  __shared__ float4v accl[NW][R][64];    // U-weighted accumulators (LDS, not registers)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const uint32_t U = args.total_units;
  const int lg = args.grid_log2;
  const uint32_t G = 1u << lg;
  // Workgroups are dealt round-robin over the XCDs; give each XCD a contiguous share of
  // the units, so the workgroups sharing an L2 also share V and U fragments.
  const uint32_t bid = blockIdx.x;
  const uint32_t L = G >= (uint32_t)kXcds ? (bid % kXcds) * (G / kXcds) + bid / kXcds : bid;
  const uint32_t u_begin = range_start(L, U, lg), u_end = range_start(L + 1, U, lg);
  const uint8_t* zero_page = static_cast<const uint8_t*>(args.zero_page);
  // A weight without blocks has no units: y = 0, the empty sum (written by workgroup 0).
  if (L == 0) {
    for (int j = 0; j < args.count; ++j)
      if (args.w[j].units == 0)
        for (int row = threadIdx.x; row < args.w[j].m; row += NW * 64) store_y(args.w[j].y, row, 0.f, args.y_fp32);
  }
  if (U == 0) return;

  // Base address of every loaded block of every weight of the launch, in LDS (a block's
  // signs, U and V share one allocation, in that order), so that the unit loop issues no
  // scalar loads: on this hardware those share a wait counter with LDS reads, and every
  // LDS wait would also wait for them.
  __shared__ uint64_t bbase[kMaxGroup][kMaxBlocks];

  // ---- cursor over the unit list (wave-uniform state)
  auto load_weight = [&](DecodeCursor& c) {
    const WeightDesc& W = args.w[c.j];
    c.nb = W.nblocks;
    c.nch = W.nch;
    c.groups = W.groups;
    c.mt = W.mt;
    c.d = W.d;
    c.rg_begin = W.rg_begin;
    c.x = W.x;
  };
  auto locate = [&](uint32_t u) {
    DecodeCursor c;
    int j = 0;
    while (j + 1 < args.count && u >= args.w[j + 1].unit_begin) ++j;
    c.j = j;
    load_weight(c);
    const uint32_t local = u - args.w[j].unit_begin;
    const uint32_t per_rg = (uint32_t)c.nch * c.nb;
    c.rg = local / per_rg;
    const uint32_t rem = local - c.rg * per_rg;
    c.i = rem / c.nch;
    c.ch = rem - c.i * c.nch;
    c.u = u;
    c.valid = true;
    return c;
  };
  auto next = [&](DecodeCursor c) {
    if (!c.valid || c.u + 1 >= u_end) {
      c.valid = false;
      return c;
    }
    ++c.u;
    if (++c.ch == c.nch) {
      c.ch = 0;
      if (++c.i == c.nb) {
        c.i = 0;
        if (++c.rg == c.groups) {
          c.rg = 0;
          do ++c.j;
          while (args.w[c.j].units == 0);
          load_weight(c);
        }
      }
    }
    return c;
  };
  // the unit closes this workgroup's share of a block / of a row group
  auto block_end = [&](const DecodeCursor& c) { return c.ch == c.nch - 1 || c.u + 1 == u_end; };
  auto group_end = [&](const DecodeCursor& c) { return (c.ch == c.nch - 1 && c.i == c.nb - 1) || c.u + 1 == u_end; };
  // Per-wave base addresses of a unit's loads (the zero page for an invalid cursor).
  struct UnitPtrs {
    const uint8_t* signs;
    const uint16_t* u;
    const uint16_t* v;
    const uint16_t* x;
    int32_t xcols;  // valid activation columns from x (the rest read zeros)
  };
  // (`direct` reads the block's base from the device table instead: the prologue does,
  // so its first loads do not wait for the LDS copy of the table)
  auto unit_ptrs = [&](const DecodeCursor& c, bool direct = false) {
    UnitPtrs p;
    if (c.valid) {
      const uint8_t* base = direct ? load_block(args.w[c.j].blocks, c.i).signs
                                   : uniform_ptr(reinterpret_cast<const uint8_t*>(bbase[c.j][c.i]));
      const size_t sign_bytes = (size_t)c.mt * c.nch * kTileBytes;
      const int rt0 = c.rg * kDecodeGroupTiles + wave * R;
      p.signs = base + ((size_t)c.ch * c.mt + rt0) * kTileBytes;
      p.u = reinterpret_cast<const uint16_t*>(base + sign_bytes) + (size_t)rt0 * 64 * 4;
      p.v = reinterpret_cast<const uint16_t*>(base + sign_bytes + (size_t)c.mt * 64 * 4 * 2) +
            ((size_t)c.ch * kPlanes + PP * wave) * 64 * 8;
      p.x = c.x + (size_t)c.ch * kChunkCols;
      p.xcols = c.d - c.ch * kChunkCols;
    } else {
      p.signs = zero_page;
      p.u = reinterpret_cast<const uint16_t*>(zero_page);
      p.v = reinterpret_cast<const uint16_t*>(zero_page);
      p.x = reinterpret_cast<const uint16_t*>(zero_page);
      p.xcols = 0;
    }
    return p;
  };

  // ---- loads.  Every load is issued unconditionally (padding rows are stored with +1
  // signs and zero U, and out-of-range addresses are redirected to the zero page), so
  // the number of loads in flight is the same on every path and the compiler's in-order
  // wait counts never drain the prefetches.
  u32x4 raw[R], rawn[R];  // sign words of the current and the next unit
  u32x2 uf[R];
  u32x4 vv[PP], xv[PP];
  auto load_signs = [&](const UnitPtrs& p, u32x4* rw) {
#pragma unroll
    for (int t = 0; t < R; ++t) rw[t] = load16_stream(p.signs + t * kTileBytes + lane * 16);
  };
  auto load_u = [&](const UnitPtrs& p) {
#pragma unroll
    for (int t = 0; t < R; ++t) uf[t] = load8(p.u + (t * 64 + lane) * 4);
  };
  auto load_vx = [&](const UnitPtrs& p) {
#pragma unroll
    for (int q = 0; q < PP; ++q) {
      vv[q] = load16(p.v + (q * 64 + lane) * 8);
      const int col = 32 * (PP * wave + q) + 8 * g;
      xv[q] = load16(col < p.xcols ? static_cast<const void*>(p.x + col) : static_cast<const void*>(zero_page));
    }
  };
  // Z fragments of this wave's PP planes (V times the plane-scaled activations).  Their
  // column sums over the chunk are added up over the block's chunks; the total goes to
  // LDS with the block's last chunk (parity `wpar` alternates per block).
  float cs_run = 0.f;
  int wpar = 0, rpar = 0;
  auto build_z = [&](int buf, const DecodeCursor& c) {
    float cs = 0.f;
#pragma unroll
    for (int q = 0; q < PP; ++q) {
      const int b = PP * wave + q;
      const half2v f = as_half2(plane_x_factor_bits_dyn(b) * 0x00010001u);
      const half2v inv = as_half2(plane_inv_factor_bits_dyn(b) * 0x00010001u);
      u32x4 z;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const half2v zq = as_half2(vv[q][k]) * (as_half2(xv[q][k]) * f);
        z[k] = as_u32(zq);
        cs = __builtin_amdgcn_fdot2(zq, inv, cs, false);
      }
      zs[buf][b][lane] = z;
    }
    cs_run += sum_over_lane_groups(cs);
    if (c.valid && block_end(c)) {
      // the sums are replicated in the four 16-lane groups; every lane stores its r's
      csum[wpar][wave][r16] = cs_run;
      cs_run = 0.f;
      wpar ^= 1;
    }
  };

  float4v acc[R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    acc[t] = (float4v){0.f, 0.f, 0.f, 0.f};
    accl[wave][t][lane] = (float4v){0.f, 0.f, 0.f, 0.f};
  }
  // After a block: U-weight the products (plus the block's column-sum term) into LDS.
  auto weight_block = [&]() {
    float cs_tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) cs_tot += csum[rpar][w][r16];
    cs_tot *= kPlaneAccScale;
    rpar ^= 1;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const half2v u01 = as_half2(uf[k][0]), u23 = as_half2(uf[k][1]);
      float4v a = accl[wave][k][lane];
      a[0] += (float)u01[0] * (acc[k][0] + cs_tot);
      a[1] += (float)u01[1] * (acc[k][1] + cs_tot);
      a[2] += (float)u23[0] * (acc[k][2] + cs_tot);
      a[3] += (float)u23[1] * (acc[k][3] + cs_tot);
      accl[wave][k][lane] = a;
      acc[k] = (float4v){0.f, 0.f, 0.f, 0.f};
    }
  };
  // After a row group: this workgroup's piece of it, summed over r.  Stored write-through
  // at device scope: the workgroup that adds the pieces may sit on another XCD.
  const int rsel = reduced_row(lane);
  auto store_piece = [&](const DecodeCursor& c) {
    const uint32_t item = c.rg_begin + c.rg;
    float* piece = args.pieces + (size_t)(item + L) * kDecodeGroupRows;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const float v = reduce_columns(accl[wave][t][lane], lane);
      accl[wave][t][lane] = (float4v){0.f, 0.f, 0.f, 0.f};
      if ((lane & 3) == 0)
        __hip_atomic_store(&piece[(wave * R + t) * kTileRows + rsel], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // ---- prologue: the first unit's signs, Z tile and U fragments, the second unit's V
  // fragments and activations
  DecodeCursor c0 = locate(u_begin);
  DecodeCursor c1 = next(c0);
  DecodeCursor c2 = next(c1);
  const UnitPtrs p0 = unit_ptrs(c0, true);
  UnitPtrs p1 = unit_ptrs(c1, true);
  UnitPtrs p2 = unit_ptrs(c2, true);
  load_vx(p0);
  load_signs(p0, raw);
  __builtin_amdgcn_sched_barrier(0);
  {
    const int j = threadIdx.x / kMaxBlocks, i = threadIdx.x % kMaxBlocks;
    if (j < args.count && i < args.w[j].nblocks) {
      const u32x2 t = load8(&args.w[j].blocks[i].signs);
      bbase[j][i] = t[0] | ((uint64_t)t[1] << 32);
    }
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  build_z(0, c0);  // (waits only for the first unit's V fragments and activations)
  __builtin_amdgcn_sched_barrier(0);
  load_signs(p1, rawn);
  load_vx(p1);
  load_u(p0);

  // ---- one unit.  On entry unit c0's signs are in `cur` and unit c1's in the other
  // buffer, c0's Z tile in zs[buf], its U fragments in uf, and unit c1's V fragments
  // and activations in vv / xv.  Unit c2's signs are fetched into `cur` as soon as the
  // tiles are done with it, so a sign tile is requested well over one unit ahead.
  auto step = [&](u32x4 (&cur)[R], const int buf) {
    lds_barrier();  // Z of c0 (and the column sums of a finished block) are complete
    {
      // Row tiles: four independent accumulator chains per plane.  Planes 6-11 are read
      // from the words as loaded; the words are then rotated right by 6 in place (planes
      // 12-15 land on bits 6-9) and by 20 more (planes 0-5 land on bits 6-11), so no
      // second copy of the words is kept.  Z fragments are read from LDS one plane ahead.
      u32x4 zf[2];
      zf[0] = zs[buf][plane_order(0)][lane];
      // (a scheduling barrier per plane keeps the compiler from computing fragments of
      // later planes early, which would raise register pressure past two waves/SIMD)
#define BSL_PLANE(S)                                                                                              \
  __builtin_amdgcn_sched_barrier(0);                                                                              \
  if ((S) + 1 < kPlanes) zf[((S) + 1) % 2] = zs[buf][plane_order((S) + 1)][lane];                              \
  _Pragma("unroll") for (int k = 0; k < R; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(                \
      as_half8(cur[k] & (0x00010001u << plane_pos(plane_order(S)))), as_half8(zf[(S) % 2]), acc[k], 0, 0, 0);
#define BSL_ROTATE(N)                                                                                             \
  _Pragma("unroll") for (int k = 0; k < R; ++k) _Pragma("unroll") for (int q = 0; q < 4; ++q) cur[k][q] =      \
      __builtin_amdgcn_alignbit(cur[k][q], cur[k][q], (N));
      BSL_PLANE(0) BSL_PLANE(1) BSL_PLANE(2) BSL_PLANE(3) BSL_PLANE(4) BSL_PLANE(5)
      BSL_ROTATE(6)
      BSL_PLANE(6) BSL_PLANE(7) BSL_PLANE(8) BSL_PLANE(9)
      BSL_ROTATE(20)
      BSL_PLANE(10) BSL_PLANE(11) BSL_PLANE(12) BSL_PLANE(13) BSL_PLANE(14) BSL_PLANE(15)
#undef BSL_ROTATE
#undef BSL_PLANE
    }
    __builtin_amdgcn_sched_barrier(0);
    load_signs(p2, cur);
    __builtin_amdgcn_sched_barrier(0);
    if (block_end(c0)) weight_block();
    __builtin_amdgcn_sched_barrier(0);
    build_z(buf ^ 1, c1);
    __builtin_amdgcn_sched_barrier(0);
    if (group_end(c0)) store_piece(c0);
    load_vx(p2);
    load_u(p1);
    c0 = c1;
    c1 = c2;
    p1 = p2;
    c2 = next(c2);
    p2 = unit_ptrs(c2);
  };

  const uint32_t n = u_end - u_begin;
  const uint32_t item_first = c0.rg_begin + c0.rg;
  for (uint32_t s = 0; s < n; s += 2) {
    step(raw, 0);
    if (s + 1 < n) step(rawn, 1);
  }

  // ---- end of the range: count this workgroup in for every row group it touched; the
  // last one to arrive at a row group adds the pieces (one per workgroup owner(first) ..
  // owner(last), in that order) and writes y.
  __shared__ uint32_t last_items[kDecodeGroupRows];
  __shared__ uint32_t n_last;
  const uint32_t tid = threadIdx.x;
  auto owner = [&](uint32_t u) {
    uint32_t o = (uint32_t)(((uint64_t)u << lg) / U);
    while (o + 1 < G && range_start(o + 1, U, lg) <= u) ++o;
    while (range_start(o, U, lg) > u) --o;
    return o;
  };
  // global row group -> its weight slot and its first and last unit
  auto group_units = [&](uint32_t item, uint32_t& first, uint32_t& last) {
    int j = 0;
    while (j + 1 < args.count && item >= args.w[j + 1].rg_begin) ++j;
    const WeightDesc& W = args.w[j];
    const uint32_t per_rg = (uint32_t)W.nblocks * W.nch;
    first = W.unit_begin + (item - W.rg_begin) * per_rg;
    last = first + per_rg - 1;
    return j;
  };
  // row group of the range's last unit
  int je = 0;
  while (je + 1 < args.count && u_end - 1 >= args.w[je + 1].unit_begin) ++je;
  const uint32_t item_last = args.w[je].rg_begin + (u_end - 1 - args.w[je].unit_begin) / ((uint32_t)args.w[je].nch * args.w[je].nblocks);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's piece stores have completed
  __syncthreads();
  // row groups of the range, 512 at a time: one thread each counts the workgroup in
  for (uint32_t k0 = 0; k0 <= item_last - item_first; k0 += kDecodeGroupRows) {
    if (tid == 0) n_last = 0;
    __syncthreads();
    if (k0 + tid <= item_last - item_first) {
      const uint32_t item = item_first + k0 + tid;
      uint32_t first, last;
      group_units(item, first, last);
      const uint32_t expected = owner(last) - owner(first) + 1;
      const uint32_t seen = __hip_atomic_fetch_add(&args.arrivals[item], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
      if (seen == expected) {
        __hip_atomic_store(&args.arrivals[item], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_items[atomicAdd(&n_last, 1u)] = item;
      }
    }
    __syncthreads();
    const uint32_t nl = n_last;
    for (uint32_t k = 0; k < nl; ++k) {
      const uint32_t item = __builtin_amdgcn_readfirstlane(last_items[k]);
      uint32_t first, last;
      const int j = group_units(item, first, last);
      const WeightDesc& W = args.w[j];
      const uint32_t o0 = owner(first), o1 = owner(last);
      const float* base = args.pieces + (size_t)item * kDecodeGroupRows + tid;
      float acc_y = 0.f;
      for (uint32_t o = o0; o <= o1; o += 32) {  // (32 loads in flight per round trip)
        float v[32];
#pragma unroll
        for (int q = 0; q < 32; ++q)
          v[q] = __hip_atomic_load(base + (size_t)min(o + q, o1) * kDecodeGroupRows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int q = 0; q < 32; ++q) acc_y += o + q <= o1 ? v[q] : 0.f;
      }
      const int row = (int)(item - W.rg_begin) * kDecodeGroupRows + tid;
      if (row < W.m) store_y(W.y, row, acc_y * kPlaneOutScale, args.y_fp32);
    }
    __syncthreads();  // n_last and last_items are rewritten by the next batch
  }
}

// ============================================================ multi-token kernel
// M >= 2.  One workgroup of 8 waves per item = (weight, 512-row group, T-token group,
// range of the (block, chunk) sequence), T = 2, 4 or 8; wave w owns rows 64 w .. 64 w + 63
// as two 32-row fragments against the T tokens as T / 2 token pairs, i.e. 2 x T / 2
// accumulators of v_mfma_f32_32x32x16_f16 (32 rows x (2 tokens x 16 r)): the N width
// 2 x 16 = 32 is filled exactly, and each +-1 A fragment feeds T / 2 MFMAs.  Z is built
// 4 planes (128 columns) at a time into double-buffered LDS as B fragments; sign words
// for the next chunk and V / activations for the next 4 planes are fetched while the
// current ones run.  After a block's K loop (or the end of the item's range) the
// accumulators are weighted by U and summed over r with a 16-lane butterfly.  When a
// weight has too few items to fill the chip its (block, chunk) sequence is cut into
// ranges; each range stores its partial sums and the last of them to finish adds all
// ranges in order.
//
// Operand layouts (v_mfma_f32_32x32x16_f16): lane l holds A[l % 32][8 (l / 32) + e] and
// B[8 (l / 32) + e][l % 32], e = 0..7; C[m][n] sits in lane n + 32 ((m / 4) % 2), value
// 4 (m / 8) + m % 4.  K step s (0, 1) of plane b covers the plane's columns 16 s .. 16 s +
// 15, which the stored tiles hold in lane group 2 s + l / 32 of row l % 32: a lane loads
// the 16 stored bytes of that (row, group) and gets every plane of it.
typedef float float16v __attribute__((ext_vector_type(16)));
constexpr int kPrefillPlanes = 4;  // planes per Z stage

// Sum 16 values over the 16 lanes of a DPP row; lane r ends with the sum of value r.
// Four butterfly stages (partners r^8, r^7, r^2, r^1) halve the values each time.
__device__ __forceinline__ float reduce16x16(float (&v)[16], int lane) {
  const int r = lane & 15;
  float a[8], b2[4], c2[2];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float keep = (r & 8) ? v[8 + k] : v[k], send = (r & 8) ? v[k] : v[8 + k];
    a[k] = keep + dpp_mov<kDppRowRor8>(send);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = (r & 4) ? a[4 + k] : a[k], send = (r & 4) ? a[k] : a[4 + k];
    b2[k] = keep + dpp_mov<kDppRowHalfMirror>(send);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = (r & 2) ? b2[2 + k] : b2[k], send = (r & 2) ? b2[k] : b2[2 + k];
    c2[k] = keep + dpp_mov<kDppQuadSwap2>(send);
  }
  const float keep = (r & 1) ? c2[1] : c2[0], send = (r & 1) ? c2[0] : c2[1];
  return keep + dpp_mov<kDppQuadSwap1>(send);
}

template <int T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(GroupArgs args, int token_groups) {
  constexpr int NP = T / 2, PL = kPrefillPlanes;
  constexpr int FRAGS = PL * 2 * NP;          // B fragments per stage (32 for 8 tokens)
  constexpr int FPW = FRAGS / 8;              // built per wave
  __shared__ u32x4 zs[2][FRAGS][64];          // [stage buffer][(plane, step, pair)][lane], 64 KiB for 8 tokens
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kg = lane >> 5;                   // K group of this lane (A and B)
  const int n32 = lane & 31;
  const WeightDesc W = find_weight(args, blockIdx.x);
  const int local = blockIdx.x - W.item_begin;
  // the (block, chunk) sequence i * nch + ch is cut into W.splits equal ranges
  const int split = local % W.splits;
  const int rest = local / W.splits;
  const int tg = rest % token_groups;
  const int rg = rest / token_groups;
  const int M = args.M;
  const int tok0 = tg * T;
  const int row0 = rg * kPrefillGroupRows + wave * 64;  // this wave's first row
  const int nch = W.nch;
  const int units = W.nblocks * nch;
  const int ups = (units + W.splits - 1) / W.splits;
  const int u_begin = min(units, split * ups);
  const int u_end = min(units, u_begin + ups);
  const uint8_t* zero_page = static_cast<const uint8_t*>(args.zero_page);

  // sign words: [fragment rf][K step s] = the 16 stored bytes of (row row0 + 32 rf + l % 32,
  // lane group 2 s + kg) of the current chunk
  auto load_signs = [&](const BlockPtrs& bp, int ch, u32x4 (&w)[2][2]) {
#pragma unroll
    for (int rf = 0; rf < 2; ++rf) {
      const int row = row0 + 32 * rf + n32;
      const uint8_t* tile = bp.signs + ((size_t)ch * W.mt + (row >> 4)) * kTileBytes;
#pragma unroll
      for (int st = 0; st < 2; ++st) w[rf][st] = load16(tile + ((row & 15) + 16 * (2 * st + kg)) * 16);
    }
  };
  // V fragment and activations of this wave's B fragments of stage (ch, q)
  auto load_vx = [&](const BlockPtrs& bp, int ch, int q, u32x4 (&vv)[FPW], u32x4 (&xv)[FPW]) {
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
      const int id = wave * FPW + f;          // (plane pl, step st, pair pp)
      const int pl = id / (2 * NP), st = (id / NP) % 2, pp = id % NP;
      const int b = q * PL + pl;
      vv[f] = load16(bp.v + (((size_t)ch * kPlanes + b) * 64 + (lane & 15) + 16 * (2 * st + kg)) * 8);
      const int tok = tok0 + 2 * pp + (n32 >> 4);
      const int col = ch * kChunkCols + 32 * b + 16 * st + 8 * kg;
      const bool ok = tok < M && col < W.d;
      xv[f] = load16(ok ? static_cast<const void*>(W.x + (size_t)tok * W.d + col) : static_cast<const void*>(zero_page));
    }
  };
  auto build = [&](int buf, const u32x4 (&vv)[FPW], const u32x4 (&xv)[FPW]) {
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
      u32x4 z;
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = as_u32(as_half2(vv[f][e]) * as_half2(xv[f][e]));
      zs[buf][wave * FPW + f][lane] = z;
    }
  };

  float yacc[2][NP];
#pragma unroll
  for (int rf = 0; rf < 2; ++rf)
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) yacc[rf][pp] = 0.f;

  const int stages = (u_end - u_begin) * (kPlanes / PL);
  if (stages > 0) {
    u32x4 w[2][2], wn[2][2];
    u32x4 vv[FPW], xv[FPW];
    float16v acc[2][NP];
#pragma unroll
    for (int rf = 0; rf < 2; ++rf)
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) acc[rf][pp] = (float16v){};
    int i = u_begin / nch, ch = u_begin % nch, q = 0;  // current stage
    BlockPtrs bp = load_block(W.blocks, i);
    load_signs(bp, ch, w);
    load_vx(bp, ch, 0, vv, xv);
    build(0, vv, xv);
    for (int sidx = 0; sidx < stages; ++sidx) {
      const int buf = sidx & 1;
      // next stage
      int ni = i, nc = ch, nq = q + 1;
      if (nq == kPlanes / PL) { nq = 0; if (++nc == nch) { nc = 0; ++ni; } }
      const bool more = sidx + 1 < stages;
      const BlockPtrs nbp = load_block(W.blocks, more ? ni : i);
      lds_barrier();  // Z of this stage is in zs[buf]; zs[buf ^ 1] is free
      if (nq == 0 && more) load_signs(nbp, nc, wn);
      load_vx(more ? nbp : bp, more ? nc : ch, more ? nq : q, vv, xv);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) {
        const int b = q * PL + pl;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const half8 a0 = as_half8(pm1_fragment(w[0][st], b));
          const half8 a1 = as_half8(pm1_fragment(w[1][st], b));
#pragma unroll
          for (int pp = 0; pp < NP; ++pp) {
            const half8 bf = as_half8(zs[buf][(pl * 2 + st) * NP + pp][lane]);
            acc[0][pp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, bf, acc[0][pp], 0, 0, 0);
            acc[1][pp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, bf, acc[1][pp], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) build(buf ^ 1, vv, xv);
      // after a block's last stage, or the range's: U weighting and the sum over r
      if ((nq == 0 && nc == 0) || !more) {
#pragma unroll
        for (int rf = 0; rf < 2; ++rf) {
          // U[row(v)][r] for v = 0..15: rows 8 (v / 4) + 4 kg + v % 4 of the fragment
          half2v uu[8];
          const int rbase = row0 + 32 * rf;
#pragma unroll
          for (int vg = 0; vg < 4; ++vg) {
            const int tile = (rbase >> 4) + (vg >> 1);
            const u32x2 u = load8(bp.u + ((size_t)tile * 64 + (lane & 15) + 16 * (2 * (vg & 1) + kg)) * 4);
            uu[2 * vg] = as_half2(u[0]);
            uu[2 * vg + 1] = as_half2(u[1]);
          }
#pragma unroll
          for (int pp = 0; pp < NP; ++pp) {
            float v[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = acc[rf][pp][e] * (float)uu[e >> 1][e & 1];
            yacc[rf][pp] += reduce16x16(v, lane);
            acc[rf][pp] = (float16v){};
          }
        }
      }
      if (nq == 0 && more) {
#pragma unroll
        for (int rf = 0; rf < 2; ++rf)
#pragma unroll
          for (int st = 0; st < 2; ++st) w[rf][st] = wn[rf][st];
      }
      bp = nbp;
      i = ni;
      ch = nc;
      q = nq;
    }
  }
  // lane l holds, for each (fragment, pair), row 8 (v / 4) + 4 kg + v % 4 with v = l % 16,
  // token 2 pair + (l % 32) / 16
  const int v = lane & 15;
  if (W.splits == 1) {
#pragma unroll
    for (int rf = 0; rf < 2; ++rf) {
      const int row = row0 + 32 * rf + 8 * (v >> 2) + 4 * kg + (v & 3);
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int tok = tok0 + 2 * pp + (n32 >> 4);
        if (row < W.m && tok < M) store_y(W.y, (size_t)tok * W.m + row, yacc[rf][pp], args.y_fp32);
      }
    }
    return;
  }
  // Split over blocks: partial[split][token][row] (write-through at device scope), then
  // the last workgroup of the (row group, token group) adds the splits in order.
  const int mpad = token_groups * T;
  const int rows_pad = W.mt * kTileRows;
#pragma unroll
  for (int rf = 0; rf < 2; ++rf) {
    const int row = row0 + 32 * rf + 8 * (v >> 2) + 4 * kg + (v & 3);
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int tok = tok0 + 2 * pp + (n32 >> 4);
      __hip_atomic_store(&W.partial[((size_t)split * mpad + tok) * rows_pad + row], yacc[rf][pp], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the write-through stores above have completed
  __syncthreads();                // ... in every wave, and every wave is done with zs
  uint32_t* last = reinterpret_cast<uint32_t*>(&zs[0][0][0]);
  if (threadIdx.x == 0)
    *last = __hip_atomic_fetch_add(&W.counters[rest], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(W.splits - 1);
  __syncthreads();
  if (!*last) return;
  const int rbeg = rg * kPrefillGroupRows;
  for (int e = threadIdx.x; e < kPrefillGroupRows * T; e += 512) {
    const int t = e / kPrefillGroupRows, row = rbeg + e % kPrefillGroupRows;
    const int tok = tok0 + t;
    float sum = 0.f;
    for (int sp = 0; sp < W.splits; ++sp)
      sum += __hip_atomic_load(&W.partial[((size_t)sp * mpad + tok) * rows_pad + row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (row < W.m && tok < M) store_y(W.y, (size_t)tok * W.m + row, sum, args.y_fp32);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&W.counters[rest], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ============================================================ debug unpack
// One wave per sign tile: unpack exactly as the forward kernels do and write +-1.
__global__ __launch_bounds__(64) void debug_unpack_kernel(BlockPtrs blk, int32_t m, int32_t d, int32_t mt, int path,
                                                          int8_t* out) {
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int ch = tile / mt, rt = tile % mt;
  const u32x4 w = load16(blk.signs + (size_t)tile * kTileBytes + lane * 16);
  const u32x4 lo = w << 6u, hi = w >> 6u;
  const int row = rt * kTileRows + (lane & 15);
  const int g = lane >> 4;
  u32x4 fr[kPlanes];
  if (path == 0) {
    fr[0] = plane_fragment<0>(w, lo, hi);
    fr[1] = plane_fragment<1>(w, lo, hi);
    fr[2] = plane_fragment<2>(w, lo, hi);
    fr[3] = plane_fragment<3>(w, lo, hi);
    fr[4] = plane_fragment<4>(w, lo, hi);
    fr[5] = plane_fragment<5>(w, lo, hi);
    fr[6] = plane_fragment<6>(w, lo, hi);
    fr[7] = plane_fragment<7>(w, lo, hi);
    fr[8] = plane_fragment<8>(w, lo, hi);
    fr[9] = plane_fragment<9>(w, lo, hi);
    fr[10] = plane_fragment<10>(w, lo, hi);
    fr[11] = plane_fragment<11>(w, lo, hi);
    fr[12] = plane_fragment<12>(w, lo, hi);
    fr[13] = plane_fragment<13>(w, lo, hi);
    fr[14] = plane_fragment<14>(w, lo, hi);
    fr[15] = plane_fragment<15>(w, lo, hi);
  } else {
#pragma unroll
    for (int b = 0; b < kPlanes; ++b) fr[b] = pm1_fragment(w, b);
  }
  if (row >= m) return;
#pragma unroll
  for (int b = 0; b < kPlanes; ++b) {
    const half8 h = as_half8(fr[b]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = ch * kChunkCols + 32 * b + 8 * g + j;
      if (col < d) {
        // bit-plane path: a set bit is a non-zero element and means -1; +-1 path: the value itself
        const float v = (float)h[j];
        out[(size_t)row * d + col] = path == 0 ? (v != 0.f ? -1 : 1) : (v < 0.f ? -1 : 1);
      }
    }
  }
}

// ============================================================ launchers
int launch_decode_m1(const GroupArgs& args, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  // 16 waves x 4 row tiles, 4 waves per SIMD (one workgroup per CU: all waves advance
  // together, so no workgroup is left running alone on a CU at the end).  With no units
  // at all (every weight empty) one workgroup still runs, to write y = 0.
  hipLaunchKernelGGL((decode_m1_kernel<kDecodeWaves, 4, 4>), dim3(1u << args.grid_log2), dim3(kDecodeWaves * 64), 0, st,
                     args);
  return (int)hipGetLastError();
}

int launch_prefill(const GroupArgs& args, int token_tile, int token_groups, void* stream) {
  if (args.total_items == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (token_tile == 2)
    hipLaunchKernelGGL(prefill_kernel<2>, dim3(args.total_items), dim3(512), 0, st, args, token_groups);
  else if (token_tile == 4)
    hipLaunchKernelGGL(prefill_kernel<4>, dim3(args.total_items), dim3(512), 0, st, args, token_groups);
  else if (token_tile == 8)
    hipLaunchKernelGGL(prefill_kernel<8>, dim3(args.total_items), dim3(512), 0, st, args, token_groups);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_debug_unpack(BlockPtrs blk, int32_t m, int32_t d, int32_t mt, int32_t nch, int path, int8_t* out,
                        void* stream) {
  hipLaunchKernelGGL(debug_unpack_kernel, dim3(mt * nch), dim3(64), 0, static_cast<hipStream_t>(stream), blk, m, d, mt,
                     path, out);
  return (int)hipGetLastError();
}

}  // namespace bsl
