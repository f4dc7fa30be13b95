// HIP kernels of libbitstack_linear for gfx950 (MI355X).
//
// The layer (BitStack OpenReview discussion, weight-restoration reply; paper-review
// page, Figure 3 caption) is y = x W_hat^T with W_hat = sum_i S_i * (U_i V_i^T).  By
// linearity,
//     y[t, j] = sum_i sum_r U_i[j, r] * P_i[j, (t, r)],   P_i = S_i Z_i,
//     Z_i[c, (t, r)] = V_i[c, r] * x[t, c],
// so each block costs one dense contraction of the sign matrix with Z_i (width 16 M)
// on the matrix cores (fp16 inputs, fp32 accumulation), a Hadamard product with U_i
// and a sum over r that is done once for all blocks.
//
// Signs stay packed at one bit per entry in HBM; the stored tiles keep each 32-column
// plane's bits at the odd or at the even bit positions of one 16-bit half of a word.
//  * single-token kernel (M = 1): the contraction runs on the 2:4 structured-sparse MFMA
//    v_smfmac_f32_16x16x64_f16, used so that the packed sign bits ARE the sparse
//    indices and no sign is ever expanded to an fp16 value.  Every 4-row group of the B
//    operand holds two activation columns a, b in both signs and the A operand is all
//    ones; the group's two index fields pick one row each:
//        "odd" form  rows [+Z_a, +Z_b, -Z_a, -Z_b]: idx0 = 2 s_a,  idx1 = 2 s_b + 1
//        "even" form rows [+Z_a, -Z_a, +Z_b, -Z_b]: idx0 = s_a,    idx1 = s_b + 2
//    (s = 1 for a -1 sign), so the MFMA adds exactly +-Z_a +- Z_b: P = S Z with no
//    rounding beyond the fp32 accumulation.  A plane's index is the stored word with the
//    other bits masked off and the two constant index bits ORed in: one v_and_or_b32
//    serves two planes (the MFMA's abid field picks the half).  The sparse MFMA issues at
//    the dense rate, so the contraction costs what the dense one does while the unpack
//    falls from four VALU operations per MFMA to half of one.
//  * multi-token kernel (M >= 2): dense v_mfma_f32_32x32x16_f16 on exact +-1 fp16 A
//    fragments (a packed 16-bit shift and one AND-OR per word); there the unpack is
//    amortised over the token pairs, and the sparse 32x32 MFMA measured slower.
//  * tile-reconstruct kernel (batches): the other formulation of the same layer.  W_hat
//    is restored tile by tile in registers (one K = 16 MFMA per block and 32 x 32 tile,
//    signs applied as +-1 fp16 pairs) and multiplied at once with up to 512 tokens, so
//    the sign and low-rank work is paid once per token group instead of once per token.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <type_traits>
#include <utility>

#include "bsl_internal.h"

namespace bsl {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef _Float16 half16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// Stored tile layout (16 rows x 512 columns, 1 KiB): lane L = 16 g + i holds row i and,
// of every 32-column plane b, the columns 8 g .. 8 g + 7, in four little-endian words.
// Plane b lives in word b / 4, half b % 2, at the odd bit positions if (b / 2) % 2 == 0
// and at the even ones otherwise: column 8 g + e of the plane is bit 16 (b % 2) + 2 e +
// 1 - (b / 2) % 2.  A set bit is a -1 sign.
__host__ __device__ constexpr int plane_word(int b) { return b >> 2; }
__host__ __device__ constexpr int plane_half(int b) { return b & 1; }
__host__ __device__ constexpr int plane_even(int b) { return (b >> 1) & 1; }

// Sparse-MFMA index of the planes kept at the odd (even = false) or even bit positions
// of stored word w: the planes' bits, plus the constant bit of every 2-bit index field
// (bit 0 of field 2n + 1 for the odd form, bit 1 of field 2n + 1 for the even form).
__device__ __forceinline__ uint32_t sign_index(uint32_t w, bool even) {
  return even ? (w & 0x55555555u) | 0x88888888u : (w & 0xAAAAAAAAu) | 0x44444444u;
}
// The same with the masks passed in registers: VOP3 instructions take no literal
// operands on this target, so with both constants literal the compiler emits an AND and
// an OR; with the mask in a VGPR it is one v_and_or_b32.
__device__ __forceinline__ uint32_t sign_index_v(uint32_t w, uint32_t vmask, bool even) {
  return (w & vmask) | (even ? 0x88888888u : 0x44444444u);
}

// B-operand words of one 4-row group from z = (Z_a, Z_b) (fp16 pair): odd form
// (Z_a, Z_b), (-Z_a, -Z_b); even form (Z_a, -Z_a), (Z_b, -Z_b).
// B operands in LDS are stored as [operand][half][lane] 16-byte pieces, so that every
// ds_read_b128 / ds_write_b128 touches 64 consecutive 16-byte slots (no bank conflicts).
__device__ __forceinline__ void store_operand(u32x4 (&slot)[2][64], int lane, const u32x8& t) {
  slot[0][lane] = (u32x4){t[0], t[1], t[2], t[3]};
  slot[1][lane] = (u32x4){t[4], t[5], t[6], t[7]};
}
__device__ __forceinline__ u32x8 load_operand(const u32x4 (&slot)[2][64], int lane) {
  const u32x4 a = slot[0][lane], b = slot[1][lane];
  return (u32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <bool EVEN>
__device__ __forceinline__ u32x2 group_words(uint32_t z) {
  const uint32_t nz = z ^ 0x80008000u;
  if (EVEN) return (u32x2){__builtin_amdgcn_perm(nz, z, 0x05040100u),   // (z.lo, -z.lo)
                           __builtin_amdgcn_perm(nz, z, 0x07060302u)};  // (z.hi, -z.hi)
  return (u32x2){z, nz};
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
// Loads at a wave-uniform 64-bit base plus a 32-bit per-lane byte offset (one VGPR per
// address instead of two: the base stays in scalar registers).
template <typename T>
__device__ __forceinline__ T load_at(const void* base, uint32_t off) {
  return *reinterpret_cast<const BSL_GLOBAL T*>(reinterpret_cast<uintptr_t>(base) + off);
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

// Partial sums go from the workgroups (or waves) that compute them to the one that adds
// them, which may sit on another XCD.  Every access to them and to the arrival counters
// is an atomic at agent scope, and the ordering is made explicit instead of with agent
// fences, following the gfx950 memory model as the compiler implements it (LLVM AMDGPU
// memory model, GFX942 family):
//  * an atomic store or read-modify-write at agent scope is issued with SC1 set and
//    writes through the XCD's L2; the vector memory counter counts it until the write is
//    acknowledged, so after s_waitcnt vmcnt(0) it is visible to every agent-scope access
//    of the device;
//  * an atomic load at agent scope (SC1) is not served from a non-coherent L2 line;
//  * publish_partials() waits for this wave's stores (vmcnt(0)) before the workgroup
//    barrier that precedes the arrival count, so every partial sum is visible before the
//    count is;
//  * the last arriver's loads of the partial sums are issued after, and only because of,
//    the returned count (a branch on it), so none is performed before the count.
// An agent-scope release fence adds buffer_wbl2 (write back every dirty L2 line) and an
// acquire fence buffer_inv (invalidate the L2); both exist for ordinary, non-atomic
// accesses, which the combines do not make.  Measured on MI355X, the fenced form costs
// 27 us per single-token launch (75 -> 102 us, 8B-shaped layer) and 50 us per split
// tile-path launch at 16 tokens.
__device__ __forceinline__ void publish_partials() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ uint32_t count_arrival(uint32_t* ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Row accumulators of the single- and few-token kernels: one 64-bit word per output row of a
// launch, zero between launches.  Bits 63..58 count the workgroups that have added their
// share of the row, bits 57..0 hold the sum of their shares in fixed point with 28
// fraction bits, each share biased by 2^51 so that the field only grows.  A workgroup
// adds its share with one atomic add that returns the previous word; the one whose add
// completes the count holds the whole sum, writes y and clears the word.  Integer
// addition is associative, so the result does not depend on the order of arrival.  A
// share is rounded to a multiple of 2^-28 (exact for every share that is a multiple of
// 2^-28 below 2^23, such as the integer-valued checks) and clamped to |share| < 2^23.
// At most kAccMaxParts workgroups share a row (the host keeps the grid within that), so
// the count and the biased sum (below 63 * 2^52 < 2^58) never overflow their fields.
constexpr int kAccCountShift = 58;
static_assert(kAccMaxParts < (1 << (64 - kAccCountShift)) && kAccMaxParts * (2ull << 51) < (1ull << kAccCountShift), "row accumulator fields");
constexpr int kAccFracBits = 28;
constexpr uint64_t kAccBias = 1ull << 51;
constexpr uint64_t kAccSumMask = (1ull << kAccCountShift) - 1;
__device__ __forceinline__ uint64_t acc_share(float v) {
  const double q = rint((double)v * (double)(1ull << kAccFracBits));
  const double lim = (double)(kAccBias - 1);
  const int64_t qi = (int64_t)fmin(fmax(q, -lim), lim);  // (NaN becomes 0)
  return (1ull << kAccCountShift) + (uint64_t)(qi + (int64_t)kAccBias);
}
__device__ __forceinline__ uint32_t acc_count(uint64_t w) { return (uint32_t)(w >> kAccCountShift); }
__device__ __forceinline__ float acc_value(uint64_t w) {
  const int64_t sum = (int64_t)(w & kAccSumMask) - (int64_t)(acc_count(w) * kAccBias);
  return (float)((double)sum * (1.0 / (double)(1ull << kAccFracBits)));
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
// For every unit the workgroup builds the chunk's B operands (+-Z in the odd or even
// group form of each plane) once, in LDS (double buffered; wave w builds plane w), and
// each wave runs its R row tiles against them with v_smfmac_f32_16x16x64_f16, the stored
// sign words of a tile giving the sparse indices of all 16 planes (one v_and_or_b32 per
// two planes), accumulating P over the chunks of a block in registers.  After a block's
// last chunk (or the end of the range) P is weighted by U (the r-sum is linear, so a
// block split over two workgroups is fine); after a row group's last unit (or the end
// of the range) each wave sums its tiles over r and adds the workgroup's share of each
// row to the row's fixed-point accumulator (acc_share); the workgroup whose add completes
// a row's count writes that row of y.  The returned words are examined a step later, so
// no wave waits for the adds, and the result does not depend on which workgroup arrives
// last.
//
// Sign tiles are fetched two units ahead, V fragments and activations one unit ahead
// (the activations by one lane of each 16-lane group, broadcast with ds_swizzle), and U
// fragments one unit ahead where a block ends, across block, row-group and weight
// boundaries, so the HBM stream never waits on compute; fetches past the end of the
// range read a page of zeros.  Sign tiles are read once, so they are loaded
// non-temporally and leave the L2 to the V and U fragments that other workgroups re-read.
// Nothing waits on outstanding loads before the end of the range.
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
  static_assert(NW * R == kDecodeGroupTiles && kPlanes % NW == 0 && NW % 2 == 0, "decode tiling");
  constexpr int PP = kPlanes / NW;       // B operands (planes) each wave builds
  __shared__ u32x4 zs[2][kPlanes][2][64];  // B operands (+-Z) of two units (64 KiB)
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
  u32x4 sgn[2][R];  // sign words of the current and the next unit
  u32x2 uf[R];
  // This wave's planes: V and x of columns 4 kk .. 4 kk + 3 and 16 + 4 kk ..; the waves
  // that build after their tiles keep them in their own registers (see step).
  struct VX {
    u32x2 v[PP][2], x[PP][2];
  } vx_early, vx_late;
  auto load_signs = [&](const UnitPtrs& p, u32x4* rw) {
#pragma unroll
    for (int t = 0; t < R; ++t) rw[t] = load16_stream(p.signs + t * kTileBytes + lane * 16);
  };
  auto load_u = [&](const UnitPtrs& p) {
#pragma unroll
    for (int t = 0; t < R; ++t) uf[t] = load8(p.u + (t * 64 + lane) * 4);
  };
  // Lane (r, kk) = (lane % 16, lane / 16) of the B operand of plane b holds the groups
  // 2 kk, 2 kk + 1, 8 + 2 kk, 9 + 2 kk, i.e. the plane's columns 4 kk .. 4 kk + 3 and
  // 16 + 4 kk .. 16 + 4 kk + 3 (group G <-> columns 2 G, 2 G + 1); in the stored V tile
  // those are the halves kk % 2 of lanes 16 (kk / 2) + r and 16 (2 + kk / 2) + r.
  const int kk = lane >> 4;
  // (the 16 lanes of a lane group need the same four activations: one of them loads them
  // and build_z broadcasts them, which spares the data-return path 15 of 16 copies)
  auto load_vx = [&](const UnitPtrs& p, VX& d) {
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int hpart = 0; hpart < 2; ++hpart) {
        d.v[pp][hpart] = load8(p.v + (pp * 64 + 16 * (2 * hpart + (kk >> 1)) + r16) * 8 + 4 * (kk & 1));
        const int col = 32 * (PP * wave + pp) + 16 * hpart + 4 * kk;
        if (r16 == 0) d.x[pp][hpart] = load8(col < p.xcols ? static_cast<const void*>(p.x + col) : static_cast<const void*>(zero_page));
      }
  };
  // B operand of this wave's plane: Z = V x (fp16 products, as the layer defines Z)
  // in the plane's group form, both signs of every column.
  auto build_z = [&](int buf, const VX& d) {
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
    const int b = PP * wave + pp;
    uint32_t z[4];
#pragma unroll
    for (int hpart = 0; hpart < 2; ++hpart)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        // lane 16 g's activations to every lane of group g (ds_swizzle, and-mask 0x10)
        const uint32_t xb = (uint32_t)__builtin_amdgcn_ds_swizzle((int)d.x[pp][hpart][k], 0x10);
        z[2 * hpart + k] = as_u32(as_half2(d.v[pp][hpart][k]) * as_half2(xb));
      }
    u32x8 t;
    if (plane_even(b)) {  // (wave-uniform branch)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x2 g2 = group_words<true>(z[k]);
        t[2 * k] = g2[0];
        t[2 * k + 1] = g2[1];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x2 g2 = group_words<false>(z[k]);
        t[2 * k] = g2[0];
        t[2 * k + 1] = g2[1];
      }
    }
    store_operand(zs[buf][b], lane, t);
    }
  };

  float4v acc[R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    acc[t] = (float4v){0.f, 0.f, 0.f, 0.f};
    accl[wave][t][lane] = (float4v){0.f, 0.f, 0.f, 0.f};
  }
  // After a block: U-weight the products into LDS.
  auto weight_block = [&]() {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const half2v u01 = as_half2(uf[k][0]), u23 = as_half2(uf[k][1]);
      float4v a = accl[wave][k][lane];
      a[0] += (float)u01[0] * acc[k][0];
      a[1] += (float)u01[1] * acc[k][1];
      a[2] += (float)u23[0] * acc[k][2];
      a[3] += (float)u23[1] * acc[k][3];
      accl[wave][k][lane] = a;
      acc[k] = (float4v){0.f, 0.f, 0.f, 0.f};
    }
  };
  // After a row group: this workgroup's share of each of its rows, summed over r, added
  // to the row's accumulator; the workgroup that completes a row's count writes y.
  const int rsel = reduced_row(lane);
  // workgroup that owns unit u
  auto owner = [&](uint32_t u) {
    uint32_t o = (uint32_t)(((uint64_t)u << lg) / U);
    while (o + 1 < G && range_start(o + 1, U, lg) <= u) ++o;
    while (range_start(o, U, lg) > u) --o;
    return o;
  };
  // The reduction leaves a row's sum in all four lanes of a quad, so lane L adds the row
  // of tile L % 4: one add per lane.  The returned word is examined only after the next
  // step's barrier (resolve), so the wave does not wait for the add's round trip, nor,
  // since loads complete in order, for the sign request issued just before it.
  const int rt = lane & 3;                                   // this lane's tile of the four
  const int rrow = (wave * R + rt) * kTileRows + rsel;       // its row in a row group
  struct PendingAdd {
    bool on;            // (uniform) an add waits to be examined
    uint64_t prev;      // the word before the add
    float v;            // the share added
    uint32_t item;      // its row group in the launch
    int32_t row;        // the lane's output row (or -1: no add)
    uint32_t parts;     // contributions the row group receives
    void* y;
  } pa = {false, 0ull, 0.f, 0u, -1, 0u, nullptr};
  auto add_shares = [&](const DecodeCursor& c) {
    const uint32_t item = c.rg_begin + c.rg;
    // workgroups that share this row group: the owners of its first and last unit and all between
    const uint32_t first = args.w[c.j].unit_begin + (uint32_t)c.rg * (uint32_t)(c.nch * c.nb);
    const uint32_t parts = owner(first + (uint32_t)(c.nch * c.nb) - 1) - owner(first) + 1;
    float v = 0.f;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const float s = reduce_columns(accl[wave][t][lane], lane);
      accl[wave][t][lane] = (float4v){0.f, 0.f, 0.f, 0.f};
      v = t == rt ? s : v;
    }
    const int row = c.rg * kDecodeGroupRows + rrow;
    pa.on = true;
    pa.v = v;
    pa.item = item;
    pa.row = row < args.w[c.j].m ? row : -1;
    pa.parts = parts;
    pa.y = args.w[c.j].y;
    pa.prev = 0;
    if (pa.row >= 0)
      pa.prev = __hip_atomic_fetch_add(&args.acc[(size_t)item * kDecodeGroupRows + rrow], acc_share(v), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  };
  // the contributor whose add completed the row's count holds the whole sum: it writes y
  // and clears the word
  auto resolve = [&]() {
    if (!pa.on) return;
    pa.on = false;
    if (pa.row < 0) return;
    const uint64_t now = pa.prev + acc_share(pa.v);
    if (acc_count(now) == pa.parts) {
      store_y(pa.y, pa.row, acc_value(now), args.y_fp32);
      __hip_atomic_store(&args.acc[(size_t)pa.item * kDecodeGroupRows + rrow], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  // Every load of the first two units is issued before anything waits: the block-table
  // entry for the LDS copy first (so that waiting for it waits for nothing else), then
  // the first unit's V / x and signs, the second unit's V / x, the first unit's U and
  // the second unit's signs.  No barrier here: the first barrier of the unit loop also
  // orders the LDS copy of the table and the first unit's B operands.
  const int bj = threadIdx.x / kMaxBlocks, bi = threadIdx.x % kMaxBlocks;
  bool bvalid = false;
  const void* bsrc = &args.w[0].blocks[0].signs;  // (always a valid entry: tables hold >= 1)
  if (bj < args.count && bi < args.w[bj].nblocks) {
    bvalid = true;
    bsrc = &args.w[bj].blocks[bi].signs;
  }
  const u32x2 btab = load8(bsrc);
  VX vx0;
  load_vx(p0, vx0);
  load_signs(p0, sgn[0]);
  if (wave >= NW / 2) load_vx(p1, vx_early);
  else load_vx(p1, vx_late);
  load_u(p0);
  load_signs(p1, sgn[1]);
  __builtin_amdgcn_sched_barrier(0);
  if (bvalid) bbase[bj][bi] = btab[0] | ((uint64_t)btab[1] << 32);
  build_z(0, vx0);  // (waits only for the table entry and the first unit's V / x)
  __builtin_amdgcn_sched_barrier(0);

  // ---- one unit.  On entry unit c0's signs are in `cur` and unit c1's in the other
  // buffer, c0's Z tile in zs[buf], its U fragments in uf (if c0 ends a block), and unit
  // c1's V fragments and activations in vx_early / vx_late.  Unit c2's signs are fetched into `cur` as soon as the
  // tiles are done with it, so a sign tile is requested well over one unit ahead.
  auto step = [&](u32x4 (&cur)[R], const int buf) __attribute__((always_inline)) {
    lds_barrier();  // the B operands of c0 are complete; zs[buf ^ 1] (unit c - 1) is free
    resolve();      // (the add of the last step's row-group end)
    // Unit c1's B operands, the next V / x loads and the cursor advance: the upper half
    // of the waves does them before its tiles and the lower half after, so on every SIMD
    // some waves keep the matrix cores busy while the others do this work.
    DecodeCursor c3;
    UnitPtrs p3;
    // (each half uses its own V / x registers: with one set, the compiler's load wait
    // before the build after the tiles would also cover the loads the other placement
    // may have issued, i.e. the sign loads just sent to HBM)
    auto prework = [&](VX& d) {
      build_z(buf ^ 1, d);
      load_vx(p2, d);
      c3 = next(c2);
      p3 = unit_ptrs(c3);
    };
    const bool early = wave >= NW / 2;  // (uniform)
    if (early) prework(vx_early);
    __builtin_amdgcn_sched_barrier(0);
    {
      // Row tiles: four independent accumulator chains per plane.  Word q of a tile's
      // stored signs gives the indices of planes 4 q .. 4 q + 3 (odd-position planes
      // 4 q, 4 q + 1, even-position planes 4 q + 2, 4 q + 3; abid picks the half); the B
      // operand of the next plane is read from LDS while the current one runs.
      const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
      u32x8 zf[2];
      zf[0] = load_operand(zs[buf][0], lane);
      uint32_t ix[2][R];
      uint32_t m_odd = 0xAAAAAAAAu, m_even = 0x55555555u;
      asm volatile("" : "+v"(m_odd), "+v"(m_even));  // (keeps the masks in VGPRs)
      // (a scheduling barrier per plane keeps the compiler from hoisting later planes'
      // work, which would raise register pressure past four waves per SIMD)
#define BSL_PLANE(B)                                                                                           \
  __builtin_amdgcn_sched_barrier(0);                                                                           \
  if ((B) % 4 == 0) {                                                                                          \
    _Pragma("unroll") for (int k = 0; k < R; ++k) {                                                            \
      ix[0][k] = sign_index_v(cur[k][plane_word(B)], m_odd, false);                                            \
      ix[1][k] = sign_index_v(cur[k][plane_word(B)], m_even, true);                                            \
    }                                                                                                          \
  }                                                                                                            \
  if ((B) + 1 < kPlanes) zf[((B) + 1) % 2] = load_operand(zs[buf][(B) + 1], lane);                          \
  _Pragma("unroll") for (int k = 0; k < R; ++k) acc[k] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(           \
      ones, __builtin_bit_cast(half16, zf[(B) % 2]), acc[k], (int)ix[plane_even(B)][k], 0, plane_half(B));
      BSL_PLANE(0) BSL_PLANE(1) BSL_PLANE(2) BSL_PLANE(3) BSL_PLANE(4) BSL_PLANE(5) BSL_PLANE(6) BSL_PLANE(7)
      BSL_PLANE(8) BSL_PLANE(9) BSL_PLANE(10) BSL_PLANE(11) BSL_PLANE(12) BSL_PLANE(13) BSL_PLANE(14) BSL_PLANE(15)
#undef BSL_PLANE
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!early) prework(vx_late);
    __builtin_amdgcn_sched_barrier(0);
    // (a row-group end's adds go out before the next sign request: the check of their
    // results after the next barrier then waits only for loads issued before them)
    if (block_end(c0)) weight_block();
    __builtin_amdgcn_sched_barrier(0);
    if (group_end(c0)) add_shares(c0);
    __builtin_amdgcn_sched_barrier(0);
    load_signs(p2, cur);
    if (block_end(c1)) load_u(p1);  // (U is needed only where a block ends)
    c0 = c1;
    c1 = c2;
    c2 = c3;
    p1 = p2;
    p2 = p3;
  };

  const uint32_t n = u_end - u_begin;
  for (uint32_t s = 0; s < n; s += 2) {
    step(sgn[0], 0);
    if (s + 1 < n) step(sgn[1], 1);
  }
  resolve();
}

// ============================================================ multi-token kernel
// M >= 2.  One workgroup of 8 waves per item = (weight, 512-row group, T-token group,
// range of the (block, chunk) sequence), T = 2, 4 or 8; wave w owns rows 64 w .. 64 w + 63
// as two 32-row fragments against the T tokens as T / 2 token pairs, i.e. 2 x T / 2
// accumulators of v_mfma_f32_32x32x16_f16 (32 rows x (2 tokens x 16 r)): the N width
// 2 x 16 = 32 is filled exactly, and each +-1 A fragment feeds T / 2 MFMAs.  Here the
// dense MFMA is used: measured on MI355X inside this kernel the 32x32 sparse MFMA runs
// about 13% slower than the dense one, while the unpack is cheap (the A fragment of a
// plane is two VALU operations per word, see pm1_fragment).  Z is built 4 planes (one
// stored word, 128 columns) at a time into double-buffered LDS as B fragments; the sign
// words of the next stage and V / activations of the next 4 planes are fetched while the
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
// word b / 4 of that (row, group) and gets the plane's 8 signs of its A fragment.
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
constexpr int kPrefillPlanes = 4;  // planes per Z stage (one stored word)

// +-1 fp16 A fragment (8 consecutive columns e = 0..7 of the lane) of plane b from its
// stored word w: column e is bit 16 h + 2 e + odd (h = b % 2, odd = 1 for the planes at
// odd positions).  A packed 16-bit shift with per-half amounts moves the bits of columns
// 2 n and 2 n + 1 to bit 15 of the two halves; masking and ORing in 1.0 gives the pair
// (one v_pk_lshlrev_b16 and one v_and_or_b32 per word; vmask holds 0x80008000).
template <int B>
__device__ __forceinline__ u32x4 pm1_fragment(uint32_t w, uint32_t vmask) {
  constexpr int H = plane_half(B), ODD = plane_even(B) ? 0 : 1;
  const unsigned short hw = (unsigned short)(w >> (16 * H));
  u32x4 a;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const ushort2v sh = {(unsigned short)(15 - 4 * n - ODD), (unsigned short)(13 - 4 * n - ODD)};
    const ushort2v v = (ushort2v){hw, hw} << sh;
    a[n] = (__builtin_bit_cast(uint32_t, v) & vmask) | 0x3C003C00u;
  }
  return a;
}

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
  constexpr int FPW = FRAGS / 8;              // built per wave (= NP: one (plane, step) per wave)
  static_assert(FPW == NP, "one (plane, step) per wave");
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

  // sign word q of [fragment rf][K step s]: word q of the 16 stored bytes of (row row0 +
  // 32 rf + l % 32, lane group 2 s + kg) of chunk ch
  auto load_sign_word = [&](const BlockPtrs& bp, int ch, int q, uint32_t (&w)[2][2]) {
    const uint8_t* chunk = bp.signs + (size_t)ch * W.mt * kTileBytes;  // (uniform)
#pragma unroll
    for (int rf = 0; rf < 2; ++rf) {
      const uint32_t row = row0 + 32 * rf + n32;
#pragma unroll
      for (int st = 0; st < 2; ++st)
        w[rf][st] = load_at<uint32_t>(chunk, (row >> 4) * kTileBytes + ((row & 15) + 16 * (2 * st + kg)) * 16 + 4 * q);
    }
  };
  // V fragment and activations of this wave's B fragments of stage (ch, q): wave w builds
  // (plane pl, step st) = (w / 2, w % 2) for all token pairs; lane (n, kg) needs columns
  // 16 st + 8 kg + 0..7 of the plane for r = n % 16 (stored V lane 16 (2 st + kg) + r)
  // and token tok0 + 2 pp + n / 16.  A token past M reads row M - 1 instead (its outputs
  // are never stored), so only a chunk that runs past column d needs the zero page.
  const int pl_w = wave >> 1, st_w = wave & 1;
  const uint16_t* xbase = W.x + (size_t)tok0 * W.d;  // (uniform; tok0 < M)
  auto xoff = [&](int pp, int col) {
    return (uint32_t)((min(tok0 + 2 * pp + (n32 >> 4), M - 1) - tok0) * W.d + col) * 2u;
  };
  auto load_vx = [&](const BlockPtrs& bp, int ch, int q, u32x4& vv, u32x4 (&xv)[NP]) {
    const int b = q * PL + pl_w;
    vv = load_at<u32x4>(bp.v, ((((uint32_t)ch * kPlanes + b) * 64 + (lane & 15) + 16 * (2 * st_w + kg)) * 8) * 2u);
    const int col = ch * kChunkCols + 32 * b + 16 * st_w + 8 * kg;
    if ((ch + 1) * kChunkCols <= W.d) {  // (uniform)
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) xv[pp] = load_at<u32x4>(xbase, xoff(pp, col));
    } else {
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) xv[pp] = col < W.d ? load_at<u32x4>(xbase, xoff(pp, col)) : load_at<u32x4>(zero_page, 0);
    }
  };
  auto build = [&](int buf, const u32x4& vv, const u32x4 (&xv)[NP]) {
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      u32x4 z;
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = as_u32(as_half2(vv[e]) * as_half2(xv[pp][e]));
      zs[buf][wave * NP + pp][lane] = z;
    }
  };

  float yacc[2][NP];
#pragma unroll
  for (int rf = 0; rf < 2; ++rf)
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) yacc[rf][pp] = 0.f;

  if (u_end > u_begin) {
    uint32_t vmask = 0x80008000u;
    asm volatile("" : "+v"(vmask));  // (a VGPR operand, so that AND and OR fuse into v_and_or_b32)
    uint32_t sw[2][2][2];            // sign words of this stage and the next: [stage parity][rf][st]
    u32x4 vv, xv[NP];
    float16v acc[2][NP];
#pragma unroll
    for (int rf = 0; rf < 2; ++rf)
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) acc[rf][pp] = (float16v){};
    int i = u_begin / nch, ch = u_begin % nch;  // current unit (block, chunk)
    BlockPtrs bp = load_block(W.blocks, i);
    load_sign_word(bp, ch, 0, sw[0]);
    load_vx(bp, ch, 0, vv, xv);
    build(0, vv, xv);
    for (int u = u_begin; u < u_end; ++u) {
      int ni = i, nc = ch + 1;
      if (nc == nch) { nc = 0; ++ni; }
      const bool more = u + 1 < u_end;
      const BlockPtrs nbp = load_block(W.blocks, more ? ni : i);
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // stage = stored word q of the chunk: planes 4 q .. 4 q + 3
        const int buf = q & 1;
        lds_barrier();  // the B fragments of this stage are in zs[buf]; zs[buf ^ 1] is free
        if (q < 3) {
          load_sign_word(bp, ch, q + 1, sw[(q + 1) & 1]);
          load_vx(bp, ch, q + 1, vv, xv);
        } else if (more) {
          load_sign_word(nbp, nc, 0, sw[0]);
          load_vx(nbp, nc, 0, vv, xv);
        }
        __builtin_amdgcn_sched_barrier(0);
#define BSL_PREFILL_PLANE(PLN)                                                                              \
  _Pragma("unroll") for (int st = 0; st < 2; ++st) {                                                        \
    const half8 a0 = as_half8(pm1_fragment<PLN>(sw[q & 1][0][st], vmask));                                  \
    const half8 a1 = as_half8(pm1_fragment<PLN>(sw[q & 1][1][st], vmask));                                  \
    _Pragma("unroll") for (int pp = 0; pp < NP; ++pp) {                                                     \
      const half8 bf = as_half8(zs[buf][((PLN) * 2 + st) * NP + pp][lane]);                                 \
      acc[0][pp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, bf, acc[0][pp], 0, 0, 0);                     \
      acc[1][pp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, bf, acc[1][pp], 0, 0, 0);                     \
    }                                                                                                       \
  }
        // (the fragment of plane 4 q + pl depends on pl only: word q is the stage's word)
        BSL_PREFILL_PLANE(0) BSL_PREFILL_PLANE(1) BSL_PREFILL_PLANE(2) BSL_PREFILL_PLANE(3)
#undef BSL_PREFILL_PLANE
        __builtin_amdgcn_sched_barrier(0);
        if (q < 3 || more) build(buf ^ 1, vv, xv);
      }
      // after a block's last chunk, or the range's: U weighting and the sum over r
      if (nc == 0 || !more) {
#pragma unroll
        for (int rf = 0; rf < 2; ++rf) {
          // U[row(v)][r] for v = 0..15: rows 8 (v / 4) + 4 kg + v % 4 of the fragment
          half2v uu[8];
          const int rbase = row0 + 32 * rf;
#pragma unroll
          for (int vg = 0; vg < 4; ++vg) {
            const int tile = (rbase >> 4) + (vg >> 1);
            const u32x2 uw = load8(bp.u + ((size_t)tile * 64 + (lane & 15) + 16 * (2 * (vg & 1) + kg)) * 4);
            uu[2 * vg] = as_half2(uw[0]);
            uu[2 * vg + 1] = as_half2(uw[1]);
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
      bp = nbp;
      i = ni;
      ch = nc;
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
  publish_partials();  // the partial sums above are visible before the arrival is counted
  __syncthreads();     // ... in every wave, and every wave is done with zs
  uint32_t* last = reinterpret_cast<uint32_t*>(&zs[0][0][0]);
  if (threadIdx.x == 0) *last = count_arrival(&W.counters[rest]) == (uint32_t)(W.splits - 1);
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


// ============================================================ tile-reconstruct kernel
// Any M (chosen for batches of tokens).  The weight restoration the pages give (add each
// block's unpacked signs times U_i V_i^T into W) is done per tile in registers and the
// rebuilt tile is multiplied with the activations at once, so the sign / low-rank work
// is paid once per group of up to 512 tokens instead of once per token:
//     W_hat[j, c] = sum_i S_i[j, c] (U_i V_i^T)[j, c],     y[t, j] = sum_c x[t, c] W_hat[j, c].
// One workgroup of 4 waves (one per SIMD; two workgroups per CU with TT = 1) per item =
// (weight, 64-row group, group of 2 x 32 TT tokens, column range); wave w owns row tile
// w / TH (32 rows) and token half w % TH (TT tiles of 32 tokens).  The column loop runs in
// steps of two planes (64 columns).  The two waves of a row tile split the blocks of a
// batch: for each step and own block, two v_mfma_f32_32x32x16_f16 with K = 16 = the rank
// give (U_i V_i^T) for the 32 rows and the step's two planes; each fp32 result pair (same
// row and column offset in both planes) is rounded to an fp16 pair and added into the
// running W_hat pair with a +-1 fp16 pair built from the stored sign word (one shift and
// one AND-OR).  The partner's share arrives through LDS; the completed pairs are split by
// plane and feed the GEMM: 4 MFMAs per 32-token tile and step, fp16 inputs, fp32
// accumulation.
//
// Layouts (lane l, h = l / 32, j = l % 32):
//  * reconstruct: A = V rows (the step plane's column sigma(j), ranks 8 h .. 8 h + 7,
//    one 16-byte load from the launch's rank-major V), B = U (row row0 + j, ranks 8 h ..);
//    result value i of lane l is column 16 h + i of the plane for row row0 + j (sigma
//    orders the A rows so).  Those columns are lane groups g = 2 h, 2 h + 1 of the stored
//    sign tile, so a lane reads the 16 stored bytes of (row, g) for its two groups.
//  * GEMM: A = activations (token t = l % 32 of the tile, 8 columns), B = W_hat (row j,
//    same 8 columns), C[t][j] in lane j + 32 ((t / 4) % 2).  The activations of a step
//    are staged in LDS as 16-byte units u = 4 z + 2 h + s (plane z of the pair, columns
//    16 h + 8 s .. + 7), [tile][u][slot], token t at slot t ^ 2 u (conflict-free writes
//    of 8 units per token and reads of 32 tokens per unit).
typedef float float2v __attribute__((ext_vector_type(2)));

// +-1 fp16 pair for planes (4 q + 2 kp, 4 q + 2 kp + 1) at column 8 g + e of lane group
// g, from that group's stored word q: their bits sit at 16 half + 2 e + 1 - kp, so one
// shift puts both at bits 15 and 31 (vmask holds 0x80008000).
__device__ __forceinline__ uint32_t tile_sign_pair(uint32_t w, int e, int kp, uint32_t vmask) {
  return ((w << (14 - 2 * e + kp)) & vmask) | 0x3C003C00u;
}

// s_waitcnt immediate for "at most 8 vector memory operations outstanding" (vmcnt in
// bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima, i.e. not waited for).
constexpr int kWaitVmcnt8 = 8 | (0x7 << 4) | (0xF << 8);

// Raw buffer loads: a descriptor in scalar registers plus a 32-bit per-lane byte offset
// (no 64-bit address arithmetic per load).  An offset at or past kBufOutOfRange reads
// zeros without touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kBufOutOfRange = 0x80000000u;
// (The base is passed through readfirstlane: should the compiler keep a uniform pointer
// in vector registers, the descriptor still ends up in scalar registers without a
// per-lane loop around the load.)
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes = kBufOutOfRange - 1) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(base)), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}
// The same for data read exactly once (sign words): non-temporal (cache policy bit 1, nt
// on this target), so the stream does not evict the L2 lines other waves re-read.
__device__ __forceinline__ u32x2 buf_load8_stream(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 2));
}
// U[row][8 h .. 8 h + 7] (eight ranks of one row, the rebuild MFMA's B operand) gathered
// from the tiled U, where rank r of row j is element j % 4 of lane 16 ((j % 16) / 4) + r
// of row tile j / 16 (8 bytes per lane, 512 bytes per row tile).  Zeros when !valid.
__device__ __forceinline__ half8 load_u_ranks(const uint16_t* u, int row, int h, bool valid) {
  const rsrc_t r = make_rsrc(u);
  const uint32_t base = valid ? (uint32_t)(row >> 4) * 512u + (uint32_t)(16 * ((row & 15) >> 2) + 8 * h) * 8u + (uint32_t)(row & 3) * 2u
                              : kBufOutOfRange;
  half8 out;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    out[k] = __builtin_bit_cast(_Float16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, base + 8u * k, 0u, 0));
  return out;
}

// V in rank order.  The stored (tiled) V of a 32-column plane gives lane L columns
// 8 (L / 16) .. + 7 of rank L % 16; the rebuild contracts over the rank and wants 8 ranks
// of one column per lane.  v_rank_order gives lane (h, j) ranks 8 h .. 8 h + 7 of column
// sigma(j) = 16 (j / 4 % 2) + 4 (j / 8) + j % 4 of each of two planes: a wave writes the
// planes to 2 KiB of LDS of its own and reads them back with the transposing 16-bit LDS
// read (ds_read_b64_tr_b16; measured on the device: in every group of 16 lanes, lane
// 4 a + b receives element b of the 8-byte rows that lanes 4 s + a address, s = 0..3).
// Lane L's 16 bytes are stored at slot L ^ 4 (L / 16 % 2) of the plane, which spreads
// every read over the banks at two dwords per bank.  LDS operations of one wave are
// performed in order, so neither the reads after the writes nor the next writes after
// the reads need a wait.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
struct VRank {
  half8 a, b;  // A operands of the step's two planes
};
struct VRankLane {
  uint32_t wpos, r0, r1;  // this lane's store offset and its two read offsets in a plane
};
__device__ __forceinline__ VRankLane vrank_lane(int lane) {
  const auto slot = [](uint32_t L) { return L ^ (((L >> 4) & 1u) << 2); };
  const uint32_t g = (uint32_t)lane >> 4, s = ((uint32_t)lane >> 2) & 3u, a = (uint32_t)lane & 3u;
  const uint32_t row = 16u * (2u * (a & 1u) + (g & 1u)) + 8u * (g >> 1) + s;  // stored lane of rank 8 (g / 2) + s
  VRankLane o;
  o.wpos = 16u * slot((uint32_t)lane);
  o.r0 = 16u * slot(row) + 8u * (a >> 1);
  o.r1 = 16u * slot(row + 4u) + 8u * (a >> 1);
  return o;
}
__device__ __forceinline__ u32x2 lds_read_tr16(lds_u8* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) s16x4*>(p)));
}
__device__ __forceinline__ VRank v_rank_order(const u32x4& pa, const u32x4& pb, lds_u8* region, const VRankLane& o) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(region + o.wpos) = pa;
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(region + 1024 + o.wpos) = pb;
  const u32x2 a0 = lds_read_tr16(region + o.r0), a1 = lds_read_tr16(region + o.r1);
  const u32x2 b0 = lds_read_tr16(region + 1024 + o.r0), b1 = lds_read_tr16(region + 1024 + o.r1);
  VRank v;
  v.a = as_half8((u32x4){a0[0], a0[1], a1[0], a1[1]});
  v.b = as_half8((u32x4){b0[0], b0[1], b1[0], b1[1]});
  return v;
}

// The rebuild's K = 16 MFMA, written out so that its result lands in VGPRs: a kernel
// that may use all 512 registers gets every compiler-built MFMA in the accumulator-
// register form, and each result would be copied back one dword per VALU operation.
// The leading s_nop covers a VALU write of an operand just before; the result is read
// only after mfma_result_ready.  (Neither statement is volatile: data dependences order
// them, and the compiler stays free to move loads across them.)
__device__ __forceinline__ float16v rebuild_mfma(const half8& a, const half8& b) {
  float16v d;
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
// Hands the results of rebuild_mfma to ordinary code after the wait states an MFMA
// result needs before a VALU operation may read it (at most 19).
__device__ __forceinline__ void mfma_result_ready(float16v& d0, float16v& d1) {
  asm("s_nop 15\n\ts_nop 3" : "+v"(d0), "+v"(d1));
}
// With one 32-token tile per wave (TT = 1: a few tokens, where the rebuild's VALU work is
// nearly all of it) the kernel fits 256 registers and two workgroups share a CU, so one
// wave's rebuild runs while the other waits on its loads (M = 16, 8B-shaped layer, n = 8:
// 310 -> 239 us); larger TT keep one wave per SIMD and all 512 registers.
// (Launched for TT = 1, groups of 64 tokens; larger groups take tile_split_kernel, which
// keeps this kernel's arithmetic and layouts.)
template <int TT, int TH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TT == 1 ? 2 : 1, TT == 1 ? 2 : 1))) void tile_kernel(GroupArgs args, int token_groups) {
  constexpr int TG = TT * TH;             // 32-token tiles per workgroup
  constexpr int RT = 4 / TH;              // 32-row tiles per workgroup
  constexpr int GROUP_ROWS = 32 * RT;
  constexpr int BPW = kTileBatch / TH;    // blocks each wave rebuilds per batch
  // activations of a step, two buffers: [token half][tile][token][slot], token t's 16-byte
  // unit u at slot u ^ ((t / 2) % 8) (the staging loads write 8 whole tokens per
  // instruction; the GEMM's reads of one unit of 16 tokens hit 16 distinct bank groups)
  __shared__ u32x4 xs0[TH][TT][32][8];
  __shared__ u32x4 xs1[TH][TT][32][8];
  __shared__ u32x4 ex[TH == 2 ? 2 : 1][TH == 2 ? 4 : 1][4][64];  // partial W_hat tiles of the wave pairs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, jl = lane & 31;
  const int rtile = wave / TH, th = wave % TH;
  const WeightDesc W = find_weight(args, blockIdx.x);
  const int local = blockIdx.x - W.item_begin;
  const int split = local % W.splits;
  const int rest = local / W.splits;
  const int rg = rest % W.groups;
  const int tg = rest / W.groups;
  const int M = args.M;
  const int tok0 = tg * 32 * TG;          // the workgroup's first token
  const int wtok0 = tok0 + th * 32 * TT;  // this wave's first token
  const int row0 = rg * GROUP_ROWS + 32 * rtile;
  const int nb = W.nblocks, d = W.d;
  const int cps = (W.nch + W.splits - 1) / W.splits;  // chunks per split
  const int c_begin = split * cps, c_end = min(W.nch, c_begin + cps);

  float16v acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[tt] = (float16v){};

  // activation staging, straight into LDS: wave w fetches tokens 8 w .. 8 w + 7 of every
  // tile, lane l the unit that belongs at slot l % 8 of token 8 w + l / 8.  The row part
  // of each address is in the per-lane offset, which the descriptor bounds: rows past M
  // read zeros.
  const uint16_t* xbase = W.x + (size_t)tok0 * d;  // (uniform)
  const uint32_t xbytes = (uint32_t)min(M - tok0, 32 * TG) * 2u * (uint32_t)d;
  const int dtok = 8 * wave + (lane >> 3);
  const int dunit = (lane & 7) ^ ((dtok >> 1) & 7);
  const uint32_t dvo = (uint32_t)dtok * 2u * (uint32_t)d + 16u * dunit, xstep = 64u * (uint32_t)d;
  // rebuild operands: A row sigma(j) of a plane; this lane's sign-tile row and groups
  const int sigma = 16 * ((jl >> 2) & 1) + 4 * (jl >> 3) + (jl & 3);
  const uint32_t voff = (uint32_t)sigma * (kRank * 2) + 16u * h;
  const int row = row0 + jl;
  const uint32_t soff = ((uint32_t)(row >> 4) * 64u + 32u * h + (row & 15)) * 16u;
  const uint32_t chunk_sign_bytes = (uint32_t)W.mt * kTileBytes;  // (a block's signs are < 2 GiB here)

  uint32_t vmask = 0x80008000u;
  asm volatile("" : "+v"(vmask));  // (a VGPR operand, so that AND and OR fuse into v_and_or_b32)

  for (int b0 = 0; b0 < nb && c_begin < c_end; b0 += kTileBatch) {
    // this wave's blocks: b0 + th BPW + i; slots past the weight's last block repeat a
    // loaded block with U = 0 (read out of range): they add exact zeros, and every load
    // stays valid, so the block loop has no branches
    const int nbw = min(BPW, max(0, nb - b0 - th * BPW));
    const uint8_t* sbase[BPW];  // (chunk offsets go in the loads' scalar offset)
    const uint16_t* vbase[BPW];
    half8 uf[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const BlockPtrs bp = load_block(W.blocks, i < nbw ? b0 + th * BPW + i : b0);
      sbase[i] = bp.signs;
      vbase[i] = W.vr + (size_t)(i < nbw ? b0 + th * BPW + i : b0) * W.nch * kChunkCols * kRank;
      // U[row][8 h .. 8 h + 7] (zeros for the repeated slots)
      uf[i] = load_u_ranks(bp.u, row, h, i < nbw);
    }
    // sign words sw[i][g2][q] of the current chunk (quads 0-1 and 2-3 refilled separately)
    uint32_t sw[BPW][2][4];
    auto load_signs = [&](int c, int half) {
      const uint32_t cb = __builtin_amdgcn_readfirstlane((uint32_t)min(c, c_end - 1) * chunk_sign_bytes);  // (uniform)
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const u32x2 v = buf_load8(make_rsrc(sbase[i]), soff + 256u * g2 + 8u * half, cb);
          sw[i][g2][2 * half] = v[0];
          sw[i][g2][2 * half + 1] = v[1];
        }
      }
    };
    // V rows of block i for step (c, qk): planes 2 qk, 2 qk + 1
    struct VP { u32x4 a, b; };
    auto load_v = [&](int c, int qk, int i) {
      const int cc = min(c, c_end - 1);
      const uint32_t cb = __builtin_amdgcn_readfirstlane((uint32_t)(cc * kChunkCols + 64 * qk) * (kRank * 2));  // (uniform)
      VP v;
      v.a = buf_load16(make_rsrc(vbase[i]), voff, cb);
      v.b = buf_load16(make_rsrc(vbase[i]), voff + 32u * kRank * 2u, cb);
      return v;
    };
    // activations of step (c, qk) into buffer `nb1` (0: xs0, 1: xs1): one 1 KiB load per
    // tile per wave.  Columns past d (only in a last, partial chunk) read zeros.
    auto stage_dma = [&](int c, int qk, int nb1) {
      const int col0 = c * kChunkCols + 64 * qk;  // (uniform)
      const uint32_t so = __builtin_amdgcn_readfirstlane(2u * (uint32_t)col0);
      const rsrc_t xr = make_rsrc(xbase, xbytes);
      uint32_t vo = dvo;
      asm volatile("" : "+v"(vo));  // (keeps the per-tile offsets below from being hoisted out of the loop)
      if (col0 + 8 * dunit >= d) vo = kBufOutOfRange;
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        __attribute__((address_space(3))) void* dst = nb1 ? (__attribute__((address_space(3))) void*)&xs1[t / TT][t % TT][8 * wave][0]
                                                            : (__attribute__((address_space(3))) void*)&xs0[t / TT][t % TT][8 * wave][0];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16, vo >= kBufOutOfRange ? vo : vo + (uint32_t)t * xstep, so, 0, 0);
      }
    };
    // one block of a step's rebuild: W_hat pairs += sign pair * (U_i V_i^T) pair
    auto recon_math = [&](const float16v& d0, const float16v& d1, int i, int qk, half2v (&wp)[16]) {
      const int q = qk >> 1, kp = qk & 1;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t sp = tile_sign_pair(sw[i][v >> 3][q], v & 7, kp, vmask);
        const half2v dp = __builtin_convertvector((float2v){d0[v], d1[v]}, half2v);
        wp[v] = as_half2(sp) * dp + wp[v];
      }
    };
    // the step's W_hat pairs, completed with the partner wave's share (TH = 2), split by
    // plane: bw[z][s] = W_hat[row][plane 2 qk + z, columns 16 h + 8 s .. + 7]
    auto finish_tile = [&](const half2v (&wp)[16], int slot, u32x4 (&bw)[2][2]) {
      half2v full[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) full[v] = wp[v];
      if constexpr (TH == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x4 o = ex[slot][wave ^ 1][k][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) full[4 * k + e] = full[4 * k + e] + as_half2(o[e]);
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int m2 = 0; m2 < 4; ++m2) {
          const uint32_t lo = as_u32(full[8 * s2 + 2 * m2]), hi = as_u32(full[8 * s2 + 2 * m2 + 1]);
          bw[0][s2][m2] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          bw[1][s2][m2] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
        }
    };
    auto publish = [&](const half2v (&wp)[16], int slot) {
      if constexpr (TH == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          ex[slot][wave][k][lane] = (u32x4){as_u32(wp[4 * k]), as_u32(wp[4 * k + 1]), as_u32(wp[4 * k + 2]), as_u32(wp[4 * k + 3])};
      }
    };
    // GEMM MFMA g = 4 tt + 2 z + s of a step: its activation fragment, then the product
    auto gemm_frag = [&](int g, int buf) -> half8 {
      const int tt = g >> 2, z = (g >> 1) & 1, s2 = g & 1;
      const int slot = (4 * z + 2 * h + s2) ^ ((jl >> 1) & 7);
      return as_half8(buf ? xs1[th][tt][jl][slot] : xs0[th][tt][jl][slot]);
    };
    auto gemm_one = [&](int g, const half8& xa, const u32x4 (&bw)[2][2]) {
      const int tt = g >> 2, z = (g >> 1) & 1, s2 = g & 1;
      acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa, as_half8(bw[z][s2]), acc[tt], 0, 0, 0);
    };

    // ---- prologue: step (c_begin, 0) rebuilt and staged
    load_signs(c_begin, 0);
    load_signs(c_begin, 1);
    VP vq[BPW];  // V rows of every block of the next step to rebuild (a full step ahead)
#pragma unroll
    for (int i = 0; i < BPW; ++i) vq[i] = load_v(c_begin, 0, i);
    half2v wp[16];  // this wave's share of the next step's W_hat pairs
    {
      stage_dma(c_begin, 0, 0);
#pragma unroll
      for (int v = 0; v < 16; ++v) wp[v] = (half2v){};
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const VP cur = vq[i];
        vq[i] = load_v(c_begin, 1, i);
        float16v d0 = rebuild_mfma(as_half8(cur.a), uf[i]);
        float16v d1 = rebuild_mfma(as_half8(cur.b), uf[i]);
        mfma_result_ready(d0, d1);
        recon_math(d0, d1, i, 0, wp);
      }
      publish(wp, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // (the staged activations are in LDS)
    lds_barrier();

    // ---- steps: the body of step (c, qk) multiplies its tile with the staged activations
    // and, interleaved, rebuilds and stages the next step (past the range's last step
    // that work repeats the last chunk and is discarded).
    for (int c = c_begin; c < c_end; ++c) {
#pragma unroll
      for (int qk = 0; qk < 8; ++qk) {
        const int buf = qk & 1;
        const int cn = qk == 7 ? c + 1 : c, qkn = (qk + 1) & 7;       // next step
        const int cnn = qk >= 6 ? c + 1 : c, qknn = (qk + 2) & 7;     // the one after
        u32x4 bw[2][2];
        finish_tile(wp, qk & 1, bw);
        if (qk == 3) load_signs(c + 1, 0);  // quads 0-1 of this chunk are done with
        if (qk == 7) load_signs(c + 1, 1);  // quads 2-3 likewise (refilled words are needed from (c + 1, 4))
        stage_dma(cn, qkn, buf ^ 1);        // the next step's activations, all requested up front
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < 16; ++v) wp[v] = (half2v){};
        // With few GEMM MFMAs per block (TT <= 4) nothing would cover the rebuild MFMAs'
        // latency, so their results are consumed one block later.
        constexpr bool PIPE = TT <= 4;
        float16v dn0, dn1;
        if constexpr (PIPE) {
          dn0 = rebuild_mfma(as_half8(vq[0].a), uf[0]);
          dn1 = rebuild_mfma(as_half8(vq[0].b), uf[0]);
        }
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
          // next step's block i: its two MFMAs, this step's share of the GEMM, then the
          // sign / accumulate work on the (by then finished) MFMA results
          const VP cur = vq[i];
          vq[i] = load_v(cnn, qknn, i);
          constexpr int GPB = (4 * TT + BPW - 1) / BPW;  // GEMM MFMAs per block (at most)
          const int g0 = (4 * TT * i) / BPW, g1 = (4 * TT * (i + 1)) / BPW;
          half8 xa[GPB];  // (all of the block's activation fragments are requested up front)
#pragma unroll
          for (int g = g0; g < g1; ++g) xa[g - g0] = gemm_frag(g, buf);
          float16v d0, d1;
          if constexpr (PIPE) {
            d0 = dn0;
            d1 = dn1;
            if (i + 1 < BPW) {
              dn0 = rebuild_mfma(as_half8(vq[i + 1].a), uf[i + 1]);
              dn1 = rebuild_mfma(as_half8(vq[i + 1].b), uf[i + 1]);
            }
          } else {
            d0 = rebuild_mfma(as_half8(cur.a), uf[i]);
            d1 = rebuild_mfma(as_half8(cur.b), uf[i]);
          }
#pragma unroll
          for (int g = g0; g < g1; ++g) gemm_one(g, xa[g - g0], bw);
          mfma_result_ready(d0, d1);
          recon_math(d0, d1, i, qkn, wp);
        }
        // Every load issued after this body's activation loads is one of the 2 BPW V loads
        // for the next body, and loads complete in order: with at most that many
        // outstanding, this wave's staging is in LDS.
        __builtin_amdgcn_sched_barrier(0);
        static_assert(2 * BPW == 8, "eight V loads follow the staging loads");
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt8);
        publish(wp, (qk + 1) & 1);
        lds_barrier();  // next step staged and published; this step's buffers are free
      }
    }
  }

  // lane (h, j) holds row row0 + j and tokens 8 (v / 4) + 4 h + v % 4 of every tile
  if (W.splits == 1) {
    if (row < W.m) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = wtok0 + 32 * tt + 8 * (v >> 2) + 4 * h + (v & 3);
          if (t < M) store_y(W.y, (size_t)t * W.m + row, acc[tt][v], args.y_fp32);
        }
    }
    return;
  }
  // Column ranges: partial[split][token][row] (write-through at device scope), then the
  // last workgroup of the (token group, row group) adds the ranges in order.
  const size_t tokpad = (size_t)token_groups * 32 * TG;
  const size_t rows_pad = (size_t)W.mt * kTileRows;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = wtok0 + 32 * tt + 8 * (v >> 2) + 4 * h + (v & 3);
      __hip_atomic_store(&W.partial[((size_t)split * tokpad + t) * rows_pad + row], acc[tt][v], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  publish_partials();  // the partial sums above are visible before the arrival is counted
  __syncthreads();     // ... in every wave, and every wave is done with xs
  uint32_t* last = reinterpret_cast<uint32_t*>(&xs0[0][0][0][0]);
  if (threadIdx.x == 0) *last = count_arrival(&W.counters[rest]) == (uint32_t)(W.splits - 1);
  __syncthreads();
  if (!*last) return;
  const int rbeg = rg * GROUP_ROWS;
  for (int e = threadIdx.x; e < GROUP_ROWS * 32 * TG; e += 256) {
    const int t = tok0 + e / GROUP_ROWS, r = rbeg + e % GROUP_ROWS;
    if (r >= W.m || t >= M) continue;
    float sum = 0.f;
    for (int sp = 0; sp < W.splits; ++sp)
      sum += __hip_atomic_load(&W.partial[((size_t)sp * tokpad + t) * rows_pad + r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    store_y(W.y, (size_t)t * W.m + r, sum, args.y_fp32);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&W.counters[rest], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ tile path, V in rank order
// First kernel of a tile-path launch: the V of every loaded block of the launch's weights
// in rank-major order, [block][d_pad][16] fp16 at WeightDesc::vr (a workspace of the
// stack), which the rebuild reads 8 ranks of one column at a time.  A block keeps V only
// in the tiled order of the single- and few-token kernels; forming this order per call
// costs one read and one write of the launch's V (32 bytes per block and column).  The
// work is the list of (weight, block, 64-column step) pairs, item_begin giving each
// weight's first pair; one pair per wave and iteration.
// One (weight, block, 64-column step) pair p of the pass; `region` is the wave's 2 KiB of LDS.
__device__ __forceinline__ void v_rank_item(const GroupArgs& args, uint32_t p, lds_u8* region, int lane) {
  const int jl = lane & 31, h = lane >> 5;
  const int sigma = 16 * ((jl >> 2) & 1) + 4 * (jl >> 3) + (jl & 3);
  const VRankLane vro = vrank_lane(lane);
  {
    int j = 0;
    while (j + 1 < args.count && p >= (uint32_t)args.w[j + 1].item_begin) ++j;
    const WeightDesc& W = args.w[j];
    const uint32_t per_block = (uint32_t)W.nch * 8u;  // steps of a block
    const uint32_t local = p - (uint32_t)W.item_begin;
    const uint32_t i = local / per_block, step = local - i * per_block;
    const rsrc_t r = make_rsrc(load_block(W.blocks, (int)i).v);
    const uint32_t off = step * 2048u + 16u * (uint32_t)lane;  // the step's two planes
    const u32x4 pa = buf_load16(r, off), pb = buf_load16(r, off + 1024u);
    const VRank t = v_rank_order(pa, pb, region, vro);
    uint16_t* out = W.vr + ((size_t)i * W.nch * kChunkCols + (size_t)step * 64 + sigma) * kRank + 8 * h;
    *reinterpret_cast<u32x4*>(out) = __builtin_bit_cast(u32x4, t.a);
    *reinterpret_cast<u32x4*>(out + 32 * kRank) = __builtin_bit_cast(u32x4, t.b);
  }
}
__global__ __launch_bounds__(256) void v_rank_major_kernel(GroupArgs args) {
  __shared__ u32x4 region[4][128];  // 2 KiB per wave
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t total = (uint32_t)args.total_items;
  for (uint32_t p = blockIdx.x * 4u + (uint32_t)wave; p < total; p += gridDim.x * 4u)
    v_rank_item(args, p, (lds_u8*)&region[wave][0], lane);
}

// ------------------------------------------------------------ tile path, split roles
// The item, arithmetic and results of tile_kernel<TT, 2>, with the rebuild and the GEMM
// in different waves: 8 waves, two per SIMD (256 registers each).  Waves 0-3 (GEMM waves)
// own row tile w / 2 and token half w % 2 (TT tiles of 32 tokens), stage the activations
// and multiply; waves 4-7 (rebuild waves) own row tile (w - 4) / 2 and block half
// (w - 4) % 2 of each batch, and hand their partial W_hat pairs of the next step to the
// GEMM waves through LDS.  A SIMD then runs one wave's sign work while the other's MFMAs
// execute, and a wave that waits for its loads or the barrier leaves the SIMD to the
// other: a wave alone on its SIMD would take the rebuild's VALU chain, the activation
// loads and the step barrier one after the other.  The two partial tiles are added in
// the order tile_kernel adds them, so both kernels give the same bits.
template <int TT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void tile_split_kernel(GroupArgs args, int token_groups) {
  constexpr int TH = 2, TG = TT * TH, GROUP_ROWS = 64, BPW = kTileBatch / 2;
  __shared__ u32x4 xs[2][TH][TT][32][8];  // activations of a step (layout of tile_kernel's xs0 / xs1), two buffers
  __shared__ u32x4 wpart[2][4][4][64];     // partial W_hat pairs of a step from the rebuild waves, two buffers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, jl = lane & 31;
  const bool gemm = wave < 4;
  const int role = gemm ? wave : wave - 4;
  const int rtile = role >> 1, half = role & 1;  // GEMM waves: token half; rebuild waves: block half
  const WeightDesc W = find_weight(args, blockIdx.x);
  const int local = blockIdx.x - W.item_begin;
  const int split = local % W.splits;
  const int rest = local / W.splits;
  const int rg = rest % W.groups;
  const int tg = rest / W.groups;
  const int M = args.M;
  const int tok0 = tg * 32 * TG;
  const int wtok0 = tok0 + half * 32 * TT;  // (GEMM waves)
  const int row0 = rg * GROUP_ROWS + 32 * rtile;
  const int row = row0 + jl;
  const int nb = W.nblocks, d = W.d;
  const int cps = (W.nch + W.splits - 1) / W.splits;
  const int c_begin = split * cps, c_end = min(W.nch, c_begin + cps);

  float16v acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[tt] = (float16v){};

  if (gemm) {
    // activation staging straight into LDS: GEMM wave g fetches tokens 8 g .. 8 g + 7 of
    // every tile (as tile_kernel's waves do)
    const uint16_t* xbase = W.x + (size_t)tok0 * d;
    const uint32_t xbytes = (uint32_t)min(M - tok0, 32 * TG) * 2u * (uint32_t)d;
    const int dtok = 8 * role + (lane >> 3);
    const int dunit = (lane & 7) ^ ((dtok >> 1) & 7);
    const uint32_t dvo = (uint32_t)dtok * 2u * (uint32_t)d + 16u * dunit, xstep = 64u * (uint32_t)d;
    auto stage_dma = [&](int c, int qk, int nb1) {
      const int col0 = c * kChunkCols + 64 * qk;  // (uniform)
      const uint32_t so = __builtin_amdgcn_readfirstlane(2u * (uint32_t)col0);
      const rsrc_t xr = make_rsrc(xbase, xbytes);
      uint32_t vo = dvo;
      asm volatile("" : "+v"(vo));  // (keeps the per-tile offsets below from being hoisted out of the loop)
      if (col0 + 8 * dunit >= d) vo = kBufOutOfRange;
#pragma unroll
      for (int t = 0; t < TG; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)&xs[nb1][t / TT][t % TT][8 * role][0], 16,
                                                 vo >= kBufOutOfRange ? vo : vo + (uint32_t)t * xstep, so, 0, 0);
    };
    for (int b0 = 0; b0 < nb && c_begin < c_end; b0 += kTileBatch) {
      stage_dma(c_begin, 0, 0);
      __builtin_amdgcn_s_waitcnt(0);  // (the staged activations are in LDS)
      lds_barrier();                  // ... and the rebuild waves' first step is published
      for (int c = c_begin; c < c_end; ++c) {
#pragma unroll
        for (int qk = 0; qk < 8; ++qk) {
          const int buf = qk & 1;
          stage_dma(qk == 7 ? c + 1 : c, (qk + 1) & 7, buf ^ 1);  // the next step's activations
          // the step's W_hat pairs: the two rebuild waves' shares, block half 0 first,
          // split by plane: bw[z][s] = W_hat[row][plane 2 qk + z, columns 16 h + 8 s .. + 7]
          u32x4 bw[2][2];
          {
            half2v full[16];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const u32x4 a = wpart[buf][2 * rtile][k][lane], b = wpart[buf][2 * rtile + 1][k][lane];
#pragma unroll
              for (int e = 0; e < 4; ++e) full[4 * k + e] = as_half2(a[e]) + as_half2(b[e]);
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
              for (int m2 = 0; m2 < 4; ++m2) {
                const uint32_t lo = as_u32(full[8 * s2 + 2 * m2]), hi = as_u32(full[8 * s2 + 2 * m2 + 1]);
                bw[0][s2][m2] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                bw[1][s2][m2] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
              }
          }
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            half8 xa[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int z = g >> 1, s2 = g & 1;
              xa[g] = as_half8(xs[buf][half][tt][jl][(4 * z + 2 * h + s2) ^ ((jl >> 1) & 7)]);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[g], as_half8(bw[g >> 1][g & 1]), acc[tt], 0, 0, 0);
          }
          __builtin_amdgcn_s_waitcnt(0);  // this wave's staging of the next step is in LDS
          lds_barrier();                  // next step staged and published; this step's buffers are free
        }
      }
    }
  } else {
    const int sigma = 16 * ((jl >> 2) & 1) + 4 * (jl >> 3) + (jl & 3);
    const uint32_t voff = (uint32_t)sigma * (kRank * 2) + 16u * h;
    const uint32_t soff = ((uint32_t)(row >> 4) * 64u + 32u * h + (row & 15)) * 16u;
    const uint32_t chunk_sign_bytes = (uint32_t)W.mt * kTileBytes;
    uint32_t vmask = 0x80008000u;
    asm volatile("" : "+v"(vmask));
    for (int b0 = 0; b0 < nb && c_begin < c_end; b0 += kTileBatch) {
      const int nbw = min(BPW, max(0, nb - b0 - half * BPW));
      const uint8_t* sbase[BPW];
      const uint16_t* vbase[BPW];
      half8 uf[BPW];
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const BlockPtrs bp = load_block(W.blocks, i < nbw ? b0 + half * BPW + i : b0);
        sbase[i] = bp.signs;
        vbase[i] = W.vr + (size_t)(i < nbw ? b0 + half * BPW + i : b0) * W.nch * kChunkCols * kRank;
        uf[i] = load_u_ranks(bp.u, row, h, i < nbw);
      }
      uint32_t sw[BPW][2][4];
      auto load_signs = [&](int c, int hq) {
        const uint32_t cb = __builtin_amdgcn_readfirstlane((uint32_t)min(c, c_end - 1) * chunk_sign_bytes);
#pragma unroll
        for (int i = 0; i < BPW; ++i)
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            const u32x2 v = buf_load8(make_rsrc(sbase[i]), soff + 256u * g2 + 8u * hq, cb);
            sw[i][g2][2 * hq] = v[0];
            sw[i][g2][2 * hq + 1] = v[1];
          }
      };
      struct VP { u32x4 a, b; };
      auto load_v = [&](int c, int qk, int i) {
        const int cc = min(c, c_end - 1);
        const uint32_t cb = __builtin_amdgcn_readfirstlane((uint32_t)(cc * kChunkCols + 64 * qk) * (kRank * 2));
        VP v;
        v.a = buf_load16(make_rsrc(vbase[i]), voff, cb);
        v.b = buf_load16(make_rsrc(vbase[i]), voff + 32u * kRank * 2u, cb);
        return v;
      };
      auto recon_math = [&](const float16v& d0, const float16v& d1, int i, int qk, half2v (&wp)[16]) {
        const int q = qk >> 1, kp = qk & 1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t sp = tile_sign_pair(sw[i][v >> 3][q], v & 7, kp, vmask);
          const half2v dp = __builtin_convertvector((float2v){d0[v], d1[v]}, half2v);
          wp[v] = as_half2(sp) * dp + wp[v];
        }
      };
      auto publish = [&](const half2v (&wp)[16], int slot) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          wpart[slot][role][k][lane] = (u32x4){as_u32(wp[4 * k]), as_u32(wp[4 * k + 1]), as_u32(wp[4 * k + 2]), as_u32(wp[4 * k + 3])};
      };
      load_signs(c_begin, 0);
      load_signs(c_begin, 1);
      VP vq[BPW];  // V rows of every block of the next step to rebuild
#pragma unroll
      for (int i = 0; i < BPW; ++i) vq[i] = load_v(c_begin, 0, i);
      half2v wp[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) wp[v] = (half2v){};
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const VP cur = vq[i];
        vq[i] = load_v(c_begin, 1, i);
        float16v d0 = rebuild_mfma(as_half8(cur.a), uf[i]);
        float16v d1 = rebuild_mfma(as_half8(cur.b), uf[i]);
        mfma_result_ready(d0, d1);
        recon_math(d0, d1, i, 0, wp);
      }
      publish(wp, 0);
      lds_barrier();
      for (int c = c_begin; c < c_end; ++c) {
#pragma unroll
        for (int qk = 0; qk < 8; ++qk) {
          const int buf = qk & 1;
          const int qkn = (qk + 1) & 7;                               // the step rebuilt now
          const int cnn = qk >= 6 ? c + 1 : c, qknn = (qk + 2) & 7;  // the one after
          if (qk == 3) load_signs(c + 1, 0);  // quads 0-1 of this chunk are done with
          if (qk == 7) load_signs(c + 1, 1);  // quads 2-3 likewise
#pragma unroll
          for (int v = 0; v < 16; ++v) wp[v] = (half2v){};
          // each block's MFMAs are issued before the previous block's sign work, which
          // covers their latency
          float16v dn0 = rebuild_mfma(as_half8(vq[0].a), uf[0]);
          float16v dn1 = rebuild_mfma(as_half8(vq[0].b), uf[0]);
#pragma unroll
          for (int i = 0; i < BPW; ++i) {
            vq[i] = load_v(cnn, qknn, i);
            float16v d0 = dn0, d1 = dn1;
            if (i + 1 < BPW) {
              dn0 = rebuild_mfma(as_half8(vq[i + 1].a), uf[i + 1]);
              dn1 = rebuild_mfma(as_half8(vq[i + 1].b), uf[i + 1]);
            }
            mfma_result_ready(d0, d1);
            recon_math(d0, d1, i, qkn, wp);
          }
          publish(wp, buf ^ 1);
          lds_barrier();
        }
      }
    }
  }

  // GEMM lane (h, j) holds row row0 + j and tokens 8 (v / 4) + 4 h + v % 4 of every tile
  if (W.splits == 1) {
    if (gemm && row < W.m) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = wtok0 + 32 * tt + 8 * (v >> 2) + 4 * h + (v & 3);
          if (t < M) store_y(W.y, (size_t)t * W.m + row, acc[tt][v], args.y_fp32);
        }
    }
    return;
  }
  const size_t tokpad = (size_t)token_groups * 32 * TG;
  const size_t rows_pad = (size_t)W.mt * kTileRows;
  if (gemm) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = wtok0 + 32 * tt + 8 * (v >> 2) + 4 * h + (v & 3);
        __hip_atomic_store(&W.partial[((size_t)split * tokpad + t) * rows_pad + row], acc[tt][v], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
  }
  publish_partials();  // the partial sums above are visible before the arrival is counted
  __syncthreads();     // ... in every wave, and every wave is done with xs
  uint32_t* last = reinterpret_cast<uint32_t*>(&xs[0][0][0][0][0]);
  if (threadIdx.x == 0) *last = count_arrival(&W.counters[rest]) == (uint32_t)(W.splits - 1);
  __syncthreads();
  if (!*last) return;
  const int rbeg = rg * GROUP_ROWS;
  for (int e = threadIdx.x; e < GROUP_ROWS * 32 * TG; e += 512) {
    const int t = tok0 + e / GROUP_ROWS, r = rbeg + e % GROUP_ROWS;
    if (r >= W.m || t >= M) continue;
    float sum = 0.f;
    for (int sp = 0; sp < W.splits; ++sp)
      sum += __hip_atomic_load(&W.partial[((size_t)sp * tokpad + t) * rows_pad + r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    store_y(W.y, (size_t)t * W.m + r, sum, args.y_fp32);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&W.counters[rest], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ============================================================ single-token kernel, wave-private operands
// One worker per wave: four waves per workgroup (one per SIMD), one workgroup per CU.  The
// work is the list of units (weight, row group of R row tiles, block, 512-column chunk) in
// that order (R = 16 for one token, fewer when the wave carries several tokens, below);
// with U units and 2^lg workers, worker o walks units [o U / 2^lg, (o + 1) U / 2^lg).  No
// operand is shared between waves, so the unit loop has no barrier.
//
// Per unit a wave contracts its R row tiles with the chunk's 16 planes on
// v_smfmac_f32_16x16x64_f16 with A = the plane's activations and B = +-V:
//  * B holds V of the plane's columns in both signs, in the odd or even group form of
//    the plane (group G = columns 2G, 2G + 1: rows (V_a, V_b, -V_a, -V_b) or (V_a, -V_a,
//    V_b, -V_b));
//  * the two compressed A values of group G are x_a and x_b, and their index fields come
//    straight from the stored sign bits (as in decode_m1_kernel), so they pick +V or -V;
//  * hence the MFMA accumulates P[j][r] = sum_c s_jc x_c V_cr with exact fp16 x fp16
//    products: Z = V (.) x is formed inside the matrix core, never rounded.
// A lane's 8 A values are the activations of the 8 columns whose signs its stored sign
// word holds (columns 8 g .. 8 g + 7 of the plane for lane group g), one 16-byte read
// from LDS, where the workgroup keeps the activations of the weights it works on.
//
// Vector memory loads retire in issue order, so a wait for one load also waits for every
// load issued before it.  The issue order keeps HBM sign loads out of the waits for L2
// operands: a unit's sign tiles are requested at the start of the previous unit, and the
// V operands of a unit are requested during the previous unit, before the next sign
// request.  (U is loaded only by a unit that ends its share of a block: making every unit
// load it, from the zero page otherwise, measured 10 us slower per launch, all waves then
// hitting the same few L2 lines.)  Plane b + 1's operands (A read, B built from V, sign indices) are prepared while plane
// b's MFMAs run, one MFMA then two VALU operations at a time; plane 0 of the next unit is
// prepared during plane 15.
struct WpPtrs {
  const uint8_t* signs;  // sign tiles of the unit's 16 row tiles (1 KiB each, consecutive)
  const uint8_t* v;      // tiled V of the unit's chunk, 16 planes x 1 KiB
  const uint8_t* u;      // tiled U of the unit's 16 row tiles (512 B each)
};

// B operand (+-V in the plane's group form) from the lane's four V words.
template <bool EVEN>
__device__ __forceinline__ u32x8 pm_v_operand(const u32x4& v) {
  u32x8 t;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x2 g2 = group_words<EVEN>(v[k]);
    t[2 * k] = g2[0];
    t[2 * k + 1] = g2[1];
  }
  return t;
}

// s_waitcnt immediate for "at most n vector memory operations outstanding" (n < 64).
__host__ __device__ constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// R row tiles per wave and T tokens (R T <= 32 accumulator tiles): the tokens share every
// B operand, sign index and load; each has its own A operand (its activations),
// accumulators and row-accumulator adds.  T is the launch's token count.  A unit's V
// (16 KiB) does not depend on its rows, so units of 128 rows or more keep the V bytes at
// most twice the sign bytes.
template <int R, int T>
__global__ __launch_bounds__(kWpWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_wp_kernel(GroupArgs args) {
  constexpr int ROWS = 16 * R;  // rows per unit
  __shared__ __attribute__((aligned(16))) uint16_t xs[kWpXBytes / 2];  // activations ([T][d_pad] per weight)
  __shared__ uint64_t bbase[kMaxGroup][kMaxBlocks];                     // block base addresses
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const uint32_t U = args.total_units;
  const int lg = args.grid_log2;  // log2 of the number of workers
  const uint32_t G = gridDim.x;
  const uint32_t bid = blockIdx.x;
  // XCD-contiguous workgroup index (workgroups are dealt round-robin over the XCDs)
  const uint32_t L = G >= (uint32_t)kXcds ? (bid % kXcds) * (G / kXcds) + bid / kXcds : bid;
  const uint32_t worker = L * kWpWaves + wave;
  const uint32_t u_begin = range_start(worker, U, lg), u_end = range_start(worker + 1, U, lg);
  const uint8_t* zero_page = static_cast<const uint8_t*>(args.zero_page);
  if (L == 0) {  // weights without blocks: y = 0, the empty sum
    for (int j = 0; j < args.count; ++j)
      if (args.w[j].units == 0)
        for (int e = threadIdx.x; e < args.w[j].m * args.M; e += kWpWaves * 64) store_y(args.w[j].y, e, 0.f, args.y_fp32);
  }
  if (U == 0) return;  // (uniform over the grid)

  auto weight_of = [&](uint32_t u) {
    int j = 0;
    while (j + 1 < args.count && u >= args.w[j + 1].unit_begin) ++j;
    return j;
  };
  // weights this workgroup works on: their activations go to LDS, back to back
  const int j0 = weight_of(range_start(L * kWpWaves, U, lg));
  const int j1 = weight_of(range_start((L + 1) * kWpWaves, U, lg) - 1);

  // ---- cursor over the unit list (wave-uniform)
  struct Cur {
    int32_t j, rg, i, ch;
    uint32_t u;
    bool valid;
    int32_t nb, nch, groups, mt, xo;  // xo: LDS offset (elements) of weight j's activations ([T][d_pad])
    uint32_t rg_begin;
  };
  auto load_weight = [&](Cur& c) {
    const WeightDesc& W = args.w[c.j];
    c.nb = W.nblocks;
    c.nch = W.nch;
    c.groups = W.groups;
    c.mt = W.mt;
    c.rg_begin = W.rg_begin;
    int xo = 0;
    for (int k = j0; k < c.j; ++k) xo += T * args.w[k].nch * kChunkCols;
    c.xo = xo;
  };
  auto locate = [&](uint32_t u) {
    Cur c;
    c.j = weight_of(u);
    load_weight(c);
    const uint32_t local = u - args.w[c.j].unit_begin;
    const uint32_t per_rg = (uint32_t)c.nch * c.nb;
    c.rg = local / per_rg;
    const uint32_t rem = local - c.rg * per_rg;
    c.i = rem / c.nch;
    c.ch = rem - c.i * c.nch;
    c.u = u;
    c.valid = true;
    return c;
  };
  auto next = [&](Cur c) {
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
  auto block_end = [&](const Cur& c) { return c.ch == c.nch - 1 || c.u + 1 == u_end; };
  auto group_end = [&](const Cur& c) { return (c.ch == c.nch - 1 && c.i == c.nb - 1) || c.u + 1 == u_end; };
  auto unit_ptrs = [&](const Cur& c, bool direct = false) {
    WpPtrs p;
    if (c.valid) {
      const uint8_t* base = direct ? load_block(args.w[c.j].blocks, c.i).signs
                                   : uniform_ptr(reinterpret_cast<const uint8_t*>(bbase[c.j][c.i]));
      const size_t sb = (size_t)c.mt * c.nch * kTileBytes;  // signs
      const size_t ub = (size_t)c.mt * 64 * 8;              // tiled U
      p.signs = base + ((size_t)c.ch * c.mt + (size_t)c.rg * R) * kTileBytes;
      p.u = base + sb + (size_t)c.rg * R * 64 * 8;
      p.v = base + sb + ub + (size_t)c.ch * kPlanes * 64 * 16;
    } else {
      p.signs = zero_page;
      p.u = zero_page;
      p.v = zero_page;
    }
    return p;
  };

  // ---- loads
  u32x4 sgn[2][R];  // sign words of the current and the next unit
  u32x4 vsl[kPlanes];  // V words of the planes (see the issue order above)
  u32x2 uw[R];
  auto load_signs = [&](const WpPtrs& p, u32x4 (&s)[R]) {
#pragma unroll
    for (int t = 0; t < R; ++t) s[t] = load16_stream(p.signs + t * kTileBytes + lane * 16);
  };
  // V words of plane b in the B-operand order (lane L = 16 kk + r: columns 4 kk .. 4 kk + 3
  // and 16 + 4 kk .. 16 + 4 kk + 3 of the plane, rank r), from the tiled copy, where lane
  // 16 g + r holds columns 8 g .. 8 g + 7: two 8-byte halves of lanes 16 (kk / 2) + r and
  // 16 (2 + kk / 2) + r
  const int vkk = lane >> 4, vr_ = lane & 15;
  const uint32_t voff0 = (uint32_t)((16 * (vkk >> 1) + vr_) * 16 + 8 * (vkk & 1));
  const uint32_t voff1 = voff0 + 32u * 16u;
  auto load_v = [&](const WpPtrs& p, int b) {
    const u32x2 lo = load8(p.v + b * 1024 + voff0), hi = load8(p.v + b * 1024 + voff1);
    return (u32x4){lo[0], lo[1], hi[0], hi[1]};
  };
  auto load_u = [&](const uint8_t* u) {
#pragma unroll
    for (int t = 0; t < R; ++t) uw[t] = load8(u + (t * 64 + lane) * 8);
  };
  // LDS address of a unit's activations of token 0 for this lane (plane 0); plane b is 64 b
  // bytes on, token t is d_pad elements on
  auto a_base = [&](const Cur& c) {
    const int off = (c.valid ? c.xo + c.ch * kChunkCols : 0) + 8 * g;
    return reinterpret_cast<const u32x4*>(&xs[off]);
  };
  auto a_stride = [&](const Cur& c) { return c.valid ? c.nch * kChunkCols / 8 : 0; };  // (in 16-byte units)
  auto read_a = [&](const u32x4* base, int stride, int t, int b) { return base[t * stride + 4 * b]; };

  // ---- prologue: the first unit's signs and V, then the block table and the
  // activations into LDS (the waits for those also cover the first unit's loads, which
  // are needed first anyway)
  Cur c0 = locate(u_begin);
  Cur c1 = next(c0);
  Cur c2 = next(c1);
  WpPtrs p0 = unit_ptrs(c0, true);
  WpPtrs p1 = unit_ptrs(c1, true);
  WpPtrs p2 = unit_ptrs(c2, true);
  load_signs(p0, sgn[0]);
#pragma unroll
  for (int b = 0; b < kPlanes; ++b) vsl[b] = load_v(p0, b);
  for (int e = threadIdx.x; e < kMaxGroup * kMaxBlocks; e += kWpWaves * 64) {
    const int bj = e / kMaxBlocks, bi = e % kMaxBlocks;
    if (bj < args.count && bi < args.w[bj].nblocks) {
      const u32x2 t = load8(&args.w[bj].blocks[bi].signs);
      bbase[bj][bi] = t[0] | ((uint64_t)t[1] << 32);
    }
  }
  {
    int off = 0;
    for (int j = j0; j <= j1; ++j) {
      const int d = args.w[j].d, dp = args.w[j].nch * kChunkCols;
      for (int t = 0; t < T; ++t) {
        const uint16_t* x = args.w[j].x + (size_t)t * d;
        const bool real = t < args.M;
        for (int c0s = threadIdx.x * 8; c0s < dp; c0s += 8 * kWpWaves * 64 * 8) {
          u32x4 v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int c = c0s + k * 8 * kWpWaves * 64;
            v[k] = real && c < d ? load16(x + c) : (u32x4){0u, 0u, 0u, 0u};
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int c = c0s + k * 8 * kWpWaves * 64;
            if (c < dp) *reinterpret_cast<u32x4*>(&xs[off + c]) = v[k];
          }
        }
        off += dp;
      }
    }
  }
  __syncthreads();

  // acc: P of the current block; accy: its U-weighted, r-summed rows over the blocks done
  // (one row per lane and tile, see reduce_columns; tile t in element t % 4 of accy[q][t / 4])
  static_assert(R % 4 == 0, "row tiles are spread over the four lanes of a quad");
  float4v acc[T][R];
  float4v accy[T][R / 4];
#pragma unroll
  for (int q = 0; q < T; ++q) {
#pragma unroll
    for (int t = 0; t < R; ++t) acc[q][t] = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < R / 4; ++s) accy[q][s] = (float4v){0.f, 0.f, 0.f, 0.f};
  }
  uint32_t m_odd = 0xAAAAAAAAu, m_even = 0x55555555u;
  asm volatile("" : "+v"(m_odd), "+v"(m_even));  // (keeps the masks in VGPRs: one v_and_or_b32 each)
  uint32_t ix_odd[R], ix_even[R];
  u32x4 av[2][T];
  u32x8 bw[2];
  // plane 0 of the first unit
#pragma unroll
  for (int t = 0; t < R; ++t) ix_odd[t] = sign_index_v(sgn[0][t][0], m_odd, false);
  const u32x4* abase = a_base(c0);
  int astride = a_stride(c0);
#pragma unroll
  for (int q = 0; q < T; ++q) av[0][q] = read_a(abase, astride, q, 0);
  bw[0] = pm_v_operand<false>(vsl[0]);
  vsl[0] = load_v(p1, 0);

  const int rsel = reduced_row(lane);
  // After a row group: this worker's share of each row of each token, added to the
  // row's fixed-point accumulator (acc_share); the worker whose add completes a row's
  // count writes that row of y.  Every lane of a quad holds the same reduced sums, so
  // lane L adds the rows of the tiles t = 4 s + (L & 3): R / 4 adds per lane, all lanes
  // busy.  The adds return the previous words, which are looked at only at the next row
  // group's end (or the end of the range): waiting for them at once would stall this
  // wave, the only one on its SIMD, on the atomics' round trip.
  constexpr int RS = R / 4;
  const int quad = lane & 3;
  const uint32_t NWK = 1u << lg;  // workers
  auto owner = [&](uint32_t u) {
    uint32_t o = (uint32_t)(((uint64_t)u << lg) / U);
    while (o + 1 < NWK && range_start(o + 1, U, lg) <= u) ++o;
    while (range_start(o, U, lg) > u) --o;
    return o;
  };
  struct Pending {
    uint64_t* words;  // [T][ROWS] accumulators of the row group (null: nothing pending)
    void* y;
    int32_t m, row0;
    uint32_t parts;
  } pend = {nullptr, nullptr, 0, 0, 0u};
  uint64_t pold[T][RS];  // previous words returned by the pending adds
  uint64_t pshare[T][RS];
  // (forced inline: called out of line, this wave's live registers would be saved to
  // scratch around every call)
  auto resolve = [&]() __attribute__((always_inline)) {
    if (pend.words == nullptr) return;
#pragma unroll
    for (int q = 0; q < T; ++q)
#pragma unroll
      for (int s = 0; s < RS; ++s) {
        const int rr = (4 * s + quad) * kTileRows + rsel;
        const int row = pend.row0 + rr;
        if (row < pend.m) {
          const uint64_t now = pold[q][s] + pshare[q][s];
          if (acc_count(now) == pend.parts) {
            store_y(pend.y, (size_t)q * pend.m + row, acc_value(now), args.y_fp32);
            __hip_atomic_store(&pend.words[q * ROWS + rr], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    pend.words = nullptr;
  };
  auto add_shares = [&](const Cur& c) __attribute__((always_inline)) {
    resolve();
    const uint32_t item = c.rg_begin + c.rg;
    const uint32_t per_rg = (uint32_t)c.nch * c.nb;
    const uint32_t first = args.w[c.j].unit_begin + (uint32_t)c.rg * per_rg;
    pend.parts = owner(first + per_rg - 1) - owner(first) + 1;
    pend.words = args.acc + (size_t)item * (ROWS * T);  // [T][ROWS]
    pend.y = args.w[c.j].y;
    pend.m = args.w[c.j].m;
    pend.row0 = c.rg * ROWS;
#pragma unroll
    for (int q = 0; q < T; ++q)
#pragma unroll
      for (int s = 0; s < RS; ++s) {
        const float v = accy[q][s][quad];  // (a vector element: selected in registers)
        const int rr = (4 * s + quad) * kTileRows + rsel;
        pshare[q][s] = acc_share(v);
        pold[q][s] = 0;
        if (pend.row0 + rr < pend.m)
          pold[q][s] = __hip_atomic_fetch_add(&pend.words[q * ROWS + rr], pshare[q][s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
    for (int q = 0; q < T; ++q)
#pragma unroll
      for (int s = 0; s < RS; ++s) accy[q][s] = (float4v){0.f, 0.f, 0.f, 0.f};
  };

  // ---- one unit: c0 with signs in `cur`; on entry plane 0's operands are ready, V of
  // planes 1..15 of c0 and of plane 0 of c1 are in vsl
  auto step = [&](u32x4 (&cur)[R], u32x4 (&nxt)[R]) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    load_signs(p1, nxt);
    __builtin_amdgcn_sched_barrier(0);
    if (block_end(c0)) load_u(p0.u);
    const Cur c3 = next(c2);
    const WpPtrs p3 = unit_ptrs(c3);
    const u32x4* abase_next = a_base(c1);
    const int astride_next = a_stride(c1);
#define BSL_WP_PLANE(B)                                                                                        \
  __builtin_amdgcn_sched_barrier(0);                                                                           \
  {                                                                                                            \
    constexpr int NB = ((B) + 1) % kPlanes; /* plane prepared in this region */                                \
    if ((B) < kPlanes - 1) {                                                                                   \
      if (NB % 4 == 0) {                                                                                       \
        _Pragma("unroll") for (int t = 0; t < R; ++t) ix_odd[t] = sign_index_v(cur[t][NB / 4], m_odd, false); \
      }                                                                                                        \
      if (NB % 4 == 2) {                                                                                       \
        _Pragma("unroll") for (int t = 0; t < R; ++t) ix_even[t] = sign_index_v(cur[t][NB / 4], m_even, true); \
      }                                                                                                        \
      _Pragma("unroll") for (int q = 0; q < T; ++q) av[NB % 2][q] = read_a(abase, astride, q, NB);              \
      bw[NB % 2] = plane_even(NB) ? pm_v_operand<true>(vsl[NB]) : pm_v_operand<false>(vsl[NB]);             \
      vsl[NB] = load_v(p1, NB);                                                                                \
    } else {                                                                                                   \
      _Pragma("unroll") for (int t = 0; t < R; ++t) ix_odd[t] = sign_index_v(nxt[t][0], m_odd, false);        \
      _Pragma("unroll") for (int q = 0; q < T; ++q) av[0][q] = read_a(abase_next, astride_next, q, 0);           \
      bw[0] = pm_v_operand<false>(vsl[0]);                                                                     \
      vsl[0] = load_v(p2, 0);                                                                                  \
    }                                                                                                          \
    _Pragma("unroll") for (int t = 0; t < R; ++t) _Pragma("unroll") for (int q = 0; q < T; ++q)              \
      acc[q][t] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(                                                    \
        __builtin_bit_cast(half8, av[(B) % 2][q]), __builtin_bit_cast(half16, bw[(B) % 2]), acc[q][t],        \
        (int)(plane_even(B) ? ix_even[t] : ix_odd[t]), 0, plane_half(B));                                      \
    /* one MFMA, then up to two VALU operations: the preparation of the next plane runs */                    \
    /* in the matrix core's shadow instead of between bursts of MFMAs */                                      \
    _Pragma("unroll") for (int t = 0; t < R * T; ++t) {                                                        \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                       \
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);                                                       \
    }                                                                                                          \
  }
    BSL_WP_PLANE(0) BSL_WP_PLANE(1) BSL_WP_PLANE(2) BSL_WP_PLANE(3) BSL_WP_PLANE(4) BSL_WP_PLANE(5)
    BSL_WP_PLANE(6) BSL_WP_PLANE(7) BSL_WP_PLANE(8) BSL_WP_PLANE(9) BSL_WP_PLANE(10) BSL_WP_PLANE(11)
    BSL_WP_PLANE(12) BSL_WP_PLANE(13) BSL_WP_PLANE(14) BSL_WP_PLANE(15)
#undef BSL_WP_PLANE
    __builtin_amdgcn_sched_barrier(0);
    if (block_end(c0)) {  // U-weight the block's products and sum them over r
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const half2v u01 = as_half2(uw[t][0]), u23 = as_half2(uw[t][1]);
#pragma unroll
        for (int q = 0; q < T; ++q) {
          float4v w;
          w[0] = (float)u01[0] * acc[q][t][0];
          w[1] = (float)u01[1] * acc[q][t][1];
          w[2] = (float)u23[0] * acc[q][t][2];
          w[3] = (float)u23[1] * acc[q][t][3];
          accy[q][t / 4][t % 4] += reduce_columns(w, lane);
          acc[q][t] = (float4v){0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    if (group_end(c0)) add_shares(c0);
    c0 = c1;
    c1 = c2;
    c2 = c3;
    p0 = p1;
    p1 = p2;
    p2 = p3;
    abase = abase_next;
    astride = astride_next;
  };

  const uint32_t n = u_end - u_begin;
  for (uint32_t s = 0; s < n; s += 2) {
    step(sgn[0], sgn[1]);
    if (s + 1 < n) step(sgn[1], sgn[0]);
  }
  resolve();
}

// ============================================================ activations in B-lane order
// Per product-index launch: x of each weight (M <= 32 tokens) rewritten as the kernel's B
// operands, so that the one of plane P, MFMA k is two 16-byte reads per lane (words 0-3
// of every lane, then words 4-7, so that each read is contiguous across the lanes): lane
// l = 32 b + t gets x[t][c + 4 b .. + 3] and x[t][c + 8 + 4 b .. + 3], c = 512 ch + 32 P
// + 16 k (zeros for t >= M and for columns >= d), each pair in both signs in the plane's
// odd or even group form.  One wave per (weight, chunk, plane, k) item p; WeightDesc::
// unit_begin holds each weight's first (weight, chunk) pair.  The pass runs in the launch
// of the rank-major V pass (layout_pass_kernel), after its V items.
__device__ __forceinline__ void x_lanes_item(const GroupArgs& args, uint32_t p, int lane) {
  const int b = lane >> 5, t = lane & 31;
  {
    const uint32_t pair = p / (kPlanes * 2), pk = p % (kPlanes * 2);  // (weight, chunk) pair; plane, k
    int j = 0;
    while (j + 1 < args.count && pair >= args.w[j + 1].unit_begin) ++j;
    const WeightDesc& W = args.w[j];
    const uint32_t ch = pair - W.unit_begin;
    const int c = (int)ch * kChunkCols + 32 * (int)(pk >> 1) + 16 * (int)(pk & 1) + 4 * b;
    u32x2 lo = {0u, 0u}, hi = {0u, 0u};
    if (t < args.M) {
      const uint16_t* row = W.x + (size_t)t * W.d;
      if (c < W.d) lo = load8(row + c);          // (d % 8 == 0: a 4-column run lies below d or past it)
      if (c + 8 < W.d) hi = load8(row + c + 8);
    }
    const u32x4 z = {lo[0], lo[1], hi[0], hi[1]};
    const u32x8 bw = plane_even((int)(pk >> 1)) ? pm_v_operand<true>(z) : pm_v_operand<false>(z);
    uint32_t* out = W.xt + ((size_t)ch * (kPlanes * 2) + pk) * 512 + 4 * lane;  // two 1 KiB halves
    *reinterpret_cast<u32x4*>(out) = (u32x4){bw[0], bw[1], bw[2], bw[3]};
    *reinterpret_cast<u32x4*>(out + 256) = (u32x4){bw[4], bw[5], bw[6], bw[7]};
  }
}
// The product-index path's two layout passes in one launch: items [0, total_items) are
// the rank-major V pass's (weight, block, 64-column step) pairs (item_begin per weight),
// items [total_items, total_items + total_units) the x pass's (weight, chunk, plane, k).
__global__ __launch_bounds__(256) void layout_pass_kernel(GroupArgs args) {
  __shared__ u32x4 region[4][128];  // 2 KiB per wave (V pass)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t nv = (uint32_t)args.total_items, total = nv + args.total_units;
  for (uint32_t p = blockIdx.x * 4u + (uint32_t)wave; p < total; p += gridDim.x * 4u) {
    if (p < nv) v_rank_item(args, p, (lds_u8*)&region[wave][0], lane);
    else x_lanes_item(args, p - nv, lane);
  }
}

// ============================================================ product-index kernel
// A few to 32 tokens.  The restoration adds, per block, the signs times the block's
// products P_i = U_i V_i^T (OpenReview discussion, weight-restoration reply).  Here each
// block's P_i, rounded to fp16 as the restoration forms it, is the value operand of the
// 2:4 sparse MFMA and the stored sign bits are its indices, against B = +-x:
//     y[t, j] = sum_i sum_c s_i[j, c] P_i[j, c] x[t, c],
// so no sign is expanded to a number and the sums over blocks and columns run in the
// fp32 accumulators.  Per 32-row tile, 32-column plane and block: one
// v_mfma_f32_32x32x16_f16 (K = 16 = the rank) gives P for the tile and the plane, eight
// conversions give two fp16 A operands, and two v_smfmac_f32_32x32x32_f16 add the plane's
// columns for up to 32 tokens.  Per 1024 (row, column) pairs of a block that is 96
// matrix-core cycles whatever the token count up to 32, against 64 per token for the
// few-token kernel and a sign-application VALU cost of 2 operations per pair for the tile
// kernel.
//
// Work: units (weight, row group of 8 x R 32-row tiles, batch of NB blocks, 512-column
// chunk) in that order.  One 8-wave workgroup per CU (two waves per SIMD) walks an equal
// contiguous share of the units; wave w owns the R tiles of rows 32 R w .. of the group.
// A batch past the weight's last block repeats a loaded block with U = 0 (read out of
// range): those slots add exact zeros and need no branch.  Each wave keeps its tiles' y
// in registers across its units and, when the row group or its range ends, stores it in
// the workgroup's slot for the row group; product_finish_kernel, next in the stream, adds
// a row group's slots in workgroup order (deterministic, and no atomics).
//
// Layouts (lane l, h = l / 32, j = l % 32):
//  * rebuild: A = V[column cp(j) of the plane][ranks 8 h .. 8 h + 7] from the launch's
//    rank-major V, B = U[row j][ranks 8 h ..]; cp(j) swaps bits 2 and 3 of j, so result
//    register v of lane l is column 8 h + v % 8 + 16 (v / 8) of the plane for row j:
//    registers 0-7 hold lane group g = h of the stored sign tile and 8-15 group 2 + h.
//  * sparse MFMA k (k = 0, 1): A = registers 8 k .. 8 k + 7 as fp16 (column 8 g + e of
//    group g = 2 k + h in value e, the order of the index fields of the stored word),
//    index = the stored word of the row and group.  B: lane l holds token j and, as
//    measured for this instruction, the 4-row groups of both A lane halves' value pairs
//    2 h and 2 h + 1, i.e. columns 16 k + 4 h + {0, 1}, {2, 3}, 16 k + 8 + 4 h + {0, 1},
//    {2, 3} of the plane in its odd or even form (the same forms as the single-token
//    kernel's +-Z).  C: lane l holds token j, rows 8 (v / 4) + 4 h + v % 4.
//
// Loads: the V of the batch and the plane's B operands (+-x, laid out per call by
// layout_pass_kernel) are the same for every wave, so the workgroup stages them in LDS:
// four planes per group and barrier, a group ahead.  Sign words are each wave's own and
// are requested (non-temporal) at planes 7 and 15 of the previous unit; U where a row
// group or batch begins.
__device__ __forceinline__ void px_result_ready(float16v& d) { asm("s_nop 15\n\ts_nop 3" : "+v"(d)); }
static_assert(kPxTiles == 1 || kPxTiles == 2, "one hand-over wait per batch of rebuilds");

template <int R, int NB>
__global__ __launch_bounds__(kPxWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void product_kernel(GroupArgs args) {
  constexpr int KA = R == 1 ? 2 : 1;  // accumulators per row tile (R > 1: the tiles' MFMAs interleave)
  constexpr int PARTS = NB + 4;       // 1 KiB parts of a plane's staging: V of the NB blocks, B for k = 0, 1 (2 KiB each)
  static_assert(PARTS <= kPxWaves, "one 1 KiB part per staging wave");
  constexpr int GP = 4;               // planes per staging group: one workgroup barrier per group
  static_assert(kPlanes % GP == 0, "a unit is whole groups");
  __shared__ __attribute__((aligned(16))) uint8_t stg[2][GP][PARTS * 1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, jl = lane & 31;
  const uint32_t U = args.total_units;
  const int lg = args.grid_log2;
  const uint32_t G = gridDim.x, bid = blockIdx.x;
  // XCD-contiguous workgroup index (workgroups are dealt round-robin over the XCDs)
  const uint32_t L = G >= (uint32_t)kXcds ? (bid % kXcds) * (G / kXcds) + bid / kXcds : bid;
  const uint32_t u_begin = range_start(L, U, lg), u_end = range_start(L + 1, U, lg);
  const int M = args.M;
  const uint8_t* zero_page = static_cast<const uint8_t*>(args.zero_page);
  if (u_begin >= u_end) return;  // (uniform over the workgroup)

  auto weight_of = [&](uint32_t u) {
    int j = 0;
    while (j + 1 < args.count && u >= args.w[j + 1].unit_begin) ++j;
    return j;
  };
  // cursor over the unit list (uniform over the workgroup): rt is the row group of
  // kPxWaves R 32-row tiles, of which this wave owns the R tiles R (kPxWaves rt + wave) ..
  struct Cur {
    int32_t j, rt, bb, ch;
    uint32_t u;
    bool valid;
    int32_t nb, nch, batches;
  };
  auto load_weight = [&](Cur& c) {
    const WeightDesc& W = args.w[c.j];
    c.nb = W.nblocks;
    c.nch = W.nch;
    c.batches = (W.nblocks + NB - 1) / NB;
  };
  auto locate = [&](uint32_t u) {
    Cur c;
    c.j = weight_of(u);
    load_weight(c);
    const uint32_t local = u - args.w[c.j].unit_begin;
    const uint32_t per_rt = (uint32_t)(c.batches * c.nch);
    c.rt = (int32_t)(local / per_rt);
    const uint32_t rem = local - (uint32_t)c.rt * per_rt;
    c.bb = (int32_t)(rem / (uint32_t)c.nch);
    c.ch = (int32_t)(rem - (uint32_t)c.bb * (uint32_t)c.nch);
    c.u = u;
    c.valid = true;
    return c;
  };
  auto next = [&](Cur c) {
    if (!c.valid || c.u + 1 >= u_end) {
      c.valid = false;
      return c;
    }
    ++c.u;
    if (++c.ch == c.nch) {
      c.ch = 0;
      if (++c.bb == c.batches) {
        c.bb = 0;
        if (++c.rt == args.w[c.j].groups) {
          c.rt = 0;
          do ++c.j;
          while (args.w[c.j].units == 0);
          load_weight(c);
        }
      }
    }
    return c;
  };
  // this wave's row group of the unit's rows (R 32-row tiles)
  auto my_rg = [&](const Cur& c) { return kPxWaves * c.rt + wave; };

  // per-lane offsets: this lane's row in the stored tiles (groups h and 2 + h), its V
  // column's 16 bytes within a plane of rank-major V
  const int cpj = (jl & 0x13) | (((jl >> 3) & 1) << 2) | (((jl >> 2) & 1) << 3);
  const uint32_t s_lane = (uint32_t)(((jl >> 4) * 64 + 16 * h + (jl & 15)) * 16);
  const uint32_t v_lane = (uint32_t)((cpj * kRank + 8 * h) * 2);

  // ---- staging: wave w < PARTS brings 1 KiB of every plane to LDS (part w), lane l 16
  // bytes at l * 16: parts 0 .. NB - 1 hold the rank-major V of the plane (1 KiB per
  // block), parts NB .. NB + 3 the plane's B operands for k = 0, 1 (2 KiB each)
  const bool stager = wave < PARTS;  // (wave-uniform)
  struct Src {
    rsrc_t r;          // this wave's part of the unit's chunk
    uint32_t pstride;  // bytes per plane in it
  };
  auto unit_src = [&](const Cur& c) {
    Src s;
    if (c.valid && stager) {
      const WeightDesc& W = args.w[c.j];
      if (wave < NB) {
        const int b0 = c.bb * NB, nok = min(NB, c.nb - b0);
        const int b = wave < nok ? b0 + wave : b0;  // (spare slots repeat the first block; their U is zero)
        s.r = make_rsrc(reinterpret_cast<const uint8_t*>(W.vr) + ((size_t)b * c.nch + c.ch) * (kChunkCols * kRank * 2));
        s.pstride = 32u * kRank * 2u;
      } else {
        s.r = make_rsrc(reinterpret_cast<const uint8_t*>(W.xt + (size_t)c.ch * (kPxLaneBytesPerChunk / 4)) + (wave - NB) * 1024,
                        (uint32_t)kPxLaneBytesPerChunk);
        s.pstride = 4096u;
      }
    } else {
      s.r = make_rsrc(zero_page, (uint32_t)kZeroPageBytes);
      s.pstride = 0;
    }
    return s;
  };
  u32x4 sr[GP];  // staged bytes of the next group's planes
  // (a V part is fetched in the order its readers take it: lane l the 16 bytes of column
  // cp(l % 32), ranks 8 (l / 32) .., so every LDS read and write is contiguous)
  auto stage_load = [&](const Src& s, int P) {
    return buf_load16(s.r, wave < NB ? v_lane : 16u * (uint32_t)lane, (uint32_t)P * s.pstride);
  };
  auto stage_write = [&](int buf, int q, const u32x4& v) {
    if (stager) *reinterpret_cast<u32x4*>(&stg[buf][q][wave * 1024 + 16 * lane]) = v;
  };

  u32x2 sw[R][NB][2][2];  // sign words [row tile][block][k][words 0-1 | 2-3] of the current unit
  half8 uf[R][NB];        // U operands of the current row group and batch
  auto load_sw = [&](const Cur& c, int half) {
    if (c.valid) {
      const WeightDesc& W = args.w[c.j];
      const uint32_t off = ((uint32_t)c.ch * (uint32_t)W.mt + 2u * (uint32_t)(R * my_rg(c))) * kTileBytes;  // (< 2 GiB)
      const int b0 = c.bb * NB, nok = min(NB, c.nb - b0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const rsrc_t rs = make_rsrc(load_block(W.blocks, i < nok ? b0 + i : b0).signs);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int k = 0; k < 2; ++k) sw[r][i][k][half] = buf_load8_stream(rs, s_lane, off + 2048u * r + 512u * k + 8u * half);
      }
    } else {
      const rsrc_t rs = make_rsrc(zero_page, (uint32_t)kZeroPageBytes);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int k = 0; k < 2; ++k) sw[r][i][k][half] = buf_load8(rs, s_lane, 2048u * r + 512u * k + 8u * half);
    }
  };
  auto load_u = [&](const Cur& c) {
    const WeightDesc& W = args.w[c.j];
    const int b0 = c.bb * NB, nok = min(NB, c.nb - b0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint16_t* u = load_block(W.blocks, i < nok ? b0 + i : b0).u;
#pragma unroll
      for (int r = 0; r < R; ++r) uf[r][i] = load_u_ranks(u, 32 * (R * my_rg(c) + r) + jl, h, i < nok);
    }
  };

  // ---- flush: this wave's share of its row tiles' y (fp32, in the MFMA result layout)
  // into the workgroup's slot for the row group, (row group + L): plain stores, each 256
  // contiguous bytes per instruction.  product_finish_kernel, next in the stream, adds
  // the slots of a row group in workgroup order.
  float16v acc[R][KA];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int a = 0; a < KA; ++a) acc[r][a] = (float16v){};
  auto flush = [&](const Cur& c) __attribute__((always_inline)) {
    float* slot = args.part + ((size_t)args.w[c.j].rg_begin + (size_t)c.rt + L) * kPxPartFloats;
    const bool live = (lane & 31) < M;  // (the finishing pass reads tokens below M only)
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (live) slot[((wave * R + r) * 16 + v) * 64 + lane] = KA == 2 ? acc[r][0][v] + acc[r][KA - 1][v] : acc[r][0][v];
#pragma unroll
      for (int a = 0; a < KA; ++a) acc[r][a] = (float16v){};
    }
  };

  uint32_t m_odd = 0xAAAAAAAAu, m_even = 0x55555555u;
  asm volatile("" : "+v"(m_odd), "+v"(m_even));  // (keeps the masks in VGPRs: one v_and_or_b32 each)

  // ---- prologue: the first unit's signs and U, planes 0 .. D - 1 staged, plane 0 in LDS
  Cur c = locate(u_begin);
  Cur cn = next(c);
  Src s0 = unit_src(c), s1 = unit_src(cn);
  load_sw(c, 0);
  load_sw(c, 1);
  load_u(c);
#pragma unroll
  for (int q = 0; q < GP; ++q) sr[q] = stage_load(s0, q);
#pragma unroll
  for (int q = 0; q < GP; ++q) stage_write(0, q, sr[q]);
  lds_barrier();
  uint32_t ix[R][NB][2];

  // One plane P of the current unit (group P / GP, in LDS buffer (P / GP) % 2): at a
  // group's first plane the staging loads of the next group, the operands from LDS, per
  // block the rebuilds, their conversion and the sparse MFMAs; after a group's last plane
  // the next group's bytes go to the other buffer and the workgroup meets.
#define BSL_PX_PLANE(P)                                                                                         \
  {                                                                                                             \
    constexpr bool EV = plane_even(P);                                                                          \
    constexpr int SB = ((P) / GP) % 2, SQ = (P) % GP;                                                          \
    if (SQ == 0) {                                                                                              \
      __builtin_amdgcn_sched_barrier(0);                                                                        \
      _Pragma("unroll") for (int q = 0; q < GP; ++q) {                                                         \
        if ((P) + GP + q < kPlanes) sr[q] = stage_load(s0, (P) + GP + q);                                      \
        else sr[q] = stage_load(s1, (P) + GP + q - kPlanes);                                                   \
      }                                                                                                         \
    }                                                                                                           \
    if ((P) == 7) load_sw(cn, 0);  /* planes 0-7 of this unit are indexed: words 0-1 free */                    \
    if ((P) == kPlanes - 1) load_sw(cn, 1);                                                                     \
    if ((P) % 2 == 0) {                                                                                         \
      _Pragma("unroll") for (int r = 0; r < R; ++r) _Pragma("unroll") for (int i = 0; i < NB; ++i)              \
        _Pragma("unroll") for (int k = 0; k < 2; ++k)                                                           \
          ix[r][i][k] = sign_index_v(sw[r][i][k][plane_word(P) / 2][plane_word(P) % 2], EV ? m_even : m_odd, EV); \
    }                                                                                                           \
    u32x4 va[NB];                                                                                               \
    _Pragma("unroll") for (int i = 0; i < NB; ++i) va[i] = *reinterpret_cast<const u32x4*>(&stg[SB][SQ][i * 1024 + 16 * lane]); \
    const u32x4 b0l = *reinterpret_cast<const u32x4*>(&stg[SB][SQ][NB * 1024 + 16 * lane]);                   \
    const u32x4 b0h = *reinterpret_cast<const u32x4*>(&stg[SB][SQ][(NB + 1) * 1024 + 16 * lane]);             \
    const u32x8 b0 = {b0l[0], b0l[1], b0l[2], b0l[3], b0h[0], b0h[1], b0h[2], b0h[3]};                        \
    const u32x4 b1l = *reinterpret_cast<const u32x4*>(&stg[SB][SQ][(NB + 2) * 1024 + 16 * lane]);             \
    const u32x4 b1h = *reinterpret_cast<const u32x4*>(&stg[SB][SQ][(NB + 3) * 1024 + 16 * lane]);             \
    const u32x8 b1 = {b1l[0], b1l[1], b1l[2], b1l[3], b1h[0], b1h[1], b1h[2], b1h[3]};                        \
    /* block i: its rebuilds were issued one step earlier (block 0 at the top of the plane);                    \
       the next block's are issued before block i's conversions, so the matrix core works                       \
       on them meanwhile */                                                                                     \
    float16v pn[R];                                                                                             \
    _Pragma("unroll") for (int r = 0; r < R; ++r) pn[r] = rebuild_mfma(as_half8(va[0]), uf[r][0]);              \
    _Pragma("unroll") for (int i = 0; i < NB; ++i) {                                                            \
      float16v pc[R];                                                                                           \
      _Pragma("unroll") for (int r = 0; r < R; ++r) pc[r] = pn[r];                                              \
      if (i + 1 < NB) {                                                                                         \
        _Pragma("unroll") for (int r = 0; r < R; ++r) pn[r] = rebuild_mfma(as_half8(va[i + 1]), uf[r][i + 1]);  \
      }                                                                                                         \
      __builtin_amdgcn_sched_barrier(0x0120);                                                                   \
      /* the wait states an MFMA result needs before a VALU read, after the last MFMA issued */                 \
      if constexpr (R == 2) mfma_result_ready(pc[0], pc[1]); else px_result_ready(pc[0]);                       \
      __builtin_amdgcn_sched_barrier(0);                                                                        \
      u32x4 a0[R], a1[R];                                                                                       \
      _Pragma("unroll") for (int r = 0; r < R; ++r) _Pragma("unroll") for (int e = 0; e < 4; ++e) {             \
        a0[r][e] = as_u32(__builtin_convertvector((float2v){pc[r][2 * e], pc[r][2 * e + 1]}, half2v));          \
        a1[r][e] = as_u32(__builtin_convertvector((float2v){pc[r][8 + 2 * e], pc[r][9 + 2 * e]}, half2v));      \
      }                                                                                                         \
      _Pragma("unroll") for (int r = 0; r < R; ++r)                                                             \
        acc[r][0] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(as_half8(a0[r]), __builtin_bit_cast(half16, b0), acc[r][0], \
                                                            (int)ix[r][i][0], 0, plane_half(P));                \
      _Pragma("unroll") for (int r = 0; r < R; ++r)                                                             \
        acc[r][KA - 1] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(as_half8(a1[r]), __builtin_bit_cast(half16, b1), \
                                                                 acc[r][KA - 1], (int)ix[r][i][1], 0, plane_half(P)); \
    }                                                                                                           \
    if (SQ == GP - 1) {                                                                                         \
      _Pragma("unroll") for (int q = 0; q < GP; ++q) stage_write(SB ^ 1, q, sr[q]);                            \
      lds_barrier();                                                                                            \
    }                                                                                                           \
  }

  while (true) {
    BSL_PX_PLANE(0) BSL_PX_PLANE(1) BSL_PX_PLANE(2) BSL_PX_PLANE(3) BSL_PX_PLANE(4) BSL_PX_PLANE(5)
    BSL_PX_PLANE(6) BSL_PX_PLANE(7) BSL_PX_PLANE(8) BSL_PX_PLANE(9) BSL_PX_PLANE(10) BSL_PX_PLANE(11)
    BSL_PX_PLANE(12) BSL_PX_PLANE(13) BSL_PX_PLANE(14) BSL_PX_PLANE(15)
    const bool group_ends = !cn.valid || cn.j != c.j || cn.rt != c.rt;
    if (group_ends) flush(c);
    if (!cn.valid) break;
    if (group_ends || cn.bb != c.bb) load_u(cn);
    c = cn;
    s0 = s1;
    cn = next(c);
    s1 = unit_src(cn);
  }
#undef BSL_PX_PLANE
}

// Finishing pass of a product-index launch: y[t][row] is the sum, in workgroup order,
// of the shares of the workgroups whose (non-empty) unit ranges hold units of the row's
// row group (zero for a weight without blocks).  The product kernel precedes this kernel
// in the stream, so its stores are complete.  One workgroup per (row group, 32-row tile):
// thread i reads floats 4 i .. 4 i + 3 of the tile's [16 registers][64 lanes] share (16
// contiguous bytes per thread and share, skipped where every token is past M), adds the
// shares in workgroup order, and the tile goes through LDS as [token][row], so that each
// token's 32 rows are stored as one contiguous run.
template <int R, int NB>
__global__ __launch_bounds__(256) void product_finish_kernel(GroupArgs args) {
  constexpr int TILES = kPxWaves * R;  // 32-row tiles of a row group
  constexpr int GROUP_ROWS = TILES * 32;
  __shared__ float tile[32][33];
  const uint32_t g = blockIdx.x / TILES;  // row group of the launch
  const int tau = (int)(blockIdx.x % TILES);  // tile wave * R + r
  if (g >= args.total_groups) return;
  int j = 0;
  while (j + 1 < args.count && args.w[j + 1].rg_begin <= g) ++j;
  const WeightDesc& W = args.w[j];
  const uint32_t rg = g - W.rg_begin;
  const int M = args.M;
  const uint32_t U = args.total_units;
  const int lg = args.grid_log2;
  const uint32_t NWK = 1u << lg;
  auto owner = [&](uint32_t u) {  // the workgroup o with range_start(o) <= u < range_start(o + 1)
    uint32_t o = (uint32_t)(((uint64_t)u << lg) / U);
    while (o + 1 < NWK && range_start(o + 1, U, lg) <= u) ++o;
    while (range_start(o, U, lg) > u) --o;
    return o;
  };
  const int i = threadIdx.x;
  const int v = i >> 4, lane0 = (i & 15) << 2;  // accumulator register, first of four lanes
  const int h = lane0 >> 5, t0 = lane0 & 31;    // lane half (row bit 2), first token
  const uint32_t per_rg = (uint32_t)(((W.nblocks + NB - 1) / NB) * W.nch);  // units of a row group
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  if (per_rg > 0 && t0 < M) {
    const uint32_t first = W.unit_begin + rg * per_rg;
    const float* share = args.part + (size_t)g * kPxPartFloats + (size_t)tau * 1024 + 4 * i;
    // four shares' loads in flight at once, then their additions in workgroup order
    const uint32_t oe = owner(first + per_rg - 1);
    for (uint32_t ob = owner(first); ob <= oe; ob += 4) {
      float4 p[4];
      bool ok[4];
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {
        const uint32_t o = ob + q;
        ok[q] = o <= oe && range_start(o, U, lg) < range_start(o + 1, U, lg);
        p[q] = ok[q] ? *reinterpret_cast<const float4*>(share + (size_t)o * kPxPartFloats) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      _Pragma("unroll") for (int q = 0; q < 4; ++q) if (ok[q]) {
        s0 += p[q].x;
        s1 += p[q].y;
        s2 += p[q].z;
        s3 += p[q].w;
      }
    }
  }
  const int mm = ((v >> 2) << 3) | (h << 2) | (v & 3);  // row of the tile
  tile[t0][mm] = s0;
  tile[t0 + 1][mm] = s1;
  tile[t0 + 2][mm] = s2;
  tile[t0 + 3][mm] = s3;
  __syncthreads();
  const int row0 = (int)rg * GROUP_ROWS + tau * 32;
  for (int e = i; e < M * 32; e += 256) {
    const int t = e >> 5, r = e & 31;
    if (row0 + r < W.m) store_y(W.y, (size_t)t * W.m + row0 + r, tile[t][r], args.y_fp32);  // y[t][row]
  }
}
static_assert(kPxTiles == 2, "product_finish_kernel indexes two tiles per wave");

// ============================================================ debug unpack
// One wave per sign tile: unpack exactly as the forward kernels do and write the signs.
// Path 0: the single-token kernel's sparse indices (odd form: field 2 s + j, even form:
// field s + 2 j for slot j of a group; s = 1 for a -1 sign).  Path 1: the multi-token
// kernel's +-1 fp16 A fragments.  Path 2: the tile-reconstruct kernel's +-1 pairs.  Lane group g holds columns 8 g .. 8 g + 7 of each plane.
template <int B>
__device__ __forceinline__ void debug_plane(const u32x4& w, int path, int g, int ch, int row, int32_t d, int8_t* out) {
  int8_t sg[8];
  if (path == 0) {
    const uint32_t half = (sign_index(w[plane_word(B)], plane_even(B)) >> (16 * plane_half(B))) & 0xFFFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t field = (half >> (2 * e)) & 3u;
      const uint32_t neg = plane_even(B) ? (field & 1u) : (field >> 1);
      sg[e] = neg ? -1 : 1;
    }
  } else if (path == 1) {
    const half8 h = as_half8(pm1_fragment<B>(w[plane_word(B)], 0x80008000u));
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = (float)h[e] < 0.f ? -1 : 1;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const half2v p = as_half2(tile_sign_pair(w[plane_word(B)], e, plane_even(B), 0x80008000u));
      sg[e] = (float)p[plane_half(B)] < 0.f ? -1 : 1;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int col = ch * kChunkCols + 32 * B + 8 * g + e;
    if (col < d) out[(size_t)row * d + col] = sg[e];
  }
}
template <int... Bs>
__device__ __forceinline__ void debug_planes(std::integer_sequence<int, Bs...>, const u32x4& w, int path, int g, int ch,
                                             int row, int32_t d, int8_t* out) {
  (debug_plane<Bs>(w, path, g, ch, row, d, out), ...);
}
__global__ __launch_bounds__(64) void debug_unpack_kernel(BlockPtrs blk, int32_t m, int32_t d, int32_t mt, int path,
                                                          int8_t* out) {
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int ch = tile / mt, rt = tile % mt;
  const u32x4 w = load16(blk.signs + (size_t)tile * kTileBytes + lane * 16);
  const int row = rt * kTileRows + (lane & 15);
  if (row >= m) return;
  debug_planes(std::make_integer_sequence<int, kPlanes>{}, w, path, lane >> 4, ch, row, d, out);
}

// ============================================================ sign repack (load time)
// Row-major sign bits (m rows of d/8 bytes, least significant bit = lowest column) into
// the tiled layout of bsl_pack_signs, on the device: one thread per 16-byte lane word.
// Lane L = 16 g + i of tile (chunk c, row tile t) holds row 16 t + i; its word q gathers
// the bytes 16 q + g, 16 q + 4 + g, 16 q + 8 + g and 16 q + 12 + g of the row's 64-byte
// segment of chunk c (planes 4 q .. 4 q + 3), each spread to every second bit and placed
// at the odd positions of half 0 / half 1 (planes 4 q, 4 q + 1) and the even positions of
// half 0 / half 1 (planes 4 q + 2, 4 q + 3).  Rows past m and columns past d are 0 (+1).
__device__ __forceinline__ uint32_t spread8(uint32_t x) {
  x = (x | (x << 4)) & 0x0F0Fu;
  x = (x | (x << 2)) & 0x3333u;
  return (x | (x << 1)) & 0x5555u;
}

__global__ __launch_bounds__(256) void repack_signs_kernel(const uint8_t* raw, int64_t m, int64_t rowbytes, int32_t mt,
                                                           uint64_t words, u32x4* out) {
  const uint64_t w = (uint64_t)blockIdx.x * 256 + threadIdx.x;  // (chunk, row tile, lane)
  if (w >= words) return;
  const int lane = (int)(w & 63);
  const uint64_t tile = w >> 6;
  const int64_t t = (int64_t)(tile % (uint64_t)mt), c = (int64_t)(tile / (uint64_t)mt);
  const int g = lane >> 4, i = lane & 15;
  const int64_t r = 16 * t + i;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < m) {
    const uint8_t* seg = raw + r * rowbytes + 64 * c;
    const int64_t have = rowbytes - 64 * c;  // bytes of this chunk present in the row (> 0)
    auto byte = [&](int k) -> uint32_t { return k < have ? (uint32_t)seg[k] : 0u; };
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = (spread8(byte(16 * q + g)) << 1) | (spread8(byte(16 * q + 4 + g)) << 17) | spread8(byte(16 * q + 8 + g)) |
             (spread8(byte(16 * q + 12 + g)) << 16);
  }
  out[w] = v;
}

int launch_repack_signs(const uint8_t* raw, int64_t m, int64_t d, int32_t mt, int32_t nch, uint8_t* out, void* stream) {
  const uint64_t words = (uint64_t)nch * mt * 64;
  const uint64_t blocks = (words + 255) / 256;
  if (blocks == 0) return 0;
  if (blocks > 0x7fffffffull) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(repack_signs_kernel, dim3((uint32_t)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), raw, m,
                     d / 8, mt, words, reinterpret_cast<u32x4*>(out));
  return (int)hipGetLastError();
}

// ============================================================ static scratch
// Scratch memory of the allocation-free forward: the row accumulators of the single- and
// few-token kernels, kStaticScratchBytes per device for the life of the
// process, shared by every such call on the device.  Host code never passes the array's
// name to a kernel or a copy (on the host it is only a stand-in for the symbol): it uses
// the device address static_scratch_setup takes once per device.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int static_scratch_setup(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return 0;
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, uint32_t n, uint32_t v) {
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = v;
}

int launch_fill_u32(uint32_t* p, uint32_t n, uint32_t v, void* stream) {
  if (n == 0) return 0;
  const uint32_t blocks = std::min<uint32_t>(64, (n + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), p, n, v);
  return (int)hipGetLastError();
}

// ============================================================ launchers
int launch_decode_m1(const GroupArgs& args, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  // 16 waves x 4 row tiles, 4 waves per SIMD (one workgroup per CU: all waves advance
  // together, so no workgroup is left running alone on a CU at the end).  With no units
  // at all (every weight empty) one workgroup still runs, to write y = 0.
  hipLaunchKernelGGL((decode_m1_kernel<kDecodeWaves, kDecodeGroupTiles / kDecodeWaves, kDecodeWaves / 4>),
                     dim3(1u << args.grid_log2), dim3(kDecodeWaves * 64), 0, st, args);
  return (int)hipGetLastError();
}

int launch_decode_wp(const GroupArgs& args, int tokens, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((1u << args.grid_log2) / kWpWaves), block(kWpWaves * 64);
  switch (tokens) {
    case 1: hipLaunchKernelGGL((decode_wp_kernel<16, 1>), grid, block, 0, st, args); break;
    case 2: hipLaunchKernelGGL((decode_wp_kernel<8, 2>), grid, block, 0, st, args); break;
    case 3: hipLaunchKernelGGL((decode_wp_kernel<8, 3>), grid, block, 0, st, args); break;
    case 4: hipLaunchKernelGGL((decode_wp_kernel<8, 4>), grid, block, 0, st, args); break;
    default: return (int)hipErrorInvalidValue;
  }
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

int launch_tile(const GroupArgs& args, int token_tiles, int token_groups, void* stream) {
  if (args.total_items == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)args.total_items);
  switch (token_tiles) {
    case 1: hipLaunchKernelGGL((tile_kernel<1, 2>), grid, dim3(256), 0, st, args, token_groups); break;
    case 2: hipLaunchKernelGGL(tile_split_kernel<2>, grid, dim3(512), 0, st, args, token_groups); break;
    case 4: hipLaunchKernelGGL(tile_split_kernel<4>, grid, dim3(512), 0, st, args, token_groups); break;
    case 8: hipLaunchKernelGGL(tile_split_kernel<8>, grid, dim3(512), 0, st, args, token_groups); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_product(const GroupArgs& args, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL((product_kernel<kPxTiles, kPxBatch>), dim3(1u << args.grid_log2), dim3(kPxWaves * 64), 0, st, args);
  return (int)hipGetLastError();
}

int launch_product_finish(const GroupArgs& args, void* stream) {
  if (args.total_groups == 0) return 0;
  const unsigned blocks = args.total_groups * (unsigned)(kPxWaves * kPxTiles);  // one per (row group, 32-row tile)
  hipLaunchKernelGGL((product_finish_kernel<kPxTiles, kPxBatch>), dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), args);
  return (int)hipGetLastError();
}

int launch_layout_pass(const GroupArgs& args, void* stream) {
  const unsigned waves = (unsigned)args.total_items + args.total_units;
  if (waves == 0) return 0;
  hipLaunchKernelGGL(layout_pass_kernel, dim3(std::min((waves + 3u) / 4u, 2048u)), dim3(256), 0, static_cast<hipStream_t>(stream), args);
  return (int)hipGetLastError();
}

int launch_v_rank_major(const GroupArgs& args, void* stream) {
  if (args.total_items == 0) return 0;
  const unsigned waves = (unsigned)args.total_items;
  const dim3 grid(std::min((waves + 3u) / 4u, 2048u));
  hipLaunchKernelGGL(v_rank_major_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), args);
  return (int)hipGetLastError();
}

int launch_debug_unpack(BlockPtrs blk, int32_t m, int32_t d, int32_t mt, int32_t nch, int path, int8_t* out,
                        void* stream) {
  hipLaunchKernelGGL(debug_unpack_kernel, dim3(mt * nch), dim3(64), 0, static_cast<hipStream_t>(stream), blk, m, d, mt,
                     path, out);
  return (int)hipGetLastError();
}

}  // namespace bsl
