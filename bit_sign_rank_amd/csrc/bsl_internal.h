// Internal declarations shared by the host side (bsl_host.cpp) and the kernels
// (bsl_kernels.hip) of libbitstack_linear.  Not part of the public interface.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

namespace bsl {

// Tile geometry of the packed sign layout (one 16x32x32 fp16 MFMA fragment per
// plane, 16 planes per 512-column chunk; see bsl_pack_signs in the public header).
constexpr int kRank = 16;         // k: rank of U_i, V_i (also the MFMA N width)
constexpr int kTileRows = 16;     // rows per sign tile
constexpr int kChunkCols = 512;   // columns per sign tile
constexpr int kPlanes = 16;       // 32-column planes per chunk
constexpr int kTileBytes = 1024;  // 16 x 512 bits
constexpr int kMaxGroup = 8;      // weights per grouped launch
constexpr int kMaxBlocks = 64;    // blocks per weight (the kernels keep the table in LDS)

// Rows are padded to a multiple of 1024 (64 tiles, the largest row group any kernel
// takes), so every kernel can read whole row groups without bounds checks; padding
// rows have +1 signs and zero U, so they add nothing.
constexpr int kRowAlign = 1024;
inline int64_t pad_rows(int64_t m) { return (m + kRowAlign - 1) / kRowAlign * kRowAlign; }
inline int64_t pad_cols(int64_t d) { return (d + kChunkCols - 1) / kChunkCols * kChunkCols; }

// Device addresses of one loaded block.  One allocation holds, in order:
//   signs: [d_pad/512][m_pad/16][64 lanes][16 B]                 (tiled bits)
//   u:     [m_pad/16][64 lanes][4] fp16  lane L holds U[16 t + 4 (L/16) + v][L % 16]
//   v:     [d_pad/512][16 planes][64 lanes][8] fp16
//          lane L of plane b holds V[512 c + 32 b + 8 (L/16) + j][L % 16], j = 0..7
//          (zero past d)
// That is the only copy of each factor.  The wave-private kernel forms its B-operand
// order from two 8-byte loads of v; the tile kernels gather each row's 8 ranks of U from
// u once per batch and read V in rank order from a copy formed per call (WeightDesc::vr).
struct BlockPtrs {
  const uint8_t* signs;
  const uint16_t* u;
  const uint16_t* v;
};

// One weight of a (grouped) forward launch; passed by value in the kernel arguments.
struct WeightDesc {
  const BlockPtrs* blocks;  // device table of the loaded blocks
  const uint16_t* x;        // [M][d] fp16
  void* y;                  // [M][m] fp16 or fp32
  float* partial;           // multi-token path: [split][token][row] partial sums (workspace)
  uint32_t* counters;       // multi-token path: arrival counters, one per (row group, token group)
                            // (workspace, zero between calls)
  uint16_t* vr;             // tile path: V of the loaded blocks in rank-major order, [block][d_pad][16]
                            // fp16 (workspace, formed by launch_v_rank_major at the start of the call)
  uint32_t* xt;             // product-index path: the sparse MFMA's B operands (+-x), [chunk][plane][k]
                            // [words 0-3 | 4-7][64 lanes][4 words] (workspace, formed by launch_layout_pass)
  int32_t m, d;             // true sizes
  int32_t mt, nch;          // row tiles (m_pad / 16), column chunks (d_pad / 512)
  int32_t nblocks;          // loaded blocks
  int32_t item_begin;       // multi-token path: first work item of this weight in the launch
  int32_t groups;           // output groups (row groups x token groups) of this weight
  int32_t splits;           // single-token path: nch; multi-token path: ranges of the (block, chunk)
                            // sequence, ceil(nblocks nch / splits) pairs each
  uint32_t unit_begin;      // single-token path: first (row group, block, chunk) unit of this weight
  uint32_t units;           // single-token path: groups * nblocks * nch
  uint32_t rg_begin;        // single-token path: first row group of this weight in the launch
};

struct GroupArgs {
  WeightDesc w[kMaxGroup];
  int32_t count;
  int32_t total_items;   // multi-token path: workgroups
  int32_t M;
  int32_t y_fp32;
  uint32_t total_units;  // single-token path: (row group, block, chunk) units over all weights
  uint32_t total_groups; // single-token path: row groups over all weights
  int32_t grid_log2;     // single-token path: log2 of the (power-of-two) grid
  const void* zero_page; // kZeroPageBytes of zeros: target of prefetches past the end of the work
  float* part;           // product-index path: each workgroup's fp32 share of each row group it works on,
                         // slot (row group + workgroup) of kPxPartFloats floats (workspace)
  uint64_t* acc;         // single- and few-token paths: row accumulators, [total_groups][rows x tokens of a
                         // row group], zero between launches (workspace)
};

// Kernel launchers (bsl_kernels.hip).  Return a hipError_t value.
int launch_decode_m1(const GroupArgs& args, void* stream);
int launch_decode_wp(const GroupArgs& args, int tokens, void* stream);  // tokens: 1 to 4
int launch_prefill(const GroupArgs& args, int token_tile, int token_groups, void* stream);
int launch_tile(const GroupArgs& args, int token_tiles, int token_groups, void* stream);
// V of every loaded block of args' weights -> WeightDesc::vr; item_begin / total_items
// count (block, 64-column step) pairs.
int launch_v_rank_major(const GroupArgs& args, void* stream);
// Product-index kernel: units and workers as args.total_units / grid_log2 (2^grid_log2
// workgroups), WeightDesc::groups = row groups, rg_begin = first 32-row tile, acc = row
// accumulators, vr / xt = the per-call layouts of V and x.
int launch_product(const GroupArgs& args, void* stream);
// After launch_product on the same stream: y from the row groups' shares, added in
// workgroup order.
int launch_product_finish(const GroupArgs& args, void* stream);
// The product-index path's layout passes in one launch: the rank-major V pass (total_items
// (weight, block, 64-column step) pairs, item_begin per weight) and x of args' weights (M
// <= kPxMaxTokens tokens) as the kernel's B operands -> WeightDesc::xt (total_units items
// of (weight, chunk, plane, k), unit_begin = each weight's first (weight, chunk) pair).
int launch_layout_pass(const GroupArgs& args, void* stream);
constexpr size_t kPxLaneBytesPerChunk = (size_t)kPlanes * 2 * 64 * 32;  // 64 KiB
// Row-major sign bits (device, m rows of d/8 bytes) -> the tiled sign layout (device, the
// first bsl_packed_sign_bytes(m, d) bytes of a block slot).
int launch_repack_signs(const uint8_t* raw, int64_t m, int64_t d, int32_t mt, int32_t nch, uint8_t* out, void* stream);
int launch_debug_unpack(BlockPtrs blk, int32_t m, int32_t d, int32_t mt, int32_t nch, int path, int8_t* out,
                        void* stream);

// Single-token path: rows are taken in row groups of 64 tiles (1024 rows), one
// persistent 16-wave workgroup per CU.  A workgroup walks an equal share of the (row
// group, block, chunk) units and adds its share of every row of a row group it touches to
// that row's 64-bit accumulator; the workgroup that completes a row writes y.
constexpr int kDecodeGroupTiles = 64;
constexpr int kDecodeWaves = 16;
constexpr int kDecodeGroupRows = kDecodeGroupTiles * 16;
constexpr int kZeroPageBytes = 65536;
// Workgroups that may share one row group of the single-token kernel: the row
// accumulators count them in 6 bits (the host shrinks the grid to stay within this).
constexpr int kAccMaxParts = 63;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin over 8 XCDs
// Single-token path, wave-private kernel: one worker per wave, four waves per workgroup
// (one per SIMD), one workgroup per CU; units of 16 row tiles (256 rows).  A workgroup
// keeps the activations of the weights its units belong to in LDS (at most kWpXBytes).
// The same kernel takes T = 2, 3 or 4 tokens with units of 8 row tiles (kWpFewRows).
constexpr int kWpTiles = 16;
constexpr int kWpRows = kWpTiles * 16;
constexpr int kWpFewRows = 128;
constexpr int kWpWaves = 4;
constexpr int kWpXBytes = 148 * 1024;
constexpr int kWpMaxTokens = 4;
// Multi-token path (M >= 2): one 8-wave workgroup per item = (512-row group, token
// group of 2, 4 or 8 tokens, range of the (block, chunk) sequence).  A weight's items are
// split along that sequence only while splits x padded tokens fit the workspace.
constexpr int kPrefillGroupRows = 512;  // rows per workgroup (8 waves x 64)
constexpr int kMaxSplits = 8;
constexpr int kSplitTokens = 128;       // splits x padded tokens the partial-sum workspace holds
// Tile-reconstruct path: one 4-wave workgroup per (64-row group, group of 64 TT tokens,
// TT = 1, 2, 4 or 8).  Each 32-row tile is shared by two waves that rebuild half of the
// blocks each, swap their partial tiles through LDS and own half of the tokens each.
constexpr int kTileGroupRows = 64;
constexpr int kTileMaxTokenTiles = 8;   // 32-token tiles per wave
constexpr int kTileBatch = 8;           // blocks whose U fragments and sign words stay in registers
constexpr int kTileAutoMinTokens = 33;  // BSL_PATH_AUTO takes the tile path from this M on
constexpr int kPxAutoMinTokens = 4;     // and the product-index path from this M to kTileAutoMinTokens - 1
// Product-index path (M = 2..32 under BSL_PATH_PRODUCT): one worker per workgroup of
// kPxWaves waves (two per SIMD, one workgroup per CU); units (weight, row group of
// kPxWaves x kPxTiles 32-row tiles, batch of kPxBatch blocks, 512-column chunk), each wave
// owning kPxTiles tiles of the group.  The shares of a row group go to slots of
// kPxPartFloats floats, in each wave's MFMA result layout [wave][tile][register][lane].
constexpr int kPxWaves = 8;
constexpr int kPxTiles = 2;
constexpr int kPxBatch = 2;
constexpr int kPxMaxTokens = 32;
constexpr int kPxPartFloats = 8 * 2 * 16 * 64;  // kPxWaves x kPxTiles x 16 registers x 64 lanes
constexpr int kPxTileRows = 32;
// Tile-path items may be cut along the columns (chunk ranges) when a launch has too few
// of them to fill the chip; the ranges' partial sums go to a workspace of the stack.
constexpr size_t kTileWorkspaceFloats = (size_t)16 << 20;  // 64 MiB
constexpr int kTileItemsPerCu = 2;     // aim of the column-range cutting
constexpr int kTileCounters = 1 << 16;

// Allocation-free forward (bsl_forward_group_static): the single- and few-token kernels
// row accumulators in one static device array per device (see bsl_kernels.hip).
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
// Address of this process's static scratch array on `device` (which must be the current
// device), taken with hipGetSymbolAddress on the first call for that device.  Returns a
// hipError_t value.
int static_scratch_setup(int device, void** out);
// p[0 .. n) = v on `stream` (a kernel, so that captured streams hold no memset node).
int launch_fill_u32(uint32_t* p, uint32_t n, uint32_t v, void* stream);

// Records the calling thread's error message (bsl_last_error) and returns code.
int set_error(int code, const std::string& msg);

// ---------------------------------------------------------------- vanilla-SVD baseline
// Factors of one weight, for n_cap blocks of rank k' padded to kp8 = roundup(k', 8)
// (padding ranks are zero):
//   vt: [n_cap kp8][d_pad512] fp16: row i kp8 + r holds V'_i[:, r] (zero past d)
//   ut: [m_pad64 / 64][n_cap kp8 / 8][64][8] fp16: lane L of row group g, column group q
//       holds U'[64 g + L][8 q .. 8 q + 7] over the blocks' concatenated ranks
// Phase 1 (one wave per row of vt): t[token][row] = x[token] . vt[row]  (fp32)
// Phase 2 (one workgroup per 64 rows): y[token][row] = sum over loaded columns of
//         ut[row][col] t[token][col]
constexpr int kLrTokens = 8;       // tokens per launch pair
constexpr int kLrColAlign = 512;
constexpr int kLrRowGroup = 64;
constexpr int kLrPhase2Waves = 8;

struct LrWeight {
  const uint16_t* vt;
  const uint16_t* ut;
  const uint16_t* x;  // [T][d] fp16
  void* y;            // [T][m]
  float* t;           // [kLrTokens][ld] workspace
  int32_t m, d, d_pad;
  int32_t ld;         // n_cap kp8: row stride of t, column groups x 8 of ut
  int32_t kcat;       // n kp8: loaded rows of vt / columns of ut
  int32_t row_begin;  // phase 1: first vt row of this weight in the launch
  int32_t rg_begin;   // phase 2: first row group of this weight in the launch
};

struct LrArgs {
  LrWeight w[kMaxGroup];
  int32_t count;
  int32_t T;          // tokens of this launch pair (1..kLrTokens)
  int32_t y_fp32;
  int32_t total_rows; // phase 1 rows (waves)
  int32_t total_rgs;  // phase 2 row groups (workgroups)
};

int launch_lowrank(const LrArgs& args, void* stream);

}  // namespace bsl
