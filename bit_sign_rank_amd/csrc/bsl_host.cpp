// Host side of libbitstack_linear: argument checking, the sign packer ("bitstack_pack"),
// the device-resident block stack and forward dispatch.  See include/bitstack_linear.h
// for the interface contract.
#include "bitstack_linear.h"

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "bsl_fp16.h"
#include "bsl_internal.h"

using namespace bsl;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  (void)hipGetLastError();  // clear the sticky error so the next call starts clean
  return fail(e == hipErrorOutOfMemory ? BSL_ENOMEM : BSL_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool shape_ok(int64_t m, int64_t d) { return m >= 1 && m <= (1 << 20) && d >= 8 && d <= (1 << 20) && d % 8 == 0; }

// ------------------------------------------------------------------ packing
// Lane L = 16 g + i of tile (row tile t, chunk c) holds row 16 t + i and, of every
// plane b (columns 512 c + 32 b .. + 31), the columns 32 b + 8 g + e, e = 0..7: these
// eight signs are bit e of byte 64 c + 4 b + g of the row-major source row.  They go to
// word b / 4, half b % 2, bit 2 e + 1 (planes with (b / 2) % 2 == 0, "odd" positions) or
// bit 2 e ("even" positions), so the word is the sum of the four planes' bytes spread
// out to every second bit.

// Spread the 8 bits of a byte to bit positions 0, 2, .., 14 (table of all 256 bytes).
struct SpreadTable {
  uint16_t v[256];
  SpreadTable() {
    for (uint32_t x = 0; x < 256; ++x) {
      uint32_t y = 0;
      for (int e = 0; e < 8; ++e) y |= ((x >> e) & 1u) << (2 * e);
      v[x] = (uint16_t)y;
    }
  }
};
const SpreadTable kSpread;

void pack_rows(const uint8_t* src, int64_t m, int64_t d, uint8_t* out, int64_t r0, int64_t r1) {
  const int64_t nch = pad_cols(d) / kChunkCols;
  const int64_t mt = pad_rows(m) / kTileRows;
  const int64_t rowbytes = d / 8;
  const uint16_t* sp = kSpread.v;
  uint8_t tail[64];
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t t = r / kTileRows, i = r % kTileRows;
    for (int64_t c = 0; c < nch; ++c) {
      uint8_t* tile = out + (c * mt + t) * kTileBytes;
      // the chunk's 64 source bytes of this row (zeros past the row's end or past m)
      const uint8_t* seg;
      if (r < m && 64 * (c + 1) <= rowbytes) {
        seg = src + r * rowbytes + 64 * c;
      } else {
        std::memset(tail, 0, sizeof(tail));
        if (r < m && 64 * c < rowbytes) std::memcpy(tail, src + r * rowbytes + 64 * c, (size_t)(rowbytes - 64 * c));
        seg = tail;
      }
      for (int g = 0; g < 4; ++g) {
        uint32_t words[4];
        for (int q = 0; q < 4; ++q) {
          // plane 4 q + k is source byte 4 (4 q + k) + g; half k % 2, odd positions for k < 2
          const uint8_t* bq = seg + 16 * q + g;
          words[q] = ((uint32_t)sp[bq[0]] << 1) | ((uint32_t)sp[bq[4]] << 17) | (uint32_t)sp[bq[8]] |
                     ((uint32_t)sp[bq[12]] << 16);
        }
        std::memcpy(tile + (16 * g + i) * 16, words, 16);  // little-endian words
      }
    }
  }
}

void pack_signs_mt(const uint8_t* src, int64_t m, int64_t d, uint8_t* out) {
  const int64_t mp = pad_rows(m);
  unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  const int64_t work = mp * pad_cols(d);
  if (work < (int64_t)1 << 22) nt = 1;
  std::vector<std::thread> th;
  const int64_t per = (mp / kTileRows + nt - 1) / nt * kTileRows;
  for (unsigned k = 0; k < nt; ++k) {
    const int64_t r0 = k * per, r1 = std::min(mp, r0 + per);
    if (r0 >= r1) break;
    th.emplace_back(pack_rows, src, m, d, out, r0, r1);
  }
  for (auto& t : th) t.join();
}

// U (m x 16, row-major fp16) -> [m_pad/16][64][4]: lane L, slot v holds U[16 t + 4 (L/16) + v][L % 16].
void tile_u(const uint16_t* u, int64_t m, uint16_t* out) {
  const int64_t mt = pad_rows(m) / kTileRows;
  for (int64_t t = 0; t < mt; ++t)
    for (int L = 0; L < 64; ++L)
      for (int v = 0; v < 4; ++v) {
        const int64_t row = 16 * t + 4 * (L / 16) + v;
        out[(t * 64 + L) * 4 + v] = row < m ? u[row * kRank + (L % 16)] : 0;
      }
}

// V (d x 16, row-major fp16) -> [d_pad/512][16][64][8]: lane L of plane b, slot j holds
// V[512 c + 32 b + 8 (L/16) + j][L % 16].
void tile_v(const uint16_t* v, int64_t d, uint16_t* out) {
  const int64_t nch = pad_cols(d) / kChunkCols;
  for (int64_t c = 0; c < nch; ++c)
    for (int b = 0; b < kPlanes; ++b)
      for (int L = 0; L < 64; ++L)
        for (int j = 0; j < 8; ++j) {
          const int64_t col = 512 * c + 32 * b + 8 * (L / 16) + j;
          out[((c * kPlanes + b) * 64 + L) * 8 + j] = col < d ? v[col * kRank + (L % 16)] : 0;
        }
}

// V (d x 16, row-major fp16) -> [d_pad][16], zero past d.
void rowmajor_v(const uint16_t* v, int64_t d, uint16_t* out) {
  std::memcpy(out, v, (size_t)d * kRank * 2);
  std::memset(out + d * kRank, 0, (size_t)(pad_cols(d) - d) * kRank * 2);
}

// U (m x 16, row-major fp16) -> [m_pad][16], zero past m.
void rowmajor_u(const uint16_t* u, int64_t m, uint16_t* out) {
  std::memcpy(out, u, (size_t)m * kRank * 2);
  std::memset(out + m * kRank, 0, (size_t)(pad_rows(m) - m) * kRank * 2);
}

// V (d x 16, row-major fp16) -> [d_pad/512][16][64][8] in the single-token kernel's
// B-operand order: lane L = 16 kk + r of plane b holds V[512 c + 32 b + 4 kk + j][r] for
// j < 4 and V[512 c + 32 b + 16 + 4 kk + j - 4][r] for j >= 4 (zero past d).
void bop_v(const uint16_t* v, int64_t d, uint16_t* out) {
  const int64_t nch = pad_cols(d) / kChunkCols;
  for (int64_t c = 0; c < nch; ++c)
    for (int b = 0; b < kPlanes; ++b)
      for (int L = 0; L < 64; ++L)
        for (int j = 0; j < 8; ++j) {
          const int kk = L / 16, r = L % 16;
          const int64_t col = 512 * c + 32 * b + (j < 4 ? 4 * kk + j : 16 + 4 * kk + j - 4);
          out[((c * kPlanes + b) * 64 + L) * 8 + j] = col < d ? v[col * kRank + r] : 0;
        }
}

// V (d x 16) with row c multiplied by inv_scale[c]: one rounding of the exact product.
bool scale_v(const uint16_t* v, int64_t d, const float* inv_scale, uint16_t* out) {
  for (int64_t c = 0; c < d; ++c)
    for (int r = 0; r < kRank; ++r)
      if (!double_to_fp16(fp16_to_double(v[c * kRank + r]) * (double)inv_scale[c], &out[c * kRank + r])) return false;
  return true;
}

}  // namespace

// ------------------------------------------------------------------ stack
struct Slot {
  void* mem = nullptr;  // one device allocation per block
  size_t bytes = 0;
};

struct Weight {
  int32_t m = 0, d = 0, mt = 0, nch = 0;
  int32_t n = 0;  // loaded blocks
  std::vector<bsl_block_src> src;
  std::vector<Slot> slots;          // [n_cap]
  std::vector<float> inv_scale;     // [d] input-channel scale folded into V at load (empty: none)
  BlockPtrs* dtable = nullptr;      // device [n_cap]
  float* partial = nullptr;         // workspace
  uint32_t* counters = nullptr;     // workspace: arrival counters of the multi-token path
  size_t partial_floats = 0, counter_count = 0;
};

struct bsl_stack {
  int device = 0;
  int32_t k = 16, n_cap = 0;
  int32_t decode_grid_max = 256;  // largest power of two <= compute units
  int32_t path = BSL_PATH_AUTO;   // multi-token formulation (bsl_set_path)
  int32_t decode = BSL_DECODE_AUTO;  // single-token kernel (bsl_set_decode)
  uint64_t budget = 0, resident = 0;
  void* zero_page = nullptr;      // kZeroPageBytes of zeros on the device
  float* pieces = nullptr;        // single-token partial sums (shared by the stack's launches)
  uint32_t* arrivals = nullptr;   // single-token arrival counters, one per row group of a launch
  float* tile_ws = nullptr;       // tile path: partial sums of column ranges (kTileWorkspaceFloats)
  uint8_t* staging[2] = {nullptr, nullptr};  // pinned host buffers of bsl_load_blocks (allocated on first use)
  size_t staging_bytes = 0;
  hipEvent_t staged[2] = {nullptr, nullptr};  // copy out of staging[k] finished
  uint32_t* tile_ctr = nullptr;   // tile path: arrival counters (kTileCounters), zero between launches
  // dense path (set up by bsl_set_path): restored W_hat of up to kMaxGroup weights, a
  // rocBLAS handle and its workspace
  uint16_t* dense_ws = nullptr;
  size_t dense_ws_bytes = 0;
  void* blas_ws = nullptr;
  rocblas_handle blas = nullptr;
  std::vector<Weight> w;
};

namespace {

// signs + tiled U + tiled V + row-major V + B-ordered V + row-major U (see BlockPtrs)
size_t slot_bytes(int64_t m, int64_t d) {
  return (size_t)pad_rows(m) * pad_cols(d) / 8 + 2 * (size_t)pad_rows(m) * kRank * 2 + 3 * (size_t)pad_cols(d) * kRank * 2;
}

BlockPtrs slot_ptrs(const Slot& s, int64_t m, int64_t d) {
  BlockPtrs p;
  const uint8_t* base = static_cast<const uint8_t*>(s.mem);
  const size_t sb = (size_t)pad_rows(m) * pad_cols(d) / 8;
  const size_t ub = (size_t)pad_rows(m) * kRank * 2;
  const size_t vb = (size_t)pad_cols(d) * kRank * 2;
  p.signs = base;
  p.u = reinterpret_cast<const uint16_t*>(base + sb);
  p.v = reinterpret_cast<const uint16_t*>(base + sb + ub);
  p.vr = reinterpret_cast<const uint16_t*>(base + sb + ub + vb);
  p.vb = reinterpret_cast<const uint16_t*>(base + sb + ub + 2 * vb);
  p.ur = reinterpret_cast<const uint16_t*>(base + sb + ub + 3 * vb);
  return p;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

// Writes table entries [lo, hi) only: entries below lo may be read meanwhile by forwards
// still running on other streams (a grown weight keeps its first blocks).
int upload_table(Weight& W, int32_t lo, int32_t hi, hipStream_t st) {
  if (hi <= lo) return BSL_OK;
  std::vector<BlockPtrs> tab(hi - lo);
  for (int32_t i = lo; i < hi; ++i)
    tab[i - lo] = W.slots[i].mem ? slot_ptrs(W.slots[i], W.m, W.d) : BlockPtrs{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  hipError_t e = hipMemcpyAsync(W.dtable + lo, tab.data(), sizeof(BlockPtrs) * (hi - lo), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return e == hipSuccess ? BSL_OK : hip_fail(e, "pointer table upload");
}

// Row groups of the single-token kernel (kDecodeGroupTiles row tiles each).
int decode_groups(const Weight& W) { return (W.mt + kDecodeGroupTiles - 1) / kDecodeGroupTiles; }
int prefill_groups(const Weight& W) { return (W.mt * kTileRows + kPrefillGroupRows - 1) / kPrefillGroupRows; }

}  // namespace

int bsl::set_error(int code, const std::string& msg) { return fail(code, msg); }

extern "C" {

const char* bsl_last_error(void) { return g_err.c_str(); }

size_t bsl_block_bytes(int64_t m, int64_t d, int32_t k) {
  if (m < 1 || d < 8 || d % 8 || k < 1) return 0;
  return (size_t)(m * d / 8 + 2 * (int64_t)k * (m + d));
}

size_t bsl_packed_sign_bytes(int64_t m, int64_t d) {
  if (!shape_ok(m, d)) return 0;
  return (size_t)pad_rows(m) * pad_cols(d) / 8;
}

int bsl_pack_signs(const uint8_t* rowmajor_bits, int64_t m, int64_t d, uint8_t* tiled_out) {
  if (!rowmajor_bits || !tiled_out) return fail(BSL_EINVAL, "bsl_pack_signs: null pointer");
  if (!shape_ok(m, d)) return fail(BSL_EUNSUPPORTED, "bsl_pack_signs: need 1 <= m, 8 <= d, d % 8 == 0");
  pack_signs_mt(rowmajor_bits, m, d, tiled_out);
  return BSL_OK;
}

int bsl_unpack_signs(const uint8_t* tiled, int64_t m, int64_t d, int8_t* pm1_out) {
  if (!tiled || !pm1_out) return fail(BSL_EINVAL, "bsl_unpack_signs: null pointer");
  if (!shape_ok(m, d)) return fail(BSL_EUNSUPPORTED, "bsl_unpack_signs: need 1 <= m, 8 <= d, d % 8 == 0");
  const int64_t mt = pad_rows(m) / kTileRows;
  for (int64_t r = 0; r < m; ++r) {
    const int64_t t = r / kTileRows, i = r % kTileRows;
    for (int64_t col = 0; col < d; ++col) {
      const int64_t c = col / kChunkCols, cc = col % kChunkCols;
      const int b = (int)(cc / 32), rem = (int)(cc % 32), g = rem / 8, e = rem % 8;
      const int q = b / 4, half = b % 2, odd = (b / 2) % 2 == 0 ? 1 : 0;
      uint32_t word;
      std::memcpy(&word, tiled + (c * mt + t) * kTileBytes + (16 * g + i) * 16 + 4 * q, 4);
      const uint32_t bit = (word >> (16 * half + 2 * e + odd)) & 1u;
      pm1_out[r * d + col] = bit ? -1 : 1;
    }
  }
  return BSL_OK;
}

int bsl_init(bsl_stack** out, int device, int32_t num_weights, const int32_t* m, const int32_t* d, int32_t k,
             int32_t n_cap, uint64_t budget_bytes) {
  if (!out || !m || !d) return fail(BSL_EINVAL, "bsl_init: null pointer");
  *out = nullptr;
  if (num_weights < 1 || num_weights > (1 << 20)) return fail(BSL_EINVAL, "bsl_init: num_weights out of range");
  if (n_cap < 1 || n_cap > kMaxBlocks) return fail(BSL_EINVAL, "bsl_init: n_cap must be in 1..64");
  if (k != kRank) return fail(BSL_EUNSUPPORTED, "bsl_init: only k = 16 is supported");
  for (int32_t w = 0; w < num_weights; ++w)
    if (!shape_ok(m[w], d[w])) return fail(BSL_EUNSUPPORTED, "bsl_init: weight " + std::to_string(w) + " has an unsupported shape");
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= ndev) return fail(BSL_EINVAL, "bsl_init: no such device");
  DeviceGuard guard(device);
  bsl_stack* s = new (std::nothrow) bsl_stack;
  if (!s) return fail(BSL_ENOMEM, "bsl_init: host allocation failed");
  s->device = device;
  s->k = k;
  s->n_cap = n_cap;
  s->budget = budget_bytes;
  s->w.resize(num_weights);
  int rc = BSL_OK;
  size_t max_groups = 0;
  int cus = 0;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device)) != hipSuccess)
    rc = hip_fail(e, "hipDeviceGetAttribute(multiprocessors)");
  else {
    s->decode_grid_max = 1;
    while (s->decode_grid_max * 2 <= std::max(1, cus)) s->decode_grid_max *= 2;
    if ((e = hipMalloc(&s->zero_page, kZeroPageBytes)) != hipSuccess) rc = hip_fail(e, "hipMalloc(zero page)");
    else if ((e = hipMemset(s->zero_page, 0, kZeroPageBytes)) != hipSuccess) rc = hip_fail(e, "hipMemset(zero page)");
  }
  for (int32_t w = 0; w < num_weights && rc == BSL_OK; ++w) {
    Weight& W = s->w[w];
    W.m = m[w];
    W.d = d[w];
    W.mt = (int32_t)(pad_rows(W.m) / kTileRows);
    W.nch = (int32_t)(pad_cols(W.d) / kChunkCols);
    W.slots.resize(n_cap);
    const size_t mpad = (size_t)pad_rows(W.m);
    W.partial_floats = (size_t)kSplitTokens * mpad;
    // split items have at most kSplitTokens / 2 padded tokens, so at most 32 token groups
    W.counter_count = (size_t)prefill_groups(W) * (kSplitTokens / 4);
    const size_t words = W.counter_count;
    max_groups = std::max<size_t>(max_groups, (size_t)decode_groups(W));
    if ((e = hipMalloc(&W.dtable, sizeof(BlockPtrs) * n_cap)) != hipSuccess) rc = hip_fail(e, "hipMalloc(table)");
    else if ((e = hipMalloc(&W.partial, W.partial_floats * sizeof(float))) != hipSuccess) rc = hip_fail(e, "hipMalloc(workspace)");
    else if ((e = hipMalloc(&W.counters, words * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMalloc(counters)");
    else if ((e = hipMemset(W.counters, 0, words * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMemset(counters)");
    else if ((e = hipMemset(W.dtable, 0, sizeof(BlockPtrs) * n_cap)) != hipSuccess) rc = hip_fail(e, "hipMemset(table)");
  }
  if (rc == BSL_OK) {
    // single- and few-token pieces: at most (row groups of one launch) + (workers) of them,
    // 1024 floats a piece for decode_m1_kernel, 256 a piece for the wave-private kernel,
    // whose row groups take 256 / T rows for T tokens
    const size_t n = ((size_t)kMaxGroup * max_groups * kWpMaxTokens + (size_t)s->decode_grid_max) * kDecodeGroupRows;
    // (arrival counters per row group: the wave-private kernel's are the smallest)
    const size_t na = (size_t)kMaxGroup * max_groups * (kDecodeGroupRows / kWpRows) * kWpMaxTokens;
    if ((e = hipMalloc(&s->pieces, n * sizeof(float))) != hipSuccess) rc = hip_fail(e, "hipMalloc(pieces)");
    else if ((e = hipMalloc(&s->arrivals, na * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMalloc(arrivals)");
    else if ((e = hipMemset(s->arrivals, 0, na * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMemset(arrivals)");
    else if ((e = hipMalloc(&s->tile_ws, kTileWorkspaceFloats * sizeof(float))) != hipSuccess) rc = hip_fail(e, "hipMalloc(tile workspace)");
    else if ((e = hipMalloc(&s->tile_ctr, kTileCounters * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMalloc(tile counters)");
    else if ((e = hipMemset(s->tile_ctr, 0, kTileCounters * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMemset(tile counters)");
  }
  if (rc == BSL_OK && (e = hipDeviceSynchronize()) != hipSuccess) rc = hip_fail(e, "hipDeviceSynchronize");
  if (rc != BSL_OK) {
    std::string msg = g_err;
    bsl_destroy(s);
    g_err = msg;
    return rc;
  }
  *out = s;
  return BSL_OK;
}

int bsl_set_source(bsl_stack* s, int32_t w, int32_t n_avail, const bsl_block_src* blocks) {
  if (!s) return fail(BSL_EINVAL, "bsl_set_source: null stack");
  if (w < 0 || w >= (int32_t)s->w.size()) return fail(BSL_EINVAL, "bsl_set_source: weight index out of range");
  if (n_avail < 0 || n_avail > s->n_cap) return fail(BSL_EINVAL, "bsl_set_source: n_avail must be in 0..n_cap");
  if (n_avail > 0 && !blocks) return fail(BSL_EINVAL, "bsl_set_source: null block array");
  for (int32_t i = 0; i < n_avail; ++i)
    if (!blocks[i].sign_bits || !blocks[i].u || !blocks[i].v) return fail(BSL_EINVAL, "bsl_set_source: block " + std::to_string(i) + " has a null array");
  s->w[w].src.assign(blocks, blocks + n_avail);
  return BSL_OK;
}

int bsl_set_input_scale(bsl_stack* s, int32_t w, const float* inv_scale) {
  if (!s) return fail(BSL_EINVAL, "bsl_set_input_scale: null stack");
  if (w < 0 || w >= (int32_t)s->w.size()) return fail(BSL_EINVAL, "bsl_set_input_scale: weight index out of range");
  Weight& W = s->w[w];
  if (W.n != 0) return fail(BSL_EINVAL, "bsl_set_input_scale: weight " + std::to_string(w) + " has loaded blocks");
  if (!inv_scale) {
    W.inv_scale.clear();
    return BSL_OK;
  }
  for (int32_t c = 0; c < W.d; ++c)
    if (!(std::isfinite(inv_scale[c]) && inv_scale[c] > 0.0f))
      return fail(BSL_EINVAL, "bsl_set_input_scale: inv_scale[" + std::to_string(c) + "] is not finite and positive");
  W.inv_scale.assign(inv_scale, inv_scale + W.d);
  return BSL_OK;
}

int bsl_load_blocks(bsl_stack* s, const int32_t* n_per_weight, void* stream) {
  if (!s || !n_per_weight) return fail(BSL_EINVAL, "bsl_load_blocks: null pointer");
  const int32_t nw = (int32_t)s->w.size();
  for (int32_t w = 0; w < nw; ++w) {
    const int32_t n = n_per_weight[w];
    if (n < 0 || n > s->n_cap) return fail(BSL_EINVAL, "bsl_load_blocks: count out of range for weight " + std::to_string(w));
    if (n > s->w[w].n && n > (int32_t)s->w[w].src.size())
      return fail(BSL_EINVAL, "bsl_load_blocks: weight " + std::to_string(w) + " has only " + std::to_string(s->w[w].src.size()) + " source blocks");
  }
  // budget check over the final state
  uint64_t after = s->resident;
  for (int32_t w = 0; w < nw; ++w) {
    const Weight& W = s->w[w];
    const uint64_t sb = slot_bytes(W.m, W.d);
    const int32_t n = n_per_weight[w];
    if (n > W.n) after += sb * (uint64_t)(n - W.n);
    else after -= sb * (uint64_t)(W.n - n);
  }
  if (s->budget && after > s->budget)
    return fail(BSL_ENOMEM, "bsl_load_blocks: " + std::to_string(after) + " bytes exceed the budget of " + std::to_string(s->budget));
  DeviceGuard guard(s->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // phase 1: allocate every new slot; undo all on failure
  struct NewSlot { int32_t w, i; };
  std::vector<NewSlot> added;
  hipError_t e = hipSuccess;
  for (int32_t w = 0; w < nw && e == hipSuccess; ++w) {
    Weight& W = s->w[w];
    for (int32_t i = W.n; i < n_per_weight[w]; ++i) {
      const size_t sb = slot_bytes(W.m, W.d);
      void* mem = nullptr;
      e = hipMalloc(&mem, sb);
      if (e != hipSuccess) break;
      W.slots[i].mem = mem;
      W.slots[i].bytes = sb;
      added.push_back({w, i});
    }
  }
  auto undo = [&]() {
    for (const NewSlot& a : added) {
      Slot& sl = s->w[a.w].slots[a.i];
      (void)hipFree(sl.mem);
      sl.mem = nullptr;
      sl.bytes = 0;
    }
  };
  if (e != hipSuccess) {
    undo();
    return hip_fail(e, "hipMalloc(block)");
  }
  // phase 2: pack on the host and copy the new blocks.  Two pinned staging buffers take
  // turns: block k is packed into one while the copy of block k - 1 runs from the other
  // (asynchronous DMA on `stream`, so forwards queued on other streams keep running).
  size_t need = 0;
  for (const NewSlot& a : added) need = std::max(need, slot_bytes(s->w[a.w].m, s->w[a.w].d));
  if (need > s->staging_bytes) {
    for (int k = 0; k < 2; ++k) {
      if (s->staging[k]) (void)hipHostFree(s->staging[k]);
      s->staging[k] = nullptr;
    }
    s->staging_bytes = 0;
    for (int k = 0; k < 2 && e == hipSuccess; ++k) e = hipHostMalloc(reinterpret_cast<void**>(&s->staging[k]), need, hipHostMallocDefault);
    for (int k = 0; k < 2 && e == hipSuccess; ++k)
      if (!s->staged[k]) e = hipEventCreateWithFlags(&s->staged[k], hipEventDisableTiming);
    if (e != hipSuccess) {
      undo();
      return hip_fail(e, "pinned staging buffers");
    }
    s->staging_bytes = need;
  }
  std::vector<uint16_t> vscaled;  // V of a scaled weight
  NewSlot overflow = {-1, -1};
  for (size_t k = 0; k < added.size() && e == hipSuccess; ++k) {
    const NewSlot& a = added[k];
    Weight& W = s->w[a.w];
    const bsl_block_src& src = W.src[a.i];
    const size_t sb = (size_t)pad_rows(W.m) * pad_cols(W.d) / 8;
    const size_t ub = (size_t)pad_rows(W.m) * kRank * 2;
    const size_t vb = (size_t)pad_cols(W.d) * kRank * 2;
    uint8_t* buf = s->staging[k % 2];
    if (k >= 2 && (e = hipEventSynchronize(s->staged[k % 2])) != hipSuccess) break;  // its last copy is done
    pack_signs_mt(src.sign_bits, W.m, W.d, buf);
    tile_u(src.u, W.m, reinterpret_cast<uint16_t*>(buf + sb));
    const uint16_t* v = src.v;
    if (!W.inv_scale.empty()) {
      vscaled.resize((size_t)W.d * kRank);
      if (!scale_v(v, W.d, W.inv_scale.data(), vscaled.data())) {
        overflow = a;
        break;
      }
      v = vscaled.data();
    }
    tile_v(v, W.d, reinterpret_cast<uint16_t*>(buf + sb + ub));
    rowmajor_v(v, W.d, reinterpret_cast<uint16_t*>(buf + sb + ub + vb));
    bop_v(v, W.d, reinterpret_cast<uint16_t*>(buf + sb + ub + 2 * vb));
    rowmajor_u(src.u, W.m, reinterpret_cast<uint16_t*>(buf + sb + ub + 3 * vb));
    e = hipMemcpyAsync(W.slots[a.i].mem, buf, sb + 2 * ub + 3 * vb, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipEventRecord(s->staged[k % 2], st);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(st);
    undo();
    return hip_fail(e, "block upload");
  }
  if (overflow.w >= 0) {  // the copies queued before it are done (synchronised above)
    undo();
    return fail(BSL_EINVAL, "bsl_load_blocks: block " + std::to_string(overflow.i) + " of weight " +
                                std::to_string(overflow.w) + ": V times the input scale overflows fp16");
  }
  // phase 3: publish the new slots in each grown weight's device table.  The table
  // lists every allocated slot; the kernels read only the first n entries, so a
  // shrink needs no table change and entries past n are never dereferenced.
  for (int32_t w = 0; w < nw; ++w) {
    if (n_per_weight[w] <= s->w[w].n) continue;
    int rc = upload_table(s->w[w], s->w[w].n, n_per_weight[w], st);
    if (rc != BSL_OK) {
      undo();
      return rc;
    }
  }
  // phase 4: commit.  Shrinking waits for the whole device: a forward that reads a slot
  // about to be released may be queued on any stream.
  bool shrink = false;
  for (int32_t w = 0; w < nw; ++w) shrink |= n_per_weight[w] < s->w[w].n;
  if (shrink && (e = hipDeviceSynchronize()) != hipSuccess) {
    undo();
    return hip_fail(e, "hipDeviceSynchronize");
  }
  for (int32_t w = 0; w < nw; ++w) {
    Weight& W = s->w[w];
    const int32_t n = n_per_weight[w];
    for (int32_t i = n; i < W.n; ++i) {
      (void)hipFree(W.slots[i].mem);
      s->resident -= W.slots[i].bytes;
      W.slots[i] = Slot{};
    }
    W.n = n;
  }
  for (const NewSlot& a : added) s->resident += s->w[a.w].slots[a.i].bytes;
  return BSL_OK;
}

int bsl_active_blocks(const bsl_stack* s, int32_t w, int32_t* n_out) {
  if (!s || !n_out) return fail(BSL_EINVAL, "bsl_active_blocks: null pointer");
  if (w < 0 || w >= (int32_t)s->w.size()) return fail(BSL_EINVAL, "bsl_active_blocks: weight index out of range");
  *n_out = s->w[w].n;
  return BSL_OK;
}

uint64_t bsl_resident_bytes(const bsl_stack* s) { return s ? s->resident : 0; }

namespace {

// Tile-reconstruct path.  Items are (weight, token group, 128-row group, column range);
// weights go longest item first, so the long items of a launch start first.  A weight's
// chunks are cut into ranges when the launch has too few items to keep every CU busy, as
// far as the stack's tile workspace holds the ranges' partial sums.
int forward_tile(bsl_stack* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y, int32_t M,
                 int32_t y_is_fp32, void* stream) {
  GroupArgs args;
  std::memset(&args, 0, sizeof(args));
  args.count = count;
  args.M = M;
  args.y_fp32 = y_is_fp32 ? 1 : 0;
  args.zero_page = s->zero_page;
  int tt = 1;  // 32-token tiles per wave (two waves per row tile): covers M, at most 8
  while (tt < kTileMaxTokenTiles && 64 * tt < M) tt *= 2;
  const int64_t token_groups = (M + 64 * tt - 1) / (64 * tt);
  const int64_t tokpad = token_groups * 64 * tt;
  struct Plan {
    int32_t j;
    int64_t rgroups, batches, splits, cps;
  };
  std::vector<Plan> plan(count);
  int64_t total = 0;  // chunk passes over all items
  for (int32_t j = 0; j < count; ++j) {
    const int32_t w = weights[j];
    if (w < 0 || w >= (int32_t)s->w.size()) return fail(BSL_EINVAL, "forward: weight index out of range");
    for (int32_t jj = 0; jj < j; ++jj)
      if (weights[jj] == w) return fail(BSL_EINVAL, "forward: a weight appears twice in one launch");
    if (!x[j] || !y[j]) return fail(BSL_EINVAL, "forward: null x or y");
    if ((reinterpret_cast<uintptr_t>(x[j]) & 15) != 0) return fail(BSL_EINVAL, "forward: x must be 16-byte aligned");
    const Weight& W = s->w[w];
    if ((uint64_t)pad_rows(W.m) * pad_cols(W.d) / 8 >= (1ull << 31))
      return fail(BSL_EUNSUPPORTED, "forward: the tile path needs each block's signs below 2 GiB");
    Plan& p = plan[j];
    p.j = j;
    p.rgroups = pad_rows(W.m) / kTileGroupRows;
    p.batches = (W.n + kTileBatch - 1) / kTileBatch;
    p.splits = 1;
    p.cps = W.nch;
    total += p.rgroups * token_groups * W.nch * p.batches;
  }
  // Items of about half a CU's share.  (Finer cutting measured slower: every range adds
  // a pipeline start and a partial-sum pass.)
  const int64_t slots = (int64_t)kTileItemsPerCu * s->decode_grid_max;
  const int64_t target = std::max<int64_t>(1, (total + slots - 1) / slots);
  size_t ws_used = 0, ctr_used = 0;
  for (Plan& p : plan) {
    const Weight& W = s->w[weights[p.j]];
    if (p.batches == 0) continue;
    const int64_t want = std::min<int64_t>(W.nch, (W.nch * p.batches + target - 1) / target);
    if (want <= 1) continue;
    const int64_t cps = (W.nch + want - 1) / want, splits = (W.nch + cps - 1) / cps;
    const size_t floats = (size_t)splits * tokpad * pad_rows(W.m);
    const size_t ctrs = (size_t)token_groups * p.rgroups;
    if (splits > 1 && ws_used + floats <= kTileWorkspaceFloats && ctr_used + ctrs <= (size_t)kTileCounters) {
      p.splits = splits;
      p.cps = cps;
      ws_used += floats;
      ctr_used += ctrs;
    }
  }
  std::stable_sort(plan.begin(), plan.end(), [](const Plan& a, const Plan& b) { return a.cps * a.batches > b.cps * b.batches; });
  int64_t items = 0;
  ws_used = ctr_used = 0;
  for (int32_t k = 0; k < count; ++k) {
    const Plan& p = plan[k];
    const Weight& W = s->w[weights[p.j]];
    WeightDesc& D = args.w[k];
    D.blocks = W.dtable;
    D.x = static_cast<const uint16_t*>(x[p.j]);
    D.y = y[p.j];
    D.m = W.m;
    D.d = W.d;
    D.mt = W.mt;
    D.nch = W.nch;
    D.nblocks = W.n;
    D.groups = (int32_t)p.rgroups;
    D.splits = (int32_t)p.splits;
    if (p.splits > 1) {
      D.partial = s->tile_ws + ws_used;
      D.counters = s->tile_ctr + ctr_used;
      ws_used += (size_t)p.splits * tokpad * pad_rows(W.m);
      ctr_used += (size_t)token_groups * p.rgroups;
    }
    D.item_begin = (int32_t)items;
    items += token_groups * p.rgroups * p.splits;
    if (items > (int64_t)INT32_MAX) return fail(BSL_EUNSUPPORTED, "forward: too many tokens for one launch");
  }
  args.total_items = (int32_t)items;
  DeviceGuard guard(s->device);
  const int e = launch_tile(args, tt, (int)token_groups, stream);
  if (e != 0) return hip_fail(static_cast<hipError_t>(e), "kernel launch");
  return BSL_OK;
}

// W_hat of a weight in the dense workspace: [m_pad][d_pad] fp16
size_t dense_bytes(const Weight& W) { return (size_t)W.mt * kTileRows * W.nch * kChunkCols * 2; }

// Dense path: restore W_hat of every weight of the launch into the workspace (one launch),
// then y = x W_hat^T per weight with a library GEMM (fp16 in, fp32 accumulate).
int forward_dense(bsl_stack* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y, int32_t M,
                  int32_t y_is_fp32, void* stream) {
  if (count < 1 || count > kMaxGroup) return fail(BSL_EINVAL, "forward: 1..8 weights per launch");
  GroupArgs args;
  std::memset(&args, 0, sizeof(args));
  args.count = count;
  args.M = M;
  args.y_fp32 = 0;
  size_t off = 0;
  uint64_t items = 0;
  for (int32_t j = 0; j < count; ++j) {
    const int32_t w = weights[j];
    if (w < 0 || w >= (int32_t)s->w.size()) return fail(BSL_EINVAL, "forward: weight index out of range");
    for (int32_t jj = 0; jj < j; ++jj)
      if (weights[jj] == w) return fail(BSL_EINVAL, "forward: a weight appears twice in one launch");
    if (!x[j] || !y[j]) return fail(BSL_EINVAL, "forward: null x or y");
    if ((reinterpret_cast<uintptr_t>(x[j]) & 15) != 0) return fail(BSL_EINVAL, "forward: x must be 16-byte aligned");
    const Weight& W = s->w[w];
    WeightDesc& D = args.w[j];
    D.blocks = W.dtable;
    D.y = reinterpret_cast<uint8_t*>(s->dense_ws) + off;
    D.m = W.m;
    D.d = W.d;
    D.mt = W.mt;
    D.nch = W.nch;
    D.nblocks = W.n;
    D.item_begin = (int32_t)items;
    items += (uint64_t)(W.mt * kTileRows / 128) * 2 * W.nch;
    off += dense_bytes(W);
  }
  if (off > s->dense_ws_bytes) return fail(BSL_EUNSUPPORTED, "forward: the dense path's workspace is too small for this launch");
  if (items > (uint64_t)INT32_MAX) return fail(BSL_EUNSUPPORTED, "forward: too many tiles for one launch");
  args.total_items = (int32_t)items;
  DeviceGuard guard(s->device);
  int e = launch_restore(args, stream);
  if (e != 0) return hip_fail(static_cast<hipError_t>(e), "restore launch");
  if (rocblas_set_stream(s->blas, static_cast<hipStream_t>(stream)) != rocblas_status_success)
    return fail(BSL_EHIP, "rocblas_set_stream failed");
  const float alpha = 1.f, beta = 0.f;
  const rocblas_datatype yt = y_is_fp32 ? rocblas_datatype_f32_r : rocblas_datatype_f16_r;
  for (int32_t j = 0; j < count; ++j) {
    const Weight& W = s->w[weights[j]];
    const int ld = W.nch * kChunkCols;
    // column-major view: y^T (m x M) = W_hat (m x d, stored as d_pad x m) ^T  x^T (d x M)
    const rocblas_status st = rocblas_gemm_ex(s->blas, rocblas_operation_transpose, rocblas_operation_none, W.m, M, W.d,
                                              &alpha, args.w[j].y, rocblas_datatype_f16_r, ld, x[j], rocblas_datatype_f16_r,
                                              W.d, &beta, y[j], yt, W.m, y[j], yt, W.m, rocblas_datatype_f32_r,
                                              rocblas_gemm_algo_standard, 0, 0);
    if (st != rocblas_status_success)
      return fail(BSL_EHIP, std::string("rocblas_gemm_ex: ") + rocblas_status_to_string(st));
  }
  return BSL_OK;
}

int forward_impl(bsl_stack* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y, int32_t M,
                 int32_t y_is_fp32, void* stream) {
  if (count < 1 || count > kMaxGroup) return fail(BSL_EINVAL, "forward: 1..8 weights per launch");
  if (M < 1 || M > (1 << 24)) return fail(BSL_EINVAL, "forward: M must be >= 1");
  GroupArgs args;
  std::memset(&args, 0, sizeof(args));
  args.count = count;
  args.M = M;
  args.y_fp32 = y_is_fp32 ? 1 : 0;
  if (s->path == BSL_PATH_DENSE && M > 1) return forward_dense(s, count, weights, x, y, M, y_is_fp32, stream);
  const bool tile = s->path == BSL_PATH_TILE || (s->path == BSL_PATH_AUTO && M >= kTileAutoMinTokens);
  if (tile) return forward_tile(s, count, weights, x, y, M, y_is_fp32, stream);
  for (int32_t j = 0; j < count; ++j) {
    const int32_t w = weights[j];
    if (w < 0 || w >= (int32_t)s->w.size()) return fail(BSL_EINVAL, "forward: weight index out of range");
    for (int32_t jj = 0; jj < j; ++jj)
      if (weights[jj] == w) return fail(BSL_EINVAL, "forward: a weight appears twice in one launch");
    if (!x[j] || !y[j]) return fail(BSL_EINVAL, "forward: null x or y");
    if ((reinterpret_cast<uintptr_t>(x[j]) & 15) != 0) return fail(BSL_EINVAL, "forward: x must be 16-byte aligned");
    const Weight& W = s->w[w];
    WeightDesc& D = args.w[j];
    D.blocks = W.dtable;
    D.x = static_cast<const uint16_t*>(x[j]);
    D.y = y[j];
    D.partial = W.partial;
    D.counters = W.counters;
    D.m = W.m;
    D.d = W.d;
    D.mt = W.mt;
    D.nch = W.nch;
    D.nblocks = W.n;
  }
  DeviceGuard guard(s->device);
  int e = 0;
  uint64_t units = 0, groups = 0;
  // Unit lists of the single- and few-token kernels: (weight, row group, block, chunk)
  // with row groups of `rows` rows.
  auto plan_units = [&](int rows) {
    units = groups = 0;
    for (int32_t j = 0; j < count; ++j) {
      const Weight& W = s->w[weights[j]];
      WeightDesc& D = args.w[j];
      D.groups = (int32_t)((W.mt * kTileRows + rows - 1) / rows);
      D.splits = W.nch;
      const uint64_t wu = (uint64_t)D.groups * W.nch * W.n;
      D.unit_begin = (uint32_t)units;
      D.units = (uint32_t)wu;
      D.rg_begin = (uint32_t)groups;
      units += wu;
      groups += D.groups;
    }
  };
  // Units [o U / 2^lg, (o + 1) U / 2^lg) of worker o, as the kernels compute them.
  auto start = [&](uint64_t o, int lg) { return (o * units) >> lg; };
  // Plan of the wave-private kernel for T tokens (row groups of 256, 128, 64 and 64 rows
  // for T = 1 to 4); false when a workgroup's activations do not fit its LDS.
  auto plan_private = [&](int T, int& lg) {
    plan_units(T == 3 ? kWpRows / 4 : kWpRows / T);
    // workers: four per workgroup, at most one workgroup per CU, at most one per unit
    int32_t workers = kWpWaves * s->decode_grid_max;
    while (workers > kWpWaves && (uint64_t)workers > units) workers /= 2;
    lg = 0;
    while ((1 << lg) < workers) ++lg;
    // (no units at all: one workgroup writes y = 0)
    bool fits = (units == 0 || units >= (uint64_t)workers) && (units << lg) < (1ull << 32);
    // every workgroup keeps the activations of the weights its units belong to in LDS
    for (int32_t L = 0; fits && units > 0 && L < workers / kWpWaves; ++L) {
      const uint64_t a = start((uint64_t)L * kWpWaves, lg), b = start((uint64_t)(L + 1) * kWpWaves, lg) - 1;
      int32_t ja = 0, jb = 0;
      while (ja + 1 < count && a >= args.w[ja + 1].unit_begin) ++ja;
      while (jb + 1 < count && b >= args.w[jb + 1].unit_begin) ++jb;
      uint64_t bytes = 0;
      for (int32_t j = ja; j <= jb; ++j) bytes += (uint64_t)T * args.w[j].nch * kChunkCols * 2;
      fits = bytes <= (uint64_t)kWpXBytes;
    }
    return fits;
  };
  auto launch_units = [&](int lg) {
    args.total_units = (uint32_t)units;
    args.total_groups = (uint32_t)groups;
    args.grid_log2 = lg;
    args.zero_page = s->zero_page;
    args.pieces = s->pieces;
    args.arrivals = s->arrivals;
  };
  if (M == 1) {
    // AUTO takes the shared-operand kernel: on the 8B-shaped layer it measured faster
    // (77 against 80 us per launch)
    const bool wp = s->decode == BSL_DECODE_PRIVATE;
    int lg = 0;
    if (wp) {
      if (!plan_private(1, lg)) return fail(BSL_EUNSUPPORTED, "forward: the wave-private single-token kernel does not fit this launch");
    } else {
      plan_units(kDecodeGroupRows);
      // Persistent grid: the largest power of two that is no more than one workgroup per
      // CU and no more than the number of units (so no workgroup's share is empty).
      int32_t grid = s->decode_grid_max;
      while (grid > 1 && (uint64_t)grid > units) grid /= 2;
      while ((1 << lg) < grid) ++lg;
      if ((units << lg) >= (1ull << 32)) return fail(BSL_EUNSUPPORTED, "forward: too much work for one launch");
    }
    launch_units(lg);
    e = wp ? launch_decode_wp(args, 1, stream) : launch_decode_m1(args, stream);
    if (e != 0) return hip_fail(static_cast<hipError_t>(e), "kernel launch");
    return BSL_OK;
  }
  if (M <= kWpMaxTokens && s->path == BSL_PATH_AUTO) {
    // a few tokens: the wave-private kernel with every operand but the activations shared
    // by the tokens, when they fit its LDS
    const int T = M;
    int lg = 0;
    if (plan_private(T, lg)) {
      launch_units(lg);
      e = launch_decode_wp(args, T, stream);
      if (e != 0) return hip_fail(static_cast<hipError_t>(e), "kernel launch");
      return BSL_OK;
    }
    // The group does not fit as a whole: the weights whose activations take at most half
    // of the LDS (so that any two neighbours fit together) go to one launch, which may
    // still fall back, and the rest to the multi-token kernel.
    int32_t narrow[kMaxGroup], wide[kMaxGroup];
    const void* xn[kMaxGroup];
    const void* xw[kMaxGroup];
    void* yn[kMaxGroup];
    void* yw[kMaxGroup];
    int32_t nn = 0, nw = 0;
    for (int32_t j = 0; j < count; ++j) {
      const uint64_t bytes = (uint64_t)T * s->w[weights[j]].nch * kChunkCols * 2;
      if (2 * bytes <= (uint64_t)kWpXBytes) {
        narrow[nn] = weights[j];
        xn[nn] = x[j];
        yn[nn++] = y[j];
      } else {
        wide[nw] = weights[j];
        xw[nw] = x[j];
        yw[nw++] = y[j];
      }
    }
    if (nn > 0 && nw > 0) {
      const int rc = forward_impl(s, nn, narrow, xn, yn, M, y_is_fp32, stream);
      if (rc != BSL_OK) return rc;
      return forward_impl(s, nw, wide, xw, yw, M, y_is_fp32, stream);
    }
  }
  const int nt = M <= 2 ? 2 : (M <= 4 ? 4 : 8);  // tokens per multi-token item
  const int token_groups = (M + nt - 1) / nt;
  // Multi-token items are cut along their (block, chunk) sequence when there are too few
  // of them: aim at about two equal items per CU, within the split-K workspace.
  uint64_t work = 0;
  for (int32_t j = 0; j < count; ++j) {
    const Weight& W = s->w[weights[j]];
    work += (uint64_t)prefill_groups(W) * token_groups * W.n * W.nch;
  }
  const uint64_t slots = 2 * (uint64_t)s->decode_grid_max;
  const uint64_t split_target = std::max<uint64_t>(1, (work + slots - 1) / slots);
  const int max_splits = std::max(1, std::min(kMaxSplits, kSplitTokens / (token_groups * nt)));
  uint64_t items = 0;
  for (int32_t j = 0; j < count; ++j) {
    const Weight& W = s->w[weights[j]];
    WeightDesc& D = args.w[j];
    D.item_begin = (int32_t)items;
    const uint64_t wunits = (uint64_t)W.n * W.nch;
    const uint64_t wgroups = (uint64_t)prefill_groups(W) * token_groups;
    const uint64_t splits = std::min<uint64_t>(max_splits, std::max<uint64_t>(1, (wunits + split_target - 1) / split_target));
    if (items + wgroups * splits > (uint64_t)INT32_MAX) return fail(BSL_EUNSUPPORTED, "forward: too many tokens for one launch");
    D.groups = (int32_t)wgroups;
    D.splits = (int32_t)splits;
    items += wgroups * splits;
  }
  args.total_items = (int32_t)items;
  args.zero_page = s->zero_page;
  e = launch_prefill(args, nt, token_groups, stream);
  if (e != 0) return hip_fail(static_cast<hipError_t>(e), "kernel launch");
  return BSL_OK;
}

}  // namespace

int bsl_forward(bsl_stack* s, int32_t w, const void* x, void* y, int32_t M, int32_t y_is_fp32, void* stream) {
  if (!s) return fail(BSL_EINVAL, "bsl_forward: null stack");
  const void* xs[1] = {x};
  void* ys[1] = {y};
  return forward_impl(s, 1, &w, xs, ys, M, y_is_fp32, stream);
}

int bsl_forward_group(bsl_stack* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y,
                      int32_t M, int32_t y_is_fp32, void* stream) {
  if (!s || !weights || !x || !y) return fail(BSL_EINVAL, "bsl_forward_group: null pointer");
  return forward_impl(s, count, weights, x, y, M, y_is_fp32, stream);
}

int bsl_set_path(bsl_stack* s, int32_t path) {
  if (!s) return fail(BSL_EINVAL, "bsl_set_path: null stack");
  if (path != BSL_PATH_AUTO && path != BSL_PATH_FACTORED && path != BSL_PATH_TILE && path != BSL_PATH_DENSE)
    return fail(BSL_EINVAL, "bsl_set_path: unknown path");
  if (path == BSL_PATH_DENSE && !s->blas) {
    // workspace for the kMaxGroup largest weights' W_hat, a rocBLAS handle and its workspace
    std::vector<size_t> sizes;
    for (const Weight& W : s->w) sizes.push_back(dense_bytes(W));
    std::sort(sizes.rbegin(), sizes.rend());
    size_t need = 0;
    for (size_t k = 0; k < sizes.size() && k < (size_t)kMaxGroup; ++k) need += sizes[k];
    DeviceGuard guard(s->device);
    hipError_t e = hipMalloc(&s->dense_ws, need);
    if (e != hipSuccess) {
      s->dense_ws = nullptr;
      return fail(BSL_ENOMEM, "bsl_set_path: " + std::to_string(need) + " bytes for the dense path's workspace");
    }
    e = hipMalloc(&s->blas_ws, kDenseBlasWorkspace);
    rocblas_handle h = nullptr;
    if (e == hipSuccess && rocblas_create_handle(&h) == rocblas_status_success &&
        rocblas_set_workspace(h, s->blas_ws, kDenseBlasWorkspace) == rocblas_status_success) {
      s->blas = h;
      s->dense_ws_bytes = need;
    } else {
      if (h) (void)rocblas_destroy_handle(h);
      if (s->blas_ws) (void)hipFree(s->blas_ws);
      (void)hipFree(s->dense_ws);
      s->blas_ws = nullptr;
      s->dense_ws = nullptr;
      return fail(BSL_ENOMEM, "bsl_set_path: rocBLAS set-up failed");
    }
  }
  s->path = path;
  return BSL_OK;
}

int bsl_set_decode(bsl_stack* s, int32_t kind) {
  if (!s) return fail(BSL_EINVAL, "bsl_set_decode: null stack");
  if (kind != BSL_DECODE_AUTO && kind != BSL_DECODE_SHARED && kind != BSL_DECODE_PRIVATE)
    return fail(BSL_EINVAL, "bsl_set_decode: unknown kernel");
  s->decode = kind;
  return BSL_OK;
}

int bsl_debug_unpack(bsl_stack* s, int32_t w, int32_t i, int32_t path, int8_t* pm1_out, void* stream) {
  if (!s || !pm1_out) return fail(BSL_EINVAL, "bsl_debug_unpack: null pointer");
  if (w < 0 || w >= (int32_t)s->w.size()) return fail(BSL_EINVAL, "bsl_debug_unpack: weight index out of range");
  const Weight& W = s->w[w];
  if (i < 0 || i >= W.n) return fail(BSL_EINVAL, "bsl_debug_unpack: block not loaded");
  if (path < 0 || path > 2) return fail(BSL_EINVAL, "bsl_debug_unpack: path must be 0, 1 or 2");
  DeviceGuard guard(s->device);
  int e = launch_debug_unpack(slot_ptrs(W.slots[i], W.m, W.d), W.m, W.d, W.mt, W.nch, path, pm1_out, stream);
  if (e != 0) return hip_fail(static_cast<hipError_t>(e), "debug unpack launch");
  return BSL_OK;
}

void bsl_destroy(bsl_stack* s) {
  if (!s) return;
  DeviceGuard guard(s->device);
  (void)hipDeviceSynchronize();
  for (Weight& W : s->w) {
    for (Slot& sl : W.slots)
      if (sl.mem) (void)hipFree(sl.mem);
    if (W.dtable) (void)hipFree(W.dtable);
    if (W.partial) (void)hipFree(W.partial);
    if (W.counters) (void)hipFree(W.counters);
  }
  if (s->zero_page) (void)hipFree(s->zero_page);
  if (s->pieces) (void)hipFree(s->pieces);
  if (s->arrivals) (void)hipFree(s->arrivals);
  if (s->tile_ws) (void)hipFree(s->tile_ws);
  if (s->tile_ctr) (void)hipFree(s->tile_ctr);
  if (s->blas) (void)rocblas_destroy_handle(s->blas);
  if (s->blas_ws) (void)hipFree(s->blas_ws);
  if (s->dense_ws) (void)hipFree(s->dense_ws);
  for (int k = 0; k < 2; ++k) {
    if (s->staging[k]) (void)hipHostFree(s->staging[k]);
    if (s->staged[k]) (void)hipEventDestroy(s->staged[k]);
  }
  delete s;
}

}  // extern "C"
