// Host side of libbitstack_linear: argument checking, the sign packer ("bitstack_pack"),
// the device-resident block stack and forward dispatch.  See include/bitstack_linear.h
// for the interface contract.
#include "bitstack_linear.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <condition_variable>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
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

// U (m x 16, row-major fp16) -> [m_pad/16][64][4]: lane L, slot v holds U[16 t + 4 (L/16) + v][L % 16]
// (row tiles [t0, t1) of it).
void tile_u(const uint16_t* u, int64_t m, uint16_t* out, int64_t t0, int64_t t1) {
  for (int64_t t = t0; t < t1; ++t)
    for (int L = 0; L < 64; ++L)
      for (int v = 0; v < 4; ++v) {
        const int64_t row = 16 * t + 4 * (L / 16) + v;
        out[(t * 64 + L) * 4 + v] = row < m ? u[row * kRank + (L % 16)] : 0;
      }
}

// V (d x 16, row-major fp16) -> [d_pad/512][16][64][8]: lane L of plane b, slot j holds
// V[512 c + 32 b + 8 (L/16) + j][L % 16] (chunks [c0, c1) of it).
void tile_v(const uint16_t* v, int64_t d, uint16_t* out, int64_t c0, int64_t c1) {
  for (int64_t c = c0; c < c1; ++c)
    for (int b = 0; b < kPlanes; ++b)
      for (int L = 0; L < 64; ++L)
        for (int j = 0; j < 8; ++j) {
          const int64_t col = 512 * c + 32 * b + 8 * (L / 16) + j;
          out[((c * kPlanes + b) * 64 + L) * 8 + j] = col < d ? v[col * kRank + (L % 16)] : 0;
        }
}

// V rows [c0, c1) (of d x 16) multiplied by inv_scale[c]: one rounding of the exact product.
bool scale_v(const uint16_t* v, int64_t c0, int64_t c1, const float* inv_scale, uint16_t* out) {
  for (int64_t c = c0; c < c1; ++c)
    for (int r = 0; r < kRank; ++r)
      if (!double_to_fp16(fp16_to_double(v[c * kRank + r]) * (double)inv_scale[c], &out[c * kRank + r])) return false;
  return true;
}

// Host threads for bsl_load_blocks' staging work (copies into pinned memory and the factor
// layouts): started on first use, joined when the stack is destroyed.  run(n, fn) calls
// fn(0) .. fn(n - 1) on the workers and the calling thread and returns when all are done.
class WorkerPool {
 public:
  ~WorkerPool() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      quit_ = true;
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  void run(int n, const std::function<void(int)>& fn) {
    if (th_.empty())
      for (int k = 0; k < kWorkers; ++k) th_.emplace_back([this] { loop(); });
    {
      std::lock_guard<std::mutex> lk(mu_);
      fn_ = &fn;
      next_ = 0;
      total_ = pending_ = n;
      ++gen_;
    }
    cv_.notify_all();
    work();
    std::unique_lock<std::mutex> lk(mu_);
    done_.wait(lk, [&] { return pending_ == 0; });
    fn_ = nullptr;
  }

 private:
  static constexpr int kWorkers = 8;
  void work() {  // take tasks until none is left
    for (;;) {
      int i;
      const std::function<void(int)>* f;
      {
        std::lock_guard<std::mutex> lk(mu_);
        if (!fn_ || next_ >= total_) return;
        i = next_++;
        f = fn_;
      }
      (*f)(i);
      std::lock_guard<std::mutex> lk(mu_);
      if (--pending_ == 0) done_.notify_all();
    }
  }
  void loop() {
    uint64_t seen = 0;
    std::unique_lock<std::mutex> lk(mu_);
    for (;;) {
      cv_.wait(lk, [&] { return quit_ || gen_ != seen; });
      if (quit_) return;
      seen = gen_;
      lk.unlock();
      work();
      lk.lock();
    }
  }
  std::vector<std::thread> th_;
  std::mutex mu_;
  std::condition_variable cv_, done_;
  const std::function<void(int)>* fn_ = nullptr;
  int next_ = 0, total_ = 0, pending_ = 0;
  uint64_t gen_ = 0;
  bool quit_ = false;
};

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
  size_t partial_floats = 0, counter_count = 0;  // its share of the multi-token path's workspace
};

struct bsl_stack {
  int device = 0;
  int32_t k = 16, n_cap = 0;
  int32_t decode_grid_max = 256;  // largest power of two <= compute units
  int32_t path = BSL_PATH_AUTO;   // multi-token formulation (bsl_set_path)
  int32_t decode = BSL_DECODE_AUTO;  // single-token kernel (bsl_set_decode)
  uint64_t budget = 0, resident = 0;
  void* zero_page = nullptr;      // kZeroPageBytes of zeros on the device
  uint64_t* acc64 = nullptr;      // single- and few-token row accumulators, one per (row, token) of a launch (zero)
  size_t acc64_words = 0;
  float* tile_ws = nullptr;       // tile path: partial sums of column ranges (kTileWorkspaceFloats)
  float* mt_partial = nullptr;    // multi-token path: split partial sums of a launch's weights
  uint32_t* mt_counters = nullptr;  // ... and their arrival counters (zero between launches)
  size_t mt_partial_floats = 0, mt_counter_words = 0;  // the kMaxGroup largest weights' shares
  uint8_t* staging[2] = {nullptr, nullptr};  // pinned host buffers of bsl_load_blocks (allocated on first use)
  size_t staging_bytes = 0;
  hipEvent_t staged[2] = {nullptr, nullptr};  // copy out of staging[k] and the repack from raw_dev[k] finished
  uint8_t* raw_dev[2] = {nullptr, nullptr};   // device buffers of row-major sign bits awaiting the repack
  size_t raw_dev_bytes = 0;
  uint32_t* tile_ctr = nullptr;   // tile path: arrival counters (kTileCounters), zero between launches
  uint16_t* vr_ws = nullptr;      // tile path: V of a launch's blocks in rank-major order (formed per call)
  uint32_t* xt_ws = nullptr;      // product-index path: a launch's x in B-lane order (formed per call)
  size_t xt_cap = 0;              // its bytes: kMaxGroup weights of the stack's most chunks
  float* px_part = nullptr;       // product-index path: workgroup shares of row groups
  size_t px_part_slots = 0;       // kMaxGroup weights of the most 512-row groups + one per workgroup
  size_t vr_cap = 0;              // its bytes: enough for the kMaxGroup weights with the most V bytes
  std::vector<void*> vr_retired;  // outgrown vr_ws buffers, freed once the device has drained
  size_t vr_retired_bytes = 0;
  void* static_scratch = nullptr; // this device's static scratch array (bsl_forward_group_static)
  uint64_t launches[BSL_KERNEL_KINDS] = {0, 0, 0, 0, 0};  // forward launches per kernel (bsl_launch_counts)
  WorkerPool loaders;             // host threads of bsl_load_blocks' staging
  std::vector<Weight> w;
};

namespace {

// Bytes of rank-major V that a tile-path launch of any group of weights may need with
// `counts` loaded blocks: the kMaxGroup largest n pad_cols(d) 32 bytes.
size_t vr_bytes_needed(const bsl_stack* s, const int32_t* counts) {
  std::vector<size_t> b(s->w.size());
  for (size_t w = 0; w < s->w.size(); ++w) b[w] = (size_t)counts[w] * pad_cols(s->w[w].d) * kRank * 2;
  const size_t k = std::min<size_t>(kMaxGroup, b.size());
  std::partial_sort(b.begin(), b.begin() + k, b.end(), std::greater<size_t>());
  size_t t = 0;
  for (size_t i = 0; i < k; ++i) t += b[i];
  return t;
}

void free_retired(bsl_stack* s) {
  for (void* p : s->vr_retired) (void)hipFree(p);
  s->vr_retired.clear();
  s->vr_retired_bytes = 0;
}

// signs + tiled U + tiled V (see BlockPtrs)
size_t slot_bytes(int64_t m, int64_t d) {
  return (size_t)pad_rows(m) * pad_cols(d) / 8 + (size_t)pad_rows(m) * kRank * 2 + (size_t)pad_cols(d) * kRank * 2;
}

BlockPtrs slot_ptrs(const Slot& s, int64_t m, int64_t d) {
  BlockPtrs p;
  const uint8_t* base = static_cast<const uint8_t*>(s.mem);
  const size_t sb = (size_t)pad_rows(m) * pad_cols(d) / 8;
  const size_t ub = (size_t)pad_rows(m) * kRank * 2;
  p.signs = base;
  p.u = reinterpret_cast<const uint16_t*>(base + sb);
  p.v = reinterpret_cast<const uint16_t*>(base + sb + ub);
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
    tab[i - lo] = W.slots[i].mem ? slot_ptrs(W.slots[i], W.m, W.d) : BlockPtrs{nullptr, nullptr, nullptr};
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
    max_groups = std::max<size_t>(max_groups, (size_t)decode_groups(W));
    if ((e = hipMalloc(&W.dtable, sizeof(BlockPtrs) * n_cap)) != hipSuccess) rc = hip_fail(e, "hipMalloc(table)");
    else if ((e = hipMemset(W.dtable, 0, sizeof(BlockPtrs) * n_cap)) != hipSuccess) rc = hip_fail(e, "hipMemset(table)");
  }
  // The multi-token path's split partial sums and counters: launches on one stack do not
  // overlap, so one workspace serves every launch, with room for the kMaxGroup weights
  // that need the most.
  if (rc == BSL_OK) {
    std::vector<size_t> pf, cw;
    for (const Weight& W : s->w) {
      pf.push_back(W.partial_floats);
      cw.push_back(W.counter_count);
    }
    const size_t k = std::min<size_t>(kMaxGroup, pf.size());
    std::partial_sort(pf.begin(), pf.begin() + k, pf.end(), std::greater<size_t>());
    std::partial_sort(cw.begin(), cw.begin() + k, cw.end(), std::greater<size_t>());
    for (size_t i = 0; i < k; ++i) {
      s->mt_partial_floats += pf[i];
      s->mt_counter_words += cw[i];
    }
    if ((e = hipMalloc(&s->mt_partial, s->mt_partial_floats * sizeof(float))) != hipSuccess) rc = hip_fail(e, "hipMalloc(workspace)");
    else if ((e = hipMalloc(&s->mt_counters, s->mt_counter_words * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMalloc(counters)");
    else if ((e = hipMemset(s->mt_counters, 0, s->mt_counter_words * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMemset(counters)");
  }
  if (rc == BSL_OK) {
    // row accumulators of the single- and few-token kernels: one per row and token of a
    // launch (at most kMaxGroup weights of at most max_groups 1024-row groups, at most
    // kWpMaxTokens tokens)
    s->acc64_words = (size_t)kMaxGroup * max_groups * kDecodeGroupRows * kWpMaxTokens;
    if ((e = hipMalloc(&s->acc64, s->acc64_words * sizeof(uint64_t))) != hipSuccess) rc = hip_fail(e, "hipMalloc(row accumulators)");
    else if ((e = hipMemset(s->acc64, 0, s->acc64_words * sizeof(uint64_t))) != hipSuccess) rc = hip_fail(e, "hipMemset(row accumulators)");
    else if ((e = hipMalloc(&s->tile_ws, kTileWorkspaceFloats * sizeof(float))) != hipSuccess) rc = hip_fail(e, "hipMalloc(tile workspace)");
    else if ((e = hipMalloc(&s->tile_ctr, kTileCounters * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMalloc(tile counters)");
    else if ((e = hipMemset(s->tile_ctr, 0, kTileCounters * sizeof(uint32_t))) != hipSuccess) rc = hip_fail(e, "hipMemset(tile counters)");
  }
  if (rc == BSL_OK) {
    // the product-index path's activations in B-lane order: kMaxGroup weights of the most
    // 512-column chunks
    int32_t max_nch = 0;
    for (const Weight& W : s->w) max_nch = std::max(max_nch, W.nch);
    s->xt_cap = (size_t)kMaxGroup * max_nch * kPxLaneBytesPerChunk;
    if ((e = hipMalloc(&s->xt_ws, s->xt_cap)) != hipSuccess) rc = hip_fail(e, "hipMalloc(x lanes)");
    // shares of row groups: a workgroup's contiguous range of units meets each row group
    // once, so (row group + workgroup) numbers the (row group, workgroup) pairs without
    // collisions and needs at most row groups + workgroups slots
    int64_t max_rg = 0;
    for (const Weight& W : s->w) max_rg = std::max<int64_t>(max_rg, (W.m + kPxWaves * kPxTiles * kPxTileRows - 1) / (kPxWaves * kPxTiles * kPxTileRows));
    s->px_part_slots = (size_t)kMaxGroup * max_rg + s->decode_grid_max;
    if (rc == BSL_OK && (e = hipMalloc(&s->px_part, s->px_part_slots * kPxPartFloats * sizeof(float))) != hipSuccess)
      rc = hip_fail(e, "hipMalloc(product shares)");
  }
  if (rc == BSL_OK) {
    const int se = static_scratch_setup(device, &s->static_scratch);
    if (se != 0) rc = hip_fail(static_cast<hipError_t>(se), "hipGetSymbolAddress(static scratch)");
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
  // The tile path's rank-major V workspace grows here, so that no forward allocates.  An
  // outgrown buffer may still be read by forwards queued on other streams: it is retired
  // and freed where the device has drained (a shrink, bsl_destroy).
  uint16_t* vr_new = nullptr;
  size_t vr_new_cap = 0;
  auto undo = [&]() {
    for (const NewSlot& a : added) {
      Slot& sl = s->w[a.w].slots[a.i];
      (void)hipFree(sl.mem);
      sl.mem = nullptr;
      sl.bytes = 0;
    }
    if (vr_new) (void)hipFree(vr_new);
    vr_new = nullptr;
  };
  if (e != hipSuccess) {
    undo();
    return hip_fail(e, "hipMalloc(block)");
  }
  if (const size_t vneed = vr_bytes_needed(s, n_per_weight); vneed > s->vr_cap) {
    vr_new_cap = std::max(vneed, s->vr_cap + s->vr_cap / 2);
    if ((e = hipMalloc(reinterpret_cast<void**>(&vr_new), vr_new_cap)) != hipSuccess) {
      vr_new = nullptr;
      undo();
      return hip_fail(e, "hipMalloc(rank-major V workspace)");
    }
  }
  // phase 2: copy the new blocks.  A block's row-major sign bits go to the device as they
  // are and a kernel repacks them into the slot's tiled layout; the factor layouts (9% of
  // an 8B-shaped block) are written on the host.  Two pinned staging buffers and two device
  // buffers of raw bits take turns: block k is staged into one pair while the copies and
  // the repack of block k - 1 run from the other (asynchronously on `stream`, so forwards
  // queued on other streams keep running).
  size_t need = 0, need_raw = 0;
  for (const NewSlot& a : added) {
    const Weight& W = s->w[a.w];
    const size_t raw = (size_t)W.m * (W.d / 8), sb = (size_t)pad_rows(W.m) * pad_cols(W.d) / 8;
    need = std::max(need, raw + slot_bytes(W.m, W.d) - sb);
    need_raw = std::max(need_raw, raw);
  }
  if (need > s->staging_bytes || need_raw > s->raw_dev_bytes) {
    for (int k = 0; k < 2; ++k) {
      if (s->staging[k]) (void)hipHostFree(s->staging[k]);
      if (s->raw_dev[k]) (void)hipFree(s->raw_dev[k]);
      s->staging[k] = nullptr;
      s->raw_dev[k] = nullptr;
    }
    s->staging_bytes = s->raw_dev_bytes = 0;
    for (int k = 0; k < 2 && e == hipSuccess; ++k) e = hipHostMalloc(reinterpret_cast<void**>(&s->staging[k]), need, hipHostMallocDefault);
    for (int k = 0; k < 2 && e == hipSuccess; ++k) e = hipMalloc(reinterpret_cast<void**>(&s->raw_dev[k]), need_raw);
    for (int k = 0; k < 2 && e == hipSuccess; ++k)
      if (!s->staged[k]) e = hipEventCreateWithFlags(&s->staged[k], hipEventDisableTiming);
    if (e != hipSuccess) {
      undo();
      return hip_fail(e, "staging buffers");
    }
    s->staging_bytes = need;
    s->raw_dev_bytes = need_raw;
  }
  std::vector<uint16_t> vscaled;  // V of a scaled weight
  NewSlot overflow = {-1, -1};
  for (size_t k = 0; k < added.size() && e == hipSuccess; ++k) {
    const NewSlot& a = added[k];
    Weight& W = s->w[a.w];
    const bsl_block_src& src = W.src[a.i];
    const size_t raw = (size_t)W.m * (W.d / 8);
    const size_t sb = (size_t)pad_rows(W.m) * pad_cols(W.d) / 8;
    const size_t ub = (size_t)pad_rows(W.m) * kRank * 2;
    const size_t vb = (size_t)pad_cols(W.d) * kRank * 2;
    uint8_t* buf = s->staging[k % 2];
    uint8_t* fac = buf + raw;  // the factor layouts, in slot order after the signs
    if (k >= 2 && (e = hipEventSynchronize(s->staged[k % 2])) != hipSuccess) break;  // its last copy and repack are done
    // The raw sign bits are copied in slices of about 1 MiB, and the factor layouts written
    // in row-tile and chunk ranges (a scaled V is scaled range by range first), all as
    // tasks of the worker threads.
    const int64_t mt = pad_rows(W.m) / kTileRows, nch = pad_cols(W.d) / kChunkCols;
    const int ncopy = (int)std::min<size_t>(8, std::max<size_t>(1, raw >> 20));
    const int nu = (int)std::min<int64_t>(4, std::max<int64_t>(1, mt / 64));
    const int nv = (int)std::min<int64_t>(4, std::max<int64_t>(1, nch / 4));
    const bool scaled = !W.inv_scale.empty();
    if (scaled) vscaled.resize((size_t)W.d * kRank);
    std::vector<char> vok(nv, 1);
    const std::function<void(int)> task = [&](int t) {
      if (t < ncopy) {
        const size_t per = (raw + ncopy - 1) / ncopy, a = (size_t)t * per, b = std::min(raw, a + per);
        if (a < b) std::memcpy(buf + a, src.sign_bits + a, b - a);
      } else if (t < ncopy + nu) {
        const int64_t k = t - ncopy, per = (mt + nu - 1) / nu;
        tile_u(src.u, W.m, reinterpret_cast<uint16_t*>(fac), k * per, std::min(mt, (k + 1) * per));
      } else {
        const int64_t k = t - ncopy - nu, per = (nch + nv - 1) / nv;
        const int64_t c0 = k * per, c1 = std::min(nch, (k + 1) * per);
        const uint16_t* v = src.v;
        if (scaled) {
          if (!scale_v(v, std::min<int64_t>(W.d, c0 * kChunkCols), std::min<int64_t>(W.d, c1 * kChunkCols), W.inv_scale.data(),
                       vscaled.data())) {
            vok[k] = 0;
            return;
          }
          v = vscaled.data();
        }
        tile_v(v, W.d, reinterpret_cast<uint16_t*>(fac + ub), c0, c1);
      }
    };
    s->loaders.run(ncopy + nu + nv, task);
    bool scaled_ok = true;
    for (char ok : vok) scaled_ok = scaled_ok && ok;
    if (!scaled_ok) {
      overflow = a;
      break;
    }
    uint8_t* slot = static_cast<uint8_t*>(W.slots[a.i].mem);
    e = hipMemcpyAsync(s->raw_dev[k % 2], buf, raw, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(slot + sb, fac, ub + vb, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = static_cast<hipError_t>(launch_repack_signs(s->raw_dev[k % 2], W.m, W.d, W.mt, W.nch, slot, st));
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
  if (shrink) free_retired(s);
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
  if (vr_new) {
    if (s->vr_ws) {
      s->vr_retired.push_back(s->vr_ws);
      s->vr_retired_bytes += s->vr_cap;
    }
    s->vr_ws = vr_new;
    s->vr_cap = vr_new_cap;
  }
  return BSL_OK;
}

int bsl_active_blocks(const bsl_stack* s, int32_t w, int32_t* n_out) {
  if (!s || !n_out) return fail(BSL_EINVAL, "bsl_active_blocks: null pointer");
  if (w < 0 || w >= (int32_t)s->w.size()) return fail(BSL_EINVAL, "bsl_active_blocks: weight index out of range");
  *n_out = s->w[w].n;
  return BSL_OK;
}

uint64_t bsl_resident_bytes(const bsl_stack* s) { return s ? s->resident : 0; }

uint64_t bsl_workspace_bytes(const bsl_stack* s) {
  if (!s) return 0;
  uint64_t t = kZeroPageBytes + s->acc64_words * sizeof(uint64_t) + kTileWorkspaceFloats * sizeof(float) +
               kTileCounters * sizeof(uint32_t) + 2 * (uint64_t)s->raw_dev_bytes + s->vr_cap + s->vr_retired_bytes + s->xt_cap +
               s->px_part_slots * kPxPartFloats * sizeof(float);
  t += s->mt_partial_floats * sizeof(float) + s->mt_counter_words * sizeof(uint32_t);
  t += sizeof(BlockPtrs) * (uint64_t)s->n_cap * s->w.size();
  return t;
}

int bsl_launch_counts(const bsl_stack* s, uint64_t* counts) {
  if (!s || !counts) return fail(BSL_EINVAL, "bsl_launch_counts: null pointer");
  for (int k = 0; k < BSL_KERNEL_KINDS; ++k) counts[k] = s->launches[k];
  return BSL_OK;
}

namespace {

// V of a launch's loaded blocks in rank-major order ([block][d_pad][16] fp16, read by the
// tile and product-index kernels), in the stack's workspace: plan_rank_major_v points
// each weight's vr into it, launch_rank_major_v runs the pass that fills it.
int plan_rank_major_v(bsl_stack* s, GroupArgs& args) {
  size_t vr_used = 0;
  int64_t pairs = 0;
  for (int32_t k = 0; k < args.count; ++k) {
    WeightDesc& D = args.w[k];
    D.vr = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(s->vr_ws) + vr_used);
    vr_used += (size_t)D.nblocks * D.nch * kChunkCols * kRank * 2;
    pairs += (int64_t)D.nblocks * D.nch * 8;
  }
  if (vr_used > s->vr_cap || pairs > (int64_t)INT32_MAX)
    return fail(BSL_EUNSUPPORTED, "forward: the rank-major V of this launch does not fit the stack's workspace");
  return BSL_OK;
}
int launch_rank_major_v(const GroupArgs& args, void* stream) {
  GroupArgs vargs = args;  // items: (weight, block, 64-column step) pairs
  int64_t pairs = 0;
  for (int32_t k = 0; k < args.count; ++k) {
    vargs.w[k].item_begin = (int32_t)pairs;
    pairs += (int64_t)args.w[k].nblocks * args.w[k].nch * 8;
  }
  vargs.total_items = (int32_t)pairs;
  return launch_v_rank_major(vargs, stream);
}

// Tile-reconstruct path.  Items are (weight, token group, 64-row group, column range);
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
  // Items of about half a CU's share (a quarter at tt = 1, where two workgroups share a
  // CU).  (Finer cutting measured slower: every range adds a pipeline start and a
  // partial-sum pass.)
  const int64_t slots = (int64_t)kTileItemsPerCu * (tt == 1 ? 2 : 1) * s->decode_grid_max;
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
  const int rc = plan_rank_major_v(s, args);
  if (rc != BSL_OK) return rc;
  DeviceGuard guard(s->device);
  int e = launch_rank_major_v(args, stream);
  if (e == 0) e = launch_tile(args, tt, (int)token_groups, stream);
  if (e == 0) ++s->launches[3];
  if (e != 0) return hip_fail(static_cast<hipError_t>(e), "kernel launch");
  return BSL_OK;
}

// Product-index path: units (weight, row group of kPxWaves x kPxTiles 32-row tiles, batch
// of kPxBatch blocks, 512-column chunk), an equal share per workgroup of kPxWaves waves;
// the shares of a row group meet in the row accumulators (one word per row and token),
// so any split of a group's units is exact up to each share's fp32 rounding.
int forward_product(bsl_stack* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y, int32_t M,
                    int32_t y_is_fp32, void* stream) {
  if (M > kPxMaxTokens) return fail(BSL_EUNSUPPORTED, "forward: the product-index path takes at most 32 tokens");
  GroupArgs args;
  std::memset(&args, 0, sizeof(args));
  args.count = count;
  args.M = M;
  args.y_fp32 = y_is_fp32 ? 1 : 0;
  args.zero_page = s->zero_page;
  uint64_t units = 0, groups = 0;
  for (int32_t j = 0; j < count; ++j) {
    const int32_t w = weights[j];
    if (w < 0 || w >= (int32_t)s->w.size()) return fail(BSL_EINVAL, "forward: weight index out of range");
    for (int32_t jj = 0; jj < j; ++jj)
      if (weights[jj] == w) return fail(BSL_EINVAL, "forward: a weight appears twice in one launch");
    if (!x[j] || !y[j]) return fail(BSL_EINVAL, "forward: null x or y");
    if ((reinterpret_cast<uintptr_t>(x[j]) & 15) != 0) return fail(BSL_EINVAL, "forward: x must be 16-byte aligned");
    const Weight& W = s->w[w];
    if ((uint64_t)pad_rows(W.m) * pad_cols(W.d) / 8 >= (1ull << 31))
      return fail(BSL_EUNSUPPORTED, "forward: the product-index path needs each block's signs below 2 GiB");
    WeightDesc& D = args.w[j];
    D.blocks = W.dtable;
    D.x = static_cast<const uint16_t*>(x[j]);
    D.y = y[j];
    D.m = W.m;
    D.d = W.d;
    D.mt = W.mt;
    D.nch = W.nch;
    D.nblocks = W.n;
    D.groups = (W.m + kPxWaves * kPxTiles * kPxTileRows - 1) / (kPxWaves * kPxTiles * kPxTileRows);  // row groups
    const uint64_t batches = (uint64_t)(W.n + kPxBatch - 1) / kPxBatch;
    D.unit_begin = (uint32_t)units;
    D.units = (uint32_t)(D.groups * batches * W.nch);
    D.rg_begin = (uint32_t)groups;  // first row group of the launch (share slots)
    units += (uint64_t)D.groups * batches * W.nch;
    groups += (uint64_t)D.groups;
  }
  if (units >= (1ull << 30)) return fail(BSL_EUNSUPPORTED, "forward: too much work for one launch");
  args.total_units = (uint32_t)units;
  args.total_groups = (uint32_t)groups;
  // Workers (workgroups): a power of two, one per CU at most, no more than the units.
  int64_t workers = s->decode_grid_max;
  while (workers > 1 && (uint64_t)workers > units) workers /= 2;
  int lg = 0;
  while ((1ll << lg) < workers) ++lg;
  // a slot per (row group, workgroup) pair: at most row groups + workgroups of them
  if (groups + ((uint64_t)1 << lg) > s->px_part_slots) return fail(BSL_EUNSUPPORTED, "forward: product share slots");
  args.part = s->px_part;
  args.grid_log2 = lg;
  // the activations as the kernel's B operands, in the stack's workspace
  int64_t chunks = 0;
  for (int32_t j = 0; j < count; ++j) {
    WeightDesc& D = args.w[j];
    D.xt = s->xt_ws + (size_t)chunks * (kPxLaneBytesPerChunk / 4);
    chunks += D.nch;
  }
  if ((size_t)chunks * kPxLaneBytesPerChunk > s->xt_cap) return fail(BSL_EUNSUPPORTED, "forward: x lanes workspace");
  const int rc = plan_rank_major_v(s, args);
  if (rc != BSL_OK) return rc;
  // one launch for both layout passes: the V pass's (weight, block, step) pairs, then the
  // x pass's (weight, chunk, plane, k) items
  GroupArgs largs = args;
  int64_t pairs = 0, xpairs = 0;
  for (int32_t j = 0; j < count; ++j) {
    largs.w[j].item_begin = (int32_t)pairs;
    largs.w[j].unit_begin = (uint32_t)xpairs;
    pairs += (int64_t)args.w[j].nblocks * args.w[j].nch * 8;
    xpairs += args.w[j].nch;
  }
  if (xpairs * kPlanes * 2 > (int64_t)UINT32_MAX - pairs) return fail(BSL_EUNSUPPORTED, "forward: too much work for one launch");
  largs.total_items = (int32_t)pairs;
  largs.total_units = (uint32_t)(xpairs * kPlanes * 2);
  DeviceGuard guard(s->device);
  int e = launch_layout_pass(largs, stream);
  if (e == 0) e = launch_product(args, stream);
  if (e == 0) e = launch_product_finish(args, stream);
  if (e == 0) ++s->launches[4];
  if (e != 0) return hip_fail(static_cast<hipError_t>(e), "kernel launch");
  return BSL_OK;
}

// use_static: the allocation-free variant (bsl_forward_group_static): 1 to 4 tokens on the
// single- and few-token kernels only, their row accumulators in the device's static
// scratch array instead of the stack's workspace.
int forward_impl(bsl_stack* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y, int32_t M,
                 int32_t y_is_fp32, void* stream, bool use_static = false) {
  if (count < 1 || count > kMaxGroup) return fail(BSL_EINVAL, "forward: 1..8 weights per launch");
  if (M < 1 || M > (1 << 24)) return fail(BSL_EINVAL, "forward: M must be >= 1");
  if (use_static && M > kWpMaxTokens)
    return fail(BSL_EUNSUPPORTED, "bsl_forward_group_static: takes 1 to 4 tokens (the single- and few-token kernels)");
  if (s->path == BSL_PATH_DECODE && M > kWpMaxTokens)
    return fail(BSL_EUNSUPPORTED, "forward: BSL_PATH_DECODE takes 1 to 4 tokens (the single- and few-token kernels)");
  GroupArgs args;
  std::memset(&args, 0, sizeof(args));
  args.count = count;
  args.M = M;
  args.y_fp32 = y_is_fp32 ? 1 : 0;
  // BSL_PATH_AUTO: 4 to 32 tokens on the product-index kernel (measured faster there than
  // the tile kernel, whose sign application is VALU work per element and block, and than
  // the few-token kernel, whose matrix work grows with every token; at 2 and 3 tokens the
  // few-token kernel is the faster)
  const bool product = !use_static && M >= 2 &&
                       (s->path == BSL_PATH_PRODUCT ||
                        (s->path == BSL_PATH_AUTO && M >= kPxAutoMinTokens && M < kTileAutoMinTokens));
  if (product) return forward_product(s, count, weights, x, y, M, y_is_fp32, stream);
  const bool tile = !use_static && (s->path == BSL_PATH_TILE || (s->path == BSL_PATH_AUTO && M >= kTileAutoMinTokens));
  if (tile) return forward_tile(s, count, weights, x, y, M, y_is_fp32, stream);
  size_t mt_floats = 0, mt_words = 0;  // this launch's shares of the multi-token workspace
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
    D.partial = s->mt_partial + mt_floats;  // (distinct weights: within the kMaxGroup largest shares)
    D.counters = s->mt_counters + mt_words;
    mt_floats += W.partial_floats;
    mt_words += W.counter_count;
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
  // Largest number of workers (2^lg of them, each with units [start(o), start(o + 1)))
  // that share one row group; the row accumulators count at most kAccMaxParts.
  auto max_parts = [&](int lg) {
    auto owner = [&](uint64_t u) {  // the kernels' owner(): o with start(o) <= u < start(o + 1)
      uint64_t o = (u << lg) / units;
      while (o + 1 < ((uint64_t)1 << lg) && start(o + 1, lg) <= u) ++o;
      while (start(o, lg) > u) --o;
      return o;
    };
    uint64_t worst = 0;
    for (int32_t j = 0; j < count; ++j) {
      const WeightDesc& D = args.w[j];
      if (D.units == 0) continue;
      const uint64_t per = D.units / (uint64_t)D.groups;
      for (int32_t g = 0; g < D.groups; ++g) {
        const uint64_t first = D.unit_begin + (uint64_t)g * per;
        worst = std::max<uint64_t>(worst, owner(first + per - 1) - owner(first) + 1);
      }
    }
    return worst;
  };
  // Plan of the wave-private kernel for T tokens (row groups of 256 rows for T = 1, 128
  // rows for T = 2 to 4); false when a workgroup's activations do not fit its LDS.
  auto plan_private = [&](int T, int& lg) {
    plan_units(T == 1 ? kWpRows : kWpFewRows);
    // workers: four per workgroup, at most one workgroup per CU, at most one per unit
    int32_t workers = kWpWaves * s->decode_grid_max;
    while (workers > kWpWaves && (uint64_t)workers > units) workers /= 2;
    lg = 0;
    while ((1 << lg) < workers) ++lg;
    // no row group shared by more workers than its accumulators count
    while (workers > kWpWaves && units > 0 && max_parts(lg) > (uint64_t)kAccMaxParts) {
      workers /= 2;
      --lg;
    }
    // (no units at all: one workgroup writes y = 0)
    bool fits = (units == 0 || units >= (uint64_t)workers) && (units << lg) < (1ull << 32) &&
                (units == 0 || max_parts(lg) <= (uint64_t)kAccMaxParts);
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
  // Row accumulators of a launch: `words` per row group (rows x tokens of the kernel about
  // to run).  In the allocation-free variant they live in the static scratch, cleared here.
  auto launch_units = [&](int lg, size_t words) {
    args.total_units = (uint32_t)units;
    args.total_groups = (uint32_t)groups;
    args.grid_log2 = lg;
    args.zero_page = s->zero_page;
    args.acc = s->acc64;
    const size_t need = groups * words * sizeof(uint64_t);
    if (!use_static) return need <= s->acc64_words * sizeof(uint64_t) ? BSL_OK : fail(BSL_EUNSUPPORTED, "forward: row accumulators");
    if (need > kStaticScratchBytes)
      return fail(BSL_EUNSUPPORTED, "bsl_forward_group_static: this launch needs " + std::to_string(need) +
                                        " bytes of row accumulators; the static scratch holds " + std::to_string(kStaticScratchBytes));
    args.acc = static_cast<uint64_t*>(s->static_scratch);
    // the kernels expect zero accumulators; a kernel, not a memset, so that captured
    // streams hold no memset node
    const int fe = launch_fill_u32(static_cast<uint32_t*>(s->static_scratch), (uint32_t)(need / sizeof(uint32_t)), 0u, stream);
    return fe == 0 ? BSL_OK : hip_fail(static_cast<hipError_t>(fe), "scratch clear");
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
      // CU and no more than the number of units (so no workgroup's share is empty), and
      // small enough that no row group is shared by more workgroups than its rows'
      // accumulators can count.
      int32_t grid = s->decode_grid_max;
      while (grid > 1 && (uint64_t)grid > units) grid /= 2;
      while ((1 << lg) < grid) ++lg;
      while (lg > 0 && units > 0 && max_parts(lg) > (uint64_t)kAccMaxParts) --lg;
      if ((units << lg) >= (1ull << 32)) return fail(BSL_EUNSUPPORTED, "forward: too much work for one launch");
    }
    const int rc = launch_units(lg, wp ? (size_t)kWpRows : (size_t)kDecodeGroupRows);
    if (rc != BSL_OK) return rc;
    e = wp ? launch_decode_wp(args, 1, stream) : launch_decode_m1(args, stream);
    if (e != 0) return hip_fail(static_cast<hipError_t>(e), "kernel launch");
    ++s->launches[wp ? 1 : 0];
    return BSL_OK;
  }
  if (M <= kWpMaxTokens && (s->path == BSL_PATH_AUTO || s->path == BSL_PATH_DECODE || use_static)) {
    // a few tokens: the wave-private kernel with every operand but the activations shared
    // by the tokens, when they fit its LDS
    const int T = M;
    int lg = 0;
    if (plan_private(T, lg)) {
      const int rc = launch_units(lg, (size_t)kWpFewRows * T);  // (rows x tokens of a row group)
      if (rc != BSL_OK) return rc;
      e = launch_decode_wp(args, T, stream);
      if (e != 0) return hip_fail(static_cast<hipError_t>(e), "kernel launch");
      ++s->launches[1];
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
    if (use_static)
      return fail(BSL_EUNSUPPORTED, "bsl_forward_group_static: the activations of this group do not fit the few-token kernel's LDS");
    // Under AUTO the wide weights take the product-index path (measured faster there than
    // the factored multi-token kernel: a 28672-column down projection at 3 tokens);
    // under DECODE the multi-token kernel.
    const bool wide_product = s->path == BSL_PATH_AUTO && nw > 0;
    if (nn > 0 && nw > 0) {
      const int rc = forward_impl(s, nn, narrow, xn, yn, M, y_is_fp32, stream);
      if (rc != BSL_OK) return rc;
      if (wide_product) return forward_product(s, nw, wide, xw, yw, M, y_is_fp32, stream);
      return forward_impl(s, nw, wide, xw, yw, M, y_is_fp32, stream);
    }
    if (wide_product && nn == 0) return forward_product(s, count, weights, x, y, M, y_is_fp32, stream);
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
  ++s->launches[2];
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

int bsl_forward_group_static(bsl_stack* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y,
                             int32_t M, int32_t y_is_fp32, void* stream) {
  if (!s || !weights || !x || !y) return fail(BSL_EINVAL, "bsl_forward_group_static: null pointer");
  if (!s->static_scratch) return fail(BSL_EHIP, "bsl_forward_group_static: no static scratch on this device");
  return forward_impl(s, count, weights, x, y, M, y_is_fp32, stream, true);
}

int bsl_set_path(bsl_stack* s, int32_t path) {
  if (!s) return fail(BSL_EINVAL, "bsl_set_path: null stack");
  if (path != BSL_PATH_AUTO && path != BSL_PATH_FACTORED && path != BSL_PATH_TILE && path != BSL_PATH_PRODUCT &&
      path != BSL_PATH_DECODE)
    return fail(BSL_EINVAL, "bsl_set_path: unknown path");
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
  }
  if (s->zero_page) (void)hipFree(s->zero_page);
  if (s->acc64) (void)hipFree(s->acc64);
  if (s->tile_ws) (void)hipFree(s->tile_ws);
  if (s->tile_ctr) (void)hipFree(s->tile_ctr);
  if (s->mt_partial) (void)hipFree(s->mt_partial);
  if (s->mt_counters) (void)hipFree(s->mt_counters);
  if (s->vr_ws) (void)hipFree(s->vr_ws);
  if (s->xt_ws) (void)hipFree(s->xt_ws);
  if (s->px_part) (void)hipFree(s->px_part);
  free_retired(s);
  for (int k = 0; k < 2; ++k) {
    if (s->staging[k]) (void)hipHostFree(s->staging[k]);
    if (s->staged[k]) (void)hipEventDestroy(s->staged[k]);
    if (s->raw_dev[k]) (void)hipFree(s->raw_dev[k]);
  }
  delete s;
}

}  // extern "C"
