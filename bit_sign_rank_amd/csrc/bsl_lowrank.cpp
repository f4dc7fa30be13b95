// Host side of the equal-size vanilla-SVD baseline stack (include/bitstack_lowrank.h):
// argument checks, factor packing, block loading and forward dispatch.
#include "bitstack_lowrank.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "bitstack_linear.h"
#include "bsl_internal.h"

using namespace bsl;

struct LrW {
  int32_t m = 0, d = 0, kp = 0, kp8 = 0, d_pad = 0, m_pad = 0, n = 0;
  std::vector<bsl_lr_block_src> src;
  uint16_t* vt = nullptr;  // [n_cap kp8][d_pad]
  uint16_t* ut = nullptr;  // [m_pad / 64][n_cap kp8 / 8][64][8]
  float* t = nullptr;      // [kLrTokens][n_cap kp8]
};

struct bsl_lr {
  int device = 0;
  int32_t n_cap = 0;
  std::vector<LrW> w;
};

namespace {

struct LrDeviceGuard {
  int prev = -1;
  explicit LrDeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    (void)hipSetDevice(dev);
  }
  ~LrDeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

int lr_hip_fail(hipError_t e, const char* what) {
  return set_error(BSL_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// V' (d x kp, row-major) -> [kp8][d_pad], zero past kp and past d.
void pack_vt(const uint16_t* v, const LrW& W, uint16_t* out) {
  std::memset(out, 0, (size_t)W.kp8 * W.d_pad * 2);
  for (int64_t c = 0; c < W.d; ++c)
    for (int32_t r = 0; r < W.kp; ++r) out[(int64_t)r * W.d_pad + c] = v[c * W.kp + r];
}

// U' (m x kp, row-major) -> [m_pad / 64][kp8 / 8][64][8], zero past kp and past m.
void pack_ut(const uint16_t* u, const LrW& W, uint16_t* out) {
  std::memset(out, 0, (size_t)W.m_pad * W.kp8 * 2);
  const int32_t qn = W.kp8 / 8;
  for (int64_t row = 0; row < W.m; ++row)
    for (int32_t r = 0; r < W.kp; ++r) {
      const int64_t g = row / kLrRowGroup, lane = row % kLrRowGroup, q = r / 8, j = r % 8;
      out[((g * qn + q) * kLrRowGroup + lane) * 8 + j] = u[row * W.kp + r];
    }
}

void release(bsl_lr* s) {
  for (LrW& W : s->w) {
    if (W.vt) (void)hipFree(W.vt);
    if (W.ut) (void)hipFree(W.ut);
    if (W.t) (void)hipFree(W.t);
    W.vt = W.ut = nullptr;
    W.t = nullptr;
  }
}

}  // namespace

extern "C" {

int32_t bsl_lr_equal_rank(int64_t m, int64_t d, int32_t k) {
  if (m < 1 || d < 1 || k < 1) return 0;
  return (int32_t)(k + (m * d) / (16 * (m + d)));
}

size_t bsl_lr_block_bytes(int64_t m, int64_t d, int32_t k_prime) {
  if (m < 1 || d < 1 || k_prime < 1) return 0;
  return (size_t)(2 * (int64_t)k_prime * (m + d));
}

int bsl_lr_init(bsl_lr** out, int device, int32_t num_weights, const int32_t* m, const int32_t* d,
                const int32_t* k_prime, int32_t n_cap) {
  if (!out || !m || !d || !k_prime) return set_error(BSL_EINVAL, "bsl_lr_init: null pointer");
  *out = nullptr;
  if (num_weights < 1) return set_error(BSL_EINVAL, "bsl_lr_init: num_weights must be >= 1");
  if (n_cap < 1 || n_cap > kMaxBlocks) return set_error(BSL_EINVAL, "bsl_lr_init: n_cap must be in 1..64");
  for (int32_t w = 0; w < num_weights; ++w) {
    if (m[w] < 1 || d[w] < 8 || d[w] % 8) return set_error(BSL_EUNSUPPORTED, "bsl_lr_init: m >= 1 and d >= 8 a multiple of 8");
    if (k_prime[w] < 1 || k_prime[w] > 1024) return set_error(BSL_EUNSUPPORTED, "bsl_lr_init: k' must be in 1..1024");
  }
  LrDeviceGuard guard(device);
  bsl_lr* s = new (std::nothrow) bsl_lr;
  if (!s) return set_error(BSL_ENOMEM, "bsl_lr_init: host allocation");
  s->device = device;
  s->n_cap = n_cap;
  s->w.resize(num_weights);
  hipError_t e = hipSuccess;
  for (int32_t w = 0; w < num_weights && e == hipSuccess; ++w) {
    LrW& W = s->w[w];
    W.m = m[w];
    W.d = d[w];
    W.kp = k_prime[w];
    W.kp8 = (int32_t)round_up(W.kp, 8);
    W.d_pad = (int32_t)round_up(W.d, kLrColAlign);
    W.m_pad = (int32_t)round_up(W.m, kLrRowGroup);
    const size_t ld = (size_t)n_cap * W.kp8;
    e = hipMalloc(&W.vt, ld * W.d_pad * 2);
    if (e == hipSuccess) e = hipMalloc(&W.ut, (size_t)W.m_pad * ld * 2);
    if (e == hipSuccess) e = hipMalloc(&W.t, (size_t)kLrTokens * ld * sizeof(float));
  }
  if (e != hipSuccess) {
    release(s);
    delete s;
    return set_error(BSL_ENOMEM, std::string("bsl_lr_init: hipMalloc: ") + hipGetErrorString(e));
  }
  *out = s;
  return BSL_OK;
}

int bsl_lr_set_source(bsl_lr* s, int32_t w, int32_t n_avail, const bsl_lr_block_src* blocks) {
  if (!s) return set_error(BSL_EINVAL, "bsl_lr_set_source: null stack");
  if (w < 0 || w >= (int32_t)s->w.size()) return set_error(BSL_EINVAL, "bsl_lr_set_source: weight index out of range");
  if (n_avail < 0 || n_avail > s->n_cap) return set_error(BSL_EINVAL, "bsl_lr_set_source: n_avail must be in 0..n_cap");
  if (n_avail > 0 && !blocks) return set_error(BSL_EINVAL, "bsl_lr_set_source: null block array");
  for (int32_t i = 0; i < n_avail; ++i)
    if (!blocks[i].u || !blocks[i].v) return set_error(BSL_EINVAL, "bsl_lr_set_source: block " + std::to_string(i) + " has a null array");
  s->w[w].src.assign(blocks, blocks + n_avail);
  return BSL_OK;
}

int bsl_lr_load_blocks(bsl_lr* s, const int32_t* n_per_weight, void* stream) {
  if (!s || !n_per_weight) return set_error(BSL_EINVAL, "bsl_lr_load_blocks: null pointer");
  const int32_t nw = (int32_t)s->w.size();
  for (int32_t w = 0; w < nw; ++w) {
    const int32_t n = n_per_weight[w];
    if (n < 0 || n > s->n_cap) return set_error(BSL_EINVAL, "bsl_lr_load_blocks: count out of range for weight " + std::to_string(w));
    if (n > s->w[w].n && n > (int32_t)s->w[w].src.size())
      return set_error(BSL_EINVAL, "bsl_lr_load_blocks: weight " + std::to_string(w) + " has only " +
                                       std::to_string(s->w[w].src.size()) + " source blocks");
  }
  LrDeviceGuard guard(s->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<uint16_t> vbuf, ubuf;
  hipError_t e = hipSuccess;
  for (int32_t w = 0; w < nw && e == hipSuccess; ++w) {
    LrW& W = s->w[w];
    const size_t ld = (size_t)s->n_cap * W.kp8;
    for (int32_t i = W.n; i < n_per_weight[w] && e == hipSuccess; ++i) {
      vbuf.resize((size_t)W.kp8 * W.d_pad);
      ubuf.resize((size_t)W.m_pad * W.kp8);
      pack_vt(W.src[i].v, W, vbuf.data());
      pack_ut(W.src[i].u, W, ubuf.data());
      e = hipMemcpyAsync(W.vt + (size_t)i * W.kp8 * W.d_pad, vbuf.data(), vbuf.size() * 2, hipMemcpyHostToDevice, st);
      // block i's column groups of every row group: a strided copy
      const size_t width = (size_t)W.kp8 * kLrRowGroup * 2;
      if (e == hipSuccess)
        e = hipMemcpy2DAsync(W.ut + (size_t)i * W.kp8 * kLrRowGroup, ld * kLrRowGroup * 2, ubuf.data(), width, width,
                             W.m_pad / kLrRowGroup, hipMemcpyHostToDevice, st);
      if (e == hipSuccess) e = hipStreamSynchronize(st);  // the host buffers are reused
    }
  }
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(st);
    return lr_hip_fail(e, "bsl_lr_load_blocks: copy");
  }
  for (int32_t w = 0; w < nw; ++w) s->w[w].n = n_per_weight[w];
  return BSL_OK;
}

uint64_t bsl_lr_resident_bytes(const bsl_lr* s) {
  if (!s) return 0;
  uint64_t b = 0;
  for (const LrW& W : s->w) b += (uint64_t)W.n * bsl_lr_block_bytes(W.m, W.d, W.kp);
  return b;
}

int bsl_lr_forward_group(bsl_lr* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y,
                         int32_t M, int32_t y_is_fp32, void* stream) {
  if (!s || !weights || !x || !y) return set_error(BSL_EINVAL, "bsl_lr_forward: null pointer");
  if (count < 1 || count > kMaxGroup) return set_error(BSL_EINVAL, "bsl_lr_forward: 1..8 weights per launch");
  if (M < 1 || M > (1 << 24)) return set_error(BSL_EINVAL, "bsl_lr_forward: M must be >= 1");
  for (int32_t j = 0; j < count; ++j) {
    const int32_t w = weights[j];
    if (w < 0 || w >= (int32_t)s->w.size()) return set_error(BSL_EINVAL, "bsl_lr_forward: weight index out of range");
    for (int32_t jj = 0; jj < j; ++jj)
      if (weights[jj] == w) return set_error(BSL_EINVAL, "bsl_lr_forward: a weight appears twice in one launch");
    if (!x[j] || !y[j]) return set_error(BSL_EINVAL, "bsl_lr_forward: null x or y");
    if ((reinterpret_cast<uintptr_t>(x[j]) & 15) != 0) return set_error(BSL_EINVAL, "bsl_lr_forward: x must be 16-byte aligned");
  }
  LrDeviceGuard guard(s->device);
  for (int32_t t0 = 0; t0 < M; t0 += kLrTokens) {
    LrArgs a;
    std::memset(&a, 0, sizeof(a));
    a.count = count;
    a.T = std::min(kLrTokens, M - t0);
    a.y_fp32 = y_is_fp32 ? 1 : 0;
    for (int32_t j = 0; j < count; ++j) {
      const LrW& W = s->w[weights[j]];
      LrWeight& D = a.w[j];
      D.vt = W.vt;
      D.ut = W.ut;
      D.x = static_cast<const uint16_t*>(x[j]) + (size_t)t0 * W.d;
      D.y = static_cast<char*>(y[j]) + (size_t)t0 * W.m * (y_is_fp32 ? 4 : 2);
      D.t = W.t;
      D.m = W.m;
      D.d = W.d;
      D.d_pad = W.d_pad;
      D.ld = s->n_cap * W.kp8;
      D.kcat = W.n * W.kp8;
      D.row_begin = a.total_rows;
      D.rg_begin = a.total_rgs;
      a.total_rows += D.kcat;
      a.total_rgs += W.m_pad / kLrRowGroup;
    }
    const int e = launch_lowrank(a, stream);
    if (e != 0) return lr_hip_fail(static_cast<hipError_t>(e), "bsl_lr_forward: launch");
  }
  return BSL_OK;
}

int bsl_lr_forward(bsl_lr* s, int32_t w, const void* x, void* y, int32_t M, int32_t y_is_fp32, void* stream) {
  if (!s) return set_error(BSL_EINVAL, "bsl_lr_forward: null stack");
  const void* xs[1] = {x};
  void* ys[1] = {y};
  return bsl_lr_forward_group(s, 1, &w, xs, ys, M, y_is_fp32, stream);
}

void bsl_lr_destroy(bsl_lr* s) {
  if (!s) return;
  LrDeviceGuard guard(s->device);
  (void)hipDeviceSynchronize();
  release(s);
  delete s;
}

}  // extern "C"
