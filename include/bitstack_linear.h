/*
 * bitstack_linear -- BitStack residual-block linear layer on one MI355X (gfx950).
 *
 * A weight W (m = out_features rows, d = in_features columns) is held as a stack of
 * residual blocks.  Block i is a +-1 sign matrix S_i (m x d, stored at one bit per
 * entry) and two rank-k factors U_i (m x k) and V_i (d x k) in fp16.  The first n
 * loaded blocks restore the weight as
 *
 *     W_hat_n = sum_{i < n} S_i (elementwise *) (U_i V_i^T)
 *
 * (BitStack OpenReview discussion, the authors' reply giving the weight restoration
 * code; residual block = packed sign matrix + singular vectors from an absolute value
 * decomposition, paper-review page, Figure 3 caption).  This library computes the
 * layer output y = x W_hat_n^T directly from the loaded blocks and never forms
 * W_hat: per block it builds Z_i = V_i (.) x, contracts S_i Z_i on the matrix cores
 * (fp16 inputs, fp32 accumulation) and reduces the row-wise dot with U_i over all
 * blocks in one pass.
 *
 * Blocks live in a device-resident stack.  The number of loaded blocks per weight
 * can grow (new blocks are copied in) or shrink (the last blocks are released)
 * without touching the blocks that stay, which mirrors BitStack's load/offload of
 * residual blocks as memory availability changes (paper-review page, Figure 2
 * caption; OpenReview reply A1.B).
 *
 * Conventions for every entry point:
 *   - Return value: BSL_OK (0) or a negative BSL_E* code; no call aborts and no
 *     C++ exception crosses this interface.  bsl_last_error() returns a message for
 *     the calling thread's most recent failure.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HIP device
 *     memory of the stack's device.  Streams are hipStream_t passed as void*; NULL
 *     means the default stream.
 *   - Host inputs are read during the call (or, for bsl_set_source, until the next
 *     bsl_set_source / bsl_destroy of that weight) and never retained otherwise.
 *   - fp16 values are passed as their IEEE binary16 bit patterns (uint16_t).
 *   - Supported shapes: k == 16, 1 <= m <= 2^20, 8 <= d <= 2^20 with d % 8 == 0.
 *     Internally rows are padded to a multiple of 1024 and columns to a multiple of
 *     512 (padding signs are +1 and padding factor entries are 0, so padding never
 *     changes a result).
 *   - A stack is not thread-safe: calls on one stack must not run concurrently.
 */
#ifndef BITSTACK_LINEAR_H
#define BITSTACK_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSL_OK 0
#define BSL_EINVAL (-1)       /* bad argument: null pointer, index or size out of range */
#define BSL_ENOMEM (-2)       /* device allocation failed or the stack's byte budget is exceeded */
#define BSL_EHIP (-3)         /* a HIP runtime call failed; the message holds HIP's error text */
#define BSL_EUNSUPPORTED (-4) /* shape, k or batch outside what this build supports */

/* Opaque handle; owns all device memory of the loaded blocks and the workspace. */
typedef struct bsl_stack bsl_stack;

/* One residual block as the caller provides it (host memory).
 *   sign_bits: m rows of d/8 bytes, row-major; bit (c % 8) of byte c/8 of a row is
 *              column c (least significant bit first); a set bit means the sign is -1.
 *   u:         fp16 [m][k] row-major.
 *   v:         fp16 [d][k] row-major (the right factor, not transposed).
 * With k = 16 the block occupies m*d/8 + 2*k*(m + d) bytes of payload (one bit per
 * sign, 16 bits per factor entry; OpenReview reply A1.A: the largest block of an 8B
 * model, 14336 x 4096, is 7.56 MB). */
typedef struct bsl_block_src {
  const uint8_t* sign_bits;
  const uint16_t* u;
  const uint16_t* v;
} bsl_block_src;

/* Payload bytes of one block: m*d/8 + 2*k*(m + d).  Returns 0 for invalid sizes. */
size_t bsl_block_bytes(int64_t m, int64_t d, int32_t k);

/* Bytes of the tiled sign layout of one m x d block (rows padded to 1024, columns to 512). */
size_t bsl_packed_sign_bytes(int64_t m, int64_t d);

/* Host-side "bitstack_pack": convert row-major sign bits (format of bsl_block_src)
 * into the tiled device layout (the sign matrix packed into a GPU data layout:
 * paper-review page, Figure 3 caption).  bsl_load_blocks produces the same layout on
 * the device; this host version serves checks and callers that pack ahead of time.  tiled_out (host) must hold bsl_packed_sign_bytes(m, d)
 * bytes.  Layout: tiles of 16 rows x 512 columns, ordered [column chunk][row tile];
 * each tile is 64 lanes x 16 bytes; lane L = 16*g + i holds row i of the tile and four
 * little-endian 32-bit words q = 0..3.  Of the chunk's 32-column plane b = 4*q + k
 * (k = 0..3), the lane keeps columns 32*b + 8*g + e (e = 0..7) in word q at bit
 * 16*(k % 2) + 2*e + 1 when k < 2 and at bit 16*(k % 2) + 2*e when k >= 2.  Each plane
 * thereby sits at the odd or the even positions of one 16-bit half, which is the form
 * the forward kernels use directly as 2:4 sparse-MFMA indices.  One 16-byte load per
 * lane fetches a whole tile (1 KiB, eight full 128-byte lines). */
int bsl_pack_signs(const uint8_t* rowmajor_bits, int64_t m, int64_t d, uint8_t* tiled_out);

/* Inverse of bsl_pack_signs, for checking: writes int8 +1/-1 into pm1_out (host,
 * m*d bytes, row-major), i.e. the unpack step of the weight restoration (OpenReview
 * discussion, weight-restoration reply).  Padding is ignored. */
int bsl_unpack_signs(const uint8_t* tiled, int64_t m, int64_t d, int8_t* pm1_out);

/* Create a stack for num_weights weights with shapes m[w] x d[w] (host arrays), rank k
 * (must be 16), at most n_cap blocks per weight (1 <= n_cap <= 64; the paper's runs
 * decompose with 16 iterations: README, "Decomposition"), on HIP device `device`.  budget_bytes caps
 * the device bytes held by loaded blocks (0 = no cap).  The per-weight workspace used
 * by bsl_forward is allocated here, so forward never allocates.  *out receives the
 * handle. */
int bsl_init(bsl_stack** out, int device, int32_t num_weights, const int32_t* m, const int32_t* d, int32_t k,
             int32_t n_cap, uint64_t budget_bytes);

/* Register the host source of weight w's blocks, in load order (the presorted order of
 * the weight's stack): blocks[0 .. n_avail-1].  The arrays must stay valid until the
 * next bsl_set_source for w or bsl_destroy; only bsl_load_blocks reads them. */
int bsl_set_source(bsl_stack* s, int32_t w, int32_t n_avail, const bsl_block_src* blocks);

/* Activation-aware scaling (paper-review page, Figure 5 caption: the "w/o scaling"
 * ablation drops the scaling of Eq. 4; the equation itself is not printed there).
 * Reading taken: the blocks of weight w decompose W diag(s), where s > 0 holds one
 * factor per input channel drawn from activation statistics, so the layer is
 *     y = (x (.) inv_scale) W_hat_n^T,   inv_scale[c] = 1 / s[c]   (c < d).
 * Column scaling commutes with the elementwise sign product, so inv_scale is folded
 * into V at load: bsl_load_blocks stores fp16(V_i[c][r] * inv_scale[c]) (exact product,
 * one rounding to nearest even) and every forward path then costs exactly what the
 * unscaled layer costs.
 *   inv_scale: host, d[w] floats, each finite and > 0; copied, so the caller may free
 *     it on return.  NULL removes the scale (inv_scale = 1).
 * Only allowed while weight w has no loaded blocks (BSL_EINVAL otherwise), so every
 * loaded block of a weight carries the same scale.  bsl_load_blocks fails with
 * BSL_EINVAL, loading nothing, if a scaled V entry would overflow fp16. */
int bsl_set_input_scale(bsl_stack* s, int32_t w, const float* inv_scale);

/* Set the number of loaded blocks of every weight to n_per_weight[w] (host array of
 * num_weights entries, 0 <= n <= min(n_cap, n_avail)).  Growing copies only the new
 * blocks [n_old, n_new): a block's row-major sign bits are copied as they are into one of
 * two pinned staging buffers (the factor layouts are written beside them on the host),
 * sent to the device asynchronously on `stream` and repacked into the tiled layout there
 * by a kernel, while the next block is staged; the call returns once the copies are
 * done.  Forwards already queued on other streams keep running meanwhile and keep using
 * the counts they were queued with (only the new entries of the device block table are
 * written).  Shrinking waits for the device to drain and then releases blocks [n_new,
 * n_old).  The call is all-or-nothing: on any failure every weight keeps its previous
 * count and no memory is leaked.  Blocks that stay loaded are never moved or rewritten.
 * (Universal stack: blocks are loaded and offloaded as memory allows; paper-review page,
 * Figure 2 caption.) */
int bsl_load_blocks(bsl_stack* s, const int32_t* n_per_weight, void* stream);

/* Number of loaded blocks of weight w: the n of W_hat_n, which sets the weight's size
 * (paper-review page, Figure 2 caption). */
int bsl_active_blocks(const bsl_stack* s, int32_t w, int32_t* n_out);

/* Device bytes currently held by loaded blocks (what budget_bytes caps).  A loaded block
 * occupies its tiled signs, U and V, with rows padded to 1024 and columns to 512, and
 * nothing else: for aligned shapes that is bsl_block_bytes(m, d, 16) exactly.  (The
 * kernels form every other operand order they need on the fly.) */
uint64_t bsl_resident_bytes(const bsl_stack* s);

/* Device bytes the stack holds besides its loaded blocks (not capped by budget_bytes):
 * the forward paths' workspaces (row accumulators, split partial sums and their counters,
 * block tables, the tile path's V in rank-major order) and bsl_load_blocks' device
 * buffers.  The rank-major V workspace holds the V of the kMaxGroup = 8 weights with the
 * most V bytes, whatever the number of weights: the tile path forms it for the launch's
 * blocks at the start of each call (one read and one write of their V). */
uint64_t bsl_workspace_bytes(const bsl_stack* s);

/* y = x W_hat_n^T for weight w with its n loaded blocks: the linear layer with the
 * weight the authors restore block by block (OpenReview discussion, weight-restoration
 * reply), computed from the packed blocks (BSL_PATH_FACTORED never forms W_hat;
 * BSL_PATH_TILE forms it only per tile in registers).
 *   x: device, fp16 [M][d] row-major, 16-byte aligned.
 *   y: device, [M][m] row-major, fp16 (y_is_fp32 == 0, round to nearest even) or fp32.
 *   M >= 1 tokens.  With n = 0 loaded blocks y is all zeros.
 * Only enqueues kernels on `stream` (no synchronisation, no allocation).  Forwards on
 * one stack must not run concurrently, even for different weights: they share the
 * stack's workspaces (row accumulators, split partial sums and their counters, the tile
 * path's rank-major V).  Forwards queued on one stream are ordered, so that is the simple
 * way to issue them. */
int bsl_forward(bsl_stack* s, int32_t w, const void* x, void* y, int32_t M, int32_t y_is_fp32, void* stream);

/* Several weights in one call (count <= 8, distinct weights): weights[j] reads x[j] and
 * writes y[j] exactly as bsl_forward would.  All share M and y_is_fp32.  The group runs
 * as one kernel launch, except
 *   - on the tile path (BSL_PATH_TILE, and BSL_PATH_AUTO from M = 33 on), which first
 *     runs a short pass that puts the V of the group's loaded blocks in rank-major order
 *     in the stack's workspace, then the tile kernel;
 *   - on the product-index path (BSL_PATH_PRODUCT at M = 2..32, BSL_PATH_AUTO at
 *     M = 4..32): one launch of the same V pass and of a pass that writes x as the
 *     kernel's B operands, the product-index kernel, then a pass that adds the
 *     workgroups' shares of every row group in a fixed order into y;
 *   - on BSL_PATH_AUTO at M = 2..3 and BSL_PATH_DECODE at M = 2..4 when the group's
 *     activations do not fit the few-token kernel as a whole: then it is split into two
 *     forwards (see bsl_set_path), the second on the product-index path under AUTO.
 *     An error returned after the first of the two was enqueued leaves the y[j] of the
 *     weights in that launch written and the others unspecified. */
int bsl_forward_group(bsl_stack* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y,
                      int32_t M, int32_t y_is_fp32, void* stream);

/* Allocation-free variant of bsl_forward_group, for callers that cannot allocate device
 * memory or must not let a call allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, same results as
 * bsl_forward_group under BSL_PATH_DECODE for 1 <= M <= 4 (the same kernels in the same
 * launch configuration),
 * with the kernels' row accumulators (one 64-bit word per output row and token) in a
 * scratch array of 8 MiB that the library holds on each device it runs on until the
 * process ends (its address is taken by bsl_init).  The call allocates nothing, on the
 * device or the host; it clears the accumulators it uses with a small kernel on
 * `stream`, then launches the forward there.
 *   M = 1 takes the single-token kernel bsl_set_decode selects; M = 2..4 the few-token
 *   kernel whatever bsl_set_path says.
 * Errors (nothing is launched): BSL_EUNSUPPORTED if M > 4, if the launch needs more
 * accumulators than the scratch holds (the message gives both sizes), or if
 * the group's activations do not fit the few-token kernel (where bsl_forward_group would
 * split the group); the argument errors of bsl_forward_group.
 * Every such call on one device shares that device's scratch: calls that may overlap in
 * time on one device (other streams, other stacks, other threads) race and give wrong
 * results.  Issue them on one stream, or order them. */
int bsl_forward_group_static(bsl_stack* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y,
                             int32_t M, int32_t y_is_fp32, void* stream);

/* Formulation of the forward for a batch of tokens (bsl_set_path):
 *   BSL_PATH_FACTORED: never form W_hat.  Per block, contract S_i with Z_i = V_i (.) x on
 *     the matrix cores and reduce with U_i (the single-token kernel at M = 1, the
 *     multi-token kernel otherwise).  Work grows as n * k * M * m * d.
 *   BSL_PATH_TILE: the weight restoration the authors give (add each block's unpacked
 *     signs times U_i V_i^T; OpenReview discussion, weight-restoration reply), done per
 *     32 x 32 tile in registers and multiplied at once with up to 512 tokens:
 *     the tile of W_hat is rounded to fp16 (each block's U_i V_i^T and the running sum
 *     over blocks), then y accumulates in fp32.  Work grows as n * k * m * d per group of
 *     512 tokens plus M * m * d, so it is the fast form for batches.
 *   BSL_PATH_PRODUCT (2 to 32 tokens; M = 1 as under FACTORED): the same restoration
 *     block by block with the sign applied inside the matrix core.  Each block's
 *     U_i V_i^T, rebuilt per 32 x 32 tile and plane in registers and rounded to fp16, is
 *     the value operand of the 2:4 sparse MFMA, and the stored sign bits are its indices
 *     against B = +x / -x, so no sign is expanded; blocks and columns sum in fp32.  Work
 *     grows as (k + 32) * n * m * d whatever the token count up to 32.  A call first runs
 *     two short passes in one launch (V in rank-major order, x as the MFMA's B operands)
 *     into the stack's workspaces; after the kernel a third adds the workgroups' fp32
 *     shares of each row group in workgroup order (deterministic: the same launch gives
 *     the same bits).  M > 32: BSL_EUNSUPPORTED.
 *   BSL_PATH_DECODE (1 to 4 tokens; M > 4: BSL_EUNSUPPORTED): M = 1 as under FACTORED;
 *     M = 2 to 4 on the wave-private kernel of BSL_DECODE_PRIVATE taking the M tokens at
 *     once, which share every sign, U and V operand and load, when their activations fit
 *     its LDS (148 KiB per workgroup); in a grouped call that does not fit as a whole, the
 *     weights whose activations take at most half of it go to that kernel and the others
 *     to the factored multi-token kernel, in a second launch.
 *   BSL_PATH_AUTO (the default): M = 1 as under FACTORED; M = 2 and 3 as under DECODE,
 *     except that the weights whose activations take more than half of the few-token
 *     kernel's LDS, when the group does not fit it as a whole, take PRODUCT instead of the
 *     factored kernel; PRODUCT for M = 4 to 32; TILE from M = 33 on. */
#define BSL_PATH_AUTO 0
#define BSL_PATH_FACTORED 1
#define BSL_PATH_TILE 2
#define BSL_PATH_PRODUCT 3
#define BSL_PATH_DECODE 4
/* Errors: BSL_EINVAL for a null stack or a value other than the five above. */
int bsl_set_path(bsl_stack* s, int32_t path);

/* Kernel of the single-token forward (M = 1; bsl_set_decode).  Both compute the same
 * sums, in different orders (results agree to fp32 rounding, not bit for bit):
 *   BSL_DECODE_SHARED: 16 waves per CU share each unit's B operands (+-Z = +-V x in fp16)
 *     through LDS, one barrier per unit.
 *   BSL_DECODE_PRIVATE: every wave builds its own B operands (+-V) and carries x in the
 *     sparse MFMA's A operand, so the products V x are exact and no barrier is needed.
 *     A workgroup keeps the activations of the weights it works on in LDS (148 KiB);
 *     a launch that does not fit fails with BSL_EUNSUPPORTED.
 *   BSL_DECODE_AUTO (the default): SHARED, the faster of the two on this hardware. */
#define BSL_DECODE_AUTO 0
#define BSL_DECODE_SHARED 1
#define BSL_DECODE_PRIVATE 2
int bsl_set_decode(bsl_stack* s, int32_t kind);

/* Run a forward kernel's own sign-unpack code on block i of weight w and write the
 * signs as int8 +1/-1, row-major m x d, to pm1_out (device, m*d bytes): the unpack
 * step of the weight restoration (OpenReview discussion, weight-restoration reply), as
 * each kernel performs it.  The `path` argument, which selects the kernel, is an
 * addition for checking.
 * path 0: the single-token kernel's sparse-MFMA indices; path 1: the multi-token
 * kernel's +-1 fp16 A fragments; path 2: the tile-reconstruct kernel's +-1 fp16 pairs. */
int bsl_debug_unpack(bsl_stack* s, int32_t w, int32_t i, int32_t path, int8_t* pm1_out, void* stream);

/* Forward kernel launches the stack has enqueued since bsl_init, per kernel: counts[0] the
 * shared-operand single-token kernel, [1] the wave-private single- and few-token kernel,
 * [2] the factored multi-token kernel, [3] the tile-reconstruct kernel, [4] the
 * product-index kernel (host array of
 * BSL_KERNEL_KINDS entries).  A diagnostic: it tells a caller which formulation a call
 * took (bsl_set_path, bsl_set_decode), and how many launches a grouped call made. */
#define BSL_KERNEL_KINDS 5
int bsl_launch_counts(const bsl_stack* s, uint64_t* counts);

/* Message for the calling thread's last failure ("" if none). */
const char* bsl_last_error(void);

/* Release all device memory of the stack (waits for the device first).  NULL is ignored. */
void bsl_destroy(bsl_stack* s);

#ifdef __cplusplus
}
#endif

#endif /* BITSTACK_LINEAR_H */
