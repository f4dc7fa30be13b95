/* libbitstack_linear: the equal-size vanilla-SVD baseline.
 *
 * The "w/o AVD" ablation (paper-review page "BitStack: Fine-Grained Size Control for
 * Compressed Large Language Models in Variable Memory Environments", Figure 5
 * caption) replaces each residual block by the plain rank-k' SVD of the residual,
 * with k' = k + m d / (16 (m + d)) so that a block takes the bytes of a 1-bit-sign
 * block: two fp16 factors U'_i (m x k') and V'_i (d x k'), no signs.  The layer with
 * n loaded blocks is
 *     y = x (sum_{i<n} U'_i V'_i^T)^T = sum_{i<n} (x V'_i) U'_i^T.
 * This stack runs that layer on the same device with the same conventions as the
 * main stack (bitstack_linear.h): fp16 x, fp16 or fp32 y, row-major, 16-byte aligned
 * device buffers, BSL_* return codes, messages through bsl_last_error().
 *
 * It is a baseline for the single-token case: the factors are read once per group
 * of up to 8 tokens, so larger batches re-read them.  Unlike the main stack it
 * reserves device memory for n_cap blocks of every weight at init (no byte budget).
 */
#ifndef BITSTACK_LOWRANK_H
#define BITSTACK_LOWRANK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bsl_lr bsl_lr;

/* One vanilla-SVD block on the host: u is fp16 [m][k'] row-major, v is fp16 [d][k']
 * row-major (column r of u and of v form the r-th rank-one term). */
typedef struct bsl_lr_block_src {
  const uint16_t* u;
  const uint16_t* v;
} bsl_lr_block_src;

/* k' = k + floor(m d / (16 (m + d))): the largest integer rank whose block
 * (2 k' (m + d) bytes) does not exceed a 1-bit-sign block of rank k.  0 if invalid. */
int32_t bsl_lr_equal_rank(int64_t m, int64_t d, int32_t k);

/* Payload bytes of one block: 2 k' (m + d).  0 for invalid sizes. */
size_t bsl_lr_block_bytes(int64_t m, int64_t d, int32_t k_prime);

/* Create a stack of num_weights weights: shapes m[w] x d[w] and ranks k_prime[w]
 * (host arrays; m >= 1, d >= 8 a multiple of 8, 1 <= k_prime <= 1024), at most n_cap
 * blocks per weight (1..64), on HIP device `device`.  Device memory for n_cap blocks
 * of every weight and the forward's workspace are allocated here. */
int bsl_lr_init(bsl_lr** out, int device, int32_t num_weights, const int32_t* m, const int32_t* d,
                const int32_t* k_prime, int32_t n_cap);

/* Register the host source of weight w's blocks (n_avail <= n_cap, in load order).
 * The arrays must stay valid until the next bsl_lr_set_source for w or
 * bsl_lr_destroy; only bsl_lr_load_blocks reads them. */
int bsl_lr_set_source(bsl_lr* s, int32_t w, int32_t n_avail, const bsl_lr_block_src* blocks);

/* Set the loaded block count of every weight (host array, 0 <= n <= n_avail).
 * Growing copies blocks [n_old, n_new) on `stream` and returns when they are on the
 * device; shrinking only lowers the count.  Forwards must not be running on the
 * stack meanwhile.  All-or-nothing: on failure every count stays as it was. */
int bsl_lr_load_blocks(bsl_lr* s, const int32_t* n_per_weight, void* stream);

/* Payload bytes of the loaded blocks: sum over weights of n_w * 2 k'_w (m_w + d_w). */
uint64_t bsl_lr_resident_bytes(const bsl_lr* s);

/* y = sum_{i<n} (x V'_i) U'_i^T for weight w (x: device fp16 [M][d]; y: device [M][m],
 * fp16 round to nearest even or fp32).  With n = 0, y = 0.  Enqueues two kernels per
 * group of 8 tokens on `stream`; no allocation, no synchronisation.  Two forwards of
 * the same weight must not run concurrently (they share its workspace). */
int bsl_lr_forward(bsl_lr* s, int32_t w, const void* x, void* y, int32_t M, int32_t y_is_fp32, void* stream);

/* Several distinct weights (count <= 8) in the same two launches, each reading x[j]
 * and writing y[j] as bsl_lr_forward would. */
int bsl_lr_forward_group(bsl_lr* s, int32_t count, const int32_t* weights, const void* const* x, void* const* y,
                         int32_t M, int32_t y_is_fp32, void* stream);

/* Release the stack's device memory (waits for the device first).  NULL is ignored. */
void bsl_lr_destroy(bsl_lr* s);

#ifdef __cplusplus
}
#endif

#endif /* BITSTACK_LOWRANK_H */
