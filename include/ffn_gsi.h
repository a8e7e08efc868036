/*
 * ffn_gsi.h -- C ABI of the gated subspace fast path for a linear map
 * (MI355X / gfx950), part of the same library as ffn_sparse.h.
 *
 * Source: "Gated Subspace Inference for Transformer Acceleration",
 *   - section 2.1: with an orthonormal rank-k basis V_k (d_in x k) of the
 *     activations, x = V_k g + r with g = V_k^T x, so y = W x = M g + W r with
 *     the cached low-rank image M = W V_k (d_out x k);
 *   - section 2.2: per token, rho = ||r|| / ||x||; rho < eps takes the fast
 *     path y = M g (reads the image, not W), rho >= eps the full product
 *     y = W x; Theorem 4 bounds the fast path's error by ||W||_2 eps ||x||.
 * A token with x = 0 has rho = 0 (fast path; y = 0 either way).
 *
 * Conventions (as in ffn_sparse.h): device pointers allocated by the caller,
 * 16-byte aligned; row-major bf16 (raw 16-bit patterns) for W [d_out x d_in],
 * V_k [d_in x k], x [m x d_in] and y [m x d_out]; fp32 accumulation; every call
 * is asynchronous on `stream` (a hipStream_t, NULL = the null stream), checks
 * its arguments before launching anything and writes nothing on an error; the
 * library never allocates device memory; calls on one handle are serialised
 * on one stream. FFN_E_HIP reports a failed launch; the handle then refuses
 * further calls.
 */
#ifndef FFN_GSI_H
#define FFN_GSI_H

#include <stddef.h>
#include <stdint.h>

#include "ffn_sparse.h"

#ifdef __cplusplus
extern "C" {
#endif

#define FFN_GSI_ABI_VERSION 1

typedef struct {
  int32_t d_in;    /* input width d: multiple of 8, 8..16384                      */
  int32_t d_out;   /* output width: 1..4194304                                    */
  int32_t k;       /* subspace rank: multiple of 8, 8..512, k <= d_in             */
  int32_t max_m;   /* largest token count a call may pass (>= 1)                  */
} ffn_gsi_config;

typedef struct ffn_gsi_handle ffn_gsi_handle;

/* Kernel kinds of the per-kernel timing. */
typedef enum {
  FFN_GSI_K_PROJ = 0,   /* g = V_k^T x                                      */
  FFN_GSI_K_RESID = 1,  /* ||x - V_k g||^2 and ||x||^2, per-workgroup parts  */
  FFN_GSI_K_OUT = 2,    /* per-token gate, then y = M g or y = W x           */
  FFN_GSI_K_DENSE = 3,  /* y = W x for every token (ffn_gsi_dense_forward)   */
  FFN_GSI_K_COUNT = 4
} ffn_gsi_kernel_kind;

/* FFN_OK, FFN_E_INVALID (field out of range) or FFN_E_UNSUPPORTED; no GPU work. */
ffn_status ffn_gsi_check_config(const ffn_gsi_config *cfg);

/* Device workspace bytes of a handle (0 for an invalid config): the transposed
 * basis V_k^T (k x d_in bf16), the image M (d_out x k bf16), the projections of
 * 16 tokens, per-workgroup norm parts and a counter. */
size_t ffn_gsi_workspace_bytes(const ffn_gsi_config *cfg);

/* Create a handle. w [d_out x d_in] and vk [d_in x k] are borrowed (not
 * copied) and must outlive the handle. Launches, on `stream`, the transpose of
 * V_k and the image M = W V_k (fp32 accumulation over d_in in index order,
 * rounded to bf16 to nearest even) into the workspace: the cached image of
 * section 2.1. The basis is used as given (r = x - V_k V_k^T x holds by
 * definition even when rounding leaves V_k only nearly orthonormal). */
ffn_status ffn_gsi_init(const ffn_gsi_config *cfg, const void *w, const void *vk, void *workspace,
                        size_t workspace_bytes, void *stream, ffn_gsi_handle **out);

/* Gated forward pass of m tokens (0 <= m <= max_m), section 2.2:
 *   x          [m x d_in] bf16
 *   eps        threshold (not NaN); eps <= 0 sends every token to the full product
 *   y          [m x d_out] bf16, written in full
 *   rho        NULL or [m] fp32: each token's ||r|| / ||x|| (fp32 evaluation)
 *   slow_list  NULL or [m] int32: the tokens with rho >= eps, ascending
 *   n_slow     NULL or one int32: their number
 * Tokens are taken 16 at a time (three kernels per group). */
ffn_status ffn_gsi_forward(ffn_gsi_handle *h, const void *x, int32_t m, float eps, void *y, float *rho,
                           int32_t *slow_list, int32_t *n_slow, void *stream);

/* y = W x for every token (the comparison baseline: every byte of W read once
 * per call). Arguments as for ffn_gsi_forward. */
ffn_status ffn_gsi_dense_forward(ffn_gsi_handle *h, const void *x, int32_t m, void *y, void *stream);

/* Device address of the cached image M [d_out x k] bf16 inside the workspace
 * (NULL for a NULL handle). Valid once the init's launches have completed. */
const void *ffn_gsi_image(const ffn_gsi_handle *h);

/* Per-kernel timing with HIP events on the launch stream, as in
 * ffn_sparse_timing_enable / ffn_sparse_timing_read, for the kinds of
 * ffn_gsi_kernel_kind. */
ffn_status ffn_gsi_timing_enable(ffn_gsi_handle *h, int32_t enable, int32_t capacity);
ffn_status ffn_gsi_timing_read(ffn_gsi_handle *h, int32_t kind, int32_t *launches, double *total_ms);

/* Release the handle's host memory and events (the workspace stays the caller's). */
void ffn_gsi_destroy(ffn_gsi_handle *h);

#ifdef __cplusplus
}
#endif

#endif /* FFN_GSI_H */
