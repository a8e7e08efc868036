/*
 * ffn_sparse.h -- C ABI of the activation-sparse gated FFN library (MI355X / gfx950).
 *
 * The block computed is y = W_down (a(z) * (W_up x)), z = G(x) + b, where G is
 * the gate projection (full rank, W_gate x, or low rank, U (V x)), a(.) is the
 * gate activation and only the neurons the selection rule keeps take part.
 *   - Gated FFN order, per-token unstructured sparsity, low-rank gate with rank
 *     ratio 1/8: LoPA page ("Meta FAIR and Inria's LoPA Gating Hits 3.31x Real
 *     GPU Speedup for LLM Inference"), section "How LoPA Gating Restructures FFN
 *     Computation".
 *   - ReLU sparsity, tile-wise ELLPACK (TwELL) written by the gate epilogue, one
 *     pass for the up and down products, dense backup for busy tokens:
 *     Sparser/Faster/Lighter page (news.neo-ai.one article 2802 on "Sparser,
 *     Faster, Lighter Transformer Language Models"), sections "稀疏不等於提速",
 *     "TwELL 減掉轉換開銷" and "Hybrid 應對非均勻稀疏".
 *   - WINA score |h_i| * ||W_down[:, i]||_2 with top-k: WINA page
 *     ("大语言模型推理加速新突破：解读WINA框架的核心原理与实践价值"), section 3.1.
 *
 * Conventions for every entry point
 *   - Pointers named w_*, x, y, pack fields, workspace and the debug outputs are
 *     DEVICE pointers allocated by the caller; the library never allocates or
 *     frees device memory and never synchronises the stream.
 *   - Matrices are row-major and dense: W_gate, W_up [d_ff x d_model];
 *     U [d_ff x rank]; V [rank x d_model]; W_down [d_model x d_ff] (output-major)
 *     or, with wdown_out_major = 0, its transpose [d_ff x d_model] (neuron-major);
 *     x, y [m x d_model]. Element type: fp32 or bf16 (raw 16-bit patterns) per
 *     config.dtype; accumulation is fp32.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream). Arguments are validated before anything is launched; on an error
 *     nothing is written. FFN_E_HIP reports a failed launch (or, through
 *     ffn_sparse_device_status, a wait that gave up), after which the handle
 *     refuses further calls until it is re-initialised.
 *   - A handle owns host memory only and is bound to the workspace it was
 *     initialised with; calls on one handle must be serialised on one stream.
 *   - Required alignment: 16 bytes for every device pointer.
 */
#ifndef FFN_SPARSE_H
#define FFN_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FFN_SPARSE_ABI_VERSION 3

typedef enum {
  FFN_OK = 0,
  FFN_E_INVALID = -1,      /* bad argument: null, misaligned, out of range      */
  FFN_E_UNSUPPORTED = -2,  /* valid but not built: shape / mode combination      */
  FFN_E_WORKSPACE = -3,    /* workspace smaller than ffn_sparse_workspace_bytes  */
  FFN_E_HIP = -4           /* a HIP launch failed                                */
} ffn_status;

typedef enum { FFN_F32 = 0, FFN_BF16 = 1 } ffn_dtype;
typedef enum { FFN_RELU = 0, FFN_SILU = 1 } ffn_act;

/* Selection rule.
 *   BIAS:   active <=> z > 0 (ReLU gate); value a = z.
 *   THRESH: active <=> z > max(tau_t, 0) (ReLU gate); value a = z (passes through).
 *   TOPK_WINA: h = a(z) * (W_up x) for every neuron, score s_i = |h_i| * c_i with
 *           c_i = ||W_down[:, i]||_2; the k largest scores per token are kept,
 *           ties to the lower index; pack values are h_i. Requires ell_w == tile_w. */
typedef enum { FFN_SEL_BIAS = 0, FFN_SEL_THRESH = 1, FFN_SEL_TOPK_WINA = 2 } ffn_select;

typedef struct {
  int32_t d_model;          /* multiple of 64, 64..4096                               */
  int32_t d_ff;             /* multiple of tile_w                                      */
  int32_t rank;             /* 0: full gate W_gate; > 0 (multiple of 32): U, V factors */
  int32_t dtype;            /* ffn_dtype                                               */
  int32_t act;              /* ffn_act (BIAS/THRESH need RELU)                         */
  int32_t sel;              /* ffn_select                                              */
  int32_t tile_w;           /* TwELL tile width T: multiple of 16, 16..1024             */
  int32_t ell_w;            /* TwELL ELL width E: 0 <= E <= T                          */
  int32_t wdown_out_major;  /* 1: w_down is [d_model x d_ff]; 0: [d_ff x d_model]      */
  int32_t max_m;            /* largest token count a call may pass (>= 1)              */
  int32_t in_keep;          /* 0: the gate reads every input channel; 1..d_model: per  */
                            /* token it keeps the in_keep channels j with the largest  */
                            /* |x_j| * ||W[:, j]||_2 (W = W_gate, or V for a low-rank  */
                            /* gate; ties to the lower index) and reads only their     */
                            /* weights (WINA page, section 3.1, applied to the gate's  */
                            /* input). bf16, bias / threshold selection, ell_w ==      */
                            /* tile_w and max_m <= 64 only.                            */
} ffn_sparse_config;

/* TwELL pack (tile-wise ELLPACK) of the selected activations, token-major.
 * With NT = d_ff / tile_w tiles per token:
 *   cnt        int32  [m x NT]      true number of active neurons in tile j
 *   idx        uint16 [m x NT x E]  first min(cnt, E) active local offsets
 *                                   (0..T-1), ascending; padding 0xFFFF
 *   val        [m x NT x E]         their values a_i (h_i for TOPK): bf16 bits for
 *                                   bf16 configs, fp32 for fp32; padding 0
 *   route      uint8  [m]           1 when some tile of the token has cnt > E
 *   dense_list int32  [m]           routed token ids, ascending (first n_dense valid)
 *   n_dense    int32  [1]           number of routed tokens
 * All device pointers, caller-owned. */
typedef struct {
  int32_t *cnt;
  uint16_t *idx;
  void *val;
  uint8_t *route;
  int32_t *dense_list;
  int32_t *n_dense;
} ffn_twell_pack;

typedef struct ffn_sparse_handle ffn_sparse_handle;

/* ABI version compiled into the library (FFN_SPARSE_ABI_VERSION). */
int32_t ffn_sparse_abi_version(void);

/* Human-readable name of a status code (static string). */
const char *ffn_sparse_status_string(ffn_status s);

/* Validate a config without touching the GPU: FFN_OK, FFN_E_INVALID or
 * FFN_E_UNSUPPORTED. */
ffn_status ffn_sparse_check_config(const ffn_sparse_config *cfg);

/* Bytes of device workspace a handle needs for this config (0 if the config
 * is not valid). The workspace holds the neuron-major (or output-major) copy of
 * W_down, WINA column norms, the low-rank intermediate, the sparse-path
 * schedule, partial sums and counters. */
size_t ffn_sparse_workspace_bytes(const ffn_sparse_config *cfg);

/* Bytes of the six pack fields for m tokens, each field rounded up to 256 bytes,
 * in the order cnt, idx, val, route, dense_list, n_dense (0 if invalid). */
size_t ffn_sparse_pack_bytes(const ffn_sparse_config *cfg, int32_t m);

/* Create a handle. w_gate_or_u is W_gate (rank 0) or U (rank > 0); v_or_null is
 * V (rank > 0) or NULL. The weights are borrowed (not copied) and must outlive
 * the handle. Launches, on `stream`, the W_down transpose into the workspace,
 * the WINA column-norm pass (TOPK configs) and the counter reset.
 * Column norms: WINA page, section 3.1. */
ffn_status ffn_sparse_init(const ffn_sparse_config *cfg, const void *w_gate_or_u,
                           const void *v_or_null, const void *w_up, const void *w_down,
                           void *workspace, size_t workspace_bytes, void *stream,
                           ffn_sparse_handle **out);

/* Gate projection + activation + selection, writing the TwELL pack directly
 * from the gate kernel's epilogue (no separate conversion pass), then routing
 * (route / dense_list / n_dense).
 *   x          [m x d_model] device
 *   bias       [m] fp32 device per-token gate bias, or NULL to use bias_scalar
 *   tau        [m] fp32 device thresholds (THRESH only), else NULL
 *   k          kept neurons per token (TOPK only), 0 <= k <= d_ff
 *   g_debug    NULL, or [m x d_ff] fp32 device: the gate projection G(x) before bias
 *   s_debug    NULL, or [m x d_ff] fp32 device: WINA scores (TOPK only)
 * Source: Sparser/Faster/Lighter page, "TwELL 減掉轉換開銷" (pack emitted in the
 * gate epilogue); "Hybrid 應對非均勻稀疏" (routing). 0 <= m <= max_m. */
ffn_status ffn_sparse_gate_pack(ffn_sparse_handle *h, const void *x, int32_t m,
                                const float *bias, float bias_scalar, const float *tau,
                                int32_t k, ffn_twell_pack *pack, float *g_debug,
                                float *s_debug, void *stream);

/* Fused sparse up + down over the pack for every non-routed token: for each
 * packed neuron i, u_i = <W_up[i,:], x>, h_i = val_i * u_i (TOPK: h_i = val_i,
 * no up product), y += h_i * W_down[:, i]; h stays in registers. Writes y rows
 * of non-routed tokens (zero rows for tokens with no active neuron); routed
 * rows are left untouched. Requires the pack written by ffn_sparse_gate_pack on
 * this handle for the same x and m.
 * Source: Sparser/Faster/Lighter page, "TwELL 減掉轉換開銷" (single pass over up
 * and down without storing h). */
ffn_status ffn_sparse_updown(ffn_sparse_handle *h, const void *x, int32_t m,
                             const ffn_twell_pack *pack, void *y, void *stream);

/* Dense backup for the routed tokens (dense_list[0..n_dense)): recomputes the
 * gate for those tokens and evaluates the same function densely on matrix
 * cores, writing their y rows. Same selection arguments as gate_pack.
 * Source: Sparser/Faster/Lighter page, "Hybrid 應對非均勻稀疏". */
ffn_status ffn_sparse_dense_fallback(ffn_sparse_handle *h, const void *x, int32_t m,
                                     const float *bias, float bias_scalar, const float *tau,
                                     int32_t k, const ffn_twell_pack *pack, void *y,
                                     void *stream);

/* gate_pack + updown + dense_fallback: the whole sparse forward pass; writes
 * every y row and the complete pack. For m <= 64 the routed tokens are
 * evaluated by the sparse kernel itself (each overflowing tile densely, gate
 * recomputed); for larger m they go through the dense backup on matrix cores.
 * Routing is done inside the sparse kernel (no separate pass).
 * Source: LoPA page, "How LoPA Gating Restructures FFN Computation" (gate
 * projection, activation, elementwise product, down projection, with only the
 * active neurons' rows read); Sparser/Faster/Lighter page, "TwELL
 * 減掉轉換開銷" and "Hybrid 應對非均勻稀疏" (pack, fused up/down, dense
 * backup; both paths give the same y); WINA page, section 3.1 (top-k score).
 * Arguments as for gate_pack; y [m x d_model] device, written in full. */
ffn_status ffn_sparse_forward(ffn_sparse_handle *h, const void *x, int32_t m,
                              const float *bias, float bias_scalar, const float *tau,
                              int32_t k, ffn_twell_pack *pack, void *y, void *stream);

/* The same function evaluated densely over every neuron (the comparison
 * baseline): bias / threshold gates keep their elementwise mask; a TOPK config
 * keeps every neuron (k = d_ff). Every weight byte is streamed once per call
 * through dense matrix products (GEMV / MFMA tiles), the "dense GPU matrix
 * operations" the sparse path is measured against (LoPA page, "How LoPA
 * Gating Restructures FFN Computation"). Arguments as for forward, without
 * k and the pack. */
ffn_status ffn_sparse_dense_forward(ffn_sparse_handle *h, const void *x, int32_t m,
                                    const float *bias, float bias_scalar, const float *tau,
                                    void *y, void *stream);

/* Bytes of the caller workspace ffn_sparse_backward needs for m tokens (0 if
 * the config has no backward pass here: it is defined for a full-rank ReLU
 * gate with bias or threshold selection, d_model <= 4096, in_keep = 0,
 * (d_ff / tile_w) * ell_w <= 8192 and, when tokens can be routed
 * (ell_w < tile_w), d_ff <= 8192). */
size_t ffn_sparse_backward_workspace_bytes(const ffn_sparse_config *cfg, int32_t m);

/* Backward pass of ffn_sparse_forward with its selection held fixed: the
 * gradients of L = sum_t <dy_t, y_t>. With a = z on the active entries,
 * u = W_up x, h = a u and dh = W_down^T dy:
 *   du = dh a, dz = dh u (active entries only),
 *   dW_down[:, i] += sum_t h_ti dy_t, dW_up[i, :] += sum_t du_ti x_t,
 *   dW_gate[i, :] += sum_t dz_ti x_t, dx_t = sum_i du_ti W_up[i, :] + dz_ti W_gate[i, :].
 * Source: Sparser/Faster/Lighter page, "Hybrid 應對非均勻稀疏" (training with
 * the compact format for most tokens and a dense backup for busy ones): the
 * compact tokens' activations come from `pack` (the forward pass's TwELL
 * pack, values a as stored: bf16 in bf16 configs), a routed token's gate row
 * is recomputed densely on matrix cores and its active neurons read from it.
 *   x, m, bias, bias_scalar, tau, pack: as passed to (and written by) the
 *               forward call on this handle
 *   dy          [m x d_model] device, config dtype
 *   dx          NULL or [m x d_model] device, config dtype: written
 *   dw_gate, dw_up  NULL or [d_ff x d_model] fp32 device: ADDED TO; only the
 *               rows of neurons active for some token change
 *   dw_down_nm  NULL or [d_ff x d_model] fp32 device: the gradient of W_down
 *               in neuron-major layout (row i = dW_down[:, i]), added to
 *   workspace   >= ffn_sparse_backward_workspace_bytes(cfg, m), 16-byte aligned;
 *               from 512 tokens in bf16 it also holds [W_up; W_gate]
 *               transposed (d_model x 2 d_ff) and the dense (du | dz) rows
 *               (m x 2 d_ff), both bf16, for dx as one matrix-core GEMM
 *               (du and dz rounded to bf16 there)
 * Every sum runs in a fixed order (tokens ascending per neuron), so the
 * result is reproducible run to run. FFN_E_UNSUPPORTED for other configs. */
ffn_status ffn_sparse_backward(ffn_sparse_handle *h, const void *x, int32_t m, const float *bias,
                               float bias_scalar, const float *tau, const ffn_twell_pack *pack,
                               const void *dy, void *dx, float *dw_gate, float *dw_up, float *dw_down_nm,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the caller workspace ffn_sparse_moe_forward needs for m tokens
 * routed to topk experts each (0 if invalid; m * topk <= 256). */
size_t ffn_sparse_moe_workspace_bytes(const ffn_sparse_config *cfg, int32_t m, int32_t topk);

/* Mixture-of-experts layer whose experts are sparse FFNs of one shape:
 * y_t = sum over t's routing slots s of weights[t, s] * FFN_{e(t, s)}(x_t).
 * Source: LoPA page, "Model Casting and Quality at 90% Sparsity" (the gating
 * carries over to mixture-of-experts layers whose experts are FFN blocks);
 * the weighted sum is the usual combination of a routed layer.
 *   experts     n_experts handles (host array), all of one config except max_m
 *   x           [m x d_model] device
 *   expert_ids  HOST [m x topk]: the experts of each token, distinct per token
 *               (the router has already run)
 *   weights     HOST [m x topk] combine weights (finite)
 *   bias, tau   NULL or DEVICE [m x topk]: the selection inputs of each
 *               (token, slot) pair (tau required for THRESH), as for forward
 *   k           kept neurons per (token, expert) for TOPK configs
 *   dense       0: the experts' sparse forward passes; 1: their dense forward
 *               passes (ffn_sparse_dense_forward, the comparison baseline)
 *   workspace   DEVICE, 16-byte aligned, >= ffn_sparse_moe_workspace_bytes
 *   y           [m x d_model] device, written in full
 * One gather kernel builds the experts' contiguous token blocks, each expert
 * with tokens runs its forward sequence on its block (expert
 * order; each expert's max_m must cover its token count), one kernel adds the
 * weighted outputs per token in slot order (fp32) and rounds once.
 * 1 <= topk <= n_experts; 0 <= m with m * topk <= 256. */
ffn_status ffn_sparse_moe_forward(ffn_sparse_handle *const *experts, int32_t n_experts, const void *x,
                                  int32_t m, int32_t topk, const int32_t *expert_ids, const float *weights,
                                  const float *bias, float bias_scalar, const float *tau, int32_t k,
                                  int32_t dense, void *workspace, size_t workspace_bytes, void *y,
                                  void *stream);

/* Which kernel sequence ffn_sparse_forward runs for m tokens (host-only
 * query, no GPU work). The decode sequences (bf16, bias / threshold
 * selection, 1 <= m <= 16; modes 1 and 2 up to 8 tokens) run the low-rank
 * first stage (rank > 0) and the gate kernel (selection + TwELL pack), then:
 *   1 = column chunks: the gate kernel computes h of its active neurons, one
 *       workgroup per 16-byte column chunk of y sums h * W_down rows;
 *   2 = partial rows: the gate kernel also sums its active neurons' down rows
 *       into a partial y row, a second kernel adds the partial rows;
 *   3 = split: an up kernel deals the union of the tokens' active neurons
 *       evenly over the chip and writes a compact (neuron, h) list, a down
 *       kernel contracts it in column slices (both on matrix cores).
 * WINA top-k selection (bf16) runs the gate + up GEMM with the score epilogue
 * and the top-k kernel, then:
 *   4 = one token: the top-k kernel also writes its kept neurons as a
 *       compact (neuron, h) list, which the split sequence's down kernel
 *       contracts;
 *   5 = several tokens (or a shape the list kernel does not take): the top-k
 *       kernel writes h rows with the other neurons zeroed, and a dense down
 *       GEMM multiplies them (the union of the tokens' kept sets covers most of
 *       W_down).
 * 6 = input-side gate selection (config in_keep > 0): the kept input
 *     channels per token, the gate from their rows of the input-major W_gate
 *     (or V) in channel groups, the selection and pack (or, low rank, t and
 *     then U t), the sparse up + down over the pack;
 * 7 = masked dense (bf16 bias / threshold selection, 17..127 tokens, or up
 *     to 256 when the pack has more than 64 TwELL tiles or 1024 slots a
 *     token, which the prefill sequence's XCD-sliced kernels cannot hold): the
 *     dense gate and up products with the selection applied to every neuron
 *     (the gate values kept), the TwELL pack built from those gate values,
 *     then a dense down GEMM; past 16 tokens the union of the tokens' active
 *     neurons covers most rows, so no sparse pass reads fewer weight bytes;
 * 0 = the general sequence (gate, sparse up + down over the TwELL pack,
 * partial-row sum, dense backup); -1 = invalid handle or m. */
int32_t ffn_sparse_forward_path(const ffn_sparse_handle *h, int32_t m);

/* Per-kernel timing with HIP events recorded on the launch stream around each
 * kernel. enable = 1 starts recording (up to `capacity` launches per kernel
 * kind), 0 stops. ffn_sparse_timing_read synchronises on the recorded events
 * and returns, for kernel kind `kind` (see ffn_kernel_kind), the number of
 * launches and their total milliseconds, then clears that kind. */
typedef enum {
  FFN_K_GATE = 0,      /* gate GEMM + selection epilogue (+ TwELL pack)        */
  FFN_K_LOWRANK_V = 1, /* low-rank gate first stage t = V x                    */
  FFN_K_TOPK = 2,      /* WINA top-k selection + pack                          */
  FFN_K_UPDOWN = 3,    /* fused sparse up + down                               */
  FFN_K_REDUCE = 4,    /* cross-workgroup sum of partial y rows                */
  FFN_K_FALLBACK = 5,  /* dense backup kernels                                 */
  FFN_K_DENSE = 6,     /* dense baseline kernels                               */
  FFN_K_ROUTE = 7,     /* routing pass of a standalone gate_pack               */
  FFN_K_UP = 8,        /* decode: up products of the union neurons (split mode) */
  FFN_K_BW_GATE = 9,   /* backward: the routed tokens' gate rows recomputed    */
  FFN_K_BW_NEURON = 10,/* backward: per-neuron du, dz and weight gradients     */
  FFN_K_BW_DX = 11,    /* backward: per-token input gradient                   */
  FFN_K_COUNT = 12
} ffn_kernel_kind;
ffn_status ffn_sparse_timing_enable(ffn_sparse_handle *h, int32_t enable, int32_t capacity);
ffn_status ffn_sparse_timing_read(ffn_sparse_handle *h, int32_t kind, int32_t *launches,
                                  double *total_ms);

/* ffn_sparse_forward for callers that cannot allocate device memory or
 * synchronise inside the call (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Same arguments, same results (the
 * same kernels on the same inputs, bit for bit), same conventions; the
 * per-call scratch (control and look-back words, low-rank intermediate,
 * sub-tile masks, hidden values, partial y rows, the compact list) comes from
 * a fixed device array that the library holds on each GPU it runs on, of
 * ffn_sparse_noalloc_scratch_bytes() bytes, instead of from the handle's
 * workspace; the handle's workspace still holds what ffn_sparse_init
 * precomputed (the other W_down layout). The call allocates and frees
 * nothing and never synchronises the stream. It covers the decode sequences
 * (bf16, bias / threshold selection, 1..16 tokens as ffn_sparse_forward_path
 * reports 1, 2 or 3) with d_ff <= 32768; other configs or token counts return
 * FFN_E_UNSUPPORTED, and a call whose scratch would exceed the array returns
 * FFN_E_WORKSPACE, both before anything is launched. The array is set up by
 * ffn_sparse_init on the current device (or by the first call on a device,
 * which then synchronises `stream` once). Every no-allocation call on one GPU
 * shares the array, which keeps the last call's contents (nothing in it needs
 * clearing between calls): calls that overlap on one GPU, on different
 * streams or from different handles, race and must not be issued. */
ffn_status ffn_sparse_forward_noalloc(ffn_sparse_handle *h, const void *x, int32_t m,
                                      const float *bias, float bias_scalar, const float *tau,
                                      int32_t k, ffn_twell_pack *pack, void *y, void *stream);

/* Size in bytes of the per-GPU scratch array of ffn_sparse_forward_noalloc. */
size_t ffn_sparse_noalloc_scratch_bytes(void);

/* Error state of the work enqueued so far on `stream` (synchronises it).
 * The kernels' cross-workgroup waits (the TwELL look-back of sub-tiled gate
 * tiles) are bounded: a wait that gives up lets its kernel finish and raises
 * an error word in the workspace. Returns FFN_OK, or FFN_E_HIP when a launch
 * failed earlier or a wait gave up; the handle is then marked failed and every
 * later call returns FFN_E_HIP until it is re-initialised with
 * ffn_sparse_init (which clears the error word). A wait that gave up in a
 * no-allocation call on this device is reported too. FFN_E_INVALID for a
 * null handle. */
ffn_status ffn_sparse_device_status(ffn_sparse_handle *h, void *stream);

/* Test hook for the give-up path of the bounded waits: from the next call on,
 * a wait expects the pass epoch plus `epoch_skew` (0 in normal use, where the
 * handle starts) and gives up after `spin_limit` polls (the default allows
 * about a second). A nonzero skew makes every wait give up after its polls,
 * so each kernel still exits and ffn_sparse_device_status then reports
 * FFN_E_HIP. Enqueued on `stream`. */
ffn_status ffn_sparse_debug_waits(ffn_sparse_handle *h, uint32_t epoch_skew, uint32_t spin_limit,
                                  void *stream);

/* Free the host-side handle (device memory belongs to the caller). */
void ffn_sparse_destroy(ffn_sparse_handle *h);

#ifdef __cplusplus
}
#endif
#endif /* FFN_SPARSE_H */
