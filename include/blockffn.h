/*
 * blockffn.h: C ABI of the MI355X (gfx950) BlockFFN layer forward.
 *
 * The layer (BlockFFN, arXiv 2507.08771; skill page "BlockFFN: Sparse
 * Mixture-of-Experts Optimized for End-Device Deployment", sections "Core Concept"
 * and "Architecture Overview"; paper-card Abstract) has two parts:
 *
 *   router      s[t,:] = RMSNorm_E( ReLU( W_r x_t ) ) * g          (no router bias)
 *   chunk FFN   y_t = sum over e in U_c(t) of s[t,e] * W2_e swish(W1_e x_t)
 *
 * where U_c is the union of the experts active (s != 0) in any token of the
 * n-token chunk c that holds t. Experts of the union that are inactive for a token
 * are computed and then masked by that token's zero score; experts outside the
 * union are never read.
 *
 * Conventions shared by every call:
 *  - All array pointers are DEVICE pointers (hipMalloc / torch CUDA memory) owned by
 *    the caller. The library never allocates or frees device or pinned memory and
 *    retains no caller pointer. It holds small static device arrays of its own (one
 *    copy per device, for the life of the process) and, per device, the result of a
 *    one-time probe of workgroup placement: blockffn_init() runs that probe
 *    explicitly; otherwise the first call on a device runs it on the caller's stream
 *    and synchronises that stream (skipped while the stream is being captured into a
 *    graph: such calls then take the schedules that need no placement facts, and a
 *    later call probes).
 *  - Arrays are dense, row-major, C-contiguous. Weights use the nn.Linear layout
 *    [out_features, in_features], stacked over experts.
 *  - `dtype` selects the element type of x, W_r, W1, W2 and y: BLOCKFFN_F32 (float)
 *    or BLOCKFFN_BF16 (bfloat16 bits, products accumulated in fp32). Scores, gain,
 *    bias and logits are always float.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls enqueue their
 *    kernels and return; BLOCKFFN_OK means "validated and enqueued". Faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Every argument is validated on the host before anything is enqueued; an
 *    invalid call writes nothing and returns a non-zero status, and
 *    blockffn_last_error() returns a message for the calling thread.
 *  - Supported sizes: 1 <= E <= 256; T, d_h, d_e, n >= 1. bf16 additionally needs
 *    d_h % 32 == 0, d_e % 16 == 0 and 16-byte aligned x, W_r, W1, W2, y; every
 *    pointer needs the alignment of its element type; the workspace 256 bytes.
 */
#ifndef BLOCKFFN_H
#define BLOCKFFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BLOCKFFN_OK = 0,
    BLOCKFFN_EINVAL = 1,        /* NULL required pointer, size <= 0, unknown dtype   */
    BLOCKFFN_EUNSUPPORTED = 2,  /* valid but outside the supported sizes/alignment   */
    BLOCKFFN_EWORKSPACE = 3,    /* workspace smaller than the query call returned    */
    BLOCKFFN_EHIP = 4,          /* the HIP runtime reported an error                 */
    BLOCKFFN_ETIMEOUT = 5       /* blockffn_workspace_check: a kernel's wait timed out */
} blockffn_status_t;

typedef enum { BLOCKFFN_F32 = 0, BLOCKFFN_BF16 = 1 } blockffn_dtype_t;

/*
 * Router (skill page, "Architecture Overview" and "Router Architecture Setup";
 * paper-card Abstract: a router integrating ReLU and RMSNorm):
 *   l[t,e] = sum_j x[t,j] W_r[e,j] (+ bias[e])
 *   s[t,e] = max(l[t,e], 0) / sqrt(mean_e max(l[t,e],0)^2 + eps) * gain[e]
 * The pages' router has no bias; `bias` is an optional per-expert logit shift for
 * callers that need one (NULL = none).
 *
 *   x       [T, d_h]  dtype         tokens
 *   w_r     [E, d_h]  dtype         router weight (nn.Linear(d_h, E) layout)
 *   gain    [E] float or NULL (=1)  RMSNorm weight
 *   bias    [E] float or NULL (=0)
 *   eps     RMSNorm epsilon (torch's default for fp32 is 1.1920929e-07)
 *   scores  [T, E] float, written   post-RMSNorm scores (exactly 0 when inactive)
 *   logits  [T, E] float or NULL    pre-ReLU logits, written when given
 *   sharpness, probs                activation probabilities (skill page, "Router
 *           Architecture Setup": the router also returns the sigmoid of the
 *           sharpened scores, which the training losses take):
 *           probs [T, E] float or NULL, written when given with
 *           probs[t,e] = 1 / (1 + exp(-sharpness * s[t,e])); sharpness must be
 *           finite (the pages' default is 1). An inactive expert gets exactly 0.5.
 *   workspace, workspace_bytes      optional device scratch (NULL, 0 = none). With a
 *           workspace of at least blockffn_router_workspace_bytes(...) bytes,
 *           ZERO-FILLED before its first use, a bf16 call with few tokens splits the
 *           d_h sum over several workgroups (fixed summation order, so results do
 *           not depend on timing). The workspace holds arrival counters that every
 *           call returns to zero; calls that may run concurrently need separate
 *           workspaces. Without one the call uses one workgroup per 32 tokens.
 * ReLU maps every logit that is not > 0 (NaN included) to 0. A row with no positive
 * logit gets all-zero scores.
 */
blockffn_status_t blockffn_router(const void *x, const void *w_r, const float *gain,
                                  const float *bias, float eps, int64_t T, int64_t d_h,
                                  int64_t E, int dtype, float *scores, float *logits,
                                  float sharpness, float *probs, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Bytes of router workspace for these sizes (>= 256; 0 when the sizes are invalid,
 * see blockffn_last_error()).
 */
size_t blockffn_router_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int dtype);

/*
 * Bytes of device workspace blockffn_chunk_ffn needs for these sizes (0 when the
 * sizes are invalid; see blockffn_last_error()).
 */
size_t blockffn_chunk_ffn_workspace_bytes(int64_t T, int64_t d_h, int64_t E,
                                          int64_t d_e, int64_t n, int dtype);

/*
 * Chunked expert FFN (skill page, "Core Concept": compute only the union of experts
 * activated across n tokens and mask unneeded activations after the computation;
 * "Architecture Overview": non-gated Swish experts, n = 32 tokens in the pages'
 * kernel). Chunk c holds tokens [c*n, min(c*n + n, T)); the last chunk may be
 * partial (skill page, "Chunk Sparsification Loss": ceil(T/n) aligned chunks).
 *
 *   x        [T, d_h]       dtype   tokens
 *   scores   [T, E]         float   router scores; expert e is active for token t
 *                                   exactly when scores[t,e] != 0 (-0 is inactive)
 *   w1       [E, d_e, d_h]  dtype   fc1 weights (nn.Linear(d_h, d_e) per expert)
 *   w2       [E, d_h, d_e]  dtype   fc2 weights (nn.Linear(d_e, d_h) per expert)
 *   n        chunk length in tokens (n >= T means one chunk)
 *   y        [T, d_h]       dtype   OVERWRITTEN with
 *                   y[t,:] = sum_{e in U_c(t)} s[t,e] * W2_e swish(W1_e x[t,:])
 *                   (swish(a) = a / (1 + exp(-a))). bf16: fp32 accumulation, the
 *                   score-scaled hidden activations are rounded to bf16 before the
 *                   second product and y is rounded to bf16 (nearest even).
 *   workspace, workspace_bytes: device scratch of at least
 *                   blockffn_chunk_ffn_workspace_bytes(...) bytes, ZERO-FILLED before
 *                   its first use (e.g. hipMemset or torch.zeros). Its first 64 KB
 *                   are a control block: arrival counters that every call returns to
 *                   zero, per-workgroup epoch flags that count the calls made with
 *                   the workspace, and a status word; a zero-filled workspace stays
 *                   valid across calls of any sizes. The rest of it is scratch.
 *                   Calls that may run concurrently need separate workspaces.
 *                   The single-chunk schedules (one launch whose workgroups hand work
 *                   to each other) wait on workgroups of the same launch, which must
 *                   all be resident at once (one per CU). A wait is bounded: if it
 *                   times out, the affected rows of y become NaN and the workspace's
 *                   status word is set, which blockffn_workspace_check reports. Causes:
 *                   a workspace that was not zero-filled (or was reused after such a
 *                   time-out), kernels of other streams or processes holding CUs so
 *                   that the launch's workgroups are not co-resident, or a faulty
 *                   device. After a time-out zero-fill the workspace before reusing it.
 *   union_masks_out   [C][ceil(E/64)] uint64 or NULL: bit e%64 of word e/64 set when
 *                   e is in U_c (C = ceil(T/n))
 *   expert_lists_out  [C][E] int32 or NULL: U_c in ascending expert id, then -1
 *   union_counts_out  [C] int32 or NULL: |U_c|
 * The optional outputs receive exactly the unions the FFN kernels used.
 */
blockffn_status_t blockffn_chunk_ffn(const void *x, const float *scores, const void *w1,
                                     const void *w2, int64_t T, int64_t d_h, int64_t E,
                                     int64_t d_e, int64_t n, int dtype, void *y,
                                     void *workspace, size_t workspace_bytes,
                                     uint64_t *union_masks_out, int32_t *expert_lists_out,
                                     int32_t *union_counts_out, void *stream);

/*
 * Bytes of workspace blockffn_layer_forward needs (0 when the sizes are invalid).
 */
size_t blockffn_layer_forward_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                              int64_t n, int dtype);

/*
 * The whole layer forward, router then chunked expert FFN (skill page, "Architecture
 * Overview" and "Core Concept"): y = blockffn_chunk_ffn(x, s, W1, W2, n) with
 * s = blockffn_router(x, W_r, gain, bias, eps). Arguments as in those two calls;
 * scores [T, E] float or NULL receives s. The workspace (at least
 * blockffn_layer_forward_workspace_bytes(...), 256-byte aligned) must be ZERO-FILLED
 * before its first use; its control block then stays consistent across calls (as in
 * blockffn_chunk_ffn, including the time-out behaviour and blockffn_workspace_check). For one chunk of at
 * most 32 tokens in bf16 with E <= 64 and d_h a multiple of 256 up to 2048 (and the
 * chunk FFN's single-chunk schedule available) the router runs inside the FFN launch:
 * the workgroups that share an XCD split the E logits between them (fp32 sums of bf16
 * products, the eight eighths of d_h added in order), exchange them through that
 * XCD's L2, and each applies bias, ReLU, RMSNorm and gain itself. The scores can then
 * differ from blockffn_router's in the last bits (summation order), within the
 * router's tolerance. Otherwise the call is blockffn_router followed by
 * blockffn_chunk_ffn.
 */
blockffn_status_t blockffn_layer_forward(const void *x, const void *w_r, const float *gain,
                                         const float *bias, float eps, const void *w1,
                                         const void *w2, int64_t T, int64_t d_h, int64_t E,
                                         int64_t d_e, int64_t n, int dtype, void *y, float *scores,
                                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * 1 when blockffn_layer_forward with these sizes runs router and FFN in one launch on
 * the current device (probing the device on first use), else 0.
 */
int blockffn_layer_forward_fused(int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n,
                                 int dtype, void *stream);

/*
 * Bytes of workspace blockffn_layer_forward_full needs (0 when the sizes are invalid).
 */
size_t blockffn_layer_forward_full_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                                   int64_t n, int dtype);

/*
 * The whole layer as the pages' layer module returns it (skill page, "Full BlockFFN
 * Layer with Combined Losses": the output is LayerNorm(FFN output + layer input) and the
 * router's probabilities come back with it; "Router Architecture Setup"):
 *   y     = blockffn_layer_forward(x, W_r, gain, bias, eps, W1, W2, n)
 *   out   = LayerNorm_{d_h}(y + x) * ln_gamma + ln_beta  (y as stored: bf16-rounded for
 *           bf16; biased variance; as blockffn_add_layernorm)
 *   probs = sigmoid(sharpness * scores)                  (when probs != NULL)
 * Expert weights: either w1 and w2 row-major (packed = NULL) or packed as
 * blockffn_pack_weights writes them (w1 = w2 = NULL; only for sizes where
 * blockffn_layer_forward_fused(...) is 1, else BLOCKFFN_EUNSUPPORTED).
 *
 *   ln_gamma, ln_beta  [d_h] float or NULL (= 1, 0), 16-byte aligned; ln_eps finite >= 0
 *   out     [T, d_h] dtype, written, 16-byte aligned; must not overlap x, y, scores, probs
 *   sharpness, probs   [T, E] float or NULL, as in blockffn_router
 *   y       [T, d_h] dtype or NULL: receives the FFN output when given
 *   scores  [T, E] float or NULL: receives the router's scores when given
 *   workspace, workspace_bytes: at least blockffn_layer_forward_full_workspace_bytes(...),
 *           ZERO-FILLED before its first use, as blockffn_layer_forward's
 * Where the router and FFN run in one launch (blockffn_layer_forward_fused), the residual
 * LayerNorm and the probabilities run in that launch too: the workgroup that finishes an
 * output tile adds x, computes the tile's per-token mean and squared deviations, and
 * after every tile's have been stored (a bounded device-wide wait, under the same
 * co-residency assumption and time-out reporting as the FFN's) combines them and writes
 * its columns of out. Otherwise the call is blockffn_router (with probs),
 * blockffn_chunk_ffn and blockffn_add_layernorm. d_h must be a multiple of 8 (bf16) or 4.
 */
blockffn_status_t blockffn_layer_forward_full(const void *x, const void *w_r, const float *gain,
                                              const float *bias, float eps, const void *w1,
                                              const void *w2, const void *packed, int64_t T,
                                              int64_t d_h, int64_t E, int64_t d_e, int64_t n,
                                              int dtype, const float *ln_gamma,
                                              const float *ln_beta, float ln_eps, void *out,
                                              float sharpness, float *probs, void *y,
                                              float *scores, void *workspace,
                                              size_t workspace_bytes, void *stream);

/*
 * blockffn_layer_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels and results as blockffn_layer_forward; the
 * workspace is a file-scope device array of the library, 16 MiB, one per device (held
 * until the process ends; its address is resolved by blockffn_init or by this call's
 * first use on a device). Sizes whose blockffn_layer_forward_workspace_bytes(...)
 * exceed 16 MiB are rejected with BLOCKFFN_EUNSUPPORTED before anything is enqueued
 * (the decode chunk, d_h=2048 E=64 d_e=128 T=32 bf16, needs 8.7 MiB). Allocates and
 * frees nothing. Each call first enqueues a one-workgroup kernel that zero-fills the
 * array's control block if an earlier call's bounded wait timed out. Every call on a
 * device shares that device's array: calls that may overlap on one device (other
 * streams, other threads) race and must not be issued.
 */
blockffn_status_t blockffn_layer_forward_noalloc(const void *x, const void *w_r, const float *gain,
                                                 const float *bias, float eps, const void *w1,
                                                 const void *w2, int64_t T, int64_t d_h, int64_t E,
                                                 int64_t d_e, int64_t n, int dtype, void *y,
                                                 float *scores, void *stream);

/*
 * Bytes of a packed copy of the expert weights (2*E*d_h*d_e bf16 elements), or 0 when
 * the sizes or dtype are not supported (bf16 only; 1 <= E <= 256; d_h and d_e positive
 * multiples of 32; E*d_h*d_e <= 2^30).
 */
size_t blockffn_pack_weights_bytes(int64_t E, int64_t d_h, int64_t d_e, int dtype);

/*
 * Rewrites W1 [E, d_e, d_h] and W2 [E, d_h, d_e] (bf16, row-major, the experts of the
 * skill page's "Architecture Overview") into packed (caller-owned device memory of
 * blockffn_pack_weights_bytes(...) bytes, 16-byte aligned): W1's tiles, then W2's.
 * Every matrix is cut into tiles of 16 rows x 32 columns (1 KB), stored in row-major
 * tile order, each tile row-major. The values are copied exactly. This is a one-time
 * layout change for weights that stay resident: it lets the one-launch layer read each
 * 16 x 32 operand fragment as one contiguous access. Asynchronous on stream;
 * BLOCKFFN_EINVAL for unsupported sizes or NULL pointers.
 */
blockffn_status_t blockffn_pack_weights(const void *w1, const void *w2, int64_t E, int64_t d_h,
                                        int64_t d_e, int dtype, void *packed, void *stream);

/*
 * blockffn_layer_forward with the expert weights given as blockffn_pack_weights wrote
 * them (same values, same result bits as the call with row-major W1 and W2). Only for
 * sizes where blockffn_layer_forward_fused(...) is 1; otherwise BLOCKFFN_EUNSUPPORTED
 * and nothing is enqueued. Other arguments, workspace and errors as in
 * blockffn_layer_forward.
 */
blockffn_status_t blockffn_layer_forward_packed(const void *x, const void *w_r, const float *gain,
                                                const float *bias, float eps, const void *packed,
                                                int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                                int64_t n, int dtype, void *y, float *scores,
                                                void *workspace, size_t workspace_bytes,
                                                void *stream);

/*
 * Residual + LayerNorm of the layer output (skill page, "Full BlockFFN Layer with
 * Combined Losses": the layer returns nn.LayerNorm(d_h) of the expert output plus
 * the layer input):
 *   v = y[t,:] + x[t,:],  mu = mean_j v_j,  var = mean_j (v_j - mu)^2  (biased)
 *   out[t,j] = (v_j - mu) / sqrt(var + eps) * gamma[j] + beta[j]
 *
 *   y      [T, d_h] dtype   expert output (e.g. blockffn_chunk_ffn's y)
 *   x      [T, d_h] dtype   layer input (the residual)
 *   gamma  [d_h] float or NULL (= 1), beta [d_h] float or NULL (= 0)
 *   eps    finite, >= 0 (nn.LayerNorm's default is 1e-5)
 *   out    [T, d_h] dtype, written. It may be the same array as y or as x (in
 *          place); any other overlap with them is rejected.
 * fp32 arithmetic (two-pass mean and variance); bf16 output rounded to nearest even.
 * Needs d_h % 8 == 0 (bf16) or d_h % 4 == 0 (fp32), d_h <= 2^20, and 16-byte aligned
 * y, x, out, gamma, beta.
 */
blockffn_status_t blockffn_add_layernorm(const void *y, const void *x, const float *gamma,
                                         const float *beta, float eps, int64_t T, int64_t d_h,
                                         int dtype, void *out, void *stream);

/*
 * Bytes of workspace blockffn_sparsity_losses needs (0 when the sizes are invalid).
 */
size_t blockffn_sparsity_losses_workspace_bytes(int64_t B, int64_t S, int64_t E, int64_t L);

/*
 * The two sparsity training losses and their gradient (skill page, "Activation
 * Locality Loss" and "Chunk Sparsification Loss"), over activation probabilities
 * p [B, S, E] (B sequences of S tokens, e.g. the router's probs):
 *   q = sigmoid(alpha (2p - 1))
 *   AL = 1/max(S-1, 1) * sum_{i < S-1} mean_{b,e} -( q[b,i,e] log(q[b,i+1,e] + 1e-8)
 *                                   + (1 - q[b,i,e]) log(1 - q[b,i+1,e] + 1e-8) )
 *   CS = 1/ceil(S/L) * sum_c mean_{b,e} ( 1 - prod_{k in chunk c} (1 - p[b,k,e]) )
 * with aligned chunks of L tokens, the last possibly partial (the pages use
 * alpha = 2, L = 8).
 *
 *   probs    [B, S, E] float, device
 *   losses   [2] float, device, written: losses[0] = AL, losses[1] = CS
 *   grad     [B, S, E] float or NULL: OVERWRITTEN with
 *            lambda_al * dAL/dp + lambda_cs * dCS/dp
 *   workspace, workspace_bytes: at least blockffn_sparsity_losses_workspace_bytes
 *            bytes, 256-byte aligned, ZERO-FILLED before its first use; it holds an
 *            arrival counter that every call returns to zero. Calls that may run
 *            concurrently need separate workspaces.
 * fp32 arithmetic per element; the loss sums are accumulated in fp64 in a fixed
 * order, so equal inputs give equal bits. probs, grad, losses and workspace must
 * not overlap. Needs B * S * E < 2^31.
 */
blockffn_status_t blockffn_sparsity_losses(const float *probs, int64_t B, int64_t S, int64_t E,
                                           float alpha, int64_t L, float lambda_al,
                                           float lambda_cs, float *losses, float *grad,
                                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace blockffn_layer_backward needs (0 when the sizes are invalid or
 * unsupported).
 */
size_t blockffn_layer_backward_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                               int64_t n, int dtype);

/*
 * Layer backward (skill page, "Architecture Overview": the ReLU + RMSNorm router is
 * differentiable and trained end to end; "Core Concept"; "Router Architecture
 * Setup"): the gradients of
 *     L = sum_{t,j} dy[t,j] y[t,j] + sum_{t,e} dprobs[t,e] probs[t,e]
 * where y = blockffn_chunk_ffn(x, scores, W1, W2, n) with scores from
 * blockffn_router(x, W_r, gain, bias, eps) and probs = sigmoid(sharpness * scores).
 * The router is recomputed inside the call. By the chain rule, for e in U_c(t) with
 * a = W1_e x_t and h = swish(a):
 *     ds[t,e] = dy_t . W2_e h,   dW2_e += s dy_t h^T,
 *     da = s (W2_e^T dy_t) * swish'(a),   dW1_e += da x_t^T,   dx_t += W1_e^T da;
 * then ds += dprobs sharpness p (1 - p), the RMSNorm backward over the experts, the
 * ReLU (derivative 0 where the logit is not > 0) and the router linear:
 *     dW_r += dl x_t^T,  dbias += dl,  dx_t += W_r^T dl,  dgain_e += ds r / rms.
 *
 *   x, w_r, gain, bias, eps, w1, w2, T, d_h, E, d_e, n: as in the forward calls
 *   dtype   BLOCKFFN_BF16 only (x, w_r, w1, w2, dy bf16); others return EUNSUPPORTED
 *   dy      [T, d_h] bf16   gradient of y
 *   dprobs  [T, E] float or NULL (no probability term); sharpness as in the router
 *   dx      [T, d_h] float, written (16-byte aligned)
 *   dw_r    [E, d_h] float, dw1 [E, d_e, d_h] float, dw2 [E, d_h, d_e] float: written
 *           (experts no chunk uses get zeros)
 *   dgain, dbias  [E] float or NULL: written when given
 *   workspace, workspace_bytes: at least blockffn_layer_backward_workspace_bytes(...),
 *           256-byte aligned, scratch only (no zero-fill needed); calls that may run
 *           concurrently need separate workspaces.
 * Needs 1 <= E <= 256, d_h % 256 == 0, d_e % 128 == 0. fp32 accumulation; the
 * recomputed hidden activations and their gradients are rounded to bf16 before the
 * weight-gradient and dx products. Every sum runs in a fixed order.
 */
blockffn_status_t blockffn_layer_backward(const void *x, const void *w_r, const float *gain,
                                          const float *bias, float eps, const void *w1,
                                          const void *w2, int64_t T, int64_t d_h, int64_t E,
                                          int64_t d_e, int64_t n, int dtype, const void *dy,
                                          const float *dprobs, float sharpness, float *dx,
                                          float *dw_r, float *dgain, float *dbias, float *dw1,
                                          float *dw2, void *workspace, size_t workspace_bytes,
                                          void *stream);

/*
 * Probes the current device for the facts some schedules need (workgroup-to-XCD
 * placement: one small kernel launch on `stream` into a static device array, then a
 * synchronisation of `stream`). Optional: without it the first call on a device does
 * the same. Call it before capturing graphs, so that captured calls can use the
 * one-launch schedules. BLOCKFFN_EINVAL while `stream` is being captured,
 * BLOCKFFN_EHIP if the probe fails.
 */
blockffn_status_t blockffn_init(void *stream);

/*
 * Reports whether a kernel that used `workspace` (a chunk-FFN or layer-forward
 * workspace, at least 64 KB) timed out in one of its bounded waits: synchronises
 * `stream`, reads the workspace's status word and returns BLOCKFFN_OK (no time-out)
 * or BLOCKFFN_ETIMEOUT (outputs of that call are NaN; zero-fill the workspace before
 * using it again). Call it on the stream the workspace's calls ran on.
 */
blockffn_status_t blockffn_workspace_check(const void *workspace, size_t workspace_bytes,
                                           void *stream);

/* Message describing the calling thread's last non-OK status ("" if none). */
const char *blockffn_last_error(void);

/* Library version string. */
const char *blockffn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKFFN_H */
