/*
 * CPU oracle for the BlockFFN layer: router and chunk-union expert FFN (forward and
 * backward), the residual + LayerNorm epilogue and the two sparsity losses.
 *
 * THIS FILE IS TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it. The GPU library shares no code with it and
 * never calls it.
 *
 * It is a plain, slow, obviously correct restatement of what the layer computes:
 * straight loops, every sum accumulated in double precision in ascending index
 * order, no blocking, no fusion, no reordering. Inputs are fp32 arrays; bf16 inputs
 * are widened to fp32 by the caller, which is exact.
 *
 * Sources (web pages on BlockFFN, arXiv 2507.08771):
 *  [S1] "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device Deployment"
 *       (skill page), section "Architecture Overview": the router is a linear map
 *       with ReLU followed by RMSNorm; experts are non-gated MLPs with Swish and a
 *       width d_e much smaller than d_h.
 *  [S2] same page, section "Core Concept": the accelerator computes only the union
 *       of experts activated across n consecutive tokens and masks the unneeded
 *       activations after the computation; the "CUTLASS Acceleration Kernel" item
 *       of "Architecture Overview" fixes n = 32 tokens.
 *  [S3] same page, "Router Architecture Setup": the router linear has no bias,
 *       RMSNorm runs over the expert axis, the expert is fc2(SiLU(fc1(x))).
 *  [S4] same page, "Chunk Sparsification Loss": chunks are consecutive, aligned,
 *       ceil(S/L) of them, the last one possibly partial.
 *  [S5] paper card (sota2), Abstract: a router integrating ReLU and RMSNorm.
 *  [S6] skill page, "Full BlockFFN Layer with Combined Losses": the layer output is
 *       a LayerNorm over d_h of (expert output + x); the router also returns
 *       probabilities sigmoid(sharpness * score) ("Router Architecture Setup").
 *  [S7] skill page, "Activation Locality Loss": binary cross entropy between the
 *       sigmoid-sharpened activation patterns of adjacent tokens.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *  - Experts carry no biases and dropout is the identity (inference).
 *  - The gate is the post-RMSNorm score s[t,e]; an expert is active for a token
 *    exactly when s[t,e] != 0 (compared in fp32, the precision scores are stored in;
 *    -0 counts as inactive).
 *  - ReLU maps every logit that is not > 0 (NaN included) to 0.
 *  - The union list is in ascending expert id; list entries past the count are -1.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the parallel loops below use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Router, per token t, following [S1] "Architecture Overview", [S3] and [S5]:
 *   l[t,e] = sum_j x[t,j] * W_r[e,j]            (+ bias[e] when bias != NULL)
 *   r[t,e] = l[t,e] if l[t,e] > 0 else 0          (ReLU)
 *   s[t,e] = r[t,e] / sqrt(mean_e r[t,e]^2 + eps) * gain[e]   (RMSNorm over experts)
 * x: [T, d_h], w_r: [E, d_h] (nn.Linear layout), gain/bias: [E] or NULL (ones/zeros).
 * Outputs logits, scores: [T, E] double.
 */
void oracle_router(const float *x, const float *w_r, const float *gain, const float *bias,
                   double eps, int64_t T, int64_t d_h, int64_t E,
                   double *logits, double *scores)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *xt = x + t * d_h;
        double *lt = logits + t * E;
        double *st = scores + t * E;

        for (int64_t e = 0; e < E; ++e) {
            const float *we = w_r + e * d_h;
            double acc = 0.0;
            for (int64_t j = 0; j < d_h; ++j)
                acc += (double)xt[j] * (double)we[j];
            if (bias)
                acc += (double)bias[e];
            lt[e] = acc;
        }

        double sumsq = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            double r = lt[e] > 0.0 ? lt[e] : 0.0;
            st[e] = r;
            sumsq += r * r;
        }
        double mean_sq = sumsq / (double)E;
        double denom = sqrt(mean_sq + eps);
        for (int64_t e = 0; e < E; ++e) {
            double g = gain ? (double)gain[e] : 1.0;
            st[e] = st[e] / denom * g;
        }
    }
}

/*
 * Chunk union, following [S2] and [S4]: chunk c holds tokens
 * [c*n, min(c*n + n, T)); expert e is in the union U_c when some token of the chunk
 * has scores[t,e] != 0. Outputs, for C = ceil(T/n) chunks and W = ceil(E/64) words:
 *   masks  [C][W]  bit (e % 64) of word (e / 64) set when e is in U_c
 *   lists  [C][E]  the members of U_c in ascending order, then -1
 *   counts [C]     |U_c|
 */
void oracle_chunk_union(const float *scores, int64_t T, int64_t E, int64_t n,
                        uint64_t *masks, int32_t *lists, int32_t *counts)
{
    int64_t C = (T + n - 1) / n;
    int64_t W = (E + 63) / 64;
    for (int64_t c = 0; c < C; ++c) {
        uint64_t *mc = masks + c * W;
        int32_t *lc = lists + c * E;
        int64_t t_end = c * n + n < T ? c * n + n : T;

        for (int64_t w = 0; w < W; ++w)
            mc[w] = 0;
        for (int64_t t = c * n; t < t_end; ++t)
            for (int64_t e = 0; e < E; ++e)
                if (scores[t * E + e] != 0.0f)
                    mc[e / 64] |= (uint64_t)1 << (e % 64);

        int32_t count = 0;
        for (int64_t e = 0; e < E; ++e)
            if (mc[e / 64] & ((uint64_t)1 << (e % 64)))
                lc[count++] = (int32_t)e;
        counts[c] = count;
        for (int64_t i = count; i < E; ++i)
            lc[i] = -1;
    }
}

/*
 * One expert applied to one token and added into y with weight s, following [S1]
 * "Architecture Overview" and [S3]: Expert_e(x) = W2_e * swish(W1_e * x), with
 * swish(a) = a / (1 + exp(-a)) (SiLU, beta = 1).
 * w1e: [d_e, d_h] (fc1 weight), w2e: [d_h, d_e] (fc2 weight), h: scratch [d_e].
 */
static void add_expert_output(const float *xt, const float *w1e, const float *w2e,
                              double s, int64_t d_h, int64_t d_e, double *h, double *yt)
{
    for (int64_t k = 0; k < d_e; ++k) {
        double a = 0.0;
        for (int64_t j = 0; j < d_h; ++j)
            a += (double)w1e[k * d_h + j] * (double)xt[j];
        h[k] = a / (1.0 + exp(-a));
    }
    for (int64_t j = 0; j < d_h; ++j) {
        double z = 0.0;
        for (int64_t k = 0; k < d_e; ++k)
            z += (double)w2e[j * d_e + k] * h[k];
        yt[j] += s * z;
    }
}

/*
 * Union-then-mask chunk FFN, following [S2]: every expert of the chunk's union is
 * evaluated for every token of the chunk and its output is weighted by that token's
 * score, which is 0 for tokens where the expert is inactive ("masking after the
 * computation"). Experts outside the union are never read.
 *   y[t,:] = sum_{e in U_c(t), ascending} s[t,e] * Expert_e(x[t,:])
 * x: [T, d_h]; scores: [T, E]; w1: [E, d_e, d_h]; w2: [E, d_h, d_e]; y: [T, d_h].
 * h_scratch: [nthreads][d_e] doubles, lists/counts: [C][E] and [C] scratch.
 */
void oracle_chunk_ffn(const float *x, const float *scores, const float *w1,
                      const float *w2, int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                      int64_t n, double *y, uint64_t *masks, int32_t *lists,
                      int32_t *counts, double *h_scratch)
{
    oracle_chunk_union(scores, T, E, n, masks, lists, counts);

#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
#ifdef _OPENMP
        double *h = h_scratch + (int64_t)omp_get_thread_num() * d_e;
#else
        double *h = h_scratch;
#endif
        int64_t c = t / n;
        double *yt = y + t * d_h;
        for (int64_t j = 0; j < d_h; ++j)
            yt[j] = 0.0;
        for (int32_t i = 0; i < counts[c]; ++i) {
            int64_t e = lists[c * E + i];
            add_expert_output(x + t * d_h, w1 + e * d_e * d_h, w2 + e * d_h * d_e,
                              (double)scores[t * E + e], d_h, d_e, h, yt);
        }
    }
}

/*
 * Per-token brute force: the same sum restricted to the experts active for the
 * token itself (scores[t,e] != 0), ascending. By the definition of the layer this is
 * the result the union-then-mask form must reproduce.
 */
void oracle_token_ffn(const float *x, const float *scores, const float *w1,
                      const float *w2, int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                      double *y, double *h_scratch)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
#ifdef _OPENMP
        double *h = h_scratch + (int64_t)omp_get_thread_num() * d_e;
#else
        double *h = h_scratch;
#endif
        double *yt = y + t * d_h;
        for (int64_t j = 0; j < d_h; ++j)
            yt[j] = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            float s = scores[t * E + e];
            if (s != 0.0f)
                add_expert_output(x + t * d_h, w1 + e * d_e * d_h, w2 + e * d_h * d_e,
                                  (double)s, d_h, d_e, h, yt);
        }
    }
}

/*
 * Router probabilities, [S6] / [S3]: p = sigmoid(sharpness * s), elementwise over n
 * scores (the pages' default sharpness is 1).
 */
void oracle_router_probs(const double *scores, int64_t n, double sharpness, double *probs)
{
    for (int64_t i = 0; i < n; ++i)
        probs[i] = 1.0 / (1.0 + exp(-sharpness * scores[i]));
}

/*
 * Residual + LayerNorm, [S6]: out[t,:] = LayerNorm(y[t,:] + x[t,:]) over the d axis,
 *   v = y + x,  mean = (1/d) sum_j v_j,  var = (1/d) sum_j (v_j - mean)^2  (biased),
 *   out_j = (v_j - mean) / sqrt(var + eps) * gamma_j + beta_j
 * (nn.LayerNorm's definition; gamma/beta NULL mean ones/zeros).
 */
void oracle_add_layernorm(const float *y, const float *x, const float *gamma,
                          const float *beta, double eps, int64_t T, int64_t d, double *out)
{
    for (int64_t t = 0; t < T; ++t) {
        double mean = 0.0;
        for (int64_t j = 0; j < d; ++j)
            mean += (double)y[t * d + j] + (double)x[t * d + j];
        mean /= (double)d;
        double var = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            double v = (double)y[t * d + j] + (double)x[t * d + j] - mean;
            var += v * v;
        }
        var /= (double)d;
        double inv = 1.0 / sqrt(var + eps);
        for (int64_t j = 0; j < d; ++j) {
            double v = (double)y[t * d + j] + (double)x[t * d + j] - mean;
            out[t * d + j] = v * inv * (gamma ? (double)gamma[j] : 1.0) +
                             (beta ? (double)beta[j] : 0.0);
        }
    }
}

/* Sigmoid sharpening of [S7]: sigmoid(alpha * (2p - 1)). */
static double sharpen(double p, double alpha)
{
    return 1.0 / (1.0 + exp(-alpha * (2.0 * p - 1.0)));
}

#define LOSS_LOG_EPS 1e-8

/*
 * Activation locality loss, [S7], over probabilities p[B][S][E]:
 *   q = sharpen(p);  for i = 0 .. S-2:
 *     bce_i = mean over (b, e) of -( q[b,i,e] log(q[b,i+1,e] + 1e-8)
 *                                    + (1 - q[b,i,e]) log(1 - q[b,i+1,e] + 1e-8) )
 *   loss = (sum_i bce_i) / max(S - 1, 1)
 */
double oracle_locality_loss(const float *p, int64_t B, int64_t S, int64_t E, double alpha)
{
    double loss = 0.0;
    for (int64_t i = 0; i + 1 < S; ++i) {
        double sum = 0.0;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t e = 0; e < E; ++e) {
                double c = sharpen(p[(b * S + i) * E + e], alpha);
                double nx = sharpen(p[(b * S + i + 1) * E + e], alpha);
                sum += -(c * log(nx + LOSS_LOG_EPS) + (1.0 - c) * log(1.0 - nx + LOSS_LOG_EPS));
            }
        loss += sum / (double)(B * E);
    }
    return loss / (double)(S - 1 > 1 ? S - 1 : 1);
}

/*
 * Chunk sparsification loss, [S4], over p[B][S][E] and chunks of L tokens (aligned,
 * ceil(S/L) of them, the last possibly partial):
 *   per chunk: mean over (b, e) of 1 - prod_{k in chunk} (1 - p[b,k,e])
 *   loss = (sum over chunks) / ceil(S/L)
 */
double oracle_chunk_sparsification_loss(const float *p, int64_t B, int64_t S, int64_t E,
                                        int64_t L)
{
    const int64_t nc = (S + L - 1) / L;
    double loss = 0.0;
    for (int64_t c = 0; c < nc; ++c) {
        const int64_t t0 = c * L, t1 = t0 + L < S ? t0 + L : S;
        double sum = 0.0;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t e = 0; e < E; ++e) {
                double none = 1.0;
                for (int64_t k = t0; k < t1; ++k)
                    none *= 1.0 - (double)p[(b * S + k) * E + e];
                sum += 1.0 - none;
            }
        loss += sum / (double)(B * E);
    }
    return loss / (double)nc;
}

/*
 * Gradient of oracle_locality_loss with respect to p (same layout), by the chain
 * rule on its definition: with q = sharpen(p), dq/dp = 2 alpha q (1 - q), and for
 * the pair (i, i+1) of one (b, e):
 *   d bce_i / d q_i     = -( log(q_{i+1} + eps) - log(1 - q_{i+1} + eps) )
 *   d bce_i / d q_{i+1} = -( q_i / (q_{i+1} + eps) - (1 - q_i) / (1 - q_{i+1} + eps) )
 * each scaled by 1 / (B E max(S - 1, 1)).
 */
void oracle_locality_loss_grad(const float *p, int64_t B, int64_t S, int64_t E,
                               double alpha, double *grad)
{
    const double scale = 1.0 / ((double)(B * E) * (double)(S - 1 > 1 ? S - 1 : 1));
    for (int64_t i = 0; i < B * S * E; ++i)
        grad[i] = 0.0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i + 1 < S; ++i)
            for (int64_t e = 0; e < E; ++e) {
                const int64_t a0 = (b * S + i) * E + e, a1 = (b * S + i + 1) * E + e;
                double c = sharpen(p[a0], alpha), nx = sharpen(p[a1], alpha);
                double dc = -(log(nx + LOSS_LOG_EPS) - log(1.0 - nx + LOSS_LOG_EPS));
                double dn = -(c / (nx + LOSS_LOG_EPS) - (1.0 - c) / (1.0 - nx + LOSS_LOG_EPS));
                grad[a0] += scale * dc * 2.0 * alpha * c * (1.0 - c);
                grad[a1] += scale * dn * 2.0 * alpha * nx * (1.0 - nx);
            }
}

/*
 * Gradient of oracle_chunk_sparsification_loss with respect to p: the chunk term
 * 1 - prod_k (1 - p_k) has derivative prod_{j != k} (1 - p_j) in p_k; scaled by
 * 1 / (B E ceil(S/L)).
 */
void oracle_chunk_sparsification_loss_grad(const float *p, int64_t B, int64_t S, int64_t E,
                                           int64_t L, double *grad)
{
    const int64_t nc = (S + L - 1) / L;
    const double scale = 1.0 / ((double)(B * E) * (double)nc);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < nc; ++c) {
            const int64_t t0 = c * L, t1 = t0 + L < S ? t0 + L : S;
            for (int64_t e = 0; e < E; ++e)
                for (int64_t k = t0; k < t1; ++k) {
                    double others = 1.0;
                    for (int64_t j = t0; j < t1; ++j)
                        if (j != k)
                            others *= 1.0 - (double)p[(b * S + j) * E + e];
                    grad[(b * S + k) * E + e] = scale * others;
                }
        }
}

/*
 * Layer backward ([S1]-[S3], [S6]): gradients of
 *     L = sum_{t,j} dy[t,j] y[t,j]  +  sum_{t,e} dprobs[t,e] probs[t,e]
 * where y is the chunk-union FFN of x under the router's scores s (computed here in
 * double from x, W_r, gain, bias, eps) and probs = sigmoid(sharpness * s). dprobs may
 * be NULL (no probability term). The chain rule on the definitions above:
 *
 *   expert e in U_c(t), a = W1_e x_t, h = swish(a), z = W2_e h, y_t += s[t,e] z:
 *     ds[t,e]  = dy_t . z
 *     dW2_e   += s[t,e] dy_t h^T
 *     da       = (s[t,e] W2_e^T dy_t) * swish'(a),  swish'(a) = sig(a) (1 + a (1 - sig(a)))
 *     dW1_e   += da x_t^T,     dx_t += W1_e^T da
 *   experts outside U_c(t) are not evaluated: their ds is left 0, which only the
 *   ReLU-killed (inactive) logits would see;
 *   probabilities: ds[t,e] += dprobs[t,e] sharpness p (1 - p), p = sigmoid(sharpness s)
 *   RMSNorm over experts, s_e = g_e r_e inv, inv = (mean_j r_j^2 + eps)^(-1/2):
 *     dr_j = g_j inv ds_j - inv^3 r_j / E * sum_e g_e r_e ds_e,  dgain_e += ds_e r_e inv
 *   ReLU: dl = dr where l > 0, else 0 (also at l == 0)
 *   router linear: dW_r += dl x_t^T, dbias += dl, dx_t += W_r^T dl
 *
 * Shapes as in the forward calls; outputs (double, overwritten): dx [T, d_h],
 * dw_r [E, d_h], dgain [E], dbias [E], dw1 [E, d_e, d_h], dw2 [E, d_h, d_e].
 * Scratch: logits, scores, ds [T, E] and da [T, E, d_e] doubles (caller-owned).
 */
void oracle_layer_backward(const float *x, const float *w_r, const float *gain,
                           const float *bias, double eps, const float *w1, const float *w2,
                           int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n,
                           const float *dy, const float *dprobs, double sharpness,
                           double *dx, double *dw_r, double *dgain, double *dbias,
                           double *dw1, double *dw2,
                           double *logits, double *scores, double *ds, double *da)
{
    const int64_t C = (T + n - 1) / n;
    oracle_router(x, w_r, gain, bias, eps, T, d_h, E, logits, scores);
    for (int64_t i = 0; i < T * E; ++i)
        ds[i] = 0.0;
    for (int64_t i = 0; i < T * E * d_e; ++i)
        da[i] = 0.0;

    /* experts: each thread owns whole experts, so dW1_e / dW2_e need no locking */
#pragma omp parallel for schedule(dynamic)
    for (int64_t e = 0; e < E; ++e) {
        double *g1 = dw1 + e * d_e * d_h, *g2 = dw2 + e * d_h * d_e;
        const float *w1e = w1 + e * d_e * d_h, *w2e = w2 + e * d_h * d_e;
        double a[4096], h[4096], sg[4096];   /* d_e <= 4096 */
        for (int64_t i = 0; i < d_e * d_h; ++i)
            g1[i] = 0.0, g2[i] = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            const int64_t t0 = c * n, t1 = t0 + n < T ? t0 + n : T;
            int used = 0;   /* e in U_c: some token of the chunk has a nonzero score */
            for (int64_t t = t0; t < t1; ++t)
                if (scores[t * E + e] != 0.0)
                    used = 1;
            if (!used)
                continue;
            for (int64_t t = t0; t < t1; ++t) {
                const float *xt = x + t * d_h, *dyt = dy + t * d_h;
                const double s = scores[t * E + e];
                for (int64_t k = 0; k < d_e; ++k) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < d_h; ++j)
                        acc += (double)w1e[k * d_h + j] * (double)xt[j];
                    a[k] = acc;
                    sg[k] = 1.0 / (1.0 + exp(-acc));
                    h[k] = acc * sg[k];
                }
                /* ds = dy . (W2 h); dW2 += s dy h^T */
                double dsv = 0.0;
                for (int64_t j = 0; j < d_h; ++j) {
                    double z = 0.0;
                    for (int64_t k = 0; k < d_e; ++k)
                        z += (double)w2e[j * d_e + k] * h[k];
                    dsv += (double)dyt[j] * z;
                    for (int64_t k = 0; k < d_e; ++k)
                        g2[j * d_e + k] += s * (double)dyt[j] * h[k];
                }
                ds[t * E + e] = dsv;
                /* da = (s W2^T dy) * swish'(a); dW1 += da x^T */
                double *dat = da + (t * E + e) * d_e;
                for (int64_t k = 0; k < d_e; ++k) {
                    double dh = 0.0;
                    for (int64_t j = 0; j < d_h; ++j)
                        dh += (double)w2e[j * d_e + k] * s * (double)dyt[j];
                    dat[k] = dh * (sg[k] * (1.0 + a[k] * (1.0 - sg[k])));
                    for (int64_t j = 0; j < d_h; ++j)
                        g1[k * d_h + j] += dat[k] * (double)xt[j];
                }
            }
        }
    }

    /* per token: dx from the experts, then the router */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double *dxt = dx + t * d_h;
        for (int64_t j = 0; j < d_h; ++j)
            dxt[j] = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            const double *dat = da + (t * E + e) * d_e;
            const float *w1e = w1 + e * d_e * d_h;
            for (int64_t k = 0; k < d_e; ++k)
                if (dat[k] != 0.0)
                    for (int64_t j = 0; j < d_h; ++j)
                        dxt[j] += (double)w1e[k * d_h + j] * dat[k];
        }
        double *dst = ds + t * E;
        const double *lt = logits + t * E;
        if (dprobs)
            for (int64_t e = 0; e < E; ++e) {
                const double p = 1.0 / (1.0 + exp(-sharpness * scores[t * E + e]));
                dst[e] += (double)dprobs[t * E + e] * sharpness * p * (1.0 - p);
            }
        double sumsq = 0.0, coup = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            const double r = lt[e] > 0.0 ? lt[e] : 0.0;
            sumsq += r * r;
        }
        const double inv = 1.0 / sqrt(sumsq / (double)E + eps);
        for (int64_t e = 0; e < E; ++e) {
            const double r = lt[e] > 0.0 ? lt[e] : 0.0;
            coup += (gain ? (double)gain[e] : 1.0) * r * dst[e];
        }
        /* dl (kept in ds's row: dst[e] becomes dl[t,e] after the gain term is read) */
        for (int64_t e = 0; e < E; ++e) {
            const int active = lt[e] > 0.0;
            const double r = active ? lt[e] : 0.0;
            const double g = gain ? (double)gain[e] : 1.0;
            const double dr = g * inv * dst[e] - inv * inv * inv * r / (double)E * coup;
            /* keep ds_e * r_e * inv for dgain in the logit's slot (the logit is no longer
               needed), dl in ds's slot */
            logits[t * E + e] = dst[e] * r * inv;
            dst[e] = active ? dr : 0.0;
        }
        for (int64_t e = 0; e < E; ++e)
            for (int64_t j = 0; j < d_h; ++j)
                dxt[j] += (double)w_r[e * d_h + j] * dst[e];
    }

    /* router parameters: sums over tokens in ascending order */
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < E; ++e) {
        double gsum = 0.0, bsum = 0.0;
        for (int64_t j = 0; j < d_h; ++j)
            dw_r[e * d_h + j] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double dl = ds[t * E + e];
            gsum += logits[t * E + e];
            bsum += dl;
            for (int64_t j = 0; j < d_h; ++j)
                dw_r[e * d_h + j] += dl * (double)x[t * d_h + j];
        }
        dgain[e] = gsum;
        dbias[e] = bsum;
    }
}
