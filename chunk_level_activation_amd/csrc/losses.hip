// Sparsity training losses of BlockFFN and their gradient with respect to the
// activation probabilities, in one pass over p [B, S, E] (skill page, "Activation
// Locality Loss" and "Chunk Sparsification Loss"):
//
//   q = sigmoid(alpha (2p - 1))                          sharpened patterns
//   AL = 1/max(S-1,1) sum_{i<S-1} mean_{b,e} BCE(target q_i, input q_{i+1}),
//        BCE(c, n) = -(c log(n + 1e-8) + (1 - c) log(1 - n + 1e-8))
//   CS = 1/ceil(S/L) sum_c mean_{b,e} (1 - prod_{k in chunk c} (1 - p_k))
//
//   dAL/dp_t = 2 alpha q_t (1 - q_t) [ dBCE(q_t, q_{t+1})/dq_t + dBCE(q_{t-1}, q_t)/dq_t ]
//              / (B E max(S-1,1))
//   dCS/dp_t = prod_{j != t in t's chunk} (1 - p_j) / (B E ceil(S/L))
//
// HBM-bound: p is read once (plus one neighbouring row at each chunk edge, which the
// caches serve) and the gradient written once. Thread <-> (b, chunk, e): consecutive
// threads take consecutive experts, so every row access of a wavefront is a
// contiguous run of floats. With L <= 32 the chunk's values sit in registers and the
// products over the other tokens come from prefix and suffix products; longer chunks
// keep the suffix products in the gradient array between two passes.
//
// The two loss sums are deterministic: fp32 terms per thread, fp64 wavefront and
// workgroup trees, per-workgroup partials in the workspace, and the last workgroup
// to arrive adds the partials in index order.
#include "plan.h"
#include "sync.h"

namespace blockffn {
namespace {

constexpr int kLossThreads = 256;
constexpr float kLogEps = 1e-8f;

__device__ __forceinline__ float sharpen(float p, float alpha)
{
    return 1.0f / (1.0f + expf(-alpha * (2.0f * p - 1.0f)));
}

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1)
        v += __shfl_xor(v, m);
    return v;
}

struct LossArgs {
    const float *p;
    float *grad;                 // NULL: losses only
    int B, S, E, L, nc;
    int64_t columns;             // B * nc * E
    float alpha;
    float g_al, g_cs;            // lambda / (B E max(S-1,1)), lambda / (B E nc)
    double al_scale, cs_scale;   // 1 / (B E max(S-1,1)), 1 / (B E nc)
    double *part;                // [gridDim.x][2]
    uint32_t *arrive;
    float *losses;
};

// The pair term of the locality loss for (t, t+1) and the pieces of its gradient:
// d/dq_t and d/dq_{t+1} of BCE(q_t, q_{t+1}).
struct PairTerm {
    float bce, d_cur, d_next;
};
__device__ __forceinline__ PairTerm pair_term(float c, float n)
{
    const float ln = logf(n + kLogEps), l1n = logf(1.0f - n + kLogEps);
    PairTerm r;
    r.bce = -(c * ln + (1.0f - c) * l1n);
    r.d_cur = -(ln - l1n);
    r.d_next = -(c / (n + kLogEps) - (1.0f - c) / (1.0f - n + kLogEps));
    return r;
}

// One column: MAXL > 0 keeps the chunk (at most MAXL tokens) and its two neighbours
// in registers; MAXL == 0 handles any L with the gradient array as temporary storage
// for the suffix products.
template <int MAXL>
__device__ __forceinline__ void column(const LossArgs &a, int64_t col, float &al, float &cs)
{
    const int e = (int)(col % a.E);
    const int64_t bc = col / a.E;
    const int c = (int)(bc % a.nc), b = (int)(bc / a.nc);
    const int t0 = c * a.L, t1 = min(t0 + a.L, a.S), len = t1 - t0;
    const float *pc = a.p + ((int64_t)b * a.S) * a.E + e;   // p[b, t, e] = pc[t * E]
    float *gc = a.grad ? a.grad + ((int64_t)b * a.S) * a.E + e : nullptr;
    const int64_t E = a.E;

    if constexpr (MAXL > 0) {
        // slot k holds token t0 - 1 + k, k = 0 .. len + 1
        float pv[MAXL + 2], q[MAXL + 2];
#pragma unroll
        for (int k = 0; k < MAXL + 2; ++k) {
            const int t = t0 - 1 + k;
            pv[k] = (k <= len + 1 && t >= 0 && t < a.S) ? pc[t * E] : 0.0f;
            q[k] = sharpen(pv[k], a.alpha);
        }
        // suffix products: suf[k] = prod_{j = k .. len} (1 - p[slot j])
        float suf[MAXL + 2];
        suf[MAXL + 1] = 1.0f;
#pragma unroll
        for (int k = MAXL; k >= 1; --k)
            suf[k] = k <= len ? suf[k + 1] * (1.0f - pv[k]) : 1.0f;
        cs = 1.0f - suf[1];
        float pre = 1.0f, prev_dn = 0.0f;
        al = 0.0f;
        // the pair (t0 - 1, t0) adds to t0's gradient
        if (t0 > 0)
            prev_dn = pair_term(q[0], q[1]).d_next;
#pragma unroll
        for (int k = 1; k <= MAXL; ++k) {
            if (k <= len) {
                const int t = t0 - 1 + k;
                float dq = prev_dn;
                prev_dn = 0.0f;
                if (t + 1 < a.S) {
                    const PairTerm pt = pair_term(q[k], q[k + 1]);
                    al += pt.bce;
                    dq += pt.d_cur;
                    prev_dn = pt.d_next;
                }
                if (gc) {
                    const float slope = 2.0f * a.alpha * q[k] * (1.0f - q[k]);
                    gc[t * E] = a.g_al * slope * dq + a.g_cs * (pre * suf[k + 1]);
                }
                pre *= 1.0f - pv[k];
            }
        }
    } else {
        // pass 1, backwards: product of the chunk, and (with a gradient) the suffix
        // product of the tokens after t parked in grad[t]
        float suf = 1.0f;
        for (int t = t1 - 1; t >= t0; --t) {
            if (gc)
                gc[t * E] = suf;
            suf *= 1.0f - pc[t * E];
        }
        cs = 1.0f - suf;
        // pass 2, forwards: locality terms and the gradient
        al = 0.0f;
        float pre = 1.0f, prev_dn = 0.0f;
        float qc = sharpen(pc[t0 * E], a.alpha);
        if (t0 > 0)
            prev_dn = pair_term(sharpen(pc[(t0 - 1) * E], a.alpha), qc).d_next;
        for (int t = t0; t < t1; ++t) {
            float dq = prev_dn;
            prev_dn = 0.0f;
            float qn = 0.0f;
            if (t + 1 < a.S) {
                qn = sharpen(pc[(t + 1) * E], a.alpha);
                const PairTerm pt = pair_term(qc, qn);
                al += pt.bce;
                dq += pt.d_cur;
                prev_dn = pt.d_next;
            }
            const float pt_ = pc[t * E];
            if (gc) {
                const float slope = 2.0f * a.alpha * qc * (1.0f - qc);
                gc[t * E] = a.g_al * slope * dq + a.g_cs * (pre * gc[t * E]);
            }
            pre *= 1.0f - pt_;
            qc = qn;
        }
    }
}

template <int MAXL>
__global__ void __launch_bounds__(kLossThreads) sparsity_losses_kernel(LossArgs a)
{
    __shared__ double red[kLossThreads / kWave][2];
    __shared__ int last;
    const int tid = threadIdx.x;
    double al_sum = 0.0, cs_sum = 0.0;
    for (int64_t col = (int64_t)blockIdx.x * kLossThreads + tid; col < a.columns;
         col += (int64_t)gridDim.x * kLossThreads) {
        float al, cs;
        column<MAXL>(a, col, al, cs);
        al_sum += (double)al;
        cs_sum += (double)cs;
    }
    al_sum = wave_sum_d(al_sum);
    cs_sum = wave_sum_d(cs_sum);
    if (tid % kWave == 0) {
        red[tid / kWave][0] = al_sum;
        red[tid / kWave][1] = cs_sum;
    }
    __syncthreads();
    if (tid == 0) {
        double s0 = 0.0, s1 = 0.0;
#pragma unroll
        for (int w = 0; w < kLossThreads / kWave; ++w) {
            s0 += red[w][0];
            s1 += red[w][1];
        }
        // device-scope stores: the last workgroup may sit on another XCD
        __hip_atomic_store(&a.part[2 * blockIdx.x], s0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.part[2 * blockIdx.x + 1], s1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        drain_memory();
        const uint32_t prev = add_counter(a.arrive, 1u);
        last = prev == gridDim.x - 1;
        if (last)
            st_counter(a.arrive, 0u);
    }
    __syncthreads();
    if (!last)
        return;
    // the last workgroup: partials in index order, thread i taking i, i + 256, ...,
    // then a fixed tree
    double s0 = 0.0, s1 = 0.0;
    for (unsigned i = tid; i < gridDim.x; i += kLossThreads) {
        s0 += __hip_atomic_load(&a.part[2 * i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s1 += __hip_atomic_load(&a.part[2 * i + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s0 = wave_sum_d(s0);
    s1 = wave_sum_d(s1);
    __syncthreads();
    if (tid % kWave == 0) {
        red[tid / kWave][0] = s0;
        red[tid / kWave][1] = s1;
    }
    __syncthreads();
    if (tid == 0) {
        double t0 = 0.0, t1 = 0.0;
#pragma unroll
        for (int w = 0; w < kLossThreads / kWave; ++w) {
            t0 += red[w][0];
            t1 += red[w][1];
        }
        a.losses[0] = (float)(t0 * a.al_scale);
        a.losses[1] = (float)(t1 * a.cs_scale);
    }
}

}  // namespace

int64_t sparsity_losses_blocks(int64_t B, int64_t S, int64_t E, int64_t L)
{
    const int64_t nc = (S + L - 1) / L;
    const int64_t cols = B * nc * E;
    const int64_t blocks = (cols + kLossThreads - 1) / kLossThreads;
    return blocks < kLossMaxBlocks ? blocks : kLossMaxBlocks;
}

size_t sparsity_losses_workspace_bytes(int64_t B, int64_t S, int64_t E, int64_t L)
{
    return kLossControlBytes + (size_t)sparsity_losses_blocks(B, S, E, L) * 2 * sizeof(double);
}

hipError_t launch_sparsity_losses(const float *p, int64_t B, int64_t S, int64_t E, float alpha,
                                  int64_t L, float lambda_al, float lambda_cs, float *losses,
                                  float *grad, void *ws, hipStream_t stream)
{
    LossArgs a;
    a.p = p;
    a.grad = grad;
    a.B = (int)B;
    a.S = (int)S;
    a.E = (int)E;
    a.L = (int)(L < S ? L : S);
    a.nc = (int)((S + L - 1) / L);
    a.columns = B * a.nc * E;
    a.alpha = alpha;
    const double den_al = (double)B * (double)E * (double)(S - 1 > 1 ? S - 1 : 1);
    const double den_cs = (double)B * (double)E * (double)a.nc;
    a.al_scale = 1.0 / den_al;
    a.cs_scale = 1.0 / den_cs;
    a.g_al = (float)(lambda_al / den_al);
    a.g_cs = (float)(lambda_cs / den_cs);
    a.arrive = static_cast<uint32_t *>(ws);
    a.part = reinterpret_cast<double *>(static_cast<char *>(ws) + kLossControlBytes);
    a.losses = losses;
    const dim3 grid((unsigned)sparsity_losses_blocks(B, S, E, L)), block(kLossThreads);
    if (a.L <= 8)
        hipLaunchKernelGGL(sparsity_losses_kernel<8>, grid, block, 0, stream, a);
    else if (a.L <= 32)
        hipLaunchKernelGGL(sparsity_losses_kernel<32>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(sparsity_losses_kernel<0>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace blockffn
