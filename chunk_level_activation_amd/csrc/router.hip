// Fused BlockFFN router: linear map, ReLU and RMSNorm over the experts in one pass.
//
// Skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
// Deployment", "Architecture Overview" and "Router Architecture Setup" (a linear
// router without bias, ReLU for sparsity, RMSNorm over the expert axis); paper-card
// Abstract (a router integrating ReLU and RMSNorm):
//     l[t,e] = sum_j x[t,j] W_r[e,j] (+ bias[e])
//     s[t,e] = max(l,0) / sqrt(mean_e max(l,0)^2 + eps) * gain[e]
// A workgroup owns all E logits of its 32 tokens, so the RMSNorm row reduction is
// done in LDS right after the product, with no second pass over memory.
#include "common.h"
#include "plan.h"

namespace blockffn {

// bf16: 32 tokens x all experts per workgroup, ET tiles of 32 experts, 8 waves. The
// 32x32x16 bf16 MFMA takes A = x rows (32 tokens x 16 k) and B = W_r rows
// transposed (16 k x 32 experts). The waves take k steps round robin, each issuing
// the loads of KB steps together; the wave sums are added in wave order in LDS.
constexpr int kRouterThreads = 512;
constexpr int kRouterWaves = kRouterThreads / kWave;

template <int ET>
__global__ void __launch_bounds__(kRouterThreads)
router_bf16_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w_r,
                   const float *__restrict__ gain, const float *__restrict__ bias,
                   float eps, int64_t T, int d_h, int E, float *__restrict__ scores,
                   float *__restrict__ logits)
{
    constexpr int KB = ET >= 8 ? 2 : (ET >= 4 ? 4 : 8);
    const int64_t t0 = (int64_t)blockIdx.x * kTileM;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int row = lane % 32;
    const int kg = lane / 32;
    const bool vt = t0 + row < T;
    const uint16_t *xr = x + (vt ? t0 + row : 0) * d_h + kg * 8;
    const uint16_t *wr[ET];
    bool ve[ET];
    f32x16 acc[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) {
        const int e = et * 32 + row;
        ve[et] = e < E;
        wr[et] = w_r + (int64_t)(ve[et] ? e : 0) * d_h + kg * 8;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc[et][i] = 0.0f;
    }
    const int KS = d_h / 16;
    for (int kb = wave; kb < KS; kb += kRouterWaves * KB) {
        bf16x8 av[KB], bv[KB][ET];
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const int ks = kb + i * kRouterWaves;
            const bool ok = ks < KS;
            av[i] = ok && vt ? load_bf16x8(xr + ks * 16) : zero_bf16x8();
#pragma unroll
            for (int et = 0; et < ET; ++et)
                bv[i][et] = ok && ve[et] ? load_bf16x8(wr[et] + ks * 16) : zero_bf16x8();
        }
#pragma unroll
        for (int i = 0; i < KB; ++i)
#pragma unroll
            for (int et = 0; et < ET; ++et)
                acc[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[i][et], acc[et], 0,
                                                                  0, 0);
    }

    // 32x32 accumulator layout: element i is row (i/4)*8 + (lane/32)*4 + i%4 (token)
    // of column lane%32 (expert).
    __shared__ float lg[kTileM][ET * 32 + 1];
    for (int w = 0; w < kRouterWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int et = 0; et < ET; ++et)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float &dst = lg[(i / 4) * 8 + kg * 4 + (i % 4)][et * 32 + row];
                    dst = w == 0 ? acc[et][i] : dst + acc[et][i];
                }
        }
        __syncthreads();
    }

    // Epilogue: 16 threads per token.
    const int tt = tid / 16, sub = tid % 16;
    const int64_t t = t0 + tt;
    float sumsq = 0.0f;
    for (int e = sub; e < E; e += 16) {
        const float l = bias ? lg[tt][e] + bias[e] : lg[tt][e];
        lg[tt][e] = l;
        const float r = l > 0.0f ? l : 0.0f;
        sumsq = fmaf(r, r, sumsq);
    }
    sumsq += __shfl_xor(sumsq, 1);
    sumsq += __shfl_xor(sumsq, 2);
    sumsq += __shfl_xor(sumsq, 4);
    sumsq += __shfl_xor(sumsq, 8);
    const float inv = 1.0f / sqrtf(sumsq / (float)E + eps);
    if (t < T) {
        for (int e = sub; e < E; e += 16) {
            const float l = lg[tt][e];
            const float r = l > 0.0f ? l : 0.0f;
            scores[t * E + e] = r * inv * (gain ? gain[e] : 1.0f);
            if (logits)
                logits[t * E + e] = l;
        }
    }
}

// fp32: one workgroup per token, one thread per expert (E <= 256), fp32 FMA.
__global__ void __launch_bounds__(256)
router_f32_kernel(const float *__restrict__ x, const float *__restrict__ w_r,
                  const float *__restrict__ gain, const float *__restrict__ bias, float eps,
                  int64_t T, int d_h, int E, float *__restrict__ scores,
                  float *__restrict__ logits)
{
    const int64_t t = blockIdx.x;
    const int e = threadIdx.x;
    float l = 0.0f;
    if (e < E) {
        const float *xr = x + t * d_h;
        const float *wr = w_r + (int64_t)e * d_h;
        for (int j = 0; j < d_h; ++j)
            l = fmaf(xr[j], wr[j], l);
        if (bias)
            l += bias[e];
    }
    const float r = (e < E && l > 0.0f) ? l : 0.0f;
    __shared__ float red[256];
    red[e] = r * r;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (e < s)
            red[e] += red[e + s];
        __syncthreads();
    }
    const float inv = 1.0f / sqrtf(red[0] / (float)E + eps);
    if (e < E) {
        scores[t * E + e] = r * inv * (gain ? gain[e] : 1.0f);
        if (logits)
            logits[t * E + e] = l;
    }
}

hipError_t launch_router_bf16(const uint16_t *x, const uint16_t *w_r, const float *gain,
                              const float *bias, float eps, int64_t T, int64_t d_h,
                              int64_t E, float *scores, float *logits, hipStream_t stream)
{
    const dim3 grid((unsigned)((T + kTileM - 1) / kTileM)), block(kRouterThreads);
    const int ET = (int)((E + 31) / 32);
    if (ET <= 1)
        hipLaunchKernelGGL(router_bf16_kernel<1>, grid, block, 0, stream, x, w_r, gain, bias,
                           eps, T, (int)d_h, (int)E, scores, logits);
    else if (ET <= 2)
        hipLaunchKernelGGL(router_bf16_kernel<2>, grid, block, 0, stream, x, w_r, gain, bias,
                           eps, T, (int)d_h, (int)E, scores, logits);
    else if (ET <= 4)
        hipLaunchKernelGGL(router_bf16_kernel<4>, grid, block, 0, stream, x, w_r, gain, bias,
                           eps, T, (int)d_h, (int)E, scores, logits);
    else
        hipLaunchKernelGGL(router_bf16_kernel<8>, grid, block, 0, stream, x, w_r, gain, bias,
                           eps, T, (int)d_h, (int)E, scores, logits);
    return hipGetLastError();
}

hipError_t launch_router_f32(const float *x, const float *w_r, const float *gain,
                             const float *bias, float eps, int64_t T, int64_t d_h,
                             int64_t E, float *scores, float *logits, hipStream_t stream)
{
    hipLaunchKernelGGL(router_f32_kernel, dim3((unsigned)T), dim3(256), 0, stream, x, w_r,
                       gain, bias, eps, T, (int)d_h, (int)E, scores, logits);
    return hipGetLastError();
}

}  // namespace blockffn
