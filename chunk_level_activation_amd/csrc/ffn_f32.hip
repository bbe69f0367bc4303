// fp32 chunk FFN: the same union-then-mask computation as the bf16 path, in plain
// fp32 fused multiply-adds (no reduced-precision matrix-core path), for workloads
// that run the layer in fp32.
//
// Skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
// Deployment", "Architecture Overview" and "Core Concept". For each chunk tile and
// each expert e of the chunk's union:
//     H_e[t,:] = s[t,e] * swish(W1_e x_t)        (up kernel, fp32 workspace)
//     y[t,:]   = sum_{e in U_c} W2_e H_e[t,:]    (down kernel)
// Sums run in ascending index order, union slots ascending, so results are
// deterministic.
#include "common.h"
#include "plan.h"

namespace blockffn {

// One workgroup per (chunk tile, union slot); a thread per (token row, hidden unit).
__global__ void __launch_bounds__(256)
up_f32_kernel(const float *__restrict__ x, const float *__restrict__ scores,
              const float *__restrict__ w1, const int32_t *__restrict__ lists,
              const int32_t *__restrict__ counts, float *__restrict__ hidden, int64_t T,
              int d_h, int E, int d_e, int64_t n, int MPC)
{
    const int slot = (int)(blockIdx.x % E);
    const int64_t ct = blockIdx.x / E;
    const int64_t c = ct / MPC;
    const int m = (int)(ct % MPC);
    if (slot >= counts[c])
        return;
    const int e = lists[c * E + slot];
    const int64_t tile_t0 = c * n + (int64_t)m * kTileM;
    const int64_t chunk_end = c * n + n < T ? c * n + n : T;
    for (int o = threadIdx.x; o < kTileM * d_e; o += 256) {
        const int tt = o / d_e, k = o % d_e;
        const int64_t t = tile_t0 + tt;
        float h = 0.0f;
        if (t < chunk_end) {
            const float *xr = x + t * d_h;
            const float *wr = w1 + ((int64_t)e * d_e + k) * d_h;
            float a = 0.0f;
            for (int j = 0; j < d_h; ++j)
                a = fmaf(wr[j], xr[j], a);
            h = swish_precise(a) * scores[t * E + e];
        }
        hidden[((ct * E + slot) * kTileM + tt) * d_e + k] = h;
    }
}

// One workgroup per (chunk tile, 256 output columns); a thread per column.
__global__ void __launch_bounds__(256)
down_f32_kernel(const float *__restrict__ hidden, const float *__restrict__ w2,
                const int32_t *__restrict__ lists, const int32_t *__restrict__ counts,
                float *__restrict__ y, int64_t T, int d_h, int E, int d_e, int64_t n,
                int MPC)
{
    const int JB = (d_h + 255) / 256;
    const int jb = (int)(blockIdx.x % JB);
    const int64_t ct = blockIdx.x / JB;
    const int64_t c = ct / MPC;
    const int m = (int)(ct % MPC);
    const int j = jb * 256 + threadIdx.x;
    if (j >= d_h)
        return;
    const int cnt = counts[c];
    const int64_t tile_t0 = c * n + (int64_t)m * kTileM;
    const int64_t chunk_end = c * n + n < T ? c * n + n : T;
    for (int tt = 0; tt < kTileM; ++tt) {
        const int64_t t = tile_t0 + tt;
        if (t >= chunk_end)
            break;
        float acc = 0.0f;
        for (int slot = 0; slot < cnt; ++slot) {
            const int e = lists[c * E + slot];
            const float *wr = w2 + ((int64_t)e * d_h + j) * d_e;
            const float *hr = hidden + ((ct * E + slot) * kTileM + tt) * d_e;
            for (int k = 0; k < d_e; ++k)
                acc = fmaf(wr[k], hr[k], acc);
        }
        y[t * d_h + j] = acc;
    }
}

hipError_t launch_ffn_f32(const FfnPlan &p, const float *x, const float *scores,
                          const float *w1, const float *w2, float *y, void *ws,
                          hipStream_t stream)
{
    char *base = static_cast<char *>(ws);
    const int32_t *lists = reinterpret_cast<const int32_t *>(base + p.off_lists);
    const int32_t *counts = reinterpret_cast<const int32_t *>(base + p.off_counts);
    float *hidden = reinterpret_cast<float *>(base + p.off_hidden);
    hipLaunchKernelGGL(up_f32_kernel, dim3((unsigned)(p.CT * p.E)), dim3(256), 0, stream, x,
                       scores, w1, lists, counts, hidden, p.T, (int)p.d_h, (int)p.E,
                       (int)p.d_e, p.n, (int)p.MPC);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int64_t JB = (p.d_h + 255) / 256;
    hipLaunchKernelGGL(down_f32_kernel, dim3((unsigned)(p.CT * JB)), dim3(256), 0, stream,
                       hidden, w2, lists, counts, y, p.T, (int)p.d_h, (int)p.E, (int)p.d_e,
                       p.n, (int)p.MPC);
    return hipGetLastError();
}

}  // namespace blockffn
