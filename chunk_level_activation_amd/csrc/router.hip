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
//
// Few tokens (decode) leave most of the chip idle with one workgroup per 32 tokens,
// so the d_h sum is split over S workgroups per token tile: each stores its 32 x E
// partial logits in the workspace, and the last of the S to arrive (an atomic
// counter) adds the S partials in split order, so the result does not depend on
// which workgroup finishes last, and applies ReLU and RMSNorm.
#include "common.h"
#include "plan.h"
#include "sync.h"

namespace blockffn {

// bf16: 32 tokens x all experts per workgroup, ET tiles of 32 experts, 8 waves. The
// workgroup's k range goes through LDS in chunks of KC: the x rows and the W_r rows of
// a chunk are loaded contiguously (16 bytes per lane, a row's pieces on consecutive
// lanes) into padded [row][k] tiles. The 32x32x16 bf16 MFMA then takes A = x rows
// (32 tokens x 16 k) and B = W_r rows transposed (16 k x 32 experts) from there. Wave
// w owns expert tile w % ET and every (8/ET)-th k step of the chunk; the 8/ET k parts
// of a tile meet in LDS after one barrier and are added in part order.
constexpr int kRouterThreads = 512;
constexpr int kRouterWaves = kRouterThreads / kWave;
constexpr int64_t kRouterTargetBlocks = 256;   // split the d_h sum until about this many (one per CU)
constexpr int kRouterMaxSplits = 8;
constexpr uint32_t kOOBRouter = 0x80000000u;   // buffer offset past every range: reads zero

// LOCAL: the S splits of a tile run on one XCD (the caller verified round-robin
// placement and laid the grid out so), and their partials meet in that XCD's L2;
// otherwise they meet in memory.
// Activation probability of a score (skill page, "Router Architecture Setup": the
// router also returns the sigmoid of the sharpened scores, used by the training
// losses).
__device__ __forceinline__ float router_prob(float s, float sharpness)
{
    return 1.0f / (1.0f + expf(-sharpness * s));
}

template <int ET, bool LOCAL>
__global__ void __launch_bounds__(kRouterThreads)
router_bf16_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w_r,
                   const float *__restrict__ gain, const float *__restrict__ bias,
                   float eps, int64_t T, int d_h, int E, int S, int X,
                   float *__restrict__ scores, float *__restrict__ logits,
                   float sharpness, float *__restrict__ probs,
                   float *__restrict__ part, uint32_t *__restrict__ arrive)
{
    constexpr int KPARTS = kRouterWaves / ET;
    constexpr int kPitch = ET * 32 + 1;
    // k per LDS chunk: (32 + 32 ET) rows of KC bf16 stay within 100 KB, so that a
    // workgroup's range (d_h / S) usually is one chunk: one memory round trip
    constexpr int KC = ET <= 2 ? 512 : (ET <= 4 ? 256 : 128);
    constexpr int KP = KC + 8;                        // row pitch (bf16): conflict-free reads
    constexpr int PPR = KC / 8;                       // 16-byte pieces per row
    constexpr int NROWS = kTileM + ET * 32;
    constexpr int NX = kTileM * PPR / kRouterThreads;                        // x pieces per thread
    constexpr int NW = (ET * 32 * PPR + kRouterThreads - 1) / kRouterThreads;   // W_r pieces
    static_assert(kTileM * PPR % kRouterThreads == 0, "x pieces fill the threads");
    __shared__ float red[KPARTS][kTileM][kPitch];
    __shared__ alignas(16) uint16_t ops[NROWS * KP];   // x rows, then the W_r rows
    __shared__ float sgain[ET * 32], sbias[ET * 32];
    __shared__ int last;

    // workgroup -> (tile, split)
    int64_t tile;
    int split;
    if (LOCAL) {
        // workgroup b runs on XCD b % X; tile t lives on XCD t % X, so its splits are
        // the workgroups (m*S + s)*X + t % X with m = t / X
        const int xcd = blockIdx.x % X;
        const int k = blockIdx.x / X;
        tile = (int64_t)(k / S) * X + xcd;
        split = k % S;
        if (tile * kTileM >= T)
            return;
    } else {
        tile = blockIdx.x / S;
        split = blockIdx.x % S;
    }
    const int64_t t0 = tile * kTileM;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int row = lane % 32;
    const int kg = lane / 32;
    const int et = wave % ET, kp = wave / ET;
    if (tid < E) {
        sgain[tid] = gain ? gain[tid] : 1.0f;
        sbias[tid] = bias ? bias[tid] : 0.0f;
    }
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        acc[i] = 0.0f;
    // this split's range of 16-wide k steps
    const int KS = d_h / 16;
    const int ks0 = (int)((int64_t)KS * split / S), ks1 = (int)((int64_t)KS * (split + 1) / S);
    const int k_end = ks1 * 16;
    // the tile's rows of x (offsets stay small whatever T is) and all of W_r
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + t0 * d_h, (uint64_t)kTileM * d_h * 2);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_r, (uint64_t)E * d_h * 2);
    for (int kc = ks0 * 16; kc < k_end; kc += KC) {
        // piece q = tid + 512 i: row q / PPR, k kc + (q % PPR) * 8, of the x rows and of the
        // W_r rows (each with its own buffer, so the descriptor stays uniform); rows past
        // T or E, pieces past the range and q past the rows read zero
        bf16x8 vx[NX], vw[NW];
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int q = tid + i * kRouterThreads;
            const int r = q / PPR, k = kc + (q % PPR) * 8;
            vx[i] = bload<0>(rx, k < k_end && t0 + r < T ? (uint32_t)((r * d_h + k) * 2) : kOOBRouter);
        }
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int q = tid + i * kRouterThreads;
            const int r = q / PPR, k = kc + (q % PPR) * 8;
            vw[i] = bload<0>(rw, q < ET * 32 * PPR && k < k_end && r < E ? (uint32_t)((r * d_h + k) * 2)
                                                                        : kOOBRouter);
        }
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int q = tid + i * kRouterThreads;
            *reinterpret_cast<bf16x8 *>(&ops[(q / PPR) * KP + (q % PPR) * 8]) = vx[i];
        }
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int q = tid + i * kRouterThreads;
            if (q < ET * 32 * PPR)
                *reinterpret_cast<bf16x8 *>(&ops[(kTileM + q / PPR) * KP + (q % PPR) * 8]) = vw[i];
        }
        __syncthreads();
        const int nsteps = (k_end - kc < KC ? k_end - kc : KC) / 16;
        for (int st = kp; st < nsteps; st += KPARTS) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&ops[row * KP + st * 16 + kg * 8]);
            const bf16x8 b =
                *reinterpret_cast<const bf16x8 *>(&ops[(kTileM + et * 32 + row) * KP + st * 16 + kg * 8]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }

    // 32x32 accumulator layout: element i is row (i/4)*8 + (lane/32)*4 + i%4 (token)
    // of column lane%32 (expert).
#pragma unroll
    for (int i = 0; i < 16; ++i)
        red[kp][(i / 4) * 8 + kg * 4 + (i % 4)][et * 32 + row] = acc[i];
    __syncthreads();
    // k parts in order -> red[0]
    for (int v = tid; v < kTileM * E; v += kRouterThreads) {
        const int tt = v / E, e = v % E;
        float sum = red[0][tt][e];
#pragma unroll
        for (int q = 1; q < KPARTS; ++q)
            sum += red[q][tt][e];
        red[0][tt][e] = sum;
    }
    __syncthreads();
    float(*lg)[kPitch] = red[0];

    if (S > 1) {
        // partial logits of this split -> workspace, then count the arrival. Four
        // floats per access.
        constexpr int kPol = LOCAL ? kSC0 : kSC1;
        const int tile_floats = kTileM * E;
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(part + (uint64_t)tile * S * tile_floats, (uint64_t)S * tile_floats * 4);
        for (int v = tid * 4; v < tile_floats; v += kRouterThreads * 4) {
            float4 o;
            o.x = lg[v / E][v % E];
            o.y = lg[(v + 1) / E][(v + 1) % E];
            o.z = lg[(v + 2) / E][(v + 2) % E];
            o.w = lg[(v + 3) / E][(v + 3) % E];
            bstore_f4<kPol>(rp, (uint32_t)((split * tile_floats + v) * 4), o);
        }
        drain_memory();
        __syncthreads();
        if (tid == 0) {
            const uint32_t prev = add_counter(&arrive[tile], 1u);
            last = prev == (uint32_t)(S - 1);
            if (last)
                st_counter(&arrive[tile], 0u);
        }
        __syncthreads();
        if (!last)
            return;
        // the last split adds all S partials in split order; all loads in flight first
        for (int v = tid * 4; v < tile_floats; v += kRouterThreads * 4) {
            float4 pv[kRouterMaxSplits];
#pragma unroll
            for (int q = 0; q < kRouterMaxSplits; ++q)
                if (q < S)
                    pv[q] = bload_f4<kPol>(rp, (uint32_t)((q * tile_floats + v) * 4));
            float4 sum = pv[0];
#pragma unroll
            for (int q = 1; q < kRouterMaxSplits; ++q)
                if (q < S) {
                    sum.x += pv[q].x;
                    sum.y += pv[q].y;
                    sum.z += pv[q].z;
                    sum.w += pv[q].w;
                }
            lg[v / E][v % E] = sum.x;
            lg[(v + 1) / E][(v + 1) % E] = sum.y;
            lg[(v + 2) / E][(v + 2) % E] = sum.z;
            lg[(v + 3) / E][(v + 3) % E] = sum.w;
        }
        __syncthreads();
    }

    // Epilogue: 16 threads per token.
    const int tt = tid / 16, sub = tid % 16;
    const int64_t t = t0 + tt;
    float sumsq = 0.0f;
    for (int e = sub; e < E; e += 16) {
        const float l = bias ? lg[tt][e] + sbias[e] : lg[tt][e];
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
            const float s = r * inv * sgain[e];
            scores[t * E + e] = s;
            if (logits)
                logits[t * E + e] = l;
            if (probs)
                probs[t * E + e] = router_prob(s, sharpness);
        }
    }
}

// fp32: one workgroup per token, one thread per expert (E <= 256), fp32 FMA.
__global__ void __launch_bounds__(256)
router_f32_kernel(const float *__restrict__ x, const float *__restrict__ w_r,
                  const float *__restrict__ gain, const float *__restrict__ bias, float eps,
                  int64_t T, int d_h, int E, float *__restrict__ scores,
                  float *__restrict__ logits, float sharpness, float *__restrict__ probs)
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
        const float s = r * inv * (gain ? gain[e] : 1.0f);
        scores[t * E + e] = s;
        if (logits)
            logits[t * E + e] = l;
        if (probs)
            probs[t * E + e] = router_prob(s, sharpness);
    }
}

int router_splits(int64_t T, int64_t d_h)
{
    const int64_t tiles = (T + kTileM - 1) / kTileM;
    // at least two 16-wide k steps per wave of a split
    const int64_t smax = d_h / (16 * 2 * kRouterWaves);
    int64_t s = (kRouterTargetBlocks + tiles - 1) / tiles;
    if (s > smax)
        s = smax;
    if (s > kRouterMaxSplits)
        s = kRouterMaxSplits;
    return s < 2 ? 1 : (int)s;
}

size_t router_workspace_bytes(int64_t T, int64_t d_h, int64_t E)
{
    const int S = router_splits(T, d_h);
    if (S == 1)
        return 0;
    const int64_t tiles = (T + kTileM - 1) / kTileM;
    return kRouterControlBytes + (size_t)tiles * S * kTileM * E * sizeof(float);
}

hipError_t launch_router_bf16(const uint16_t *x, const uint16_t *w_r, const float *gain,
                              const float *bias, float eps, int64_t T, int64_t d_h,
                              int64_t E, float *scores, float *logits, float sharpness,
                              float *probs, void *ws, int xcds, hipStream_t stream)
{
    const int64_t tiles = (T + kTileM - 1) / kTileM;
    const int S = ws ? router_splits(T, d_h) : 1;
    uint32_t *arrive = static_cast<uint32_t *>(ws);
    float *part = ws ? reinterpret_cast<float *>(static_cast<char *>(ws) + kRouterControlBytes)
                     : nullptr;
    const bool local = S > 1 && xcds > 1;
    const int X = local ? xcds : 1;
    const int64_t blocks = local ? (tiles + X - 1) / X * S * X : tiles * S;
    const dim3 grid((unsigned)blocks), block(kRouterThreads);
    const int ET = (int)((E + 31) / 32);
#define ROUTER_LAUNCH(N, L)                                                                 \
    hipLaunchKernelGGL((router_bf16_kernel<N, L>), grid, block, 0, stream, x, w_r, gain,    \
                       bias, eps, T, (int)d_h, (int)E, S, X, scores, logits, sharpness, probs,    \
                       part, arrive)
#define ROUTER_LAUNCH_ET(L)   \
    if (ET <= 1)              \
        ROUTER_LAUNCH(1, L);  \
    else if (ET <= 2)         \
        ROUTER_LAUNCH(2, L);  \
    else if (ET <= 4)         \
        ROUTER_LAUNCH(4, L);  \
    else                      \
        ROUTER_LAUNCH(8, L);
    if (local) {
        ROUTER_LAUNCH_ET(true)
    } else {
        ROUTER_LAUNCH_ET(false)
    }
#undef ROUTER_LAUNCH_ET
#undef ROUTER_LAUNCH
    return hipGetLastError();
}

hipError_t launch_router_f32(const float *x, const float *w_r, const float *gain,
                             const float *bias, float eps, int64_t T, int64_t d_h,
                             int64_t E, float *scores, float *logits, float sharpness,
                             float *probs, hipStream_t stream)
{
    hipLaunchKernelGGL(router_f32_kernel, dim3((unsigned)T), dim3(256), 0, stream, x, w_r,
                       gain, bias, eps, T, (int)d_h, (int)E, scores, logits, sharpness, probs);
    return hipGetLastError();
}

}  // namespace blockffn
