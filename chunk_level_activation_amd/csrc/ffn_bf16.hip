// bf16 chunk FFN on the gfx950 matrix cores: gathered up-projection with Swish and
// score scaling, then the down-projection summed over the chunk's union.
//
// Skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
// Deployment": "Architecture Overview" (experts are non-gated MLPs with Swish,
// d_e << d_h; the pages' kernel processes n = 32 tokens at once and computes only the
// union of activated experts) and "Core Concept" (unneeded activations are masked
// after the computation). For each chunk tile (32 token rows) and each expert e of
// the chunk's union U_c:
//     Ht_e[t,:] = bf16( s[t,e] * swish(W1_e x_t) )          (up kernel)
//     y[t,:]    = bf16( sum_{e in U_c} W2_e Ht_e[t,:] )        (down kernel)
// Scaling the hidden row by s before W2 equals scaling the expert output after it
// (the map is linear); a token whose score is 0 gets an all-zero hidden row, which
// is the masking. Experts outside U_c are never read.
//
// Data layout (all row-major): x [T, d_h], W1 [E, d_e, d_h], W2 [E, d_h, d_e],
// hidden workspace Ht [chunk tile][union slot][32][d_e] bf16, so a chunk's union
// occupies consecutive slots 0..|U_c|-1.
#include "common.h"
#include "plan.h"

namespace blockffn {

// ------------------------------------------------------------------ up-projection
// One workgroup (4 waves) per (chunk tile, union slot, 16 rows of d_e). The 16x16x32
// bf16 MFMA takes A = x rows (16 tokens x 32 k) and B = W1 rows transposed (32 k x
// 16 hidden units); the two token halves of the tile share every W1 fragment. The
// four waves interleave over the k steps of d_h and their partial sums are added in
// a fixed order through LDS. W1 is read once per tile with 16-byte loads, each wave
// instruction covering 16 rows x 64 contiguous bytes.
constexpr int kUpRows = 16;

__global__ void __launch_bounds__(256)
up_bf16_kernel(const uint16_t *__restrict__ x, const float *__restrict__ scores,
               const uint16_t *__restrict__ w1, const int32_t *__restrict__ lists,
               const int32_t *__restrict__ counts, uint16_t *__restrict__ hidden,
               int64_t T, int d_h, int E, int d_e, int64_t n, int MPC)
{
    const int RT = d_e / kUpRows;
    int64_t item = blockIdx.x;
    const int rt = (int)(item % RT);
    item /= RT;
    const int slot = (int)(item % E);
    const int64_t ct = item / E;
    const int64_t c = ct / MPC;
    const int m = (int)(ct % MPC);
    if (slot >= counts[c])
        return;
    const int e = lists[c * E + slot];

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int r = lane % 16;         // A: token row within a half; B: hidden unit
    const int kg = lane / 16;        // k group of 8 within the 32-wide k step
    const int64_t tile_t0 = c * n + (int64_t)m * kTileM;
    const int64_t chunk_end = c * n + n < T ? c * n + n : T;

    const int64_t ta = tile_t0 + r, tb = tile_t0 + 16 + r;
    const bool va = ta < chunk_end, vb = tb < chunk_end;
    const uint16_t *xa = x + (va ? ta : 0) * d_h + kg * 8;
    const uint16_t *xb = x + (vb ? tb : 0) * d_h + kg * 8;
    const uint16_t *wr = w1 + ((int64_t)e * d_e + rt * kUpRows + r) * d_h + kg * 8;

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc1 = {0.f, 0.f, 0.f, 0.f};
    const int KS = d_h / 32;
#pragma unroll 4
    for (int ks = wave; ks < KS; ks += 4) {
        const int k0 = ks * 32;
        const bf16x8 b = load_bf16x8_stream(wr + k0);
        const bf16x8 a0 = va ? load_bf16x8(xa + k0) : zero_bf16x8();
        const bf16x8 a1 = vb ? load_bf16x8(xb + k0) : zero_bf16x8();
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc1, 0, 0, 0);
    }

    // 16x16 accumulator layout: lane holds rows (lane/16)*4 + i of column lane%16.
    __shared__ float red[4][kTileM][kUpRows + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        red[wave][kg * 4 + i][r] = acc0[i];
        red[wave][16 + kg * 4 + i][r] = acc1[i];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < kTileM * kUpRows; o += 256) {
        const int tt = o / kUpRows, rr = o % kUpRows;
        const float a = ((red[0][tt][rr] + red[1][tt][rr]) + red[2][tt][rr]) + red[3][tt][rr];
        const int64_t t = tile_t0 + tt;
        const float s = t < chunk_end ? scores[t * E + e] : 0.0f;
        const float h = t < chunk_end ? swish_fast(a) * s : 0.0f;
        hidden[((ct * E + slot) * kTileM + tt) * d_e + rt * kUpRows + rr] = f32_to_bf16(h);
    }
}

// ------------------------------------------------------------------ down-projection
// One workgroup per (chunk tile, 32 columns of d_h, expert group). The 32x32x16 bf16
// MFMA takes A = hidden rows (32 tokens x 16 k) and B = W2 rows transposed (16 k x
// 32 output columns). The four waves take every fourth union slot of the group and
// are summed in a fixed order through LDS. With G > 1 groups the partial tiles go to
// the workspace and the last group to arrive (an atomic counter per tile, reset by
// the union kernel of the same call) adds them in group order and writes y.
__global__ void __launch_bounds__(256)
down_bf16_kernel(const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ w2,
                 const int32_t *__restrict__ lists, const int32_t *__restrict__ counts,
                 uint16_t *__restrict__ y, float *__restrict__ partials,
                 uint32_t *__restrict__ ctrl, int64_t T, int d_h, int E, int d_e,
                 int64_t n, int MPC, int G)
{
    const int JT = d_h / 32;
    int64_t item = blockIdx.x;
    const int g = (int)(item % G);
    item /= G;
    const int jt = (int)(item % JT);
    const int64_t ct = item / JT;
    const int64_t c = ct / MPC;
    const int m = (int)(ct % MPC);
    const int cnt = counts[c];
    const int per = (cnt + G - 1) / G;
    const int s_begin = g * per < cnt ? g * per : cnt;
    const int s_end = s_begin + per < cnt ? s_begin + per : cnt;

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int col = lane % 32;      // A: token row; B: output column
    const int kg = lane / 32;       // k group of 8 within the 16-wide k step
    const int KS = d_e / 16;

    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        acc[i] = 0.0f;
    for (int slot = s_begin + wave; slot < s_end; slot += 4) {
        const int e = lists[c * E + slot];
        const uint16_t *hr = hidden + ((ct * E + slot) * kTileM + col) * d_e + kg * 8;
        const uint16_t *wr = w2 + ((int64_t)e * d_h + jt * 32 + col) * d_e + kg * 8;
#pragma unroll 4
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = load_bf16x8(hr + ks * 16);
            const bf16x8 b = load_bf16x8_stream(wr + ks * 16);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
    }

    // 32x32 accumulator layout: element i of a lane is row (i/4)*8 + (lane/32)*4 +
    // i%4 of column lane%32.
    __shared__ float red[4][kTileM][33];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        red[wave][(i / 4) * 8 + kg * 4 + (i % 4)][col] = acc[i];
    __syncthreads();

    const int64_t tile_t0 = c * n + (int64_t)m * kTileM;
    const int64_t chunk_end = c * n + n < T ? c * n + n : T;
    float out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int o = threadIdx.x + q * 256;
        const int tt = o / 32, jj = o % 32;
        out[q] = ((red[0][tt][jj] + red[1][tt][jj]) + red[2][tt][jj]) + red[3][tt][jj];
    }

    if (G > 1) {
        float *mine = partials + ((ct * JT + jt) * G + g) * (kTileM * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            mine[threadIdx.x + q * 256] = out[q];
        __threadfence();
        __syncthreads();
        __shared__ int is_last;
        if (threadIdx.x == 0)
            is_last = atomicAdd(&ctrl[ct * JT + jt], 1u) == (unsigned)(G - 1);
        __syncthreads();
        if (!is_last)
            return;
        __threadfence();
        const float *all = partials + (ct * JT + jt) * G * (kTileM * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float sum = 0.0f;
            for (int gg = 0; gg < G; ++gg)
                sum += all[gg * (kTileM * 32) + threadIdx.x + q * 256];
            out[q] = sum;
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int o = threadIdx.x + q * 256;
        const int tt = o / 32, jj = o % 32;
        const int64_t t = tile_t0 + tt;
        if (t < chunk_end)
            y[t * d_h + jt * 32 + jj] = f32_to_bf16(out[q]);
    }
}

hipError_t launch_ffn_bf16(const FfnPlan &p, const uint16_t *x, const float *scores,
                           const uint16_t *w1, const uint16_t *w2, uint16_t *y, void *ws,
                           hipStream_t stream)
{
    char *base = static_cast<char *>(ws);
    const int32_t *lists = reinterpret_cast<const int32_t *>(base + p.off_lists);
    const int32_t *counts = reinterpret_cast<const int32_t *>(base + p.off_counts);
    uint16_t *hidden = reinterpret_cast<uint16_t *>(base + p.off_hidden);
    const int64_t up_items = p.CT * p.E * (p.d_e / kUpRows);
    hipLaunchKernelGGL(up_bf16_kernel, dim3((unsigned)up_items), dim3(256), 0, stream, x,
                       scores, w1, lists, counts, hidden, p.T, (int)p.d_h, (int)p.E,
                       (int)p.d_e, p.n, (int)p.MPC);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int64_t down_items = p.CT * p.JT * p.G;
    hipLaunchKernelGGL(down_bf16_kernel, dim3((unsigned)down_items), dim3(256), 0, stream,
                       hidden, w2, lists, counts, y,
                       reinterpret_cast<float *>(base + p.off_partials),
                       reinterpret_cast<uint32_t *>(base + p.off_ctrl), p.T, (int)p.d_h,
                       (int)p.E, (int)p.d_e, p.n, (int)p.MPC, (int)p.G);
    return hipGetLastError();
}

}  // namespace blockffn
