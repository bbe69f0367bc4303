// Layer backward of BlockFFN: gradients of the router + chunk-union expert FFN with
// respect to x, W_r, gain, bias, W1 and W2, for bf16 inputs, in fp32.
//
// Skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
// Deployment": "Architecture Overview" (ReLU + RMSNorm router, non-gated Swish
// experts; the router is trained end to end through these differentiable parts),
// "Core Concept" (each chunk evaluates the union of its tokens' experts and masks by
// the scores), "Router Architecture Setup" (probabilities sigmoid(sharpness * s)).
// For an upstream gradient dy of y and, optionally, dprobs of the probabilities:
//
//   e in U_c(t):  a = W1_e x_t,  h = swish(a),  G_t = W2_e^T dy_t
//                 ds[t,e] = G_t . h                      (= dy_t . W2_e h)
//                 dA[t,e] = s[t,e] G_t * swish'(a),      SH[t,e] = s[t,e] h
//                 dW1_e = sum_t dA^T x_t,  dW2_e = sum_t dy_t SH^T,  dx_t = sum_e W1_e^T dA
//   router:       ds += dprobs sharpness p (1 - p);  RMSNorm and ReLU backward give dl,
//                 dx += W_r^T dl,  dW_r = sum_t dl x_t^T,  dbias = sum_t dl,
//                 dgain_e = sum_t ds r inv
//
// Kernels, in stream order (all products on 32x32x16 bf16 MFMA, fp32 accumulation):
//   0. the forward router (recomputed: logits and scores, with its d_h split when it
//      takes one), the chunk unions and the per-expert tile lists (the forward's
//      kernels);
//   1. transpose_tiles_kernel: x and dy copied per 32-token chunk tile as
//      [tile][d_h][32 tokens], so the weight-gradient products, whose k is the token,
//      read k-contiguous operands;
//   2. expert_pass_kernel, workgroup = (expert e, 4 of its tiles), 8 waves: a = X W1_e^T
//      on waves 0-3 and G = DY W2_e on waves 4-7 over d_h (B = W2^T rows), both on the
//      128 x 128 tile loop of tile_gemm.h; then ds, and dA and SH in bf16 in both
//      [token][unit] and [unit][token] order;
//   3. wgrad_kernel, workgroup = (expert, dW1 or dW2, 128 x 128 output tile): k over the
//      expert's tiles' tokens; every output element is owned by one workgroup (an
//      expert no chunk uses gets zeros);
//   4. dx_kernel, workgroup = (4 tiles, 128 columns, expert split): k over the union of
//      the 4 chunks' unions x d_e, B = W1^T rows (W1 and W2 are transposed once per call
//      into the workspace, for the experts some chunk uses, so every product reads
//      k-contiguous operands); with few tiles the experts are split over workgroups
//      and the fp32 partials added in split order;
//   5. router_token_kernel: per token, dl and the router's share of dx;
//      router_param_kernel: dW_r, dgain, dbias as sums over the tokens in order.
// Every sum runs in a fixed order, so equal inputs give equal bits.
#include "common.h"
#include "plan.h"
#include "sync.h"
#include "tile_gemm.h"

namespace blockffn {

namespace {

constexpr int kBT = 256;                  // threads per workgroup, 4 waves
constexpr int kTM = 128;                  // 128 x 128 output tiles
constexpr int kXN = 256;                  // dx columns per workgroup
constexpr int kPassTiles = 4;             // chunk tiles per expert-pass workgroup
constexpr int kTrCols = 256;              // d_h columns per transpose workgroup
using tile::acc_row;
using tile::kDepth;
using tile::kloop_128x128;
using tile::kOOB;
using tile::kPK;
using tile::kPKP;
using tile::load16;
using tile::mma_64x64;
static_assert(kBT == tile::kThreads, "the 128 x 128 tile loop runs on 4 waves");

struct Dims {
    int64_t T;
    int n, d_h, E, d_e, C, W, MPC, CT;
};

// Token of row r of chunk tile `tile`, or -1 when the row holds no token.
__device__ __forceinline__ int64_t tile_token(const Dims &d, int tile, int r)
{
    if (tile < 0)
        return -1;
    const int c = tile / d.MPC, m = tile % d.MPC;
    const int in_chunk = m * kTileM + r;
    const int64_t t = (int64_t)c * d.n + in_chunk;
    return (in_chunk < d.n && t < d.T) ? t : -1;
}

// The weight-gradient kernel keeps k = one tile's 32 tokens per step with one step of
// prefetch: its grid (E x 2 x 128-square tiles) already gives each CU several
// workgroups, and the deeper loop's registers would cost that occupancy.
constexpr int kWBK = 32;
constexpr int kWLP = kWBK + 8;

__device__ __forceinline__ void zero_acc(f32x16 &a)
{
#pragma unroll
    for (int v = 0; v < 16; ++v)
        a[v] = 0.0f;
}

// ------------------------------------------------------------------ 1. tile transposes
// dst[tile][j][r] = src[token(tile, r)][j] (zero for rows without a token).
__global__ void __launch_bounds__(kBT) transpose_tiles_kernel(const uint16_t *src, Dims d,
                                                              uint16_t *dst)
{
    __shared__ alignas(16) uint16_t t[kTileM][kTrCols + 8];
    const int tile = blockIdx.x, jb = blockIdx.y * kTrCols, tid = threadIdx.x;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint64_t)d.T * d.d_h * 2);
#pragma unroll
    for (int q = 0; q < kTileM * kTrCols / 8 / kBT; ++q) {
        const int v = q * kBT + tid, row = v / (kTrCols / 8), jv = v % (kTrCols / 8);
        const int64_t tok = tile_token(d, tile, row);
        const uint32_t off = tok >= 0 ? (uint32_t)((tok * d.d_h + jb + jv * 8) * 2) : kOOB;
        *reinterpret_cast<u32x4 *>(&t[row][jv * 8]) = load16(rs, off);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kTileM * kTrCols / 8 / kBT; ++q) {
        const int v = q * kBT + tid, j = v / 4, tv = v % 4;
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = (uint32_t)t[tv * 8 + 2 * i][j] | ((uint32_t)t[tv * 8 + 2 * i + 1][j] << 16);
        *reinterpret_cast<u32x4 *>(&dst[(((int64_t)tile * d.d_h + jb + j) * kTileM) + tv * 8]) = o;
    }
}

// Per expert, dst[e] = src[e]^T for an R x Cc bf16 matrix (64 x 64 blocks through LDS);
// experts that no chunk uses are skipped (their copy is never read).
__global__ void __launch_bounds__(kBT) transpose_weights_kernel(const uint16_t *src, int R, int Cc,
                                                                const int32_t *tile_count,
                                                                uint16_t *dst)
{
    __shared__ alignas(16) uint16_t t[64][64 + 8];
    const int e = blockIdx.z;
    if (tile_count[e] == 0)
        return;
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64, tid = threadIdx.x;
    const uint16_t *s = src + (int64_t)e * R * Cc;
    uint16_t *o = dst + (int64_t)e * R * Cc;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int v = q * kBT + tid, row = v / 8, cv = v % 8;
        *reinterpret_cast<u32x4 *>(&t[row][cv * 8]) =
            *reinterpret_cast<const u32x4 *>(&s[(int64_t)(r0 + row) * Cc + c0 + cv * 8]);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int v = q * kBT + tid, col = v / 8, rv = v % 8;
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)t[rv * 8 + 2 * i][col] | ((uint32_t)t[rv * 8 + 2 * i + 1][col] << 16);
        *reinterpret_cast<u32x4 *>(&o[(int64_t)(c0 + col) * R + r0 + rv * 8]) = w;
    }
}

// ------------------------------------------------------------------ 2. expert pass
struct PassArgs {
    const uint16_t *x, *dy, *w1, *w2t;    // w2t [E][d_e][d_h]: W2 transposed
    const float *scores;          // recomputed forward scores [T][E]
    const int32_t *tile_list, *tile_count;
    float *ds;                    // [T][E], written for e in U_c(t)
    uint16_t *da_tu, *da_ut, *sh_ut;
    Dims d;
};

constexpr int kPP = kPKP;                 // the expert pass's LDS pitch (same k step)
constexpr int kPassThreads = 2 * kBT;     // two 4-wave groups: X W1^T and DY W2

// Waves 0-3 multiply X by W1_e^T and waves 4-7 DY by W2_e (the same 128 x 128 tile
// loop on their own LDS tiles, three k steps of loads in flight); the second group then
// hands G to the first through LDS (each thread's accumulators to the thread with the
// same position in the first group), which applies the epilogue.
__global__ void __launch_bounds__(kPassThreads, 2) expert_pass_kernel(PassArgs a)
{
    const Dims &d = a.d;
    const int e = blockIdx.x % d.E, grp = blockIdx.x / d.E;
    const int cnt = a.tile_count[e];
    if (grp * kPassTiles >= cnt)
        return;
    // operand tiles As1 Bs1 As2 Bs2, reused after the k loop for the hand-over of G
    __shared__ alignas(16) uint16_t ops[4 * kTM * kPP];
    static_assert(sizeof(ops) >= (size_t)kBT * 64 * sizeof(float), "G hand-over fits the operand tiles");
    __shared__ float red[kTM][65];
    __shared__ float dsacc[kTM], scol[kTM];
    __shared__ int64_t tok[kTM];
    __shared__ int tiles[kPassTiles];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int g = __builtin_amdgcn_readfirstlane(wave >> 2);   // 0: X W1^T, 1: DY W2
    const int gt = tid & (kBT - 1);                            // thread within the group
    const int wm = wave & 1, wn = (wave >> 1) & 1;
    if (tid < kPassTiles)
        tiles[tid] = grp * kPassTiles + tid < cnt ? a.tile_list[(int64_t)e * d.CT + grp * kPassTiles + tid] : -1;
    __syncthreads();
    if (tid < kTM) {
        const int64_t t = tile_token(d, tiles[tid / kTileM], tid % kTileM);
        tok[tid] = t;
        scol[tid] = t >= 0 ? a.scores[t * d.E + e] : 0.0f;
        dsacc[tid] = 0.0f;
    }
    __syncthreads();

    // the group's operands: token rows of x or dy, hidden-unit rows of W1 or W2^T (both
    // [E][d_e][d_h], so the same offsets serve either)
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(g ? a.dy : a.x, (uint64_t)d.T * d.d_h * 2);
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc(g ? a.w2t : a.w1, (uint64_t)d.E * d.d_e * d.d_h * 2);
    uint16_t *As = ops + (2 * g) * kTM * kPP, *Bs = ops + (2 * g + 1) * kTM * kPP;
    // piece i of this thread: row (gt + 256 i) / 8, k offset (gt % 8) * 8
    constexpr int kV = kTM * kPK / 8 / kBT;    // 4
    uint32_t xoff[kV], xmask[kV];
#pragma unroll
    for (int i = 0; i < kV; ++i) {
        const int q = gt + i * kBT;
        const int64_t t = tok[q >> 3];
        xmask[i] = 0u - (uint32_t)(t >= 0);
        xoff[i] = t >= 0 ? (uint32_t)((t * d.d_h + (q & 7) * 8) * 2) : 0u;
    }
    const int KS = d.d_h / kPK;
    float *gbuf = reinterpret_cast<float *>(ops);   // [64 values][256 threads]
    for (int u0 = 0; u0 < d.d_e; u0 += kTM) {
        uint32_t woff[kV];
#pragma unroll
        for (int i = 0; i < kV; ++i) {
            const int q = gt + i * kBT;
            woff[i] = (uint32_t)((((int64_t)e * d.d_e + u0 + (q >> 3)) * d.d_h + (q & 7) * 8) * 2);
        }
        auto load = [&](int s, u32x4(&ra)[4], u32x4(&rb)[4]) {
            const uint32_t okm = 0u - (uint32_t)(s < KS);
            const uint32_t ko = (uint32_t)(s * kPK * 2);
#pragma unroll
            for (int i = 0; i < kV; ++i) {
                const uint32_t am = okm & xmask[i];
                ra[i] = load16(rA, ((xoff[i] + ko) & am) | (kOOB & ~am));
                rb[i] = load16(rB, ((woff[i] + ko) & okm) | (kOOB & ~okm));
            }
        };
        f32x16 acc[2][2];
        tile::zero_acc(acc);
        kloop_128x128(load, KS, As, Bs, acc, gt, wm, wn, lane);
        // the k loop ended with a barrier: the operand tiles are free for G
        if (g == 1) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        gbuf[((i * 2 + j) * 16 + v) * kBT + gt] = acc[i][j][v];
        }
        __syncthreads();
        if (g == 0) {
            // epilogue: Swish, its slope, the score
            float part[2][16];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    part[i][v] = 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int unit = u0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
                    for (int vg = 0; vg < 4; ++vg) {
                        uint32_t da_pk[2] = {0u, 0u}, sh_pk[2] = {0u, 0u};
                        const int row0 = wm * 64 + i * 32 + acc_row(vg * 4, lane);   // 4 consecutive rows
                        const int tile = tiles[row0 / kTileM];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int v = vg * 4 + q, row = row0 + q;
                            const float av = acc[i][j][v], s = scol[row];
                            const float gv = gbuf[((i * 2 + j) * 16 + v) * kBT + gt];
                            const float sig = 1.0f / (1.0f + expf(-av));
                            const float h = av * sig;
                            part[i][v] += gv * h;
                            const float dA = s * gv * (sig * (1.0f + av * (1.0f - sig)));
                            const float sh = s * h;
                            const uint32_t b_da = f32_to_bf16(dA), b_sh = f32_to_bf16(sh);
                            da_pk[q >> 1] |= b_da << ((q & 1) * 16);
                            sh_pk[q >> 1] |= b_sh << ((q & 1) * 16);
                            if (tile >= 0)
                                a.da_tu[(((int64_t)tile * d.E + e) * kTileM + row % kTileM) * d.d_e + unit] =
                                    (uint16_t)b_da;
                        }
                        if (tile >= 0) {
                            const int64_t o = (((int64_t)tile * d.E + e) * d.d_e + unit) * kTileM + row0 % kTileM;
                            *reinterpret_cast<uint64_t *>(&a.da_ut[o]) = (uint64_t)da_pk[0] | ((uint64_t)da_pk[1] << 32);
                            *reinterpret_cast<uint64_t *>(&a.sh_ut[o]) = (uint64_t)sh_pk[0] | ((uint64_t)sh_pk[1] << 32);
                        }
                    }
                }
            // ds: per-lane row partials -> LDS [row][64 columns] -> summed in column order
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    red[wm * 64 + i * 32 + acc_row(v, lane)][wn * 32 + (lane & 31)] = part[i][v];
        }
        __syncthreads();
        if (tid < kTM) {
            float sum = 0.0f;
            for (int c = 0; c < 64; ++c)
                sum += red[tid][c];
            dsacc[tid] += sum;
        }
        __syncthreads();
    }
    if (tid < kTM && tok[tid] >= 0)
        a.ds[tok[tid] * d.E + e] = dsacc[tid];
}

// ------------------------------------------------------------------ 3. weight gradients
struct WgradArgs {
    const uint16_t *xt, *dyt;             // [CT][d_h][32]
    const uint16_t *da_ut, *sh_ut;        // [CT][E][d_e][32]
    const int32_t *tile_list, *tile_count;
    float *dw1, *dw2;
    Dims d;
};

__global__ void __launch_bounds__(kBT, 2) wgrad_kernel(WgradArgs a)
{
    const Dims &d = a.d;
    const int e = blockIdx.x % d.E;
    const int rest = blockIdx.x / d.E;
    const int kind = rest & 1, t2 = rest >> 1;
    const int M = kind == 0 ? d.d_e : d.d_h, N = kind == 0 ? d.d_h : d.d_e;
    const int MT = M / kTM;
    const int mt = t2 % MT, nt = t2 / MT;
    __shared__ alignas(16) uint16_t As[kTM * kWLP], Bs[kTM * kWLP];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave & 1, wn = wave >> 1;
    const int cnt = a.tile_count[e];
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(a.xt, (uint64_t)d.CT * d.d_h * kTileM * 2);
    const __amdgpu_buffer_rsrc_t rdt = make_rsrc(a.dyt, (uint64_t)d.CT * d.d_h * kTileM * 2);
    const __amdgpu_buffer_rsrc_t rda = make_rsrc(a.da_ut, (uint64_t)d.CT * d.E * d.d_e * kTileM * 2);
    const __amdgpu_buffer_rsrc_t rsh = make_rsrc(a.sh_ut, (uint64_t)d.CT * d.E * d.d_e * kTileM * 2);
    // A rows = m (unit for dW1, hidden column for dW2), B rows = n; k = the tile's tokens
    int srow[2], skv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + i * kBT;
        srow[i] = q >> 2;
        skv[i] = (q & 3) * 8;
    }
    auto a_off = [&](int tile, int m) -> uint32_t {
        return kind == 0 ? (uint32_t)(((((int64_t)tile * d.E + e) * d.d_e + m) * kTileM) * 2)
                         : (uint32_t)((((int64_t)tile * d.d_h + m) * kTileM) * 2);
    };
    auto b_off = [&](int tile, int nn) -> uint32_t {
        return kind == 0 ? (uint32_t)((((int64_t)tile * d.d_h + nn) * kTileM) * 2)
                         : (uint32_t)(((((int64_t)tile * d.E + e) * d.d_e + nn) * kTileM) * 2);
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            zero_acc(acc[i][j]);
    u32x4 ra[2], rb[2];
    auto load_step = [&](int s) {
        const int tile = a.tile_list[(int64_t)e * d.CT + s];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t ao = a_off(tile, mt * kTM + srow[i]) + skv[i] * 2;
            const uint32_t bo = b_off(tile, nt * kTM + srow[i]) + skv[i] * 2;
            ra[i] = kind == 0 ? load16(rda, ao) : load16(rdt, ao);
            rb[i] = kind == 0 ? load16(rt, bo) : load16(rsh, bo);
        }
    };
    if (cnt > 0)
        load_step(0);
    for (int s = 0; s < cnt; ++s) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<u32x4 *>(&As[srow[i] * kWLP + skv[i]]) = ra[i];
            *reinterpret_cast<u32x4 *>(&Bs[srow[i] * kWLP + skv[i]]) = rb[i];
        }
        __syncthreads();
        if (s + 1 < cnt)
            load_step(s + 1);
        mma_64x64<kWBK>(As, Bs, acc, wm, wn, lane);
        __syncthreads();
    }
    float *out = kind == 0 ? a.dw1 + (int64_t)e * d.d_e * d.d_h : a.dw2 + (int64_t)e * d.d_h * d.d_e;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = mt * kTM + wm * 64 + i * 32 + acc_row(v, lane);
                const int nn = nt * kTM + wn * 64 + j * 32 + (lane & 31);
                out[(int64_t)m * N + nn] = acc[i][j][v];
            }
}

// ------------------------------------------------------------------ 4. dx from the experts
struct DxArgs {
    const uint16_t *w1t;                  // [E][d_h][d_e]: W1 transposed
    const uint16_t *da_tu;                // [CT][E][32][d_e]
    const uint64_t *masks;                // [C][W] chunk unions
    float *dx;                            // [T][d_h] (splits == 1)
    float *part;                          // [splits][CT][32][d_h] (splits > 1)
    int splits;
    Dims d;
};

constexpr int kXTiles = 4;                // chunk tiles (128 rows) per dx workgroup

// Workgroup = (4 consecutive tiles, 128 output columns, expert split z): k runs over the
// experts of the 4 tiles' chunks' unions (ascending; split z takes a contiguous share)
// x d_e. A = dA rows (a tile whose chunk does not use the expert reads zeros), B = W1^T
// rows; both k-contiguous.
__global__ void __launch_bounds__(kBT, 2) dx_kernel(DxArgs a)
{
    const Dims &d = a.d;
    const int tg = blockIdx.x, nb = blockIdx.y * kTM, z = blockIdx.z;
    __shared__ alignas(16) uint16_t As[kTM * kPKP], Bs[kTM * kPKP];
    __shared__ uint64_t um[kXTiles][4];     // union masks of the 4 tiles' chunks
    __shared__ int elist[256];
    __shared__ int ecount;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave & 1, wn = wave >> 1;
    if (tid < kXTiles * 4) {
        const int q = tid / 4, w = tid % 4, tile = tg * kXTiles + q;
        um[q][w] = (tile < d.CT && w < d.W) ? a.masks[(int64_t)(tile / d.MPC) * d.W + w] : 0ull;
    }
    __syncthreads();
    if (tid == 0) {
        int c = 0;
        for (int e = 0; e < d.E; ++e) {
            const uint64_t bit = 1ull << (e & 63);
            if ((um[0][e >> 6] | um[1][e >> 6] | um[2][e >> 6] | um[3][e >> 6]) & bit)
                elist[c++] = e;
        }
        ecount = c;
    }
    __syncthreads();
    const int ne = ecount;
    const int e_lo = (int)((int64_t)z * ne / a.splits), e_hi = (int)((int64_t)(z + 1) * ne / a.splits);
    const __amdgpu_buffer_rsrc_t rda = make_rsrc(a.da_tu, (uint64_t)d.CT * d.E * kTileM * d.d_e * 2);
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(a.w1t, (uint64_t)d.E * d.d_e * d.d_h * 2);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            zero_acc(acc[i][j]);
    const int US = d.d_e / kPK;
    const int steps = (e_hi - e_lo) * US;
    auto load = [&](int st, u32x4 (&ra)[4], u32x4 (&rb)[4]) {
        // no branch here, so the compiler keeps every step's loads in flight: the list
        // is read at a valid position even past the last step (masked to an expert
        // index; such steps read zeros)
        const uint32_t vmask = 0u - (uint32_t)(st < steps);   // all ones on a real step
        const int e = elist[e_lo + (st < steps ? st / US : 0)] & 255;
        const int u0 = (st % US) * kPK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + i * kBT, row = q >> 3, kk = (q & 7) * 8;
            const int qt = row / kTileM, tile = tg * kXTiles + qt;
            const uint64_t word = um[qt][e >> 6];               // (qt < 4 always)
            const uint32_t umask = vmask & (0u - (uint32_t)((tile < d.CT) & (int)((word >> (e & 63)) & 1ull)));
            const uint32_t ao = (uint32_t)(((((int64_t)tile * d.E + e) * kTileM + row % kTileM) * d.d_e + u0 + kk) * 2);
            const uint32_t bo = (uint32_t)((((int64_t)e * d.d_h + nb + row) * d.d_e + u0 + kk) * 2);
            ra[i] = load16(rda, (ao & umask) | (kOOB & ~umask));
            rb[i] = load16(rw1, (bo & vmask) | (kOOB & ~vmask));
        }
    };
    kloop_128x128(load, steps, As, Bs, acc, tid, wm, wn, lane);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * 64 + i * 32 + acc_row(v, lane);
                const int tile = tg * kXTiles + row / kTileM;
                const int col = nb + wn * 64 + j * 32 + (lane & 31);
                if (tile >= d.CT)
                    continue;
                if (a.splits == 1) {
                    const int64_t t = tile_token(d, tile, row % kTileM);
                    if (t >= 0)
                        a.dx[t * d.d_h + col] = acc[i][j][v];
                } else {
                    a.part[(((int64_t)z * d.CT + tile) * kTileM + row % kTileM) * d.d_h + col] = acc[i][j][v];
                }
            }
}

// dx = the expert splits' partials added in split order (rows with a token only).
__global__ void __launch_bounds__(kBT) dx_reduce_kernel(DxArgs a)
{
    const Dims &d = a.d;
    const int64_t i = (int64_t)blockIdx.x * kBT + threadIdx.x;    // over CT * 32 * d_h
    if (i >= (int64_t)d.CT * kTileM * d.d_h)
        return;
    const int col = (int)(i % d.d_h);
    const int64_t rt = i / d.d_h;
    const int tile = (int)(rt / kTileM), r = (int)(rt % kTileM);
    const int64_t t = tile_token(d, tile, r);
    if (t < 0)
        return;
    float sum = 0.0f;
    for (int z = 0; z < a.splits; ++z)
        sum += a.part[((int64_t)z * d.CT * kTileM + rt) * d.d_h + col];
    a.dx[t * d.d_h + col] = sum;
}

// ------------------------------------------------------------------ 5. router backward
struct RouterArgs {
    const uint16_t *x, *w_r;
    const float *gain, *dprobs;
    const float *logits, *scores, *ds;    // [T][E]
    const uint64_t *masks;                // [C][W]
    float *dl, *gt;                       // [T][E]
    float *dx, *dw_r, *dgain, *dbias;
    float eps, sharpness;
    Dims d;
};

constexpr int kRtTokens = 4;              // tokens per router-token workgroup (one per wave)
constexpr int kRtPer = 256 / kWave;       // experts per lane (E <= 256)

// Per token (one wavefront each, kRtTokens per workgroup): ds (masked to the chunk's
// union, plus the probability term), the RMSNorm and ReLU backward -> dl, and the gain
// term; then dx[t] += W_r^T dl for the workgroup's tokens, each W_r row loaded once for
// all of them (experts in order, eight rows in flight).
// p[0 .. n) = 0 (the recomputed router's arrival counters: this workspace is not
// zero-filled by the caller)
__global__ void __launch_bounds__(kBT) zero_words_kernel(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kBT + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

__global__ void __launch_bounds__(kBT) router_token_kernel(RouterArgs a)
{
    const Dims &d = a.d;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int64_t t0 = (int64_t)blockIdx.x * kRtTokens;
    __shared__ float dl_s[kRtTokens][256];
    {
        const int64_t t = t0 + wave;
        const bool vt = t < d.T;
        const int c = vt ? (int)(t / d.n) : 0;
        float l[kRtPer], r[kRtPer], ds[kRtPer], g[kRtPer];
        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < kRtPer; ++i) {
            const int e = lane + i * kWave;
            const bool ve = vt && e < d.E;
            l[i] = ve ? a.logits[t * d.E + e] : 0.0f;
            r[i] = l[i] > 0.0f ? l[i] : 0.0f;
            sq = fmaf(r[i], r[i], sq);
            ds[i] = 0.0f;
            if (ve) {
                if ((a.masks[(int64_t)c * d.W + (e >> 6)] >> (e & 63)) & 1ull)
                    ds[i] = a.ds[t * d.E + e];
                if (a.dprobs) {
                    const float p = 1.0f / (1.0f + expf(-a.sharpness * a.scores[t * d.E + e]));
                    ds[i] += a.dprobs[t * d.E + e] * a.sharpness * p * (1.0f - p);
                }
            }
            g[i] = ve && a.gain ? a.gain[e] : 1.0f;
        }
        const float inv = 1.0f / sqrtf(wave_sum_f32(sq) / (float)d.E + a.eps);
        float cp = 0.0f;
#pragma unroll
        for (int i = 0; i < kRtPer; ++i)
            cp = fmaf(g[i] * r[i], ds[i], cp);
        const float coup = wave_sum_f32(cp);
#pragma unroll
        for (int i = 0; i < kRtPer; ++i) {
            const int e = lane + i * kWave;
            const float dr = g[i] * inv * ds[i] - inv * inv * inv * r[i] / (float)d.E * coup;
            const float dl = l[i] > 0.0f ? dr : 0.0f;
            dl_s[wave][e] = dl;
            if (vt && e < d.E) {
                a.dl[t * d.E + e] = dl;
                a.gt[t * d.E + e] = ds[i] * r[i] * inv;
            }
        }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w_r, (uint64_t)d.E * d.d_h * 2);
    for (int jv = tid; jv < d.d_h / 8; jv += kBT) {
        float acc[kRtTokens][8];
#pragma unroll
        for (int k = 0; k < kRtTokens; ++k)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[k][q] = 0.0f;
        for (int k0 = 0; k0 < d.E; k0 += 8) {
            u32x4 w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                w[u] = load16(rw, k0 + u < d.E ? (uint32_t)((((int64_t)(k0 + u)) * d.d_h + jv * 8) * 2) : kOOB);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int k = 0; k < kRtTokens; ++k) {
                    const float dk = k0 + u < d.E ? dl_s[k][k0 + u] : 0.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[k][2 * q] = fmaf(dk, __uint_as_float(w[u][q] << 16), acc[k][2 * q]);
                        acc[k][2 * q + 1] = fmaf(dk, __uint_as_float(w[u][q] & 0xffff0000u), acc[k][2 * q + 1]);
                    }
                }
        }
#pragma unroll
        for (int k = 0; k < kRtTokens; ++k) {
            const int64_t t = t0 + k;
            if (t >= d.T)
                continue;
            float4 *o = reinterpret_cast<float4 *>(&a.dx[t * d.d_h + jv * 8]);
            float4 o0 = o[0], o1 = o[1];
            o0.x += acc[k][0], o0.y += acc[k][1], o0.z += acc[k][2], o0.w += acc[k][3];
            o1.x += acc[k][4], o1.y += acc[k][5], o1.z += acc[k][6], o1.w += acc[k][7];
            o[0] = o0;
            o[1] = o1;
        }
    }
}

constexpr int kRpE = 8;       // experts per router-parameter workgroup
constexpr int kRpTargetBlocks = 1024;

// Token splits of the router-parameter sums: enough workgroups to fill the chip,
// at least 32 tokens per split.
int router_param_splits(int64_t T, int64_t d_h, int64_t E)
{
    const int64_t base = ((E + kRpE - 1) / kRpE) * (d_h / kBT);
    int64_t s = (kRpTargetBlocks + base - 1) / base;
    const int64_t smax = (T + 31) / 32;
    if (s > smax)
        s = smax;
    return s < 1 ? 1 : (int)s;
}

// Partial dW_r over token split z: part[z][e][j] = sum_{t in split z} dl[t][e] x[t][j],
// tokens in order.
__global__ void __launch_bounds__(kBT) router_param_kernel(RouterArgs a, int splits, float *part)
{
    const Dims &d = a.d;
    const int e0 = blockIdx.x * kRpE, j = blockIdx.y * kBT + threadIdx.x, z = blockIdx.z;
    const int64_t per = (d.T + splits - 1) / splits;
    const int64_t t0 = z * per, t1 = t0 + per < d.T ? t0 + per : d.T;
    // dl[t][e0 .. e0+8) of 128 tokens at a time staged in LDS (read back as broadcasts);
    // x of 16 tokens in flight at a time
    __shared__ float dls[128][kRpE];
    const int tid = threadIdx.x;
    float acc[kRpE];
#pragma unroll
    for (int q = 0; q < kRpE; ++q)
        acc[q] = 0.0f;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint64_t)d.T * d.d_h * 2);
    for (int64_t tb = t0; tb < t1; tb += 128) {
        {
            const int64_t t = tb + tid / 2;
            const int q0 = (tid % 2) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dls[tid / 2][q0 + q] = (t < t1 && e0 + q0 + q < d.E) ? a.dl[t * d.E + e0 + q0 + q] : 0.0f;
        }
        __syncthreads();
        const int nt = (int)(t1 - tb < 128 ? t1 - tb : 128);
        for (int u0 = 0; u0 < nt; u0 += 16) {
            float xv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const uint32_t off = u0 + u < nt ? (uint32_t)(((tb + u0 + u) * d.d_h + j) * 2) : kOOB;
                xv[u] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rx, (int)off, 0, 0)
                                        << 16);
            }
#pragma unroll
            for (int u = 0; u < 16; ++u)
#pragma unroll
                for (int q = 0; q < kRpE; ++q)
                    acc[q] = fmaf(dls[u0 + u][q], xv[u], acc[q]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < kRpE; ++q)
        if (e0 + q < d.E)
            part[((int64_t)z * d.E + e0 + q) * d.d_h + j] = acc[q];
}

// dW_r = the splits' partials added in split order; the workgroups of column block 0
// also sum dgain and dbias (thread = (expert q = tid % 8, token slice tid / 8 of 32),
// then the 32 slices in order).
__global__ void __launch_bounds__(kBT) router_param_reduce_kernel(RouterArgs a, int splits,
                                                                  const float *part)
{
    const Dims &d = a.d;
    const int e0 = blockIdx.x * kRpE, j = blockIdx.y * kBT + threadIdx.x, tid = threadIdx.x;
    // the kRpE experts' partials of up to 16 splits requested together, then added in
    // split order (experts past E and splits past `splits` read zero and are not added)
    const __amdgpu_buffer_rsrc_t rpp = make_rsrc(part, (uint64_t)splits * d.E * d.d_h * 4);
    for (int z0 = 0; z0 < splits; z0 += 16) {
        float pv[16][kRpE];
#pragma unroll
        for (int z = 0; z < 16; ++z)
#pragma unroll
            for (int q = 0; q < kRpE; ++q) {
                const bool ok = z0 + z < splits && e0 + q < d.E;
                pv[z][q] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(
                               rpp, ok ? (int)((((int64_t)(z0 + z) * d.E + e0 + q) * d.d_h + j) * 4) : (int)kOOB, 0, 0));
            }
#pragma unroll
        for (int q = 0; q < kRpE; ++q)
            if (e0 + q < d.E) {
                float sum = z0 == 0 ? 0.0f : a.dw_r[(int64_t)(e0 + q) * d.d_h + j];
#pragma unroll
                for (int z = 0; z < 16; ++z)
                    if (z0 + z < splits)
                        sum += pv[z][q];
                a.dw_r[(int64_t)(e0 + q) * d.d_h + j] = sum;
            }
    }
    if (blockIdx.y != 0)
        return;
    __shared__ float pg[kBT], pb[kBT];
    const int q = tid % kRpE, sl = tid / kRpE;
    float sg = 0.0f, sb = 0.0f;
    if (e0 + q < d.E) {
#pragma unroll 16
        for (int64_t t = sl; t < d.T; t += kBT / kRpE) {
            sg += a.gt[t * d.E + e0 + q];
            sb += a.dl[t * d.E + e0 + q];
        }
    }
    pg[tid] = sg;
    pb[tid] = sb;
    __syncthreads();
    if (tid < kRpE && e0 + tid < d.E) {
        float g = 0.0f, b = 0.0f;
        for (int s2 = 0; s2 < kBT / kRpE; ++s2) {
            g += pg[s2 * kRpE + tid];
            b += pb[s2 * kRpE + tid];
        }
        if (a.dgain)
            a.dgain[e0 + tid] = g;
        if (a.dbias)
            a.dbias[e0 + tid] = b;
    }
}

// ------------------------------------------------------------------ workspace layout
struct BwdLayout {
    FfnPlan p;
    size_t masks, lists, counts, tile_list, tile_count;
    size_t logits, scores, ds, dl, gt;
    size_t xt, dyt, da_tu, da_ut, sh_ut, rp_part, w1t, w2t, dx_part;
    size_t router;        // the forward router's split workspace (0 bytes when it takes none)
    int dx_splits;
    size_t total;
};

constexpr int kDxTargetBlocks = 256;

// Expert splits of the dx products: enough workgroups for one per CU.
int dx_splits(int64_t CT, int64_t d_h, int64_t E)
{
    const int64_t base = ((CT + kXTiles - 1) / kXTiles) * (d_h / kTM);
    int64_t s = (kDxTargetBlocks + base - 1) / base;
    if (s > E)
        s = E;
    if (s > 32)
        s = 32;
    return s < 1 ? 1 : (int)s;
}

BwdLayout bwd_layout(int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n)
{
    BwdLayout L;
    L.p = make_plan(T, d_h, E, d_e, n, 1);
    const FfnPlan &p = L.p;
    size_t off = kControlBytes;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    L.masks = take(8 * p.C * p.W);
    L.lists = take(4 * p.C * E);
    L.counts = take(4 * p.C);
    L.tile_list = take(4 * E * p.CT);
    L.tile_count = take(4 * E);
    L.logits = take(4 * T * E);
    L.scores = take(4 * T * E);
    L.ds = take(4 * T * E);
    L.dl = take(4 * T * E);
    L.gt = take(4 * T * E);
    L.xt = take(2 * p.CT * d_h * kTileM);
    L.dyt = take(2 * p.CT * d_h * kTileM);
    L.da_tu = take(2 * p.CT * E * kTileM * d_e);
    L.da_ut = take(2 * p.CT * E * kTileM * d_e);
    L.sh_ut = take(2 * p.CT * E * kTileM * d_e);
    L.rp_part = take(4 * (size_t)router_param_splits(T, d_h, E) * E * d_h);
    L.router = take(router_workspace_bytes(T, d_h, E));
    L.w1t = take(2 * (size_t)E * d_e * d_h);
    L.w2t = take(2 * (size_t)E * d_e * d_h);
    L.dx_splits = dx_splits(p.CT, d_h, E);
    L.dx_part = take(L.dx_splits > 1 ? 4 * (size_t)L.dx_splits * p.CT * kTileM * d_h : 0);
    L.total = off;
    L.p.off_masks = L.masks;
    L.p.off_lists = L.lists;
    L.p.off_counts = L.counts;
    return L;
}

}  // namespace

bool backward_supported(int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n)
{
    if (T < 1 || n < 1 || E < 1 || E > 256 || d_h % kXN != 0 || d_e % kTM != 0)
        return false;
    const FfnPlan p = make_plan(T, d_h, E, d_e, n, 1);
    const uint64_t lim = 0x7fffffffull;
    return (uint64_t)T * d_h * 2 < lim && (uint64_t)E * d_e * d_h * 2 < lim &&
           (uint64_t)p.CT * E * kTileM * d_e * 2 < lim && (uint64_t)p.CT * d_h * kTileM * 2 < lim &&
           p.CT * E < ((int64_t)1 << 31);
}

size_t backward_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n)
{
    return bwd_layout(T, d_h, E, d_e, n).total;
}

hipError_t launch_layer_backward(const BackwardArgs &b, void *ws, hipStream_t stream)
{
    const BwdLayout L = bwd_layout(b.T, b.d_h, b.E, b.d_e, b.n);
    const FfnPlan &p = L.p;
    char *base = static_cast<char *>(ws);
    auto at = [&](size_t off) { return base + off; };
    float *logits = reinterpret_cast<float *>(at(L.logits));
    float *scores = reinterpret_cast<float *>(at(L.scores));
    // the forward router with its d_h split when it takes one (few tokens): its arrival
    // counters are cleared first
    void *rws = nullptr;
    if (router_workspace_bytes(b.T, b.d_h, b.E) > 0) {
        rws = at(L.router);
        const int64_t tiles = (b.T + kTileM - 1) / kTileM;
        hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((tiles + kBT - 1) / kBT)), dim3(kBT), 0, stream,
                           static_cast<uint32_t *>(rws), tiles);
    }
    hipError_t err = launch_router_bf16(b.x, b.w_r, b.gain, b.bias, b.eps, b.T, b.d_h, b.E, scores,
                                        logits, 1.0f, nullptr, rws, 0, stream);
    if (err != hipSuccess)
        return err;
    if ((err = launch_union(p, scores, ws, nullptr, nullptr, nullptr, stream)) != hipSuccess)
        return err;
    const uint64_t *masks = reinterpret_cast<const uint64_t *>(at(L.masks));
    int32_t *tile_list = reinterpret_cast<int32_t *>(at(L.tile_list));
    int32_t *tile_count = reinterpret_cast<int32_t *>(at(L.tile_count));
    if ((err = launch_expert_tiles(p, masks, tile_list, tile_count, stream)) != hipSuccess)
        return err;
    Dims d;
    d.T = b.T;
    d.n = (int)p.n;
    d.d_h = (int)b.d_h;
    d.E = (int)b.E;
    d.d_e = (int)b.d_e;
    d.C = (int)p.C;
    d.W = (int)p.W;
    d.MPC = (int)p.MPC;
    d.CT = (int)p.CT;
    uint16_t *w1t = reinterpret_cast<uint16_t *>(at(L.w1t));
    uint16_t *w2t = reinterpret_cast<uint16_t *>(at(L.w2t));
    // W1 [E][d_e][d_h] -> [E][d_h][d_e], W2 [E][d_h][d_e] -> [E][d_e][d_h], used experts only
    hipLaunchKernelGGL(transpose_weights_kernel, dim3((unsigned)(b.d_h / 64), (unsigned)(b.d_e / 64), (unsigned)b.E),
                       dim3(kBT), 0, stream, b.w1, (int)b.d_e, (int)b.d_h, tile_count, w1t);
    hipLaunchKernelGGL(transpose_weights_kernel, dim3((unsigned)(b.d_e / 64), (unsigned)(b.d_h / 64), (unsigned)b.E),
                       dim3(kBT), 0, stream, b.w2, (int)b.d_h, (int)b.d_e, tile_count, w2t);
    uint16_t *xt = reinterpret_cast<uint16_t *>(at(L.xt));
    uint16_t *dyt = reinterpret_cast<uint16_t *>(at(L.dyt));
    const dim3 tgrid((unsigned)p.CT, (unsigned)(b.d_h / kTrCols));
    hipLaunchKernelGGL(transpose_tiles_kernel, tgrid, dim3(kBT), 0, stream, b.x, d, xt);
    hipLaunchKernelGGL(transpose_tiles_kernel, tgrid, dim3(kBT), 0, stream, b.dy, d, dyt);

    PassArgs pa;
    pa.x = b.x;
    pa.dy = b.dy;
    pa.w1 = b.w1;
    pa.w2t = w2t;
    pa.scores = scores;
    pa.tile_list = tile_list;
    pa.tile_count = tile_count;
    pa.ds = reinterpret_cast<float *>(at(L.ds));
    pa.da_tu = reinterpret_cast<uint16_t *>(at(L.da_tu));
    pa.da_ut = reinterpret_cast<uint16_t *>(at(L.da_ut));
    pa.sh_ut = reinterpret_cast<uint16_t *>(at(L.sh_ut));
    pa.d = d;
    const int64_t pass_blocks = b.E * ((p.CT + kPassTiles - 1) / kPassTiles);
    hipLaunchKernelGGL(expert_pass_kernel, dim3((unsigned)pass_blocks), dim3(kPassThreads), 0, stream, pa);

    WgradArgs wa;
    wa.xt = xt;
    wa.dyt = dyt;
    wa.da_ut = pa.da_ut;
    wa.sh_ut = pa.sh_ut;
    wa.tile_list = tile_list;
    wa.tile_count = tile_count;
    wa.dw1 = b.dw1;
    wa.dw2 = b.dw2;
    wa.d = d;
    const int64_t wblocks = b.E * 2 * (b.d_e / kTM) * (b.d_h / kTM);
    hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)wblocks), dim3(kBT), 0, stream, wa);

    DxArgs xa;
    xa.w1t = w1t;
    xa.da_tu = pa.da_tu;
    xa.masks = masks;
    xa.dx = b.dx;
    xa.part = reinterpret_cast<float *>(at(L.dx_part));
    xa.splits = L.dx_splits;
    xa.d = d;
    hipLaunchKernelGGL(dx_kernel,
                       dim3((unsigned)((p.CT + kXTiles - 1) / kXTiles), (unsigned)(b.d_h / kTM),
                            (unsigned)L.dx_splits),
                       dim3(kBT), 0, stream, xa);
    if (L.dx_splits > 1) {
        const int64_t nel = p.CT * kTileM * b.d_h;
        hipLaunchKernelGGL(dx_reduce_kernel, dim3((unsigned)((nel + kBT - 1) / kBT)), dim3(kBT), 0,
                           stream, xa);
    }

    RouterArgs ra;
    ra.x = b.x;
    ra.w_r = b.w_r;
    ra.gain = b.gain;
    ra.dprobs = b.dprobs;
    ra.logits = logits;
    ra.scores = scores;
    ra.ds = pa.ds;
    ra.masks = masks;
    ra.dl = reinterpret_cast<float *>(at(L.dl));
    ra.gt = reinterpret_cast<float *>(at(L.gt));
    ra.dx = b.dx;
    ra.dw_r = b.dw_r;
    ra.dgain = b.dgain;
    ra.dbias = b.dbias;
    ra.eps = b.eps;
    ra.sharpness = b.sharpness;
    ra.d = d;
    hipLaunchKernelGGL(router_token_kernel, dim3((unsigned)((b.T + kRtTokens - 1) / kRtTokens)), dim3(kBT), 0,
                       stream, ra);
    const int splits = router_param_splits(b.T, b.d_h, b.E);
    float *rp = reinterpret_cast<float *>(at(L.rp_part));
    const unsigned eb = (unsigned)((b.E + kRpE - 1) / kRpE), jb = (unsigned)(b.d_h / kBT);
    hipLaunchKernelGGL(router_param_kernel, dim3(eb, jb, (unsigned)splits), dim3(kBT), 0, stream,
                       ra, splits, rp);
    hipLaunchKernelGGL(router_param_reduce_kernel, dim3(eb, jb), dim3(kBT), 0, stream, ra,
                       splits, static_cast<const float *>(rp));
    return hipGetLastError();
}

}  // namespace blockffn
