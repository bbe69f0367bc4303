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
//   0. the forward router (recomputed: logits and scores), the chunk unions and the
//      per-expert tile lists (the forward's kernels);
//   1. transpose_tiles_kernel: x and dy copied per 32-token chunk tile as
//      [tile][d_h][32 tokens], so the weight-gradient products, whose k is the token,
//      read k-contiguous operands;
//   2. expert_pass_kernel, workgroup = (expert e, 4 of its tiles): a = X W1_e^T and
//      G = DY W2_e over d_h (W2 tiles transposed in LDS), then ds, and dA and SH in bf16
//      in both [token][unit] and [unit][token] order;
//   3. wgrad_kernel, workgroup = (expert, dW1 or dW2, 128 x 128 output tile): k over the
//      expert's tiles' tokens; every output element is owned by one workgroup (an
//      expert no chunk uses gets zeros);
//   4. dx_kernel, workgroup = (tile, 256 columns): k over the chunk's union experts x
//      d_e (W1 tiles transposed in LDS);
//   5. router_token_kernel: per token, dl and the router's share of dx;
//      router_param_kernel: dW_r, dgain, dbias as sums over the tokens in order.
// Every sum runs in a fixed order, so equal inputs give equal bits.
#include "common.h"
#include "plan.h"
#include "sync.h"

namespace blockffn {

namespace {

constexpr int kBT = 256;                  // threads per workgroup, 4 waves
constexpr int kBK = 32;                   // k per staged step
constexpr int kLP = kBK + 8;              // LDS pitch (bf16) of a [row][k] tile: 80 bytes
constexpr int kTM = 128;                  // 128 x 128 output tiles
constexpr int kXN = 256;                  // dx columns per workgroup
constexpr int kPassTiles = 4;             // chunk tiles per expert-pass workgroup
constexpr int kTrCols = 256;              // d_h columns per transpose workgroup
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset past every range: reads zero

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

// 32x32 accumulator layout: element v of a lane is row (v/4)*8 + (lane/32)*4 + v%4 of
// column lane%32.
__device__ __forceinline__ int acc_row(int v, int lane) { return (v / 4) * 8 + (lane >> 5) * 4 + (v % 4); }

__device__ __forceinline__ void zero_acc(f32x16 &a)
{
#pragma unroll
    for (int v = 0; v < 16; ++v)
        a[v] = 0.0f;
}

// One k step (kBK = 32) of a wave's 64 x 64 block: rows [wm*64, +64) of As, columns
// [wn*64, +64) of Bs, both stored [row][k] with pitch kLP.
__device__ __forceinline__ void mma_64x64(const uint16_t *As, const uint16_t *Bs, f32x16 (&acc)[2][2],
                                          int wm, int wn, int lane)
{
    const int r = lane & 31, kg = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            a[i] = *reinterpret_cast<const bf16x8 *>(&As[(wm * 64 + i * 32 + r) * kLP + ks * 16 + kg * 8]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[(wn * 64 + j * 32 + r) * kLP + ks * 16 + kg * 8]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

// Stores eight bf16 values (one 16-byte global load of 8 consecutive n at one k) into
// a [n][k] LDS tile: element i goes to row n0 + i, column k.
__device__ __forceinline__ void store_transposed(uint16_t *S, int n0, int k, u32x4 v)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        S[(n0 + 2 * q) * kLP + k] = (uint16_t)(v[q] & 0xffffu);
        S[(n0 + 2 * q + 1) * kLP + k] = (uint16_t)(v[q] >> 16);
    }
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// ------------------------------------------------------------------ 1. tile transposes
// dst[tile][j][r] = src[token(tile, r)][j] (zero for rows without a token).
__global__ void __launch_bounds__(kBT) transpose_tiles_kernel(const uint16_t *src, Dims d,
                                                              uint16_t *dst)
{
    __shared__ uint16_t t[kTileM][kTrCols + 8];
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

// ------------------------------------------------------------------ 2. expert pass
struct PassArgs {
    const uint16_t *x, *dy, *w1, *w2;
    const float *scores;          // recomputed forward scores [T][E]
    const int32_t *tile_list, *tile_count;
    float *ds;                    // [T][E], written for e in U_c(t)
    uint16_t *da_tu, *da_ut, *sh_ut;
    Dims d;
};

__global__ void __launch_bounds__(kBT, 1) expert_pass_kernel(PassArgs a)
{
    const Dims &d = a.d;
    const int e = blockIdx.x % d.E, grp = blockIdx.x / d.E;
    const int cnt = a.tile_count[e];
    if (grp * kPassTiles >= cnt)
        return;
    __shared__ uint16_t As1[kTM * kLP], Bs1[kTM * kLP], As2[kTM * kLP], Bs2[kTM * kLP];
    __shared__ float red[kTM][65];
    __shared__ float dsacc[kTM], scol[kTM];
    __shared__ int64_t tok[kTM];
    __shared__ int tiles[kPassTiles];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave & 1, wn = wave >> 1;
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

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint64_t)d.T * d.d_h * 2);
    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, (uint64_t)d.T * d.d_h * 2);
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(a.w1, (uint64_t)d.E * d.d_e * d.d_h * 2);
    const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(a.w2, (uint64_t)d.E * d.d_h * d.d_e * 2);
    // k-contiguous staging: vector q = tid + 256 i is row q / 4, k offset (q % 4) * 8.
    // Transposed W2 staging: wave group g = 2 wave + i covers k [8 (g % 4), +8) x
    // n [64 (g / 4), +64); lane: k = lane % 8, n = 8 (lane / 8) .. +8.
    int srow[2], skv[2], tk[2], tn[2];
    uint32_t xoff[2], dyoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + i * kBT;
        srow[i] = q >> 2;
        skv[i] = (q & 3) * 8;
        const int64_t t = tok[srow[i]];
        xoff[i] = t >= 0 ? (uint32_t)((t * d.d_h + skv[i]) * 2) : kOOB;
        dyoff[i] = xoff[i];
        const int g = 2 * wave + i;
        tk[i] = (g & 3) * 8 + (lane & 7);
        tn[i] = (g >> 2) * 64 + (lane >> 3) * 8;
    }
    const int KS = d.d_h / kBK;
    for (int u0 = 0; u0 < d.d_e; u0 += kTM) {
        f32x16 acc1[2][2], acc2[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                zero_acc(acc1[i][j]);
                zero_acc(acc2[i][j]);
            }
        u32x4 rxv[2], rw1v[2], rdyv[2], rw2v[2];
        auto load_step = [&](int s) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t ko = (uint32_t)(s * kBK * 2);
                rxv[i] = load16(rx, xoff[i] == kOOB ? kOOB : xoff[i] + ko);
                rdyv[i] = load16(rdy, dyoff[i] == kOOB ? kOOB : dyoff[i] + ko);
                rw1v[i] = load16(rw1, (uint32_t)((((int64_t)e * d.d_e + u0 + srow[i]) * d.d_h + s * kBK + skv[i]) * 2));
                rw2v[i] = load16(rw2, (uint32_t)((((int64_t)e * d.d_h + s * kBK + tk[i]) * d.d_e + u0 + tn[i]) * 2));
            }
        };
        load_step(0);
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                *reinterpret_cast<u32x4 *>(&As1[srow[i] * kLP + skv[i]]) = rxv[i];
                *reinterpret_cast<u32x4 *>(&Bs1[srow[i] * kLP + skv[i]]) = rw1v[i];
                *reinterpret_cast<u32x4 *>(&As2[srow[i] * kLP + skv[i]]) = rdyv[i];
                store_transposed(Bs2, tn[i], tk[i], rw2v[i]);
            }
            __syncthreads();
            if (s + 1 < KS)
                load_step(s + 1);
            mma_64x64(As1, Bs1, acc1, wm, wn, lane);
            mma_64x64(As2, Bs2, acc2, wm, wn, lane);
            __syncthreads();
        }
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
                        const float av = acc1[i][j][v], g = acc2[i][j][v], s = scol[row];
                        const float sig = 1.0f / (1.0f + expf(-av));
                        const float h = av * sig;
                        part[i][v] += g * h;
                        const float dA = s * g * (sig * (1.0f + av * (1.0f - sig)));
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
    __shared__ uint16_t As[kTM * kLP], Bs[kTM * kLP];
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
            *reinterpret_cast<u32x4 *>(&As[srow[i] * kLP + skv[i]]) = ra[i];
            *reinterpret_cast<u32x4 *>(&Bs[srow[i] * kLP + skv[i]]) = rb[i];
        }
        __syncthreads();
        if (s + 1 < cnt)
            load_step(s + 1);
        mma_64x64(As, Bs, acc, wm, wn, lane);
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
    const uint16_t *w1;
    const uint16_t *da_tu;                // [CT][E][32][d_e]
    const int32_t *lists, *counts;        // chunk unions
    float *dx;
    Dims d;
};

__global__ void __launch_bounds__(kBT, 2) dx_kernel(DxArgs a)
{
    const Dims &d = a.d;
    const int tile = blockIdx.x, nb = blockIdx.y * kXN;
    const int c = tile / d.MPC;
    const int ne = a.counts[c];
    __shared__ uint16_t As[kTileM * kLP], Bs[kXN * kLP];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const __amdgpu_buffer_rsrc_t rda = make_rsrc(a.da_tu, (uint64_t)d.CT * d.E * kTileM * d.d_e * 2);
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(a.w1, (uint64_t)d.E * d.d_e * d.d_h * 2);
    // A: 32 rows x 32 k = 128 vectors (threads 0..127): row tid / 4, k (tid % 4) * 8.
    // B (transposed W1): wave group g = 4 wave + i covers k [8 (g % 4), +8) x
    // n [64 (g / 4), +64); lane: k = lane % 8, n = 8 (lane / 8) .. +8.
    const int arow = (tid & 127) >> 2, akv = (tid & 3) * 8;
    int tk[4], tn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * wave + i;
        tk[i] = (g & 3) * 8 + (lane & 7);
        tn[i] = (g >> 2) * 64 + (lane >> 3) * 8;
    }
    f32x16 acc[2];
    zero_acc(acc[0]);
    zero_acc(acc[1]);
    const int US = d.d_e / kBK;
    const int steps = ne * US;
    u32x4 ra, rb[4];
    auto load_step = [&](int s) {
        const int e = a.lists[(int64_t)c * d.E + s / US];
        const int u0 = (s % US) * kBK;
        ra = load16(rda, tid < 128 ? (uint32_t)(((((int64_t)tile * d.E + e) * kTileM + arow) * d.d_e + u0 + akv) * 2) : kOOB);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rb[i] = load16(rw1, (uint32_t)((((int64_t)e * d.d_e + u0 + tk[i]) * d.d_h + nb + tn[i]) * 2));
    };
    if (steps > 0)
        load_step(0);
    const int r = lane & 31, kg = lane >> 5;
    for (int s = 0; s < steps; ++s) {
        if (tid < 128)
            *reinterpret_cast<u32x4 *>(&As[arow * kLP + akv]) = ra;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            store_transposed(Bs, tn[i], tk[i], rb[i]);
        __syncthreads();
        if (s + 1 < steps)
            load_step(s + 1);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&As[r * kLP + ks * 16 + kg * 8]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8 bv =
                    *reinterpret_cast<const bf16x8 *>(&Bs[(wave * 64 + j * 32 + r) * kLP + ks * 16 + kg * 8]);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[j], 0, 0, 0);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t t = tile_token(d, tile, acc_row(v, lane));
            if (t >= 0)
                a.dx[t * d.d_h + nb + wave * 64 + j * 32 + (lane & 31)] = acc[j][v];
        }
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

__device__ __forceinline__ float block_sum(float v, float *sh)
{
    // fixed order: wave DPP trees, then the 4 wave sums in order
    v = wave_sum_f32(v);
    const int tid = threadIdx.x;
    __syncthreads();
    if (tid % kWave == 0)
        sh[tid / kWave] = v;
    __syncthreads();
    return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

__global__ void __launch_bounds__(kBT) router_token_kernel(RouterArgs a)
{
    const Dims &d = a.d;
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x, e = tid;
    const int c = (int)(t / d.n);
    __shared__ float red[4];
    __shared__ float dl_s[256];
    const bool ve = e < d.E;
    const float l = ve ? a.logits[t * d.E + e] : 0.0f;
    const float r = l > 0.0f ? l : 0.0f;
    const float inv = 1.0f / sqrtf(block_sum(r * r, red) / (float)d.E + a.eps);
    float ds = 0.0f;
    if (ve) {
        if ((a.masks[(int64_t)c * d.W + (e >> 6)] >> (e & 63)) & 1ull)
            ds = a.ds[t * d.E + e];
        if (a.dprobs) {
            const float p = 1.0f / (1.0f + expf(-a.sharpness * a.scores[t * d.E + e]));
            ds += a.dprobs[t * d.E + e] * a.sharpness * p * (1.0f - p);
        }
    }
    const float g = ve && a.gain ? a.gain[e] : 1.0f;
    const float coup = block_sum(ve ? g * r * ds : 0.0f, red);
    const float dr = g * inv * ds - inv * inv * inv * r / (float)d.E * coup;
    const float dl = (ve && l > 0.0f) ? dr : 0.0f;
    dl_s[tid] = dl;
    if (ve) {
        a.dl[t * d.E + e] = dl;
        a.gt[t * d.E + e] = ds * r * inv;
    }
    __syncthreads();
    // dx[t] += W_r^T dl, eight columns per thread, experts in order
    for (int jv = tid; jv < d.d_h / 8; jv += kBT) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < d.E; ++k) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(&a.w_r[(int64_t)k * d.d_h + jv * 8]);
            const float dk = dl_s[k];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(dk, __uint_as_float(w[q] << 16), acc[2 * q]);
                acc[2 * q + 1] = fmaf(dk, __uint_as_float(w[q] & 0xffff0000u), acc[2 * q + 1]);
            }
        }
        float4 *o = reinterpret_cast<float4 *>(&a.dx[t * d.d_h + jv * 8]);
        float4 o0 = o[0], o1 = o[1];
        o0.x += acc[0], o0.y += acc[1], o0.z += acc[2], o0.w += acc[3];
        o1.x += acc[4], o1.y += acc[5], o1.z += acc[6], o1.w += acc[7];
        o[0] = o0;
        o[1] = o1;
    }
}

constexpr int kRpE = 8;       // experts per router-parameter workgroup

// dW_r[e][j] = sum_t dl[t][e] x[t][j] (tokens in order); the workgroups of column block
// 0 also sum dgain and dbias.
__global__ void __launch_bounds__(kBT) router_param_kernel(RouterArgs a)
{
    const Dims &d = a.d;
    const int e0 = blockIdx.x * kRpE, j = blockIdx.y * kBT + threadIdx.x, tid = threadIdx.x;
    float acc[kRpE];
#pragma unroll
    for (int q = 0; q < kRpE; ++q)
        acc[q] = 0.0f;
    for (int64_t t = 0; t < d.T; ++t) {
        const float xv = bf16_to_f32(a.x[t * d.d_h + j]);
#pragma unroll
        for (int q = 0; q < kRpE; ++q)
            if (e0 + q < d.E)
                acc[q] = fmaf(a.dl[t * d.E + e0 + q], xv, acc[q]);
    }
#pragma unroll
    for (int q = 0; q < kRpE; ++q)
        if (e0 + q < d.E)
            a.dw_r[(int64_t)(e0 + q) * d.d_h + j] = acc[q];
    if (blockIdx.y != 0)
        return;
    // dgain, dbias: thread = (expert q = tid % 8, token slice tid / 8 of 32), then the
    // 32 slices in order
    __shared__ float pg[kBT], pb[kBT];
    const int q = tid % kRpE, sl = tid / kRpE;
    float sg = 0.0f, sb = 0.0f;
    if (e0 + q < d.E)
        for (int64_t t = sl; t < d.T; t += kBT / kRpE) {
            sg += a.gt[t * d.E + e0 + q];
            sb += a.dl[t * d.E + e0 + q];
        }
    pg[tid] = sg;
    pb[tid] = sb;
    __syncthreads();
    if (tid < kRpE && e0 + tid < d.E) {
        float g = 0.0f, b = 0.0f;
        for (int s = 0; s < kBT / kRpE; ++s) {
            g += pg[s * kRpE + tid];
            b += pb[s * kRpE + tid];
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
    size_t xt, dyt, da_tu, da_ut, sh_ut;
    size_t total;
};

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
    hipError_t err = launch_router_bf16(b.x, b.w_r, b.gain, b.bias, b.eps, b.T, b.d_h, b.E, scores,
                                        logits, 1.0f, nullptr, nullptr, 0, stream);
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
    uint16_t *xt = reinterpret_cast<uint16_t *>(at(L.xt));
    uint16_t *dyt = reinterpret_cast<uint16_t *>(at(L.dyt));
    const dim3 tgrid((unsigned)p.CT, (unsigned)(b.d_h / kTrCols));
    hipLaunchKernelGGL(transpose_tiles_kernel, tgrid, dim3(kBT), 0, stream, b.x, d, xt);
    hipLaunchKernelGGL(transpose_tiles_kernel, tgrid, dim3(kBT), 0, stream, b.dy, d, dyt);

    PassArgs pa;
    pa.x = b.x;
    pa.dy = b.dy;
    pa.w1 = b.w1;
    pa.w2 = b.w2;
    pa.scores = scores;
    pa.tile_list = tile_list;
    pa.tile_count = tile_count;
    pa.ds = reinterpret_cast<float *>(at(L.ds));
    pa.da_tu = reinterpret_cast<uint16_t *>(at(L.da_tu));
    pa.da_ut = reinterpret_cast<uint16_t *>(at(L.da_ut));
    pa.sh_ut = reinterpret_cast<uint16_t *>(at(L.sh_ut));
    pa.d = d;
    const int64_t pass_blocks = b.E * ((p.CT + kPassTiles - 1) / kPassTiles);
    hipLaunchKernelGGL(expert_pass_kernel, dim3((unsigned)pass_blocks), dim3(kBT), 0, stream, pa);

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
    xa.w1 = b.w1;
    xa.da_tu = pa.da_tu;
    xa.lists = reinterpret_cast<const int32_t *>(at(L.lists));
    xa.counts = reinterpret_cast<const int32_t *>(at(L.counts));
    xa.dx = b.dx;
    xa.d = d;
    hipLaunchKernelGGL(dx_kernel, dim3((unsigned)p.CT, (unsigned)(b.d_h / kXN)), dim3(kBT), 0,
                       stream, xa);

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
    hipLaunchKernelGGL(router_token_kernel, dim3((unsigned)b.T), dim3(kBT), 0, stream, ra);
    hipLaunchKernelGGL(router_param_kernel, dim3((unsigned)((b.E + kRpE - 1) / kRpE), (unsigned)(b.d_h / kBT)),
                       dim3(kBT), 0, stream, ra);
    return hipGetLastError();
}

}  // namespace blockffn
