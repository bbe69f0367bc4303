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
//      takes one); then union_tiles_kernel: the chunk union masks and the per-expert
//      tile lists in one launch;
//   1. transpose_tiles_kernel: x and dy copied per 32-token chunk tile as
//      [tile][d_h][32 tokens], so the weight-gradient products, whose k is the token,
//      read k-contiguous operands;
//   2. expert_pass_kernel, workgroup = (expert e, 4 of its tiles), 16 waves: a = X W1_e^T
//      on waves 0-7 and G = DY W2_e on waves 8-15 over d_h (B = W2^T rows), each a
//      128 x 128 tile on 8 waves; then ds, and dA and SH in bf16 in both [token][unit]
//      and [unit][token] order;
//   3. wgrad_kernel, workgroup = (expert, dW1 or dW2, 128 x 128 output tile): k over the
//      expert's tiles' tokens; every output element is owned by one workgroup (an
//      expert no chunk uses gets zeros);
//   4. dx = sum_e dA_e W1_e, B = W1^T rows (W1 and W2 are transposed once per call into
//      the workspace, for the experts some chunk uses, so every product reads
//      k-contiguous operands). With two or more chunk tiles it is the forward's grouped
//      down-projection (dA in the hidden rows' layout), with an fp32 result; with one
//      tile, dx_kernel, workgroup = (4 tiles, 128 columns, expert split): k over the
//      union of the 4 chunks' unions x d_e, the experts split over workgroups. Split
//      partials (either path) are added in split order by the router backward as it
//      adds its own term, so dx is written once;
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
// workgroups, and the deeper loop's registers would cost that occupancy (a 4-deep
// register ring with double-buffered LDS, 168 registers, was timed slower).
constexpr int kWBK = 32;
constexpr int kWLP = kWBK + 8;

__device__ __forceinline__ void zero_acc(f32x16 &a)
{
#pragma unroll
    for (int v = 0; v < 16; ++v)
        a[v] = 0.0f;
}

// ------------------------------------------------------------------ 0. unions and tile lists
// From the recomputed scores, in one launch (expert e of a chunk is in its union when
// some token of the chunk has s[t,e] != 0; -0 is inactive, NaN active, as in the
// forward's union):
//   blocks [0, C): chunk c's union mask words, wave w -> word w, lane -> expert;
//   blocks [C, C + E): expert e's ascending list of the chunk tiles whose chunk holds
//     it (a chunk's rank is the count of earlier chunks holding e), and their count.
// Whether s[t,e] != 0 for some t in [t0, t1): 32 loads in flight at a time (tokens past
// t1 re-read the last one and are masked), so no load waits on its own.
__device__ __forceinline__ bool any_active(const float *__restrict__ scores, int E, int e, int64_t t0,
                                           int64_t t1)
{
    constexpr int kB = 32;
    bool f = false;
    for (int64_t tb = t0; tb < t1; tb += kB) {
        float v[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i)
            v[i] = scores[(tb + i < t1 ? tb + i : t1 - 1) * E + e];
#pragma unroll
        for (int i = 0; i < kB; ++i)
            f |= tb + i < t1 && v[i] != 0.0f;
    }
    return f;
}

__global__ void __launch_bounds__(kBT) union_tiles_kernel(const float *__restrict__ scores, Dims d,
                                                          uint64_t *masks, int32_t *tile_list,
                                                          int32_t *tile_count)
{
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    if (blockIdx.x < (unsigned)d.C) {
        const int64_t c = blockIdx.x;
        const int64_t t0 = c * d.n, t1 = t0 + d.n < d.T ? t0 + d.n : d.T;
        for (int w = wave; w < d.W; w += kBT / kWave) {
            const int e = w * kWave + lane;
            const bool active = e < d.E && any_active(scores, d.E, e, t0, t1);
            const uint64_t word = __ballot(active);
            if (lane == 0)
                masks[c * d.W + w] = word;
        }
        return;
    }
    const int e = (int)(blockIdx.x - (unsigned)d.C);
    __shared__ int wsum[kBT / kWave];
    __shared__ int base;
    if (tid == 0)
        base = 0;
    __syncthreads();
    for (int c0 = 0; c0 < d.C; c0 += kBT) {
        const int c = c0 + tid;
        bool f = false;
        if (c < d.C) {
            const int64_t t0 = (int64_t)c * d.n, t1 = t0 + d.n < d.T ? t0 + d.n : d.T;
            f = any_active(scores, d.E, e, t0, t1);
        }
        const uint64_t bal = __ballot(f);
        const int below = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0)
            wsum[wave] = __popcll(bal);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w)
            off += wsum[w];
        if (f)
            for (int m = 0; m < d.MPC; ++m)
                tile_list[(int64_t)e * d.CT + (int64_t)(off + below) * d.MPC + m] = c * d.MPC + m;
        __syncthreads();
        if (tid == 0)
            for (int w = 0; w < kBT / kWave; ++w)
                base += wsum[w];
        __syncthreads();
    }
    if (tid == 0)
        tile_count[e] = base * d.MPC;
}

// ------------------------------------------------------------------ 1. tile transposes
// dst[tile][j][r] = src[token(tile, r)][j] (zero for rows without a token), for two
// sources in one launch (blockIdx.z: x, then dy).
__global__ void __launch_bounds__(kBT) transpose_tiles_kernel(const uint16_t *src0, const uint16_t *src1,
                                                              Dims d, uint16_t *dst0, uint16_t *dst1)
{
    __shared__ alignas(16) uint16_t t[kTileM][kTrCols + 8];
    const uint16_t *src = blockIdx.z == 0 ? src0 : src1;
    uint16_t *dst = blockIdx.z == 0 ? dst0 : dst1;
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
// experts that no chunk uses are skipped (their copy is never read). Two matrices of
// equal size per launch: blockIdx.z = job * E + e, blockIdx.x = the 64 x 64 block.
struct TransposeJob {
    const uint16_t *src;
    int R, Cc;
    uint16_t *dst;
};
__global__ void __launch_bounds__(kBT) transpose_weights_kernel(TransposeJob j0, TransposeJob j1, int E,
                                                                const int32_t *tile_count)
{
    __shared__ alignas(16) uint16_t t[64][64 + 8];
    const TransposeJob &j = blockIdx.z < (unsigned)E ? j0 : j1;
    const int e = (int)(blockIdx.z % (unsigned)E);
    if (tile_count[e] == 0)
        return;
    const int R = j.R, Cc = j.Cc, nbx = Cc / 64;
    const int r0 = (int)(blockIdx.x / nbx) * 64, c0 = (int)(blockIdx.x % nbx) * 64, tid = threadIdx.x;
    const uint16_t *s = j.src + (int64_t)e * R * Cc;
    uint16_t *o = j.dst + (int64_t)e * R * Cc;
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
constexpr int kPassGroup = 2 * kBT;       // 8 waves per product
constexpr int kPassThreads = 2 * kPassGroup;
constexpr int kPassDepth = 2;             // k steps of loads in flight
static_assert(kPassDepth % 2 == 0, "the LDS double buffer alternates with the ring slot");

// Two 8-wave groups, one workgroup per CU: group 0 forms a = X W1_e^T and group 1
// G = DY W2_e at the same time, each on its own LDS double buffer, each wave a 32 x 64
// block of the 128 x 128 tile (wm = 32-row tile, wn = 64-unit half) with two k steps of
// loads in flight (at most 128 registers: 16 waves per CU). Group 1 then hands G to
// group 0 through LDS (each thread's accumulators to the thread at the same position),
// which applies the epilogue.
__global__ void __launch_bounds__(kPassThreads, 4) expert_pass_kernel(PassArgs a)
{
    const Dims &d = a.d;
    const int e = blockIdx.x % d.E, grp = blockIdx.x / d.E;
    const int cnt = a.tile_count[e];
    if (grp * kPassTiles >= cnt)
        return;
    // [group][A, B][buffer]; afterwards group 1's hold G and group 0's the ds partials
    __shared__ alignas(16) uint16_t ops[2][2][2][kTM * kPP];
    static_assert(sizeof(ops[1]) >= (size_t)kPassGroup * 32 * sizeof(float), "G fits group 1's buffers");
    static_assert(sizeof(ops[0]) >= (size_t)kTM * 65 * sizeof(float), "the ds partials fit group 0's buffers");
    __shared__ float dsacc[kTM], scol[kTM];
    __shared__ int64_t tok[kTM];
    __shared__ int tiles[kPassTiles];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int g = __builtin_amdgcn_readfirstlane(wave >> 3);   // 0: X W1^T, 1: DY W2
    const int gt = tid & (kPassGroup - 1);                     // thread within the group
    const int wm = wave & 3, wn = (wave >> 2) & 1;
    const int col = lane & 31, kg = lane >> 5;
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
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g ? a.dy : a.x, (uint64_t)d.T * d.d_h * 2);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g ? a.w2t : a.w1, (uint64_t)d.E * d.d_e * d.d_h * 2);
    uint16_t *const As0 = ops[g][0][0], *const As1 = ops[g][0][1];
    uint16_t *const Bs0 = ops[g][1][0], *const Bs1 = ops[g][1][1];
    // piece i of this thread per k step: row (gt + 512 i) / 8, k offset (gt % 8) * 8
    uint32_t aoff[2], amask[2];
    int lrow[2], lcol[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = gt + i * kPassGroup;
        lrow[i] = q >> 3;
        lcol[i] = (q & 7) * 8;
        const int64_t t = tok[lrow[i]];
        amask[i] = 0u - (uint32_t)(t >= 0);
        aoff[i] = t >= 0 ? (uint32_t)((t * d.d_h + lcol[i]) * 2) : 0u;
    }
    const int KS = d.d_h / kPK;
    float *gbuf = reinterpret_cast<float *>(ops[1]);   // [32 values][512 threads]
    float *red = reinterpret_cast<float *>(ops[0]);    // [128 rows][65]
    const int tile = __builtin_amdgcn_readfirstlane(tiles[wm]);
    // the epilogue's stores: wave-uniform descriptors of this (tile, expert) block of
    // the [token][unit] and [unit][token] arrays, one lane offset each; the (row group,
    // row, unit block) parts are uniform
    const int64_t blk = ((int64_t)(tile < 0 ? 0 : tile) * d.E + e) * kTileM * d.d_e;
    const uint32_t blk_bytes = (uint32_t)(kTileM * d.d_e * 2);
    const __amdgpu_buffer_rsrc_t rtu = make_rsrc(a.da_tu + blk, blk_bytes);
    const __amdgpu_buffer_rsrc_t rdut = make_rsrc(a.da_ut + blk, blk_bytes);
    const __amdgpu_buffer_rsrc_t rsut = make_rsrc(a.sh_ut + blk, blk_bytes);
    const uint32_t tu_lane = (uint32_t)(((lane >> 5) * 4 * d.d_e + wn * 64 + col) * 2);
    const uint32_t ut_lane = (uint32_t)(((wn * 64 + col) * kTileM + (lane >> 5) * 4) * 2);
    for (int u0 = 0; u0 < d.d_e; u0 += kTM) {
        uint32_t boff[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            boff[i] = (uint32_t)((((int64_t)e * d.d_e + u0 + lrow[i]) * d.d_h + lcol[i]) * 2);
        f32x16 acc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            zero_acc(acc[j]);
        {
            u32x4 ra[kPassDepth][2], rb[kPassDepth][2];
            // every load is issued: rows without a token, and steps past KS, read zeros
            auto issue = [&](int st, int dd) {
                const uint32_t okm = 0u - (uint32_t)(st < KS);
                const uint32_t kb = (uint32_t)(st * kPK * 2);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint32_t am = okm & amask[i];
                    ra[dd][i] = load16(rA, ((aoff[i] + kb) & am) | (kOOB & ~am));
                    rb[dd][i] = load16(rB, ((boff[i] + kb) & okm) | (kOOB & ~okm));
                }
            };
            // in ring order (the scheduling barriers keep it), so that the wait before a
            // slot's LDS store counts only the younger slots' loads
#pragma unroll
            for (int dd = 0; dd < kPassDepth; ++dd) {
                issue(dd, dd);
                __builtin_amdgcn_sched_barrier(0);
            }
            // whole turns of the ring (steps past KS add zeros); both groups take the
            // same steps, so the workgroup barriers pair up
            for (int s0 = 0; s0 < KS; s0 += kPassDepth) {
#pragma unroll
                for (int dd = 0; dd < kPassDepth; ++dd) {
                    uint16_t *As = (dd & 1) ? As1 : As0;
                    uint16_t *Bs = (dd & 1) ? Bs1 : Bs0;
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        *reinterpret_cast<u32x4 *>(&As[lrow[i] * kPP + lcol[i]]) = ra[dd][i];
                        *reinterpret_cast<u32x4 *>(&Bs[lrow[i] * kPP + lcol[i]]) = rb[dd][i];
                    }
                    __syncthreads();
                    issue(s0 + dd + kPassDepth, dd);
#pragma unroll
                    for (int ks = 0; ks < kPK / 16; ++ks) {
                        const bf16x8 fa =
                            *reinterpret_cast<const bf16x8 *>(&As[(wm * 32 + col) * kPP + ks * 16 + kg * 8]);
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const bf16x8 fb = *reinterpret_cast<const bf16x8 *>(
                                &Bs[(wn * 64 + j * 32 + col) * kPP + ks * 16 + kg * 8]);
                            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[j], 0, 0, 0);
                        }
                    }
                }
            }
        }
        // every wave is done with the operand buffers: group 1's take G
        __syncthreads();
        if (g == 1) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    gbuf[(j * 16 + v) * kPassGroup + gt] = acc[j][v];
        }
        __syncthreads();
        if (g == 0) {
            // epilogue: Swish, its slope, the score; element v of accumulator j is row
            // wm * 32 + acc_row(v) (row acc_row(v) of tile wm) and unit u0 + wn * 64 +
            // j * 32 + col
            float part[16];
#pragma unroll
            for (int v = 0; v < 16; ++v)
                part[v] = 0.0f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    uint32_t da_pk[2] = {0u, 0u}, sh_pk[2] = {0u, 0u};
                    const int r0 = acc_row(vg * 4, lane);   // 4 consecutive rows of the tile
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int v = vg * 4 + q, r = r0 + q;
                        const float av = acc[j][v], s = scol[wm * 32 + r];
                        const float gv = gbuf[(j * 16 + v) * kPassGroup + gt];
                        const float sig = 1.0f / (1.0f + expf(-av));
                        const float h = av * sig;
                        part[v] += gv * h;
                        const float dA = s * gv * (sig * (1.0f + av * (1.0f - sig)));
                        const uint32_t b_da = f32_to_bf16(dA), b_sh = f32_to_bf16(s * h);
                        da_pk[q >> 1] |= b_da << ((q & 1) * 16);
                        sh_pk[q >> 1] |= b_sh << ((q & 1) * 16);
                        // row r = (lane / 32) * 4 + 8 vg + q, unit u0 + j * 32 + wn * 64 + col
                        if (tile >= 0)
                            __builtin_amdgcn_raw_buffer_store_b16(
                                (unsigned short)b_da, rtu, (int)tu_lane,
                                (int)(((vg * 8 + q) * d.d_e + u0 + j * 32) * 2), 0);
                    }
                    if (tile >= 0) {
                        const uint32_t so = (uint32_t)(((u0 + j * 32) * kTileM + vg * 8) * 2);
                        const uint64_t dpk = (uint64_t)da_pk[0] | ((uint64_t)da_pk[1] << 32);
                        const uint64_t spk = (uint64_t)sh_pk[0] | ((uint64_t)sh_pk[1] << 32);
                        __builtin_amdgcn_raw_buffer_store_b64(
                            __builtin_bit_cast(unsigned int __attribute__((ext_vector_type(2))), dpk), rdut,
                            (int)ut_lane, (int)so, 0);
                        __builtin_amdgcn_raw_buffer_store_b64(
                            __builtin_bit_cast(unsigned int __attribute__((ext_vector_type(2))), spk), rsut,
                            (int)ut_lane, (int)so, 0);
                    }
                }
            }
            // ds: row partials (units j * 32 + col of this wave's half, j summed) -> LDS
            // [row][64] -> summed in column order
#pragma unroll
            for (int v = 0; v < 16; ++v)
                red[(wm * 32 + acc_row(v, lane)) * 65 + wn * 32 + col] = part[v];
        }
        __syncthreads();
        if (tid < kTM) {
            float sum = 0.0f;
            for (int c = 0; c < 64; ++c)
                sum += red[tid * 65 + c];
            dsacc[tid] += sum;
        }
        __syncthreads();
    }
    if (tid < kTM && tok[tid] >= 0)
        a.ds[tok[tid] * d.E + e] = dsacc[tid];
}

// For few tiles (a backward of a decode-sized batch) the expert pass above would run
// one workgroup per expert and leave most CUs idle. Here each workgroup takes 32 of
// the expert's hidden units, so there are d_e / 32 times as many: waves 0-3 form
// a = X W1_e^T and waves 4-7 G = DY W2_e for the 128 token rows x 32 units (one 32 x 32
// block per wave, two k steps in flight), G goes to the first group through LDS, and
// the epilogue is the one above. The workgroup's share of ds (its 32 units) goes to
// slice ub of ds, [d_e / 32][T][E]; the router backward adds the slices in order.
constexpr int kNarrowUnits = 32;
constexpr int kNarrowGroup = kBT;             // 4 waves per product
constexpr int kNarrowThreads = 2 * kNarrowGroup;
// k steps of loads in flight: 2 (at most 128 registers, two workgroups per CU), or 4
// (153 registers, one per CU) when the grid has no more workgroups than CUs: the
// weight stream then has twice the bytes in flight (T = 32 call 112.7 -> 110.2 us)

template <int DEPTH>
__global__ void __launch_bounds__(kNarrowThreads, DEPTH == 2 ? 2 : 1) expert_pass_narrow_kernel(PassArgs a)
{
    static_assert(DEPTH % 2 == 0, "the LDS double buffer alternates with the ring slot");
    const Dims &d = a.d;
    const int nub = d.d_e / kNarrowUnits;
    const int e = blockIdx.x % d.E;
    const int rest = blockIdx.x / d.E;
    const int ub = rest % nub, grp = rest / nub;
    const int cnt = a.tile_count[e];
    if (grp * kPassTiles >= cnt)
        return;
    __shared__ alignas(16) uint16_t As[2][2][kTM * kPP];            // [group][buffer] token rows
    __shared__ alignas(16) uint16_t Bs[2][2][kNarrowUnits * kPP];   // [group][buffer] unit rows
    __shared__ float gbuf[16][kNarrowGroup];                         // G of group 1
    __shared__ float red[kTM][kNarrowUnits + 1];
    __shared__ float scol[kTM];
    __shared__ int64_t tok[kTM];
    __shared__ int tiles[kPassTiles];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int g = __builtin_amdgcn_readfirstlane(wave >> 2);   // 0: X W1^T, 1: DY W2
    const int gt = tid & (kNarrowGroup - 1);
    const int wm = wave & 3;                                   // 32-row tile
    const int col = lane & 31, kg = lane >> 5;
    if (tid < kPassTiles)
        tiles[tid] = grp * kPassTiles + tid < cnt ? a.tile_list[(int64_t)e * d.CT + grp * kPassTiles + tid] : -1;
    __syncthreads();
    if (tid < kTM) {
        const int64_t t = tile_token(d, tiles[tid / kTileM], tid % kTileM);
        tok[tid] = t;
        scol[tid] = t >= 0 ? a.scores[t * d.E + e] : 0.0f;
    }
    __syncthreads();

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g ? a.dy : a.x, (uint64_t)d.T * d.d_h * 2);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g ? a.w2t : a.w1, (uint64_t)d.E * d.d_e * d.d_h * 2);
    // per k step: A pieces gt + 256 i (row q / 8, k (q % 8) * 8) of the 128 x 64 token
    // tile, and B piece gt (row gt / 8) of the 32 x 64 unit tile
    uint32_t aoff[4], amask[4];
    int arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = gt + i * kNarrowGroup;
        arow[i] = q >> 3;
        const int64_t t = tok[arow[i]];
        amask[i] = 0u - (uint32_t)(t >= 0);
        aoff[i] = t >= 0 ? (uint32_t)((t * d.d_h + (q & 7) * 8) * 2) : 0u;
    }
    const int acol = (gt & 7) * 8, brow = gt >> 3;
    const uint32_t boff = (uint32_t)((((int64_t)e * d.d_e + ub * kNarrowUnits + brow) * d.d_h + acol) * 2);
    const int KS = d.d_h / kPK;
    f32x16 acc;
    zero_acc(acc);
    {
        u32x4 ra[DEPTH][4], rb[DEPTH];
        auto issue = [&](int st, int dd) {
            const uint32_t okm = 0u - (uint32_t)(st < KS);
            const uint32_t kb = (uint32_t)(st * kPK * 2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t am = okm & amask[i];
                ra[dd][i] = load16(rA, ((aoff[i] + kb) & am) | (kOOB & ~am));
            }
            rb[dd] = load16(rB, ((boff + kb) & okm) | (kOOB & ~okm));
        };
#pragma unroll
        for (int dd = 0; dd < DEPTH; ++dd) {
            issue(dd, dd);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int s0 = 0; s0 < KS; s0 += DEPTH) {
#pragma unroll
            for (int dd = 0; dd < DEPTH; ++dd) {
                const int buf = dd & 1;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<u32x4 *>(&As[g][buf][arow[i] * kPP + ((gt + i * kNarrowGroup) & 7) * 8]) =
                        ra[dd][i];
                *reinterpret_cast<u32x4 *>(&Bs[g][buf][brow * kPP + acol]) = rb[dd];
                __syncthreads();
                issue(s0 + dd + DEPTH, dd);
#pragma unroll
                for (int ks = 0; ks < kPK / 16; ++ks) {
                    const bf16x8 fa =
                        *reinterpret_cast<const bf16x8 *>(&As[g][buf][(wm * 32 + col) * kPP + ks * 16 + kg * 8]);
                    const bf16x8 fb =
                        *reinterpret_cast<const bf16x8 *>(&Bs[g][buf][col * kPP + ks * 16 + kg * 8]);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
                }
            }
        }
    }
    if (g == 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
            gbuf[v][gt] = acc[v];
    }
    __syncthreads();
    if (g == 0) {
        // element v: row acc_row(v) of tile wm, unit ub * 32 + col
        const int tile = __builtin_amdgcn_readfirstlane(tiles[wm]);
        const int unit = ub * kNarrowUnits + col;
        if (tile >= 0) {
            const int64_t blk = ((int64_t)tile * d.E + e) * kTileM * d.d_e;
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                uint32_t da_pk[2] = {0u, 0u}, sh_pk[2] = {0u, 0u};
                const int r0 = acc_row(vg * 4, lane);   // 4 consecutive rows of the tile
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int v = vg * 4 + q, r = r0 + q;
                    const float av = acc[v], s = scol[wm * 32 + r], gv = gbuf[v][gt];
                    const float sig = 1.0f / (1.0f + expf(-av));
                    const float h = av * sig;
                    red[wm * 32 + r][col] = gv * h;
                    const float dA = s * gv * (sig * (1.0f + av * (1.0f - sig)));
                    const uint32_t b_da = f32_to_bf16(dA), b_sh = f32_to_bf16(s * h);
                    da_pk[q >> 1] |= b_da << ((q & 1) * 16);
                    sh_pk[q >> 1] |= b_sh << ((q & 1) * 16);
                    a.da_tu[blk + (int64_t)r * d.d_e + unit] = (uint16_t)b_da;
                }
                const int64_t o = blk + (int64_t)unit * kTileM + r0;
                *reinterpret_cast<uint64_t *>(&a.da_ut[o]) = (uint64_t)da_pk[0] | ((uint64_t)da_pk[1] << 32);
                *reinterpret_cast<uint64_t *>(&a.sh_ut[o]) = (uint64_t)sh_pk[0] | ((uint64_t)sh_pk[1] << 32);
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v)
                red[wm * 32 + acc_row(v, lane)][col] = 0.0f;
        }
    }
    __syncthreads();
    // this unit block's share of ds, summed over its 32 units in order
    if (tid < kTM && tok[tid] >= 0) {
        float sum = 0.0f;
        for (int c = 0; c < kNarrowUnits; ++c)
            sum += red[tid][c];
        a.ds[((int64_t)ub * d.T + tok[tid]) * d.E + e] = sum;
    }
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

// ------------------------------------------------------------------ 5. router backward
struct RouterArgs {
    const uint16_t *x, *w_r;
    const float *gain, *dprobs;
    const float *logits, *scores;        // [T][E]
    const float *ds;                      // [ds_splits][T][E]: slices added in order
    const uint64_t *masks;                // [C][W]
    float *dl, *gt;                       // [T][E]
    float *dx, *dw_r, *dgain, *dbias;
    // the expert products' dx: dx itself (dx_splits == 1), or dx_splits partials
    // [dx_splits][CT][32][d_h] that the router backward adds in split order
    const float *dx_part;
    int dx_splits;
    float eps, sharpness;
    int ds_splits;
    int rt_slices;                        // 256-column slices of dx per router-token workgroup
    Dims d;
};

// The expert products' dx of token t at columns j .. j + 3: read from dx, or the sum of
// the k-split partials in split order (the same additions the split sum would make).
__device__ __forceinline__ float4 expert_dx4(const RouterArgs &a, int64_t t, int j)
{
    const Dims &d = a.d;
    if (a.dx_splits <= 1)
        return *reinterpret_cast<const float4 *>(&a.dx[t * d.d_h + j]);
    const int64_t c = t / d.n;
    const int ic = (int)(t - c * d.n);
    const int64_t row = (c * d.MPC + ic / kTileM) * kTileM + ic % kTileM;
    const int64_t stride = (int64_t)d.CT * kTileM * d.d_h;
    const float *p = a.dx_part + row * d.d_h + j;
    float4 sum = *reinterpret_cast<const float4 *>(p);
    for (int z = 1; z < a.dx_splits; ++z) {
        const float4 v = *reinterpret_cast<const float4 *>(p + z * stride);
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
    }
    return sum;
}

constexpr int kRtTokens = 4;              // tokens per router-token workgroup (one per wave)
constexpr int kRtPer = 256 / kWave;       // experts per lane (E <= 256)
constexpr int kRtCols = 256;              // d_h columns of dx per router-token workgroup
constexpr int kRtPieces = kRtCols / 8;    // 8-column pieces: 32
constexpr int kRtGroups = kBT / kRtPieces;   // expert groups: 8
static_assert(kRtGroups * kRtPieces == kBT, "thread = (piece, expert group)");
constexpr int64_t kRtMinBlocks = 512;

// p[0 .. n) = 0 (the recomputed router's arrival counters: this workspace is not
// zero-filled by the caller)
__global__ void __launch_bounds__(kBT) zero_words_kernel(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kBT + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

// Per token (one wavefront each, kRtTokens per workgroup): ds (masked to the chunk's
// union, plus the probability term), the RMSNorm and ReLU backward -> dl, and the gain
// term; then dx[t] += W_r^T dl for the workgroup's tokens, each W_r row piece loaded
// once for all of them. !SPLIT: one workgroup per token group, over all of d_h. SPLIT
// (few token groups): one workgroup per token group and run of rt_slices 256-column
// slices of d_h, so that more workgroups share the W_r stream; the first run writes dl
// and the gain term.
template <bool SPLIT>
__global__ void __launch_bounds__(kBT) router_token_kernel(RouterArgs a)
{
    const Dims &d = a.d;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int nsb = SPLIT ? d.d_h / kRtCols / a.rt_slices : 1;   // slice blocks per token group
    const int64_t t0 = (int64_t)(blockIdx.x / nsb) * kRtTokens;
    const int slice0 = (blockIdx.x % nsb) * a.rt_slices;
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
                    for (int q = 0; q < a.ds_splits; ++q)
                        ds[i] += a.ds[((int64_t)q * d.T + t) * d.E + e];
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
            if (vt && e < d.E && slice0 == 0) {
                a.dl[t * d.E + e] = dl;
                a.gt[t * d.E + e] = ds[i] * r[i] * inv;
            }
        }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w_r, (uint64_t)d.E * d.d_h * 2);
    if constexpr (!SPLIT) {
        // dx[t] += W_r^T dl, all of d_h: thread -> 8 columns, the experts in order
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
                float4 o0 = expert_dx4(a, t, jv * 8), o1 = expert_dx4(a, t, jv * 8 + 4);
                o0.x += acc[k][0], o0.y += acc[k][1], o0.z += acc[k][2], o0.w += acc[k][3];
                o1.x += acc[k][4], o1.y += acc[k][5], o1.z += acc[k][6], o1.w += acc[k][7];
                o[0] = o0;
                o[1] = o1;
            }
        }
    } else {
        // dx[t, slice columns] += W_r^T dl: thread (8-column piece pc, expert group eg) sums
        // experts eg, eg + 8, ... (all of its W_r loads in flight at once); the 8 groups'
        // partials are added in group order through LDS
        __shared__ float part[kRtGroups][kRtTokens][kRtCols + 4];
        const int pc = tid % kRtPieces, eg = tid / kRtPieces;
        for (int slice = slice0; slice < slice0 + a.rt_slices; ++slice) {
            const int j0 = slice * kRtCols + pc * 8;
            float acc[kRtTokens][8];
#pragma unroll
            for (int k = 0; k < kRtTokens; ++k)
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[k][q] = 0.0f;
            for (int e0 = eg; e0 < d.E; e0 += kRtGroups * 8) {
                u32x4 w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + u * kRtGroups;
                    w[u] = load16(rw, e < d.E ? (uint32_t)(((int64_t)e * d.d_h + j0) * 2) : kOOB);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + u * kRtGroups;
#pragma unroll
                    for (int k = 0; k < kRtTokens; ++k) {
                        const float dk = e < d.E ? dl_s[k][e] : 0.0f;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            acc[k][2 * q] = fmaf(dk, __uint_as_float(w[u][q] << 16), acc[k][2 * q]);
                            acc[k][2 * q + 1] = fmaf(dk, __uint_as_float(w[u][q] & 0xffff0000u), acc[k][2 * q + 1]);
                        }
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < kRtTokens; ++k)
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    part[eg][k][pc * 8 + q] = acc[k][q];
            __syncthreads();
            // thread -> (token k, 4 columns c4): the groups in order, then dx += the sum
            for (int v = tid; v < kRtTokens * kRtCols / 4; v += kBT) {
                const int k = v / (kRtCols / 4), c4 = (v % (kRtCols / 4)) * 4;
                const int64_t t = t0 + k;
                if (t >= d.T)
                    continue;
                float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int g = 0; g < kRtGroups; ++g) {
                    sum.x += part[g][k][c4];
                    sum.y += part[g][k][c4 + 1];
                    sum.z += part[g][k][c4 + 2];
                    sum.w += part[g][k][c4 + 3];
                }
                float4 *o = reinterpret_cast<float4 *>(&a.dx[t * d.d_h + slice * kRtCols + c4]);
                float4 o0 = expert_dx4(a, t, slice * kRtCols + c4);
                o0.x += sum.x, o0.y += sum.y, o0.z += sum.z, o0.w += sum.w;
                *o = o0;
            }
            __syncthreads();   // part is refilled by the next slice
        }
    }
}

constexpr int kRpE = 8;       // experts per router-parameter workgroup
constexpr int kRpTargetBlocks = 512;
constexpr int kRpMaxSplits = 16;

// Token splits of the router-parameter sums: about kRpTargetBlocks workgroups (two per
// CU), at most kRpMaxSplits splits, at least 32 tokens per split.
int router_param_splits(int64_t T, int64_t d_h, int64_t E)
{
    const int64_t base = ((E + kRpE - 1) / kRpE) * (d_h / kBT);
    int64_t s = (kRpTargetBlocks + base - 1) / base;
    int64_t smax = (T + 31) / 32;
    if (smax > kRpMaxSplits)
        smax = kRpMaxSplits;
    if (s > smax)
        s = smax;
    return s < 1 ? 1 : (int)s;
}

constexpr int kRpTok = 128;   // tokens of dl (and gt) staged in LDS at a time
constexpr int kRpLanes = 8;   // token lanes: thread = (8-column piece, token lane)
constexpr int kRpCols = 256;  // columns per router-parameter workgroup
static_assert((kRpCols / 8) * kRpLanes == kBT, "thread = (piece, token lane)");

// Partial sums over token split z, tokens ascending within each token lane:
//   part[z][e][j] = sum_{t in z} dl[t][e] x[t][j]      (dW_r)
//   gpart[z][e]   = (sum_{t in z} gt[t][e], sum_{t in z} dl[t][e])   (dgain, dbias)
// Thread (piece pc, token lane tl) takes 8 columns of x (one 16-byte load per token)
// over the tokens tl, tl + 8, ... of the split, 8 of them in flight; the 8 lanes are
// added in lane order through LDS. The workgroups of column block 0 also sum gt and
// dl per expert (thread (expert tid % 8, slice tid / 8 of 32), slices in order).
// With one split (direct) part is dW_r itself and the gain and bias sums go straight to
// dgain and dbias: no reduction launch follows.
__global__ void __launch_bounds__(kBT) router_param_kernel(RouterArgs a, int splits, float *part,
                                                           float *gpart, bool direct)
{
    const Dims &d = a.d;
    const int e0 = blockIdx.x * kRpE, jb = blockIdx.y, z = blockIdx.z, tid = threadIdx.x;
    const int64_t per = (d.T + splits - 1) / splits;
    const int64_t t0 = z * per, t1 = t0 + per < d.T ? t0 + per : d.T;
    __shared__ alignas(16) float dls[kRpTok][kRpE];
    __shared__ float gts[kRpTok][kRpE];
    __shared__ float red[kRpLanes][kRpE][kRpCols + 4];
    const int pc = tid % (kRpCols / 8), tl = tid / (kRpCols / 8);
    const int j0 = jb * kRpCols + pc * 8;
    const int gq = tid % kRpE, gsl = tid / kRpE;
    float acc[kRpE][8];
#pragma unroll
    for (int q = 0; q < kRpE; ++q)
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[q][c] = 0.0f;
    float sg = 0.0f, sb = 0.0f;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint64_t)d.T * d.d_h * 2);
    for (int64_t tb = t0; tb < t1; tb += kRpTok) {
        const int nt = (int)(t1 - tb < kRpTok ? t1 - tb : kRpTok);
        {
            const int u = tid / 2, q0 = (tid % 2) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool ok = u < nt && e0 + q0 + q < d.E;
                const int64_t o = (tb + u) * d.E + e0 + q0 + q;
                dls[u][q0 + q] = ok ? a.dl[o] : 0.0f;
                if (jb == 0)
                    gts[u][q0 + q] = ok ? a.gt[o] : 0.0f;
            }
        }
        __syncthreads();
        if (jb == 0)
            for (int u = gsl; u < nt; u += kBT / kRpE) {
                sg += gts[u][gq];
                sb += dls[u][gq];
            }
        for (int u0 = tl; u0 < nt; u0 += kRpLanes * 8) {
            u32x4 xv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int u = u0 + i * kRpLanes;
                xv[i] = load16(rx, u < nt ? (uint32_t)(((tb + u) * d.d_h + j0) * 2) : kOOB);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int u = u0 + i * kRpLanes;
                if (u < nt) {
                    const float4 dA = *reinterpret_cast<const float4 *>(&dls[u][0]);
                    const float4 dB = *reinterpret_cast<const float4 *>(&dls[u][4]);
                    const float dv[kRpE] = {dA.x, dA.y, dA.z, dA.w, dB.x, dB.y, dB.z, dB.w};
#pragma unroll
                    for (int q = 0; q < kRpE; ++q)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            acc[q][2 * c] = fmaf(dv[q], __uint_as_float(xv[i][c] << 16), acc[q][2 * c]);
                            acc[q][2 * c + 1] =
                                fmaf(dv[q], __uint_as_float(xv[i][c] & 0xffff0000u), acc[q][2 * c + 1]);
                        }
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < kRpE; ++q)
#pragma unroll
        for (int c = 0; c < 8; ++c)
            red[tl][q][pc * 8 + c] = acc[q][c];
    float *const pg = &red[0][0][0], *const pb = pg + kBT;   // reused after the lane sums
    __syncthreads();
    // thread -> (expert q, 8 columns): the token lanes in order
    {
        const int q = tid / (kRpCols / 8), c0 = (tid % (kRpCols / 8)) * 8;
        float sum[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
            sum[c] = 0.0f;
#pragma unroll
        for (int l = 0; l < kRpLanes; ++l)
#pragma unroll
            for (int c = 0; c < 8; ++c)
                sum[c] += red[l][q][c0 + c];
        if (e0 + q < d.E) {
            float4 *o = reinterpret_cast<float4 *>(&part[((int64_t)z * d.E + e0 + q) * d.d_h + jb * kRpCols + c0]);
            o[0] = make_float4(sum[0], sum[1], sum[2], sum[3]);
            o[1] = make_float4(sum[4], sum[5], sum[6], sum[7]);
        }
    }
    if (jb != 0)
        return;
    __syncthreads();
    pg[tid] = sg;
    pb[tid] = sb;
    __syncthreads();
    if (tid < kRpE && e0 + tid < d.E) {
        float g = 0.0f, bsum = 0.0f;
        for (int s2 = 0; s2 < kBT / kRpE; ++s2) {
            g += pg[s2 * kRpE + tid];
            bsum += pb[s2 * kRpE + tid];
        }
        if (direct) {
            if (a.dgain)
                a.dgain[e0 + tid] = g;
            if (a.dbias)
                a.dbias[e0 + tid] = bsum;
        } else {
            gpart[((int64_t)z * d.E + e0 + tid) * 2] = g;
            gpart[((int64_t)z * d.E + e0 + tid) * 2 + 1] = bsum;
        }
    }
}

// dW_r, dgain and dbias = the splits' partials added in split order: workgroup =
// (expert e, 256 columns), thread = column, all of its ZC >= splits loads requested
// together (past the last split they read zero and are not added). The workgroups of
// column block 0 also add the expert's dgain and dbias partials.
template <int ZC>
__global__ void __launch_bounds__(kBT) router_param_reduce_kernel(RouterArgs a, int splits,
                                                                  const float *part,
                                                                  const float *gpart)
{
    const Dims &d = a.d;
    const int e = blockIdx.x, j = blockIdx.y * kBT + threadIdx.x, tid = threadIdx.x;
    const __amdgpu_buffer_rsrc_t rpp = make_rsrc(part, (uint64_t)splits * d.E * d.d_h * 4);
    float pv[ZC];
#pragma unroll
    for (int z = 0; z < ZC; ++z)
        pv[z] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       rpp, z < splits ? (int)((((int64_t)z * d.E + e) * d.d_h + j) * 4) : (int)kOOB, 0, 0));
    float sum = 0.0f;
#pragma unroll
    for (int z = 0; z < ZC; ++z)
        if (z < splits)
            sum += pv[z];
    a.dw_r[(int64_t)e * d.d_h + j] = sum;
    if (blockIdx.y != 0 || tid != 0)
        return;
    float g = 0.0f, bsum = 0.0f;
    for (int z = 0; z < splits; ++z) {
        g += gpart[((int64_t)z * d.E + e) * 2];
        bsum += gpart[((int64_t)z * d.E + e) * 2 + 1];
    }
    if (a.dgain)
        a.dgain[e] = g;
    if (a.dbias)
        a.dbias[e] = bsum;
}

// ------------------------------------------------------------------ workspace layout
struct BwdLayout {
    FfnPlan p;
    size_t masks, tile_list, tile_count;
    size_t logits, scores, ds, dl, gt;
    size_t xt, dyt, da_tu, da_ut, sh_ut, rp_part, rp_gpart, w1t, w2t, dx_part;
    size_t router;        // the forward router's split workspace (0 bytes when it takes none)
    int dx_splits;
    bool dx_grouped;      // dx on the forward's grouped down-projection (two or more tiles)
    int ds_splits;        // 1, or d_e / 32 with the narrow expert pass
    size_t total;
};

constexpr int kDxTargetBlocks = 256;

// The narrow expert pass when the (expert, 4 tiles) workgroups would not fill the CUs.
bool pass_narrow(int64_t E, int64_t CT, int64_t d_e)
{
    return E * ((CT + kPassTiles - 1) / kPassTiles) < 256 && d_e % kNarrowUnits == 0;
}

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
    L.tile_list = take(4 * E * p.CT);
    L.tile_count = take(4 * E);
    L.logits = take(4 * T * E);
    L.scores = take(4 * T * E);
    L.ds_splits = pass_narrow(E, p.CT, d_e) ? (int)(d_e / kNarrowUnits) : 1;
    L.ds = take(4 * (size_t)L.ds_splits * T * E);
    L.dl = take(4 * T * E);
    L.gt = take(4 * T * E);
    L.xt = take(2 * p.CT * d_h * kTileM);
    L.dyt = take(2 * p.CT * d_h * kTileM);
    L.da_tu = take(2 * p.CT * E * kTileM * d_e);
    L.da_ut = take(2 * p.CT * E * kTileM * d_e);
    L.sh_ut = take(2 * p.CT * E * kTileM * d_e);
    L.rp_part = take(4 * (size_t)router_param_splits(T, d_h, E) * E * d_h);
    L.rp_gpart = take(8 * (size_t)router_param_splits(T, d_h, E) * E);
    L.router = take(router_workspace_bytes(T, d_h, E));
    L.w1t = take(2 * (size_t)E * d_e * d_h);
    L.w2t = take(2 * (size_t)E * d_e * d_h);
    L.dx_grouped = p.grouped;
    L.dx_splits = dx_splits(p.CT, d_h, E);
    L.dx_part = take(L.dx_grouped ? grouped_partial_bytes(p.CT, d_h)
                     : L.dx_splits > 1 ? 4 * (size_t)L.dx_splits * p.CT * kTileM * d_h
                                       : 0);
    L.total = off;
    L.p.off_masks = L.masks;
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
                                        logits, 1.0f, nullptr, rws, rws ? b.xcds : 0, stream);
    if (err != hipSuccess)
        return err;
    uint64_t *masks = reinterpret_cast<uint64_t *>(at(L.masks));
    int32_t *tile_list = reinterpret_cast<int32_t *>(at(L.tile_list));
    int32_t *tile_count = reinterpret_cast<int32_t *>(at(L.tile_count));
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
    hipLaunchKernelGGL(union_tiles_kernel, dim3((unsigned)(p.C + b.E)), dim3(kBT), 0, stream, scores, d,
                       masks, tile_list, tile_count);
    uint16_t *w1t = reinterpret_cast<uint16_t *>(at(L.w1t));
    uint16_t *w2t = reinterpret_cast<uint16_t *>(at(L.w2t));
    // W1 [E][d_e][d_h] -> [E][d_h][d_e], W2 [E][d_h][d_e] -> [E][d_e][d_h], used experts only
    const TransposeJob tw1{b.w1, (int)b.d_e, (int)b.d_h, w1t}, tw2{b.w2, (int)b.d_h, (int)b.d_e, w2t};
    hipLaunchKernelGGL(transpose_weights_kernel,
                       dim3((unsigned)((b.d_h / 64) * (b.d_e / 64)), 1u, (unsigned)(2 * b.E)), dim3(kBT), 0,
                       stream, tw1, tw2, (int)b.E, tile_count);
    uint16_t *xt = reinterpret_cast<uint16_t *>(at(L.xt));
    uint16_t *dyt = reinterpret_cast<uint16_t *>(at(L.dyt));
    const dim3 tgrid((unsigned)p.CT, (unsigned)(b.d_h / kTrCols), 2u);
    hipLaunchKernelGGL(transpose_tiles_kernel, tgrid, dim3(kBT), 0, stream, b.x, b.dy, d, xt, dyt);

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
    if (L.ds_splits > 1 && pass_blocks * L.ds_splits <= 256)
        hipLaunchKernelGGL(expert_pass_narrow_kernel<4>, dim3((unsigned)(pass_blocks * L.ds_splits)),
                           dim3(kNarrowThreads), 0, stream, pa);
    else if (L.ds_splits > 1)
        hipLaunchKernelGGL(expert_pass_narrow_kernel<2>, dim3((unsigned)(pass_blocks * L.ds_splits)),
                           dim3(kNarrowThreads), 0, stream, pa);
    else
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

    // the expert products' dx, or (k split) their partials, which the router backward
    // adds up in split order
    const float *dx_part = reinterpret_cast<const float *>(at(L.dx_part));
    int dx_parts = 1;
    if (L.dx_grouped) {
        // two or more chunk tiles: dx = sum_e dA_e W1_e is the grouped down-projection's
        // product (dA in the hidden rows' layout, W1^T in W2's), in fp32
        const hipError_t gerr = launch_grouped_down_f32(
            p, pa.da_tu, w1t, masks, b.dx, reinterpret_cast<float *>(at(L.dx_part)), false, stream);
        if (gerr != hipSuccess)
            return gerr;
        dx_parts = grouped_down_splits(p.CT, b.d_h);
    } else {
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
        dx_parts = L.dx_splits;
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
    ra.ds_splits = L.ds_splits;
    ra.dx_part = dx_part;
    ra.dx_splits = dx_parts;
    ra.d = d;
    // a long batch: one workgroup per token group over all of d_h; a short one: the
    // columns split into 256-column slices, rt_slices of them per workgroup, as many as
    // keep at least kRtMinBlocks workgroups
    const int64_t tgroups = (b.T + kRtTokens - 1) / kRtTokens, nslice = b.d_h / kRtCols;
    ra.rt_slices = 1;
    if (tgroups >= kRtMinBlocks) {
        ra.rt_slices = (int)nslice;
        hipLaunchKernelGGL(router_token_kernel<false>, dim3((unsigned)tgroups), dim3(kBT), 0, stream, ra);
    } else {
        while (ra.rt_slices < nslice && nslice % (2 * ra.rt_slices) == 0 &&
               tgroups * (nslice / (2 * ra.rt_slices)) >= kRtMinBlocks)
            ra.rt_slices *= 2;
        hipLaunchKernelGGL(router_token_kernel<true>, dim3((unsigned)(tgroups * (nslice / ra.rt_slices))),
                           dim3(kBT), 0, stream, ra);
    }
    const int splits = router_param_splits(b.T, b.d_h, b.E);
    float *rp = reinterpret_cast<float *>(at(L.rp_part));
    float *rg = reinterpret_cast<float *>(at(L.rp_gpart));
    const unsigned eb = (unsigned)((b.E + kRpE - 1) / kRpE);
    // (dW_r takes 16-byte stores; a dW_r the caller did not align that far takes the
    // reduction path)
    if (splits == 1 && reinterpret_cast<uintptr_t>(b.dw_r) % 16 == 0) {
        hipLaunchKernelGGL(router_param_kernel, dim3(eb, (unsigned)(b.d_h / kRpCols), 1u), dim3(kBT), 0,
                           stream, ra, 1, b.dw_r, rg, true);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(router_param_kernel, dim3(eb, (unsigned)(b.d_h / kRpCols), (unsigned)splits),
                       dim3(kBT), 0, stream, ra, splits, rp, rg, false);
    const dim3 rgrid((unsigned)b.E, (unsigned)(b.d_h / kBT));
#define RP_REDUCE(ZC)                                                                        \
    hipLaunchKernelGGL(router_param_reduce_kernel<ZC>, rgrid, dim3(kBT), 0, stream, ra, splits, \
                       static_cast<const float *>(rp), static_cast<const float *>(rg))
    if (splits <= 1)
        RP_REDUCE(1);
    else if (splits <= 4)
        RP_REDUCE(4);
    else if (splits <= 8)
        RP_REDUCE(8);
    else
        RP_REDUCE(kRpMaxSplits);
#undef RP_REDUCE
    return hipGetLastError();
}

}  // namespace blockffn
