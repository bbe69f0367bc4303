// Multi-chunk bf16 chunk FFN with expert-grouped up-projection (prefill shapes).
//
// Skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
// Deployment": "Core Concept" (each chunk evaluates the union of its tokens' experts
// and masks the results by the scores afterwards) and "Architecture Overview"
// (non-gated Swish experts):
//     Ht[c,e][t,:] = bf16( s[t,e] * swish(W1_e x_t) )   e in U_c, t in chunk c
//     y[t,:]       = bf16( sum_{e in U_c} W2_e Ht[c,e][t,:] )
//
// Over many chunks an expert's weights serve every chunk whose union holds it, so
// each launch should read them once, not once per chunk:
//   1. union_kernel: per-chunk union masks, lists and counts.
//   2. up_grouped_kernel: workgroup = (expert e, 4 of e's tiles): a 128 x d_e x d_h
//      GEMM (x rows gathered, W1_e read once per workgroup and shared through the
//      XCD's L2 by the workgroups of the same expert, which the grid places on one
//      XCD), double-buffered through LDS with kUpDepth k steps of loads in flight
//      (few enough registers for two 8-wave workgroups per CU), 32x32x16 bf16 MFMA,
//      then Swish and the score (staged in LDS with the rows' tokens); the bf16 hidden
//      rows go to Ht[tile][e].
//   3. down_grouped_kernel: workgroup = (2 or 4 chunk tiles, 256 output columns): a
//      64 (128) x 256 GEMM over k = the union of the tiles' chunks' experts x d_e
//      (four tiles from four chunk tiles up), ascending,
//      with the hidden rows of a tile whose chunk does not use the expert read as
//      zero (those terms are exactly zero: the scores are zero there). Every output
//      element is owned by one workgroup, so there is no cross-workgroup sum, and the
//      column tiles map to XCDs so each W2 column slice stays in one L2. When those
//      workgroups would not fill the chip (few chunks, e.g. 16 chunks of a d_h = 4096
//      layer: 128 workgroups), k is split in 2 or 4 contiguous ranges, each
//      workgroup writes its fp32 partial tile, and 4. down_reduce_kernel adds the
//      partials in split order into y.
#include "common.h"
#include "plan.h"
#include "sync.h"

namespace blockffn {

namespace {

constexpr int kGThreads = 512;            // 8 waves
constexpr int kKStep = 64;                // k per pipeline step
constexpr int kPitch = kKStep + 8;        // LDS row pitch (bf16): 144 bytes, conflict-free
constexpr int kUpTiles = 4;               // chunk tiles (32 rows each) per up workgroup
constexpr int kUpRows = kUpTiles * kTileM;    // 128
constexpr int kUpCols = 128;              // hidden units per pass
constexpr int kDnCols = 256;              // output columns per down workgroup
constexpr int kMaxWords = 4;
constexpr int kDepth = 4;                 // k steps whose loads are in flight ahead of use
constexpr int kUpDepth = 2;               // up: the same, in 32 registers, so two workgroups fit a CU
static_assert(kDepth % 2 == 0 && kUpDepth % 2 == 0, "the LDS double buffer alternates with the ring slot");
// A buffer offset beyond every range used here: the load returns zero, no memory access.
constexpr uint32_t kOutOfRange = 0x80000000u;

struct GroupedArgs {
    const uint16_t *x;
    const float *scores;
    const uint16_t *w1;
    const uint16_t *w2;
    uint16_t *y;
    uint16_t *hidden;            // [CT][E][32][d_e]
    const uint64_t *masks;       // [C][W]
    float *dn_part;              // [splits][CT * 32][d_h] when splits > 1
    float *y32;                  // fp32 output instead of y (the layer backward's dx)
    int64_t T;
    int n, d_h, E, d_e, C, MPC, CT, W;
    int splits;
};

// Token of row r of chunk tile `tile`, or -1 when the row holds no token.
__device__ __forceinline__ int64_t tile_token(const GroupedArgs &a, int tile, int r)
{
    if (tile < 0)
        return -1;
    const int c = tile / a.MPC, m = tile % a.MPC;
    const int in_chunk = m * kTileM + r;
    const int64_t t = (int64_t)c * a.n + in_chunk;
    return (in_chunk < a.n && t < a.T) ? t : -1;
}

// 32x32 accumulator layout: element i of a lane is row (i/4)*8 + (lane/32)*4 + i%4 of
// column lane%32.
__device__ __forceinline__ int acc_row(int i, int lane) { return (i / 4) * 8 + (lane >> 5) * 4 + (i % 4); }

// ------------------------------------------------------------------ up (grouped GEMM)
// At least 4 waves per SIMD (at most 128 registers): two 8-wave workgroups per CU.
__global__ void __launch_bounds__(kGThreads, 4) up_grouped_kernel(GroupedArgs a)
{
    const int e = blockIdx.x % a.E;
    const int b = blockIdx.x / a.E;
    __shared__ alignas(16) uint16_t As[2][kUpRows * kPitch];   // x rows x 64 k
    __shared__ alignas(16) uint16_t Bs[2][kUpCols * kPitch];   // W1 rows (hidden units) x 64 k
    __shared__ int64_t tok[kUpRows];
    __shared__ float scol[kUpRows];   // score of (row's token, e), zero for rows without one
    __shared__ int tiles[kUpTiles];

    __shared__ int ntiles;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave & 3, wn = wave >> 2;       // 32-row tile, 64-unit half
    const int col = lane & 31, kg = lane >> 5;
    // Tiles 4b .. 4b + 3 of e's ascending tile list, from the chunks' union masks: lane
    // c of the first wave tests chunk c0 + c, and a chunk's rank among e's chunks is
    // the count of set ballot bits below it (plus the earlier blocks' counts).
    if (wave == 0) {
        if (lane < kUpTiles)
            tiles[lane] = -1;
        int base = 0;
        for (int c0 = 0; c0 < a.C; c0 += kWave) {
            const int c = c0 + lane;
            const bool f = c < a.C && ((a.masks[(int64_t)c * a.W + (e >> 6)] >> (e & 63)) & 1ull);
            const uint64_t bal = __ballot(f);
            const int rank = base + __popcll(bal & ((1ull << lane) - 1ull));
            if (f)
                for (int m = 0; m < a.MPC; ++m) {
                    const int i = rank * a.MPC + m - b * kUpTiles;
                    if (i >= 0 && i < kUpTiles)
                        tiles[i] = c * a.MPC + m;
                }
            base += __popcll(bal);
        }
        if (lane == 0)
            ntiles = base * a.MPC;
    }
    __syncthreads();
    if (b * kUpTiles >= ntiles)
        return;
    if (tid < kUpRows) {
        const int64_t t = tile_token(a, tiles[tid / kTileM], tid % kTileM);
        tok[tid] = t;
        scol[tid] = t >= 0 ? a.scores[t * a.E + e] : 0.0f;
    }
    __syncthreads();

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint64_t)a.T * a.d_h * 2);
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(a.w1, (uint64_t)a.E * a.d_e * a.d_h * 2);
    // per thread: 2 A chunks and 2 B chunks (16 bytes) per k step; chunk q = tid + 512 i:
    // row q / 8, k offset (q % 8) * 8
    uint32_t aoff[2], boff[2];
    bool av[2];
    int lrow[2], lcol[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + i * kGThreads;
        lrow[i] = q >> 3;
        lcol[i] = (q & 7) * 8;
        const int64_t t = tok[lrow[i]];
        av[i] = t >= 0;
        aoff[i] = av[i] ? (uint32_t)((t * a.d_h + lcol[i]) * 2) : 0u;
    }
    const int KS = a.d_h / kKStep;
    for (int nb = 0; nb < a.d_e; nb += kUpCols) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            boff[i] = (uint32_t)((((int64_t)e * a.d_e + nb + lrow[i]) * a.d_h + lcol[i]) * 2);
        f32x16 acc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[j][v] = 0.0f;
        // kUpDepth k steps of loads in flight, every load issued: rows without a token,
        // and steps past KS, read zeros
        bf16x8 ra[kUpDepth][2], rb[kUpDepth][2];
        auto issue = [&](int st, int d) {
            const uint32_t okm = 0u - (uint32_t)(st < KS);
            const uint32_t kb = (uint32_t)(st * kKStep * 2);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t am = okm & (0u - (uint32_t)av[i]);
                ra[d][i] = bload<0>(rx, ((aoff[i] + kb) & am) | (kOutOfRange & ~am));
                rb[d][i] = bload<0>(rw1, ((boff[i] + kb) & okm) | (kOutOfRange & ~okm));
            }
        };
        // issued in ring order (the scheduling barriers keep it) so that the wait before
        // a slot's LDS store counts only the younger slots' loads
#pragma unroll
        for (int d = 0; d < kUpDepth; ++d) {
            issue(d, d);
            __builtin_amdgcn_sched_barrier(0);
        }
        // whole turns of the ring: the steps past KS add zeros, and the loop has no exit
        // that would leave the wait counts unknown
        for (int s0 = 0; s0 < KS; s0 += kUpDepth) {
#pragma unroll
            for (int d = 0; d < kUpDepth; ++d) {
                const int buf = d & 1;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    *reinterpret_cast<bf16x8 *>(&As[buf][lrow[i] * kPitch + lcol[i]]) = ra[d][i];
                    *reinterpret_cast<bf16x8 *>(&Bs[buf][lrow[i] * kPitch + lcol[i]]) = rb[d][i];
                }
                __syncthreads();
                issue(s0 + d + kUpDepth, d);
#pragma unroll
                for (int ks = 0; ks < kKStep / 16; ++ks) {
                    const bf16x8 fa =
                        *reinterpret_cast<const bf16x8 *>(&As[buf][(wm * 32 + col) * kPitch + ks * 16 + kg * 8]);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const bf16x8 fb = *reinterpret_cast<const bf16x8 *>(
                            &Bs[buf][(wn * 64 + j * 32 + col) * kPitch + ks * 16 + kg * 8]);
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[j], 0, 0, 0);
                    }
                }
            }
        }
        // Swish, score, bf16 -> Ht[tile][e][row][unit]
        const int tile = tiles[wm];
        if (tile >= 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int unit = nb + wn * 64 + j * 32 + col;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = acc_row(v, lane);
                    const float h = swish_fast(acc[j][v]) * scol[wm * 32 + r];
                    a.hidden[(((int64_t)tile * a.E + e) * kTileM + r) * a.d_e + unit] = f32_to_bf16(h);
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ down (grouped GEMM)
// Workgroup = (TILES consecutive chunk tiles, 256 output columns, k split): a
// TILES*32 x 256 GEMM over k = the union of the tiles' chunks' experts x d_e. Wave
// (wm, wn) holds rows wm * TILES * 16 .. (TILES / 2 blocks of 32) x columns wn * 64 ..
// +64 (two blocks of 32). Four tiles halve the L2 bytes per product of two (48 KB of
// operands per 4.2 MFLOP and k step, against 40 KB per 2.1), for a union of four
// chunks instead of two.
// F32: the result goes to y32 in fp32 (the same products serve the layer backward's
// dx = sum_e dA_e W1_e, with dA in the hidden rows' layout and W1^T in W2's).
template <bool F32, int TILES>
__global__ void __launch_bounds__(kGThreads, 1) down_grouped_kernel(GroupedArgs a)
{
    static_assert(TILES == 2 || TILES == 4, "two or four chunk tiles per workgroup");
    constexpr int ROWS = TILES * kTileM;              // 64 or 128
    constexpr int RB = TILES / 2;                     // 32-row blocks per wave
    constexpr int AC = ROWS * (kKStep / 8) / kGThreads;   // A chunks per thread and k step
    const int NCT = a.d_h / kDnCols;
    const int NBT = (a.CT + TILES - 1) / TILES;
    const int ct = blockIdx.x % NCT;
    const int bt = (blockIdx.x / NCT) % NBT;
    const int split = blockIdx.x / NCT / NBT;
    __shared__ alignas(16) uint16_t As[2][ROWS * kPitch];      // hidden rows x 64 units
    __shared__ alignas(16) uint16_t Bs[2][kDnCols * kPitch];   // W2 rows (output columns) x 64 units
    __shared__ uint64_t m_tile[TILES][kMaxWords];
    __shared__ int list[256];
    __shared__ int nlist;

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave & 1, wn = wave >> 1;       // row half (RB blocks), 64-column quarter
    const int col = lane & 31, kg = lane >> 5;
    if (tid < TILES * kMaxWords) {
        const int i = tid / kMaxWords, w = tid % kMaxWords, tile = bt * TILES + i;
        m_tile[i][w] = (tile < a.CT && w < a.W) ? a.masks[(int64_t)(tile / a.MPC) * a.W + w] : 0ull;
    }
    __syncthreads();
    // ascending list of the experts of the union of the tiles' chunks
    auto union_word = [&](int w) {
        uint64_t u = 0ull;
#pragma unroll
        for (int i = 0; i < TILES; ++i)
            u |= m_tile[i][w];
        return u;
    };
    if (tid < a.E) {
        const int w = tid >> 6, bit = tid & 63;
        const uint64_t word = union_word(w);
        if ((word >> bit) & 1ull) {
            int pos = __popcll(word & ((1ull << bit) - 1ull));
            for (int v = 0; v < w; ++v)
                pos += __popcll(union_word(v));
            list[pos] = tid;
        }
    }
    if (tid == 0) {
        int c = 0;
        for (int w = 0; w < a.W; ++w)
            c += __popcll(union_word(w));
        nlist = c;
    }
    __syncthreads();

    const __amdgpu_buffer_rsrc_t rhid =
        make_rsrc(a.hidden, (uint64_t)a.CT * a.E * kTileM * a.d_e * 2);
    const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(a.w2, (uint64_t)a.E * a.d_h * a.d_e * 2);
    // per thread per k step: AC A chunks (ROWS rows x 8 chunks) and 4 B chunks (256 rows
    // x 8); A chunk j is row (tid + 512 j) / 8
    int arow[AC], acol[AC], a_ti[AC], a_tile[AC];
#pragma unroll
    for (int j = 0; j < AC; ++j) {
        const int q = tid + j * kGThreads;
        arow[j] = q >> 3;
        acol[j] = (q & 7) * 8;
        a_ti[j] = arow[j] / kTileM;
        a_tile[j] = bt * TILES + a_ti[j] < a.CT ? bt * TILES + a_ti[j] : -1;
    }
    const int DK = a.d_e / kKStep;
    // this split's contiguous range [st0, st1) of the k steps
    const int steps_all = nlist * DK;
    const int st0 = (int)((int64_t)split * steps_all / a.splits);
    const int st1 = (int)((int64_t)(split + 1) * steps_all / a.splits);
    f32x16 acc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[rb][j][v] = 0.0f;

    // kDepth k steps in flight: every load is issued (a tile whose chunk does not use
    // the expert, and steps past the end, read beyond the buffer and get zero)
    bf16x8 ra[kDepth][AC], rb[kDepth][4];
    auto issue = [&](int st, int d) {
        // branch-free: the list entry is read even past the end (masked to a valid
        // expert index) and the offsets are replaced afterwards
        const bool ok = st < st1;
        const int li = st / DK;
        const int e = list[li < 255 ? li : 255] & 255;
        const int k0 = (st - li * DK) * kKStep;
#pragma unroll
        for (int j = 0; j < AC; ++j) {
            const bool use = ok && a_tile[j] >= 0 && ((m_tile[a_ti[j]][e >> 6] >> (e & 63)) & 1ull);
            const uint32_t aoffs = (uint32_t)((((a_tile[j] * a.E + e) * kTileM + arow[j] % kTileM) * a.d_e +
                                               k0 + acol[j]) * 2);
            ra[d][j] = bload<0>(rhid, use ? aoffs : kOutOfRange);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + i * kGThreads;
            const int r = q >> 3, c8 = (q & 7) * 8;
            const uint32_t boffs =
                (uint32_t)(((e * a.d_h + ct * kDnCols + r) * a.d_e + k0 + c8) * 2);
            rb[d][i] = bload<0>(rw2, ok ? boffs : kOutOfRange);
        }
    };
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        issue(st0 + d, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int s0 = st0; s0 < st1; s0 += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int st = s0 + d;
            const int buf = d & 1;
#pragma unroll
            for (int j = 0; j < AC; ++j)
                *reinterpret_cast<bf16x8 *>(&As[buf][arow[j] * kPitch + acol[j]]) = ra[d][j];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = tid + i * kGThreads;
                *reinterpret_cast<bf16x8 *>(&Bs[buf][(q >> 3) * kPitch + (q & 7) * 8]) = rb[d][i];
            }
            __syncthreads();
            issue(st + kDepth, d);
#pragma unroll
            for (int ks = 0; ks < kKStep / 16; ++ks) {
                bf16x8 fa[RB];
#pragma unroll
                for (int r = 0; r < RB; ++r)
                    fa[r] = *reinterpret_cast<const bf16x8 *>(
                        &As[buf][((wm * RB + r) * 32 + col) * kPitch + ks * 16 + kg * 8]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const bf16x8 fb = *reinterpret_cast<const bf16x8 *>(
                        &Bs[buf][(wn * 64 + j * 32 + col) * kPitch + ks * 16 + kg * 8]);
#pragma unroll
                    for (int r = 0; r < RB; ++r)
                        acc[r][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[r], fb, acc[r][j], 0, 0, 0);
                }
            }
        }
    }
    // y rows of the wave's tiles (rows without a token are not written)
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int tile = bt * TILES + wm * RB + r;
        if (tile >= a.CT)
            continue;
        if (a.splits > 1) {
            // the split's fp32 partial of the tile's rows
            float *dst = a.dn_part + ((int64_t)split * a.CT + tile) * kTileM * a.d_h;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int cidx = ct * kDnCols + wn * 64 + j * 32 + col;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    dst[(int64_t)acc_row(v, lane) * a.d_h + cidx] = acc[r][j][v];
            }
            continue;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int cidx = ct * kDnCols + wn * 64 + j * 32 + col;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t t = tile_token(a, tile, acc_row(v, lane));
                if (t >= 0) {
                    if constexpr (F32)
                        a.y32[t * a.d_h + cidx] = acc[r][j][v];
                    else
                        a.y[t * a.d_h + cidx] = f32_to_bf16(acc[r][j][v]);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ split sum
// y[t][c] = bf16(sum over the splits, in order, of the partials of t's tile row), or
// the fp32 sum into y32 (F32); thread -> 4 consecutive columns of one tile row.
template <bool F32>
__global__ void __launch_bounds__(256) down_reduce_kernel(GroupedArgs a)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int c4 = a.d_h / 4;
    const int64_t rows = (int64_t)a.CT * kTileM;
    if (q >= rows * c4)
        return;
    const int64_t row = q / c4;
    const int c = (int)(q - row * c4) * 4;
    const int64_t t = tile_token(a, (int)(row / kTileM), (int)(row % kTileM));
    if (t < 0)
        return;
    float4 sum = *reinterpret_cast<const float4 *>(a.dn_part + row * a.d_h + c);
    for (int s = 1; s < a.splits; ++s) {
        const float4 v = *reinterpret_cast<const float4 *>(a.dn_part + ((int64_t)s * rows + row) * a.d_h + c);
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
    }
    if constexpr (F32) {
        *reinterpret_cast<float4 *>(a.y32 + t * a.d_h + c) = sum;
        return;
    }
    const uint64_t packed = (uint64_t)f32_to_bf16(sum.x) | ((uint64_t)f32_to_bf16(sum.y) << 16) |
                            ((uint64_t)f32_to_bf16(sum.z) << 32) | ((uint64_t)f32_to_bf16(sum.w) << 48);
    *reinterpret_cast<uint64_t *>(a.y + t * a.d_h + c) = packed;
}

}  // namespace

// k splits for a grid of `blocks` (tiles, column tile) workgroups: doubled while the
// grid would not fill the chip's 256 CUs, at most 4
static int down_splits_for(int64_t blocks)
{
    int s = 1;
    while (s < 4 && blocks * s < 256)
        s *= 2;
    return s;
}

// Four tiles per workgroup read fewer L2 bytes per product than two, at the price of
// a four-chunk union and, where the grid halves below the CU count, a doubled k split
// (fp32 partials); timed, that pays except for very sparse unions (TLS 90%).
int grouped_down_tiles(int64_t CT, int64_t d_h)
{
    (void)d_h;
    return CT >= 4 ? 4 : 2;
}

int grouped_down_splits(int64_t CT, int64_t d_h)
{
    const int tiles = grouped_down_tiles(CT, d_h);
    return down_splits_for(((CT + tiles - 1) / tiles) * (d_h / kDnCols));
}

// The down-projection launch: TILES chunk tiles per workgroup (grouped_down_tiles),
// a.splits k ranges.
template <bool F32>
static void launch_down(const FfnPlan &p, const GroupedArgs &a, hipStream_t stream)
{
    const int tiles = grouped_down_tiles(p.CT, p.d_h);
    const int64_t dn_blocks = ((p.CT + tiles - 1) / tiles) * (p.d_h / kDnCols) * a.splits;
    if (tiles == 4)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(down_grouped_kernel<F32, 4>), dim3((unsigned)dn_blocks), dim3(kGThreads),
                           0, stream, a);
    else
        hipLaunchKernelGGL(HIP_KERNEL_NAME(down_grouped_kernel<F32, 2>), dim3((unsigned)dn_blocks), dim3(kGThreads),
                           0, stream, a);
}

size_t grouped_partial_bytes(int64_t CT, int64_t d_h)
{
    const int s = grouped_down_splits(CT, d_h);
    return s > 1 ? (size_t)s * CT * kTileM * d_h * 4 : 0;
}

bool grouped_supported(int64_t T, int64_t CT, int64_t d_h, int64_t E, int64_t d_e)
{
    return CT >= 2 && d_h % kDnCols == 0 && d_e % kUpCols == 0 && E <= 256 &&
           (uint64_t)T * d_h * 2 < 0x7fffffffull &&
           (uint64_t)CT * E * kTileM * d_e * 2 < 0x7fffffffull &&
           (uint64_t)E * d_e * d_h * 2 < 0x7fffffffull;
}

hipError_t launch_ffn_bf16_grouped(const FfnPlan &p, const uint16_t *x, const float *scores,
                                   const uint16_t *w1, const uint16_t *w2, uint16_t *y, void *ws,
                                   uint64_t *masks_out, int32_t *lists_out, int32_t *counts_out,
                                   hipStream_t stream)
{
    hipError_t err = launch_union(p, scores, ws, masks_out, lists_out, counts_out, stream);
    if (err != hipSuccess)
        return err;
    char *base = static_cast<char *>(ws);
    GroupedArgs a;
    a.x = x;
    a.scores = scores;
    a.w1 = w1;
    a.w2 = w2;
    a.y = y;
    a.hidden = reinterpret_cast<uint16_t *>(base + p.off_hidden);
    a.masks = reinterpret_cast<const uint64_t *>(base + p.off_masks);
    a.T = p.T;
    a.n = (int)p.n;
    a.d_h = (int)p.d_h;
    a.E = (int)p.E;
    a.d_e = (int)p.d_e;
    a.C = (int)p.C;
    a.MPC = (int)p.MPC;
    a.CT = (int)p.CT;
    a.W = (int)p.W;
    a.splits = grouped_down_splits(p.CT, p.d_h);
    a.dn_part = reinterpret_cast<float *>(base + p.off_dnpart);
    const int64_t up_blocks = p.E * ((p.CT + kUpTiles - 1) / kUpTiles);
    hipLaunchKernelGGL(up_grouped_kernel, dim3((unsigned)up_blocks), dim3(kGThreads), 0, stream, a);
    launch_down<false>(p, a, stream);
    if (a.splits > 1) {
        const int64_t q = p.CT * kTileM * (p.d_h / 4);
        hipLaunchKernelGGL(down_reduce_kernel<false>, dim3((unsigned)((q + 255) / 256)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_grouped_down_f32(const FfnPlan &p, const uint16_t *act, const uint16_t *w,
                                   const uint64_t *masks, float *out, float *part,
                                   bool sum_splits, hipStream_t stream)
{
    GroupedArgs a{};
    a.hidden = const_cast<uint16_t *>(act);
    a.w2 = w;
    a.masks = masks;
    a.y32 = out;
    a.dn_part = part;
    a.T = p.T;
    a.n = (int)p.n;
    a.d_h = (int)p.d_h;
    a.E = (int)p.E;
    a.d_e = (int)p.d_e;
    a.C = (int)p.C;
    a.MPC = (int)p.MPC;
    a.CT = (int)p.CT;
    a.W = (int)p.W;
    a.splits = grouped_down_splits(p.CT, p.d_h);
    launch_down<true>(p, a, stream);
    if (a.splits > 1 && sum_splits) {
        const int64_t q = p.CT * kTileM * (p.d_h / 4);
        hipLaunchKernelGGL(down_reduce_kernel<true>, dim3((unsigned)((q + 255) / 256)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

}  // namespace blockffn
