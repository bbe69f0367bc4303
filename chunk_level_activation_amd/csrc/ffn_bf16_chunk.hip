// One-launch bf16 chunk FFN for a single 32-token chunk tile (the decode /
// speculative-verification shape: the pages' kernel evaluates n = 32 tokens at once).
//
// Skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
// Deployment": "Architecture Overview" (non-gated Swish experts, n = 32, only the
// union of activated experts is computed) and "Core Concept" (unneeded activations
// are masked after the computation):
//     Ht_e[t,:] = bf16( s[t,e] * swish(W1_e x_t) )     e in U, every token t
//     y[t,:]    = bf16( sum_{e in U} W2_e Ht_e[t,:] )
//
// At this size the layer is bound by how many bytes each CU can pull, not by math:
// the union experts' W1 and W2 (about 36 MiB at 80% token sparsity) must stream from
// HBM while the small operands (x, the hidden rows, partial sums) are shared. The
// schedule keeps every CU busy and re-reads as little as possible:
//
//   * The grid is two workgroups per CU. Workgroup b runs on
//     XCD b mod X (round-robin dispatch; verified by the library before use), and the
//     union's slots are split into X contiguous groups, group g on XCD g, so all
//     exchanges of a group stay in that XCD's L2.
//   * Every workgroup computes the union itself from the 32 x E scores.
//   * Up items: (slot, 128 hidden units, 512-wide slice of d_h). The x slice (32 x
//     512) is staged once in LDS; eight waves (4 row quarters x 2 k halves) stream the
//     W1 block, partial sums meet in LDS, and the item's 32 x 128 fp32 partial goes to
//     the XCD's L2. The last of the d_h/512 slices to arrive adds them in slice order,
//     applies Swish and the score, and writes the bf16 hidden tile.
//   * Down items: (64 output columns, expert group). W2 for the group's slots is
//     loaded first (it depends only on the union), then the item waits for the
//     group's hidden tiles and reads them from the XCD's L2. Eight waves (2 column
//     halves x 4 parts of the slots' k range) meet in LDS.
//   * The X group tiles of an output tile are on different XCDs: they go to memory
//     with device-scope stores, and the last of the X to arrive (an atomic counter)
//     adds them in group order and writes y.
// The lower workgroups of each XCD run up items, the upper ones down items (the split
// follows the group's size: one workgroup per up item where possible).
// A down workgroup waits only on up workgroups of its own XCD with smaller indices,
// which the in-order dispatcher has placed first, so every wait ends (it is bounded
// anyway: on time-out the outputs of the tile become NaN and the workspace's status
// word is set). The cross-XCD sum and the k-slice sum are done by whichever workgroup
// arrives last, which never waits. All
// counters return to zero before the kernel ends; they live in the workspace's fixed
// control block.
#include "common.h"
#include "plan.h"
#include "sync.h"

namespace blockffn {

namespace {

constexpr int kThreads = 512;
constexpr int kKSlice = 512;        // d_h elements per up item
constexpr int kUpRows = 128;        // hidden units per up item
constexpr int kDnCols = 64;         // output columns per down item
constexpr int kXPitch = kKSlice + 8;   // LDS row pitch (bf16) of the staged x slice
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kMaxWords = 4;

struct Chunk1Args {
    const uint16_t *x;
    const float *scores;
    const uint16_t *w1;
    const uint16_t *w2;
    uint16_t *y;
    uint16_t *hidden;       // [E][32][d_e] bf16
    float *up_part;         // [E][RT][KP][32][128] fp32 partial pre-activations
    float *dn_part;         // [JT][X][32][64] fp32 group tiles
    uint32_t *up_arrive;    // [E][RT] k slices stored per up tile
    uint32_t *up_done;      // [E]     finished hidden tiles per slot
    uint32_t *cons_done;    // [X]     down items done with the group's hidden rows
    uint32_t *dn_arrive;    // [JT]    group tiles stored per output tile
    uint32_t *status;       // the workspace's status word: set when a wait times out
    uint64_t *masks_out;
    int32_t *lists_out;
    int32_t *counts_out;
    int T, d_h, E, d_e;
    int X;                  // XCDs = expert groups
    int WPX;                // workgroups per XCD
    int RT, KP, JT;         // d_e / 128, d_h / 512, d_h / 64
};

// 32x32 accumulator layout: element i of a lane is row (i/4)*8 + (lane/32)*4 + i%4 of
// column lane%32.
__device__ __forceinline__ int acc_row(int i, int lane) { return (i / 4) * 8 + (lane >> 5) * 4 + (i % 4); }

struct Shared {
    uint64_t mask[kMaxWords];
    int list[256];
    int flag;
    float s_col[kTileM];
    alignas(16) float red[4][2][kTileM][33];  // up: [row quarter][k half]; down: [part][half]
    alignas(16) uint16_t xs[kTileM * kXPitch];  // staged x slice (up items)
};

struct Rsrc {
    __amdgpu_buffer_rsrc_t x, w1, w2, hid, upp, dnp;
};

// Union of the experts active in the chunk (all T <= 32 tokens), ascending list in
// LDS; returns |U|.
__device__ int union_of_chunk(const Chunk1Args &a, Shared &sh)
{
    const int tid = threadIdx.x;
    if (tid < kMaxWords)
        sh.mask[tid] = 0;
    __syncthreads();
    const int total = a.T * a.E;
    for (int idx = tid; idx < total; idx += kThreads)
        if (a.scores[idx] != 0.0f) {
            const int e = idx % a.E;
            atomicOr(reinterpret_cast<unsigned long long *>(&sh.mask[e >> 6]), 1ull << (e & 63));
        }
    __syncthreads();
    const int W = (a.E + 63) >> 6;
    int cnt = 0;
    for (int w = 0; w < W; ++w)
        cnt += __popcll(sh.mask[w]);
    if (tid < a.E) {
        const int w = tid >> 6, bit = tid & 63;
        const uint64_t word = sh.mask[w];
        if ((word >> bit) & 1ull) {
            int pos = __popcll(word & ((1ull << bit) - 1ull));
            for (int v = 0; v < w; ++v)
                pos += __popcll(sh.mask[v]);
            sh.list[pos] = tid;
        }
    }
    __syncthreads();
    return cnt;
}

// ------------------------------------------------------------------ up item
__device__ void up_item(const Chunk1Args &a, const Rsrc &r, Shared &sh, int slot, int rt, int kq)
{
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int e = sh.list[slot];
    const int k0 = kq * kKSlice;
    // wave -> (row quarter rq, k half kh): rows rt*128 + rq*32 .. +32, k k0 + kh*256 .. +256
    const int rq = wave & 3, kh = wave >> 2;
    const int col = lane & 31, kg = lane >> 5;
    const uint32_t w1_off = (uint32_t)e * ((uint32_t)a.d_e * (uint32_t)a.d_h * 2u) +
                            (uint32_t)(rt * kUpRows + rq * 32 + col) * ((uint32_t)a.d_h * 2u) +
                            (uint32_t)(k0 + kh * 256 + kg * 8) * 2u;
    // W1 first: the weight stream is the long pole, x comes from L2
    bf16x8 bw[16];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
        bw[ks] = bload<kNT>(r.w1, w1_off + ks * 32);
    // stage x[:, k0:k0+512] in LDS (rows past T read as zero): 4 loads per thread
    constexpr int kXLoads = kTileM * (kKSlice / 8) / kThreads;
    bf16x8 xv[kXLoads];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int v = tid + i * kThreads;
        const int row = v / (kKSlice / 8), c8 = v % (kKSlice / 8);
        xv[i] = row < a.T ? bload<0>(r.x, (uint32_t)((row * a.d_h + k0 + c8 * 8) * 2))
                          : zero_bf16x8();
    }
    if (tid < kTileM)
        sh.s_col[tid] = tid < a.T ? a.scores[tid * a.E + e] : 0.0f;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int v = tid + i * kThreads;
        const int row = v / (kKSlice / 8), c8 = v % (kKSlice / 8);
        *reinterpret_cast<bf16x8 *>(&sh.xs[row * kXPitch + c8 * 8]) = xv[i];
    }
    __syncthreads();     // x slice staged
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        acc[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 ax =
            *reinterpret_cast<const bf16x8 *>(&sh.xs[col * kXPitch + kh * 256 + ks * 16 + kg * 8]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax, bw[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
        sh.red[rq][kh][acc_row(i, lane)][col] = acc[i];
    __syncthreads();
    // 32 tokens x 128 units; thread -> (token tt, units u0 .. u0 + 7), u0 within one quarter
    const int tt = tid >> 4, u0 = (tid & 15) * 8;
    float pv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int u = u0 + q, quarter = u >> 5, uc = u & 31;
        pv[q] = sh.red[quarter][0][tt][uc] + sh.red[quarter][1][tt][uc];
    }
    const uint32_t tile_bytes = kTileM * kUpRows * 4;
    const uint32_t tile_off = (uint32_t)((slot * a.RT + rt) * a.KP) * tile_bytes;
    const uint32_t elem_off = (uint32_t)((tt * kUpRows + u0) * 4);
    bstore_f4<kSC0>(r.upp, tile_off + kq * tile_bytes + elem_off,
                    make_float4(pv[0], pv[1], pv[2], pv[3]));
    bstore_f4<kSC0>(r.upp, tile_off + kq * tile_bytes + elem_off + 16,
                    make_float4(pv[4], pv[5], pv[6], pv[7]));
    drain_memory();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = add_counter(&a.up_arrive[slot * a.RT + rt], 1u);
        sh.flag = prev == (uint32_t)(a.KP - 1);
        if (sh.flag)
            st_counter(&a.up_arrive[slot * a.RT + rt], 0u);
    }
    __syncthreads();
    if (!sh.flag)
        return;
    // Last slice of the tile: add the KP partials in slice order, Swish, score, bf16.
    float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < a.KP; ++q) {
        const float4 v0 = bload_f4<kSC0>(r.upp, tile_off + q * tile_bytes + elem_off);
        const float4 v1 = bload_f4<kSC0>(r.upp, tile_off + q * tile_bytes + elem_off + 16);
        sum[0] += v0.x;
        sum[1] += v0.y;
        sum[2] += v0.z;
        sum[3] += v0.w;
        sum[4] += v1.x;
        sum[5] += v1.y;
        sum[6] += v1.z;
        sum[7] += v1.w;
    }
    const float sc = sh.s_col[tt];
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        h[q] = (uint32_t)f32_to_bf16(swish_fast(sum[2 * q]) * sc) |
               ((uint32_t)f32_to_bf16(swish_fast(sum[2 * q + 1]) * sc) << 16);
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{h[0], h[1], h[2], h[3]}, r.hid,
        (int)(((slot * kTileM + tt) * a.d_e + rt * kUpRows + u0) * 2), 0, kSC0);
    drain_memory();
    __syncthreads();
    if (tid == 0)
        add_counter(&a.up_done[slot], 1u);
}

// ------------------------------------------------------------------ down item
// Group g's slots [s0, s1); unit u = (slot s0 + u / KSe, k step u % KSe), KSe = d_e/16.
// Wave -> (column half ch, part pp): units u with u % 4 == pp.
constexpr int kDnMaxUnitsPerWave = 6;   // W2 units per wave whose loads are in flight together
constexpr int kDnSub = 2;                // hidden-row loads in flight together
struct DownState {
    int s0, s1, units, KSe, jt, ch, pp;
    uint32_t w2_expert_bytes;   // d_h * d_e * 2
    uint32_t w2_row_off;        // byte offset of this lane's W2 row in an expert
    uint32_t hid_slot_bytes;    // 32 * d_e * 2
    uint32_t hid_row_off;       // byte offset of this lane's hidden row in a slot
    bf16x8 bw[kDnMaxUnitsPerWave];
};

__device__ void down_issue_w2(const Chunk1Args &a, const Rsrc &r, const Shared &sh, DownState &d,
                              int batch)
{
    const int lane = threadIdx.x % kWave, kg = lane >> 5;
#pragma unroll
    for (int i = 0; i < kDnMaxUnitsPerWave; ++i) {
        const int u = d.pp + 4 * (batch * kDnMaxUnitsPerWave + i);
        if (u < d.units) {
            const uint32_t e = (uint32_t)sh.list[d.s0 + u / d.KSe];
            d.bw[i] = bload<kNT>(r.w2, e * d.w2_expert_bytes + d.w2_row_off +
                                           (uint32_t)(u % d.KSe) * 32u + (uint32_t)kg * 16u);
        } else {
            d.bw[i] = zero_bf16x8();
        }
    }
}

__device__ void down_item(const Chunk1Args &a, const Rsrc &r, Shared &sh, int g, DownState &d)
{
    const int tid = threadIdx.x, lane = tid % kWave;
    const int col = lane & 31, kg = lane >> 5;
    // wait for the group's hidden tiles (one thread per slot)
    if (tid == 0)
        sh.flag = 0;
    __syncthreads();
    if (tid < d.s1 - d.s0) {
        uint32_t spins = 0;
        while (ld_counter(&a.up_done[d.s0 + tid]) < (uint32_t)a.RT) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                sh.flag = 1;
                break;
            }
        }
    }
    __syncthreads();
    const bool timed_out = sh.flag != 0;
    if (timed_out && tid == 0)
        __hip_atomic_fetch_or(a.status, kStatusTimedOut, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        acc[i] = 0.0f;
    // batch 0 of W2 was issued before the wait; later batches are loaded here
    const int per_wave = (d.units - d.pp + 3) / 4;
    for (int batch = 0; batch * kDnMaxUnitsPerWave < per_wave; ++batch) {
        if (batch > 0)
            down_issue_w2(a, r, sh, d, batch);
        // hidden rows from the XCD's L2 in sub-batches (bounds the live registers)
#pragma unroll
        for (int i0 = 0; i0 < kDnMaxUnitsPerWave; i0 += kDnSub) {
            bf16x8 ha[kDnSub];
#pragma unroll
            for (int i = 0; i < kDnSub; ++i) {
                const int u = d.pp + 4 * (batch * kDnMaxUnitsPerWave + i0 + i);
                ha[i] = u < d.units
                            ? bload<kSC0>(r.hid, (uint32_t)(d.s0 + u / d.KSe) * d.hid_slot_bytes +
                                                     d.hid_row_off + (uint32_t)(u % d.KSe) * 32u +
                                                     (uint32_t)kg * 16u)
                            : zero_bf16x8();
            }
#pragma unroll
            for (int i = 0; i < kDnSub; ++i)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha[i], d.bw[i0 + i], acc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // hidden rows consumed: the last of the JT down items of the group resets counters
    drain_memory();
    __syncthreads();
    if (tid == 0 && add_counter(&a.cons_done[g], 1u) == (uint32_t)(a.JT - 1)) {
        for (int s = d.s0; s < d.s1; ++s)
            st_counter(&a.up_done[s], 0u);
        st_counter(&a.cons_done[g], 0u);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
        sh.red[d.pp][d.ch][acc_row(i, lane)][col] = acc[i];
    __syncthreads();
    // 32 tokens x 64 columns; thread -> (token tt, columns c0 .. c0 + 3)
    const int tt = tid >> 4, c0 = (tid & 15) * 4;
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = c0 + q, h = c >> 5, cc = c & 31;
        o[q] = ((sh.red[0][h][tt][cc] + sh.red[1][h][tt][cc]) + sh.red[2][h][tt][cc]) +
               sh.red[3][h][tt][cc];
        if (timed_out)
            o[q] = __builtin_nanf("");
    }
    const uint32_t tile_off = (uint32_t)(d.jt * kMaxGroups * (kTileM * kDnCols) * 4);
    const uint32_t elem_off = (uint32_t)((tt * kDnCols + c0) * 4);
    bstore_f4<kSC1>(r.dnp, tile_off + g * (kTileM * kDnCols * 4) + elem_off,
                    make_float4(o[0], o[1], o[2], o[3]));
    drain_memory();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = add_counter(&a.dn_arrive[d.jt], 1u);
        sh.flag = prev == (uint32_t)(a.X - 1);
        if (sh.flag)
            st_counter(&a.dn_arrive[d.jt], 0u);
    }
    __syncthreads();
    if (!sh.flag)
        return;
    // add the X group tiles in group order, eight groups' loads in flight at a time
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < a.X; q0 += 8) {
        float4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = q0 + j < a.X
                       ? bload_f4<kSC1>(r.dnp, tile_off + (q0 + j) * (kTileM * kDnCols * 4) + elem_off)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (q0 + j < a.X) {
                sum[0] += v[j].x;
                sum[1] += v[j].y;
                sum[2] += v[j].z;
                sum[3] += v[j].w;
            }
    }
    if (tt < a.T) {
        const uint64_t packed = (uint64_t)f32_to_bf16(sum[0]) | ((uint64_t)f32_to_bf16(sum[1]) << 16) |
                                ((uint64_t)f32_to_bf16(sum[2]) << 32) |
                                ((uint64_t)f32_to_bf16(sum[3]) << 48);
        *reinterpret_cast<uint64_t *>(a.y + (int64_t)tt * a.d_h + d.jt * kDnCols + c0) = packed;
    }
}

__global__ void __launch_bounds__(kThreads, 4)
ffn_bf16_chunk1_kernel(Chunk1Args a)
{
    __shared__ Shared sh;
    const int g = blockIdx.x % a.X;
    const int k = blockIdx.x / a.X;
    const int tid = threadIdx.x, wave = tid / kWave;
    Rsrc r;
    r.x = make_rsrc(a.x, (uint64_t)a.T * a.d_h * 2);
    r.w1 = make_rsrc(a.w1, (uint64_t)a.E * a.d_e * a.d_h * 2);
    r.w2 = make_rsrc(a.w2, (uint64_t)a.E * a.d_h * a.d_e * 2);
    r.hid = make_rsrc(a.hidden, (uint64_t)a.E * kTileM * a.d_e * 2);
    r.upp = make_rsrc(a.up_part, (uint64_t)a.E * a.RT * a.KP * kTileM * kUpRows * 4);
    r.dnp = make_rsrc(a.dn_part, (uint64_t)a.JT * kMaxGroups * kTileM * kDnCols * 4);
    const int cnt = union_of_chunk(a, sh);

    if (blockIdx.x == 0) {
        const int W = (a.E + 63) >> 6;
        if (a.counts_out && tid == 0)
            a.counts_out[0] = cnt;
        if (a.lists_out)
            for (int i = tid; i < a.E; i += kThreads)
                a.lists_out[i] = i < cnt ? sh.list[i] : -1;
        if (a.masks_out && tid < W)
            a.masks_out[tid] = sh.mask[tid];
    }

    const int s0 = (int)((int64_t)g * cnt / a.X), s1 = (int)((int64_t)(g + 1) * cnt / a.X);
    const int sg = s1 - s0;
    const int U = sg * a.RT * a.KP;           // up items of this group
    // Role split of this XCD's workgroups, decided per group from the union: up items
    // finish with a k-slice sum and a hidden-tile handoff, so a second round of them is
    // dear; give them one workgroup each where possible and let the down workgroups
    // (at least a quarter of the XCD) loop over the column tiles instead.
    const int n_up = U < a.WPX - a.WPX / 4 ? U : a.WPX - a.WPX / 4;
    if (k < n_up) {
        // up workgroups: items k, k + n_up, ...
        for (int u = k; u < U; u += n_up) {
            const int slot = s0 + u / (a.RT * a.KP);
            const int rt = (u / a.KP) % a.RT;
            const int kq = u % a.KP;
            up_item(a, r, sh, slot, rt, kq);
            __syncthreads();
        }
    } else {
        // down workgroups: W2 is in flight while the group's up items run
        DownState d;
        d.s0 = s0;
        d.s1 = s1;
        d.KSe = a.d_e / 16;
        d.units = sg * d.KSe;
        d.ch = wave & 1;
        d.pp = wave >> 1;
        const int lane = tid % kWave;
        d.w2_expert_bytes = (uint32_t)a.d_h * (uint32_t)a.d_e * 2u;
        d.hid_slot_bytes = (uint32_t)kTileM * (uint32_t)a.d_e * 2u;
        d.hid_row_off = (uint32_t)(lane & 31) * (uint32_t)a.d_e * 2u;
        for (int dn = k - n_up; dn < a.JT; dn += a.WPX - n_up) {
            d.jt = dn;
            d.w2_row_off = (uint32_t)(dn * kDnCols + d.ch * 32 + (lane & 31)) * (uint32_t)a.d_e * 2u;
            down_issue_w2(a, r, sh, d, 0);
            down_item(a, r, sh, g, d);
            __syncthreads();
        }
    }
}

}  // namespace

bool chunk1_supported(int64_t CT, int64_t d_h, int64_t d_e)
{
    return CT == 1 && d_h % kKSlice == 0 && d_e % kUpRows == 0 &&
           (uint64_t)d_h * (uint64_t)d_e * 2u * 256u < 0x7fffffffull;
}

// Occupancy of the chunk kernel (workgroups per CU), 0 on error.
int chunk1_blocks_per_cu()
{
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ffn_bf16_chunk1_kernel, kThreads, 0) !=
        hipSuccess)
        return 0;
    return nb;
}

hipError_t launch_ffn_bf16_chunk1(const FfnPlan &p, int xcds, int wg_per_xcd,
                                  const uint16_t *x, const float *scores, const uint16_t *w1,
                                  const uint16_t *w2, uint16_t *y, void *ws,
                                  uint64_t *masks_out, int32_t *lists_out, int32_t *counts_out,
                                  hipStream_t stream)
{
    char *base = static_cast<char *>(ws);
    uint32_t *control = reinterpret_cast<uint32_t *>(base);
    Chunk1Args a;
    a.x = x;
    a.scores = scores;
    a.w1 = w1;
    a.w2 = w2;
    a.y = y;
    a.T = (int)p.T;
    a.d_h = (int)p.d_h;
    a.E = (int)p.E;
    a.d_e = (int)p.d_e;
    a.X = xcds;
    a.WPX = wg_per_xcd;
    a.RT = (int)(p.d_e / kUpRows);
    a.KP = (int)(p.d_h / kKSlice);
    a.JT = (int)(p.d_h / kDnCols);
    a.hidden = reinterpret_cast<uint16_t *>(base + p.off_hidden);
    a.up_part = reinterpret_cast<float *>(base + p.off_partials);
    a.dn_part = a.up_part + (size_t)p.E * a.RT * a.KP * kTileM * kUpRows;
    a.up_arrive = control;
    a.up_done = a.up_arrive + p.E * a.RT;
    a.cons_done = a.up_done + p.E;
    a.dn_arrive = a.cons_done + kMaxGroups;
    a.status = control + kStatusWord;
    a.masks_out = masks_out;
    a.lists_out = lists_out;
    a.counts_out = counts_out;
    hipLaunchKernelGGL(ffn_bf16_chunk1_kernel, dim3((unsigned)(xcds * wg_per_xcd)),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

size_t chunk1_partial_bytes(int64_t d_h, int64_t E, int64_t d_e)
{
    const int64_t RT = d_e / kUpRows, KP = d_h / kKSlice, JT = d_h / kDnCols;
    return sizeof(float) * ((size_t)E * RT * KP * kTileM * kUpRows +
                            (size_t)JT * kMaxGroups * kTileM * kDnCols);
}

}  // namespace blockffn
