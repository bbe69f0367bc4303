// One-launch bf16 chunk FFN for a single chunk of at most 32 tokens, the decode /
// speculative-verification shape (the pages' kernel evaluates n = 32 tokens at once).
//
// Skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
// Deployment": "Architecture Overview" (non-gated Swish experts, n = 32, only the
// union of activated experts is computed) and "Core Concept" (unneeded activations
// are masked after the computation):
//     Ht_e[t,:] = bf16( s[t,e] * swish(W1_e x_t) )     e in U, every token t
//     y[t,:]    = bf16( sum_{e in U} W2_e Ht_e[t,:] )
//
// The layer is a stream of the union experts' W1 and W2 (about 36 MiB at 80% token
// sparsity) that every CU should pull in equal shares, with as few dependent global
// round trips after the stream as possible. Schedule:
//
//   * One workgroup of 8 waves per CU. Workgroup b runs on XCD g = b mod X (verified
//     by the library before use) and is member k = b / X of group g. The union's
//     slots are split into X contiguous groups, group g on XCD g, so the hidden rows
//     a group produces and consumes stay in that XCD's L2.
//   * Every workgroup computes the union itself from the scores. The scores are
//     loaded first, then x (which does not depend on the union) with contiguous 1 KB
//     accesses, staged whole in LDS (XOR-swizzled 16-byte chunks, so the MFMA operand
//     reads are conflict-free). A CU's load pipe handles contiguous accesses several
//     times faster than the row-strided ones of MFMA operand layouts, and x is the
//     one operand every CU reads whole.
//   * Up: member k owns hidden units [k*upw, k*upw + upw) of every slot of its group
//     (upw = d_e / P for P members) over the whole of d_h, so no split-k partial ever
//     leaves the workgroup. Wave w = (16-row half rh, quarter kq of d_h): A = the W1
//     rows (16 x 32 k, straight from memory into registers: 16 rows x 64 bytes per
//     access), B = x from LDS, 16x16x32 MFMAs for both 16-token halves; the 4 k
//     quarters meet in LDS and are added in order, then Swish and the score.
//   * Down: member k owns the 64 output columns [64k, 64k + 64) for every slot of its
//     group. Its W2 block is loaded together with W1, right after the union, so both
//     halves of the weight stream are in flight at once. Wave w = (16-column quarter
//     ct, half kh of the hidden units): A = W2 rows, B = the hidden rows from L2.
//     After the group's barrier (an arrival counter all P members bump once their
//     hidden rows are in L2) each wave loads its hidden operand and runs the MFMAs;
//     the 2 unit halves meet in LDS.
//   * The X group tiles of an output tile come from different XCDs: they go to
//     memory with device-scope stores, and the last of the X to arrive (an atomic
//     counter) adds them in group order and writes y.
// Every wait is bounded: on time-out the affected outputs become NaN. Waits are on the
// members of one group, which are all resident at once (one workgroup per CU, as many
// members as the XCD has CUs). The group barrier uses per-member epoch flags that all
// advance by one per call (from zero), the cross-XCD sum an arrival counter that
// returns to zero; both live in the workspace's fixed control block.
#include "common.h"
#include "plan.h"
#include "sync.h"

namespace blockffn {

namespace {

constexpr int kThreads = 512;        // 8 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxXLoads = 16;       // 16-byte x chunks per thread: d_h <= 2048
constexpr int kMaxScoreLoads = 8;    // scores per thread: T * E <= 4096
constexpr int kMaxKSteps = 16;       // 32-wide k steps per up wave: d_h / 4 <= 512
constexpr int kMaxSlots = 8;         // union slots per group
constexpr int kMaxRows = 32;         // W1 rows per member: slots * upw
constexpr int kDnCols = 64;          // output columns per member
constexpr int kMaxDnSteps = 2;       // 32-wide k steps per slot and down wave: d_e / 64
constexpr int kMaxWords = 4;
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kMaxDh = 2048;
constexpr int kDecodeMaxJT = kMaxDh / kDnCols;
constexpr int kMaxMembers = 64;
constexpr int kRedPitch = kTileM + 1;     // LDS pitch of the partials [part][row][token]

struct DecodeArgs {
    const uint16_t *x;
    const float *scores;
    const uint16_t *w1;
    const uint16_t *w2;
    uint16_t *y;
    uint16_t *hidden;       // [X][kMaxSlots] blocks of 32 x d_e bf16, fragment order
    float *dn_part;         // [JT][X][32][64] fp32 group tiles
    uint32_t *flags;        // [X][P] per member: calls whose hidden rows it has stored
    uint32_t *dn_arrive;    // [JT] group tiles stored per output tile
    uint64_t *masks_out;
    int32_t *lists_out;
    int32_t *counts_out;
    int T, d_h, E, d_e;
    int X, P;               // groups (XCDs), members per group
    int upw;                // hidden units per member and slot, d_e / P
    int JT;                 // d_h / 64 output tiles
};

struct Shared {
    uint64_t mask[kMaxWords];
    int list[256];
    int flag;
    int last;
    float s_col[kMaxSlots][kTileM];
    // up partials [4 k quarters][32 rows][32 tokens], later down partials
    // [2 unit halves][64 columns][32 tokens]
    float red[2 * kDnCols * kRedPitch];
    uint16_t xs[kTileM * kMaxDh];   // x, 16-byte chunk c of token t at chunk c ^ (t & 15)
};

// Union of the experts active in the chunk from the scores each thread holds (entry
// tid + 512 i of the T x E array; entries past the end read as zero), ascending list
// in LDS; returns |U|. sh.mask must be zero and visible on entry.
__device__ int union_from_scores(const DecodeArgs &a, Shared &sh, const float (&sv)[kMaxScoreLoads])
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kMaxScoreLoads; ++i)
        if (sv[i] != 0.0f) {
            const int e = (tid + i * kThreads) % a.E;
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

// Byte offset in LDS of the 16-byte chunk c of token t of the staged x (row pitch
// d_h elements); XOR with the low token bits spreads 16 tokens over all banks.
__device__ __forceinline__ int xs_chunk(int t, int c, int chunks_per_row)
{
    return t * chunks_per_row + (c ^ (t & 15));
}

// Byte offset of Ht[slot][token][unit] of group g. The hidden block of a slot is kept
// in the order the down products read it: fragment (unit / 32, token / 16) of 1 KB
// holds, at lane kgrp*16 + token%16, the 8 units 8*kgrp .. +8 of its 32 (kgrp =
// (unit % 32) / 8), so each operand load of a down wave is one contiguous access.
__device__ __forceinline__ uint32_t hid_offset(int g, int sl, int t, int unit, int d_e)
{
    const int frag = (unit >> 5) * 2 + (t >> 4);
    const int ln = ((unit & 31) >> 3) * 16 + (t & 15);
    return (uint32_t)(((((g * kMaxSlots + sl) * (d_e / 32) * 2 + frag) * kWave + ln) * 8 +
                       (unit & 7)) *
                      2);
}

__global__ void __launch_bounds__(kThreads, 1) ffn_bf16_decode_kernel(DecodeArgs a)
{
    __shared__ Shared sh;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane & 15, kgrp = lane >> 4;
    const int g = blockIdx.x % a.X;      // group = XCD
    const int k = blockIdx.x / a.X;      // member within the group

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint64_t)a.T * a.d_h * 2);
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(a.w1, (uint64_t)a.E * a.d_e * a.d_h * 2);
    const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(a.w2, (uint64_t)a.E * a.d_h * a.d_e * 2);
    const __amdgpu_buffer_rsrc_t rhid =
        make_rsrc(a.hidden, (uint64_t)a.X * kMaxSlots * kTileM * a.d_e * 2);
    const __amdgpu_buffer_rsrc_t rdnp =
        make_rsrc(a.dn_part, (uint64_t)a.JT * a.X * kTileM * kDnCols * 4);
    const __amdgpu_buffer_rsrc_t rflag = make_rsrc(a.flags, (uint64_t)a.X * a.P * 4);
    // this call's epoch: one more than the member's flag, which (like every flag of
    // the group) holds the number of calls so far
    const uint32_t epoch = 1u + ld_counter(&a.flags[g * a.P + k]);

    // Prologue loads, all unconditional (entries past a buffer's end read as zero) so
    // the compiler can wait for the scores alone: the union's scores first, then x.
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scores, (uint64_t)a.T * a.E * 4);
    float sv[kMaxScoreLoads];
#pragma unroll
    for (int i = 0; i < kMaxScoreLoads; ++i)
        sv[i] = bload_f1<0>(rs, (uint32_t)((tid + i * kThreads) * 4));
    // x, contiguous: 16-byte chunk q = i * 512 + tid of the 32 x d_h tile (token
    // q / cpr, chunk q % cpr); tokens past T read as zero.
    const int cpr = a.d_h / 8;
    const int nxl = kTileM * cpr / kThreads;
    bf16x8 xv[kMaxXLoads];
#pragma unroll
    for (int i = 0; i < kMaxXLoads; ++i)
        xv[i] = bload<0>(rx, (uint32_t)((i * kThreads + tid) * 16));
    if (tid < kMaxWords)
        sh.mask[tid] = 0;
    __syncthreads();
    const int cnt = union_from_scores(a, sh, sv);

    if (blockIdx.x == 0) {
        const int W = (a.E + 63) >> 6;
        if (a.masks_out && tid < W)
            a.masks_out[tid] = sh.mask[tid];
        if (a.lists_out)
            for (int i = tid; i < a.E; i += kThreads)
                a.lists_out[i] = i < cnt ? sh.list[i] : -1;
        if (a.counts_out && tid == 0)
            a.counts_out[0] = cnt;
    }
    const int s0 = (int)((int64_t)g * cnt / a.X);
    const int ns = (int)((int64_t)(g + 1) * cnt / a.X) - s0;
    const int nrows = ns * a.upw;

    // W1 as the A operand (16 rows x 32 k): wave (row half rh, k quarter kq); lane
    // (row l16, k group kgrp) holds row rh*16 + l16 of the member's W1 block (slot
    // row / upw, unit k*upw + row % upw) at k = kq*d_h/4 + 32 ks + 8 kgrp .. +8.
    const int rh = wave & 1, kq = wave >> 1;
    const int KSU = a.d_h / 128;          // 32-wide k steps per quarter
    const int kq0 = kq * (a.d_h / 4);
    bf16x8 wa[kMaxKSteps];
    {
        const int row = rh * 16 + l16;
        const bool vr = row < nrows;
        const int e = vr ? sh.list[s0 + row / a.upw] : 0;
        const int unit = k * a.upw + row % a.upw;
        const uint32_t base = (uint32_t)(((e * a.d_e + unit) * a.d_h + kq0 + kgrp * 8) * 2);
#pragma unroll
        for (int ks = 0; ks < kMaxKSteps; ++ks)
            wa[ks] = vr && ks < KSU ? bload<kNT>(rw1, base + ks * 64) : zero_bf16x8();
    }

    // W2 as the A operand of the down products (16 columns x 32 units): wave (column
    // quarter ct, unit half kh); lane (column l16, k group kgrp) holds
    // W2[e][64 jt + 16 ct + l16][uh + 32 ds + 8 kgrp .. +8] per slot, uh = kh*d_e/2.
    const int jt = k;
    const bool has_dn = jt < a.JT;
    const int ct = wave & 3, kh = wave >> 2;
    const int DS = a.d_e / 64;
    const int uh = kh * (a.d_e / 2);
    bf16x8 wb[kMaxSlots * kMaxDnSteps];
#pragma unroll
    for (int sl = 0; sl < kMaxSlots; ++sl) {
        const bool vs = has_dn && sl < ns;
        const int e = vs ? sh.list[s0 + sl] : 0;
        const uint32_t base =
            (uint32_t)(((e * a.d_h + jt * kDnCols + ct * 16 + l16) * a.d_e + uh + kgrp * 8) * 2);
#pragma unroll
        for (int ds = 0; ds < kMaxDnSteps; ++ds)
            wb[sl * kMaxDnSteps + ds] =
                vs && ds < DS ? bload<kNT>(rw2, base + ds * 64) : zero_bf16x8();
    }

    // the group's score columns, zero past T
    if (tid < ns * kTileM) {
        const int sl = tid / kTileM, t = tid % kTileM;
        sh.s_col[sl][t] = t < a.T ? a.scores[t * a.E + sh.list[s0 + sl]] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kMaxXLoads; ++i)
        if (i < nxl) {
            const int q = i * kThreads + tid;
            *reinterpret_cast<bf16x8 *>(&sh.xs[xs_chunk(q / cpr, q % cpr, cpr) * 8]) = xv[i];
        }
    __syncthreads();

    // ---- up: pre-activations of the member's rows over this wave's k quarter.
    // B = x^T (32 k x 16 tokens): lane (token l16 (+16), k group kgrp).
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    if (rh * 16 < nrows) {
#pragma unroll
        for (int ks = 0; ks < kMaxKSteps; ++ks)
            if (ks < KSU) {
                const int c = (kq0 + ks * 32) / 8 + kgrp;
                const bf16x8 b0 = *reinterpret_cast<const bf16x8 *>(&sh.xs[xs_chunk(l16, c, cpr) * 8]);
                const bf16x8 b1 =
                    *reinterpret_cast<const bf16x8 *>(&sh.xs[xs_chunk(l16 + 16, c, cpr) * 8]);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ks], b0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ks], b1, acc1, 0, 0, 0);
            }
    }
    // 16x16 accumulator layout: element i of a lane is row (lane/16)*4 + i of column
    // lane%16 (here: W1 row, token)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = rh * 16 + kgrp * 4 + i;
        sh.red[(kq * kTileM + row) * kRedPitch + l16] = acc0[i];
        sh.red[(kq * kTileM + row) * kRedPitch + l16 + 16] = acc1[i];
    }
    __syncthreads();
    // k quarters in order, Swish, score, bf16: thread -> (token tt, rows r0, r0 + 1),
    // both of one slot (upw is even)
    {
        const int tt = tid >> 4, r0 = (tid & 15) * 2;
        if (r0 < nrows) {
            float h[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float sum = 0.0f;
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    sum += sh.red[(p * kTileM + r0 + q) * kRedPitch + tt];
                h[q] = swish_fast(sum) * sh.s_col[r0 / a.upw][tt];
            }
            const int sl = r0 / a.upw, unit = k * a.upw + r0 % a.upw;
            const uint32_t off = hid_offset(g, sl, tt, unit, a.d_e);
            const uint32_t packed = (uint32_t)f32_to_bf16(h[0]) | ((uint32_t)f32_to_bf16(h[1]) << 16);
            __builtin_amdgcn_raw_buffer_store_b32(packed, rhid, (int)off, 0, kSC0);
        }
    }
    drain_memory();
    __syncthreads();

    // ---- group barrier: every member's hidden rows are in the XCD's L2. Each member
    // publishes the call's epoch in its own flag; the first wave polls all P flags.
    if (tid == 0)
        xcd_flag_store(rflag, (uint32_t)((g * a.P + k) * 4), epoch);
    if (wave == 0) {
        const uint32_t *flag = &a.flags[g * a.P + (lane < a.P ? lane : 0)];
        uint32_t spins = 0;
        bool ready = false;
        while (!ready && spins < kSpinLimit) {
            const uint32_t v = ld_counter(flag);
            ready = __all(lane >= a.P || v == epoch);
            if (!ready) {
                ++spins;
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0)
            sh.flag = !ready;
    }
    __syncthreads();
    const bool timed_out = sh.flag != 0;
    if (!has_dn)
        return;

    // ---- down: B = the hidden rows (32 units x 16 tokens): lane (token l16 (+16),
    // k group kgrp) holds Ht[slot][token][uh + 32 ds + 8 kgrp .. +8], from L2; in the
    // fragment order each of these loads is one contiguous 1 KB access
    bf16x8 hv[kMaxSlots * kMaxDnSteps][2];
#pragma unroll
    for (int sl = 0; sl < kMaxSlots; ++sl)
#pragma unroll
        for (int ds = 0; ds < kMaxDnSteps; ++ds)
#pragma unroll
            for (int th = 0; th < 2; ++th)
                hv[sl * kMaxDnSteps + ds][th] =
                    sl < ns && ds < DS
                        ? bload<kSC0>(rhid, hid_offset(g, sl, th * 16 + l16,
                                                       uh + ds * 32 + kgrp * 8, a.d_e))
                        : zero_bf16x8();
    acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < kMaxSlots; ++sl)
#pragma unroll
        for (int ds = 0; ds < kMaxDnSteps; ++ds)
            if (sl < ns && ds < DS) {
                const int i = sl * kMaxDnSteps + ds;
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i], hv[i][0], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i], hv[i][1], acc1, 0, 0, 0);
            }
    // element i: column ct*16 + kgrp*4 + i, token l16 (+16)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = ct * 16 + kgrp * 4 + i;
        sh.red[(kh * kDnCols + c) * kRedPitch + l16] = acc0[i];
        sh.red[(kh * kDnCols + c) * kRedPitch + l16 + 16] = acc1[i];
    }
    __syncthreads();

    // group tile: the 2 unit halves in order; thread -> (token tt, columns c0 .. +3)
    const int tt = tid >> 4, c0 = (tid & 15) * 4;
    {
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float sum = sh.red[(c0 + q) * kRedPitch + tt] +
                              sh.red[(kDnCols + c0 + q) * kRedPitch + tt];
            o[q] = timed_out ? __builtin_nanf("") : sum;
        }
        bstore_f4<kSC1>(rdnp, (uint32_t)((((jt * a.X + g) * kTileM + tt) * kDnCols + c0) * 4),
                        make_float4(o[0], o[1], o[2], o[3]));
    }
    drain_memory();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = add_counter(&a.dn_arrive[jt], 1u);
        sh.last = prev == (uint32_t)(a.X - 1);
        if (sh.last)
            st_counter(&a.dn_arrive[jt], 0u);
    }
    __syncthreads();
    if (!sh.last)
        return;
    // last group tile of this output tile: add the X tiles in group order
    float4 pv[kMaxGroups];
#pragma unroll
    for (int q = 0; q < kMaxGroups; ++q)
        if (q < a.X)
            pv[q] = bload_f4<kSC1>(
                rdnp, (uint32_t)((((jt * a.X + q) * kTileM + tt) * kDnCols + c0) * 4));
    float4 sum = pv[0];
#pragma unroll
    for (int q = 1; q < kMaxGroups; ++q)
        if (q < a.X) {
            sum.x += pv[q].x;
            sum.y += pv[q].y;
            sum.z += pv[q].z;
            sum.w += pv[q].w;
        }
    if (tt < a.T) {
        const uint64_t packed = (uint64_t)f32_to_bf16(sum.x) | ((uint64_t)f32_to_bf16(sum.y) << 16) |
                                ((uint64_t)f32_to_bf16(sum.z) << 32) |
                                ((uint64_t)f32_to_bf16(sum.w) << 48);
        *reinterpret_cast<uint64_t *>(a.y + (int64_t)tt * a.d_h + jt * kDnCols + c0) = packed;
    }
}

}  // namespace

bool decode_supported(int64_t CT, int64_t d_h, int64_t E, int64_t d_e, int xcds, int members)
{
    if (CT != 1 || xcds < 1 || xcds > kMaxGroups || members < 1 || members > kMaxMembers)
        return false;
    if (d_h % 128 != 0 || d_h > kMaxDh || d_h / kDnCols > members)
        return false;
    if (d_e % 64 != 0 || d_e / 64 > kMaxDnSteps || d_e % members != 0)
        return false;
    if (E * kTileM > kMaxScoreLoads * kThreads)
        return false;
    const int64_t upw = d_e / members;
    const int64_t slots = (E + xcds - 1) / xcds;
    return upw % 2 == 0 && slots <= kMaxSlots && slots * upw <= kMaxRows;
}

size_t decode_scratch_bytes(int64_t d_h, int64_t d_e)
{
    const size_t hidden = (size_t)kMaxGroups * kMaxSlots * kTileM * d_e * 2;
    const size_t part = (size_t)(d_h / kDnCols) * kMaxGroups * kTileM * kDnCols * 4;
    return align_up(hidden, 256) + part;
}

int decode_blocks_per_cu()
{
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ffn_bf16_decode_kernel, kThreads, 0) !=
        hipSuccess)
        return 0;
    return nb;
}

hipError_t launch_ffn_bf16_decode(const FfnPlan &p, int xcds, int members, const uint16_t *x,
                                  const float *scores, const uint16_t *w1, const uint16_t *w2,
                                  uint16_t *y, void *ws, uint64_t *masks_out,
                                  int32_t *lists_out, int32_t *counts_out, hipStream_t stream)
{
    char *base = static_cast<char *>(ws);
    uint32_t *ctrl = reinterpret_cast<uint32_t *>(base) + kDecodeControlWord;
    DecodeArgs a;
    a.x = x;
    a.scores = scores;
    a.w1 = w1;
    a.w2 = w2;
    a.y = y;
    a.hidden = reinterpret_cast<uint16_t *>(base + p.off_partials);
    a.dn_part = reinterpret_cast<float *>(
        base + p.off_partials + align_up((size_t)kMaxGroups * kMaxSlots * kTileM * p.d_e * 2, 256));
    a.dn_arrive = ctrl;
    a.flags = ctrl + kDecodeMaxJT;
    a.masks_out = masks_out;
    a.lists_out = lists_out;
    a.counts_out = counts_out;
    a.T = (int)p.T;
    a.d_h = (int)p.d_h;
    a.E = (int)p.E;
    a.d_e = (int)p.d_e;
    a.X = xcds;
    a.P = members;
    a.upw = (int)(p.d_e / members);
    a.JT = (int)(p.d_h / kDnCols);
    hipLaunchKernelGGL(ffn_bf16_decode_kernel, dim3((unsigned)(xcds * members)), dim3(kThreads),
                       0, stream, a);
    return hipGetLastError();
}

}  // namespace blockffn
