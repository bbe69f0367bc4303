// The 128 x 128 bf16 output tile of the backward's weight-gradient and dx products:
// 256 threads = 4 waves, each wave a 64 x 64 block of 2 x 2 32x32x16 MFMA
// accumulators, operands staged through LDS as [row][k] tiles of 64 k.
//
// A 64 x 64 wave block reads 16 KB of LDS per 64-wide k step for 512 KFLOP (32 flops
// per byte), twice the ratio of a 32 x 64 block, so with LDS delivering about 150
// bytes per clock per CU four waves can keep the matrix cores fed. (The expert pass
// instead runs 16 waves of 32 x 64 blocks per CU: more waves in flight, at half the
// LDS ratio.)
#pragma once

#include "common.h"

namespace blockffn {
namespace tile {

constexpr int kThreads = 256;             // 4 waves
constexpr int kPK = 64;                   // k per step
constexpr int kPKP = kPK + 8;             // LDS pitch of the [row][k] tiles: 144 bytes
constexpr int kDepth = 3;                 // default number of k steps whose loads are in flight
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset past every range: reads zero

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// 32x32 accumulator layout: element v of a lane is row (v/4)*8 + (lane/32)*4 + v%4 of
// column lane%32.
__device__ __forceinline__ int acc_row(int v, int lane) { return (v / 4) * 8 + (lane >> 5) * 4 + (v % 4); }

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[2][2])
{
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;
}

// One k step (BK) of a wave's 64 x 64 block: rows [wm*64, +64) of As, columns
// [wn*64, +64) of Bs, both stored [row][k] with pitch BK + 8.
template <int BK>
__device__ __forceinline__ void mma_64x64(const uint16_t *As, const uint16_t *Bs, f32x16 (&acc)[2][2],
                                          int wm, int wn, int lane)
{
    constexpr int P = BK + 8;
    const int r = lane & 31, kg = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            a[i] = *reinterpret_cast<const bf16x8 *>(&As[(wm * 64 + i * 32 + r) * P + ks * 16 + kg * 8]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[(wn * 64 + j * 32 + r) * P + ks * 16 + kg * 8]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

// The k loop of a 128 x 128 output tile, k in steps of kPK = 64, with kDepth steps in
// flight: the operands of step s + kDepth are requested while step s is multiplied, so
// the memory latency is covered by kDepth steps of products instead of one. load(s,
// ra, rb) fills this thread's four 16-byte pieces of A and of B of step s (piece i:
// row (tid + 256 i) / 8, k (tid % 8) * 8 of the [128][64] tiles) and must read zeros
// (out-of-range offsets) for s >= steps: the loop runs a multiple of kDepth steps so
// that every thread always has the same loads in flight. As and Bs hold 128 * kPKP
// bf16 each, 16-byte aligned; the caller's accumulators are added to. DEPTH = kDepth
// holds 96 registers of operands in flight; DEPTH = 2 (64) lets three workgroups share
// a CU.
template <int DEPTH = kDepth, typename Load>
__device__ __forceinline__ void kloop_128x128(Load load, int steps, uint16_t *As, uint16_t *Bs,
                                              f32x16 (&acc)[2][2], int tid, int wm, int wn,
                                              int lane)
{
    constexpr int kDepth = DEPTH;
    u32x4 ra[kDepth][4], rb[kDepth][4];
    // issued in ring order (the scheduling barriers keep it) so that the wait before a
    // slot's LDS store counts only the younger slots' loads
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        load(d, ra[d], rb[d]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int s0 = 0; s0 < steps; s0 += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = tid + i * kThreads;
                *reinterpret_cast<u32x4 *>(&As[(q >> 3) * kPKP + (q & 7) * 8]) = ra[d][i];
                *reinterpret_cast<u32x4 *>(&Bs[(q >> 3) * kPKP + (q & 7) * 8]) = rb[d][i];
            }
            __syncthreads();
            load(s0 + d + kDepth, ra[d], rb[d]);
            mma_64x64<kPK>(As, Bs, acc, wm, wn, lane);
            __syncthreads();
        }
    }
}

}  // namespace tile
}  // namespace blockffn
