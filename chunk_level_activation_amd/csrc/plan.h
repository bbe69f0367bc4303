// Host-side launch plan and workspace layout of the chunk FFN.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace blockffn {

// Problem sizes plus everything derived from them that the kernels and the
// workspace layout need. Built once per call by make_plan().
struct FfnPlan {
    int64_t T, d_h, E, d_e, n;
    int dtype;            // BLOCKFFN_F32 or BLOCKFFN_BF16
    int64_t C;            // chunks, ceil(T / n)
    int64_t MPC;          // 32-token tiles per chunk, ceil(n / 32) (n capped at T)
    int64_t CT;           // chunk tiles, C * MPC
    int64_t W;            // 64-bit mask words per chunk, ceil(E / 64)
    int64_t JT;           // 32-column tiles of d_h in the down-projection
    int64_t G;            // expert groups the down-projection splits a union into
    size_t off_ctrl, off_masks, off_lists, off_counts, off_hidden, off_partials;
    size_t total_bytes;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline FfnPlan make_plan(int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n,
                         int dtype)
{
    FfnPlan p{};
    p.T = T; p.d_h = d_h; p.E = E; p.d_e = d_e; p.dtype = dtype;
    p.n = n < T ? n : T;                  // n >= T: one chunk of all the tokens
    p.C = (T + p.n - 1) / p.n;
    p.MPC = (p.n + 31) / 32;
    p.CT = p.C * p.MPC;
    p.W = (E + 63) / 64;
    p.JT = (d_h + 31) / 32;
    // Split each union over G expert groups when there are too few (tile, column
    // tile) pairs to give every compute unit work; partial sums are then combined
    // in a fixed order by the last group to finish.
    int64_t tiles = p.CT * p.JT;
    p.G = 1;
    while (p.G < 8 && tiles * p.G * 2 <= 256)
        p.G *= 2;
    const size_t helem = dtype == 1 ? 2 : 4;   // hidden activations: bf16 or fp32
    size_t off = 0;
    p.off_ctrl = off;     off = align_up(off + sizeof(uint32_t) * p.CT * p.JT, 256);
    p.off_masks = off;    off = align_up(off + sizeof(uint64_t) * p.C * p.W, 256);
    p.off_lists = off;    off = align_up(off + sizeof(int32_t) * p.C * E, 256);
    p.off_counts = off;   off = align_up(off + sizeof(int32_t) * p.C, 256);
    p.off_hidden = off;   off = align_up(off + helem * p.CT * E * 32 * d_e, 256);
    p.off_partials = off;
    if (p.G > 1)
        off = align_up(off + sizeof(float) * p.CT * p.JT * p.G * 32 * 32, 256);
    p.total_bytes = off;
    return p;
}

// Launchers, one per kernel file. Each returns the hipError_t of its launches.
hipError_t launch_union(const FfnPlan &p, const float *scores, void *ws,
                        uint64_t *masks_out, int32_t *lists_out, int32_t *counts_out,
                        hipStream_t stream);
hipError_t launch_ffn_bf16(const FfnPlan &p, const uint16_t *x, const float *scores,
                           const uint16_t *w1, const uint16_t *w2, uint16_t *y, void *ws,
                           hipStream_t stream);
hipError_t launch_ffn_f32(const FfnPlan &p, const float *x, const float *scores,
                          const float *w1, const float *w2, float *y, void *ws,
                          hipStream_t stream);
hipError_t launch_router_bf16(const uint16_t *x, const uint16_t *w_r, const float *gain,
                              const float *bias, float eps, int64_t T, int64_t d_h,
                              int64_t E, float *scores, float *logits, hipStream_t stream);
hipError_t launch_router_f32(const float *x, const float *w_r, const float *gain,
                             const float *bias, float eps, int64_t T, int64_t d_h,
                             int64_t E, float *scores, float *logits, hipStream_t stream);

}  // namespace blockffn
