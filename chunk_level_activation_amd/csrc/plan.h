// Host-side launch plan and workspace layout of the chunk FFN.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace blockffn {

// The workspace starts with a control block of fixed size (64 KB of 32-bit words),
// in three disjoint regions:
//   words [0, kDecodeControlWord): the single-chunk schedule's arrival counters
//       (ffn_bf16_chunk.hip); every call returns the ones it used to zero;
//   words [kDecodeControlWord, kStatusWord): the decode schedule's arrival counters,
//       which return to zero, and its per-member epoch flags, which count the calls
//       made with this workspace and only ever increase (a zero-filled workspace
//       starts them at a consistent state; the first word past them is
//       kDecodeControlEnd);
//   word kStatusWord: set to a non-zero value by a kernel whose bounded wait timed
//       out (its outputs are then NaN); only zero-filling the workspace clears it.
// A workspace zero-filled once therefore stays valid across calls of any sizes until
// a wait times out. Scratch data always lies after the block.
constexpr size_t kControlBytes = 64 * 1024;
constexpr int64_t kControlWords = kControlBytes / sizeof(uint32_t);
constexpr int64_t kMaxGroups = 16;   // XCDs the one-launch kernels may spread groups over
constexpr int64_t kStatusWord = kControlWords - 1;
constexpr uint32_t kStatusTimedOut = 1u;

// One-launch bf16 schedule for a single chunk tile (defined in ffn_bf16_chunk.hip).
bool chunk1_supported(int64_t CT, int64_t d_h, int64_t d_e);
size_t chunk1_partial_bytes(int64_t d_h, int64_t E, int64_t d_e);
int chunk1_blocks_per_cu();

// One-launch bf16 decode schedule, one workgroup per CU (ffn_bf16_decode.hip).
// decode_shape(): sizes that may use it on some device (the workspace is sized for
// it); decode_supported(): sizes usable with `xcds` groups of `members` workgroups.
// Its counters and flags occupy words [kDecodeControlWord, kDecodeControlEnd) of the
// control block: 32 output-tile counters, two flag arrays of kMaxGroups x 64 members,
// then the fused LayerNorm's arrival and departure counters.
constexpr int64_t kDecodeControlWord = kControlWords / 2;
constexpr int64_t kDecodeControlEnd = kDecodeControlWord + 32 + 2 * kMaxGroups * 64 + 2;
static_assert(kDecodeControlEnd <= kStatusWord, "the decode flags stay below the status word");
// Words the single-chunk schedule uses for E experts of width d_e and d_h columns.
inline int64_t chunk1_control_words(int64_t E, int64_t d_h, int64_t d_e)
{
    return E * (d_e / 128) + E + kMaxGroups + d_h / 64;
}
inline bool decode_shape(int dtype, int64_t CT, int64_t d_h, int64_t d_e)
{
    return dtype == 1 && CT == 1 && d_h % 128 == 0 && d_h <= 2048 && d_e % 64 == 0 &&
           d_e <= 512;
}
bool decode_supported(int64_t CT, int64_t d_h, int64_t E, int64_t d_e, int xcds, int members);
size_t decode_scratch_bytes(int64_t d_h, int64_t E, int64_t d_e);
int decode_blocks_per_cu();

// Expert-grouped multi-chunk bf16 schedule (ffn_bf16_grouped.hip): the sizes it takes.
bool grouped_supported(int64_t T, int64_t CT, int64_t d_h, int64_t E, int64_t d_e);
// Its down-projection: chunk tiles per workgroup (4 from four chunk tiles up, else 2)
// and k splits (1, or 2 / 4 when the (tiles, column tile) workgroups
// would not fill the chip's 256 CUs); the splits' fp32 partials need
// grouped_partial_bytes() of scratch.
int grouped_down_tiles(int64_t CT, int64_t d_h);
int grouped_down_splits(int64_t CT, int64_t d_h);
size_t grouped_partial_bytes(int64_t CT, int64_t d_h);

// Problem sizes plus everything derived from them that the kernels and the
// workspace layout need. Built once per call by make_plan().
struct FfnPlan {
    int64_t T, d_h, E, d_e, n;
    int dtype;            // BLOCKFFN_F32 or BLOCKFFN_BF16
    int64_t C;            // chunks, ceil(T / n)
    int64_t MPC;          // 32-token tiles per chunk, ceil(n / 32) (n capped at T)
    int64_t CT;           // chunk tiles, C * MPC
    int64_t W;            // 64-bit mask words per chunk, ceil(E / 64)
    int64_t JT;           // 32-column tiles of d_h in the two-launch down-projection
    bool chunk1;          // sizes admit the one-launch single-tile bf16 schedule
    bool decode;          // sizes may admit the one-workgroup-per-CU decode schedule
    bool grouped;         // sizes admit the expert-grouped multi-chunk schedule
    // scratch after the control block (byte offsets)
    size_t off_masks, off_lists, off_counts;   // fp32 path union
    size_t off_hidden, off_partials;
    size_t off_dnpart;    // grouped schedule: the down-projection's split partials
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
    p.chunk1 = dtype == 1 && chunk1_supported(p.CT, d_h, d_e) &&
               chunk1_control_words(E, d_h, d_e) <= kDecodeControlWord;
    p.decode = decode_shape(dtype, p.CT, d_h, d_e);
    p.grouped = dtype == 1 && grouped_supported(T, p.CT, d_h, E, d_e);
    const size_t helem = dtype == 1 ? 2 : 4;   // hidden activations: bf16 or fp32
    size_t off = kControlBytes;
    p.off_masks = off;    off = align_up(off + sizeof(uint64_t) * p.C * p.W, 256);
    p.off_lists = off;    off = align_up(off + sizeof(int32_t) * p.C * E, 256);
    p.off_counts = off;   off = align_up(off + sizeof(int32_t) * p.C, 256);
    p.off_hidden = off;   off = align_up(off + helem * p.CT * E * 32 * d_e, 256);
    p.off_partials = off;
    size_t partials = 0;
    if (p.chunk1)
        partials = chunk1_partial_bytes(d_h, E, d_e);
    if (p.decode && decode_scratch_bytes(d_h, E, d_e) > partials)
        partials = decode_scratch_bytes(d_h, E, d_e);
    off = align_up(off + partials, 256);
    p.off_dnpart = off;
    if (p.grouped)
        off = align_up(off + grouped_partial_bytes(p.CT, d_h), 256);
    p.total_bytes = off;
    return p;
}

// Launchers, one per kernel file. Each returns the hipError_t of its launches.
hipError_t launch_union(const FfnPlan &p, const float *scores, void *ws,
                        uint64_t *masks_out, int32_t *lists_out, int32_t *counts_out,
                        hipStream_t stream);
hipError_t launch_ffn_bf16(const FfnPlan &p, const uint16_t *x, const float *scores,
                           const uint16_t *w1, const uint16_t *w2, uint16_t *y, void *ws,
                           uint64_t *masks_out, int32_t *lists_out, int32_t *counts_out,
                           hipStream_t stream);
// One launch for a single chunk tile, `xcds` expert groups of `wg_per_xcd`
// workgroups each (requires round-robin placement and that many resident workgroups).
hipError_t launch_ffn_bf16_chunk1(const FfnPlan &p, int xcds, int wg_per_xcd,
                                  const uint16_t *x, const float *scores, const uint16_t *w1,
                                  const uint16_t *w2, uint16_t *y, void *ws,
                                  uint64_t *masks_out, int32_t *lists_out, int32_t *counts_out,
                                  hipStream_t stream);
// One launch for a single chunk tile of at most 32 tokens: `xcds` groups of `members`
// workgroups, one per CU, group g on XCD g (requires round-robin placement and every
// workgroup resident at once).
hipError_t launch_ffn_bf16_decode(const FfnPlan &p, int xcds, int members, const uint16_t *x,
                                  const float *scores, const uint16_t *w1, const uint16_t *w2,
                                  uint16_t *y, void *ws, uint64_t *masks_out,
                                  int32_t *lists_out, int32_t *counts_out, hipStream_t stream);
// The same schedule with the router computed inside the launch (E <= 64 and at most
// two experts per member, d_h % 256 == 0 and <= 2048, on top of the decode sizes);
// scores_out [T][E] is written when given. packed: w1 and w2 are in the tiled layout
// of launch_pack_weights.
bool layer_decode_supported(int64_t E, int64_t d_h, int members);
// The rest of the pages' layer around the FFN, fused into the one-launch layer when
// given: ln_out = LayerNorm(y + x) (y rounded to bf16 first; NULL = no epilogue, and
// y may then be NULL too) and probs = sigmoid(sharpness * scores) (NULL = none).
struct LayerEpilogue {
    const float *ln_gamma, *ln_beta;
    float ln_eps;
    uint16_t *ln_out;
    float sharpness;
    float *probs;
};
hipError_t launch_layer_bf16_decode(const FfnPlan &p, int xcds, int members, const uint16_t *x,
                                    const uint16_t *w_r, const float *gain, const float *bias,
                                    float eps, const uint16_t *w1, const uint16_t *w2,
                                    bool packed, uint16_t *y, float *scores_out, void *ws,
                                    const LayerEpilogue *ep, hipStream_t stream);
// W1 [E][d_e][d_h] and W2 [E][d_h][d_e] (bf16) into packed = [W1 tiles][W2 tiles], each
// matrix as 16 x 32 tiles of 1 KB in row-major tile order, row-major inside a tile.
hipError_t launch_pack_weights(const uint16_t *w1, const uint16_t *w2, int64_t E, int64_t d_h,
                               int64_t d_e, uint16_t *packed, hipStream_t stream);
// Four launches: union, per-expert tile lists, expert-grouped up-projection,
// tile-pair x column-tile down-projection.
hipError_t launch_ffn_bf16_grouped(const FfnPlan &p, const uint16_t *x, const float *scores,
                                   const uint16_t *w1, const uint16_t *w2, uint16_t *y, void *ws,
                                   uint64_t *masks_out, int32_t *lists_out, int32_t *counts_out,
                                   hipStream_t stream);
// The grouped down-projection with an fp32 result: out[t][c] = sum over the experts e of
// the union of t's chunk of act[tile][e][row] . w[e][c], act [CT][E][32][d_e] and
// w [E][d_h][d_e] (bf16), masks [C][W]; part holds grouped_partial_bytes(CT, d_h) bytes
// (the split partials, when k is split). With sum_splits the partials are then added
// into out; without, out is left alone and the caller adds the grouped_down_splits()
// partials [splits][CT][32][d_h] in split order. Sizes as grouped_supported admits.
hipError_t launch_grouped_down_f32(const FfnPlan &p, const uint16_t *act, const uint16_t *w,
                                   const uint64_t *masks, float *out, float *part,
                                   bool sum_splits, hipStream_t stream);
hipError_t launch_ffn_f32(const FfnPlan &p, const float *x, const float *scores,
                          const float *w1, const float *w2, float *y, void *ws,
                          hipStream_t stream);
// Router: the bf16 kernel splits the d_h sum over workgroups when it has a workspace
// (ws != NULL, at least router_workspace_bytes, zero-filled once; its counters return
// to zero after every call). router_workspace_bytes is 0 when no split pays. xcds > 1
// states that workgroup b runs on XCD b % xcds (verified on this device); the splits
// of a tile then share an XCD. xcds <= 1: no placement assumption.
constexpr size_t kRouterControlBytes = 64 * 1024;   // arrival counters, one per token tile
int router_splits(int64_t T, int64_t d_h);
size_t router_workspace_bytes(int64_t T, int64_t d_h, int64_t E);
hipError_t launch_router_bf16(const uint16_t *x, const uint16_t *w_r, const float *gain,
                              const float *bias, float eps, int64_t T, int64_t d_h,
                              int64_t E, float *scores, float *logits, float sharpness,
                              float *probs, void *ws, int xcds, hipStream_t stream);
// Checks that workgroup b of a launch runs on XCD b % nxcd (round-robin dispatch): one
// probe launch on `stream` into a static device array, then a synchronisation of that
// stream. Allocates nothing.
hipError_t probe_xcd_placement(int nxcd, hipStream_t stream, bool *round_robin);
hipError_t launch_router_f32(const float *x, const float *w_r, const float *gain,
                             const float *bias, float eps, int64_t T, int64_t d_h,
                             int64_t E, float *scores, float *logits, float sharpness,
                             float *probs, hipStream_t stream);

// Residual + LayerNorm of the layer output over d_h (one wavefront per row). d_h is a
// multiple of 8 (bf16) or 4 (fp32); out may be y or x.
hipError_t launch_add_layernorm(int dtype_bf16, const void *y, const void *x, const float *gamma,
                                const float *beta, float eps, int64_t T, int64_t d_h, void *out,
                                hipStream_t stream);

// Sparsity losses over probabilities [B, S, E] with chunks of L tokens. The workspace
// (zero-filled once; its counters return to zero after every call) holds the arrival
// counters (a top counter and 64 group counters, 128 bytes apart) and one fp64 pair
// of partial sums per workgroup.
constexpr size_t kLossControlBytes = 65 * 128;   // top counter + 64 group counters
constexpr int64_t kLossMaxBlocks = 2048;
int64_t sparsity_losses_blocks(int64_t B, int64_t S, int64_t E, int64_t L);
size_t sparsity_losses_workspace_bytes(int64_t B, int64_t S, int64_t E, int64_t L);
hipError_t launch_sparsity_losses(const float *p, int64_t B, int64_t S, int64_t E, float alpha,
                                  int64_t L, float lambda_al, float lambda_cs, float *losses,
                                  float *grad, void *ws, hipStream_t stream);

// Layer backward (bf16): sizes it takes, workspace bytes, launches.
bool backward_supported(int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n);
size_t backward_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n);
struct BackwardArgs {
    const uint16_t *x, *w_r, *w1, *w2, *dy;
    const float *gain, *bias, *dprobs;
    float eps, sharpness;
    int64_t T, d_h, E, d_e, n;
    float *dx, *dw_r, *dgain, *dbias, *dw1, *dw2;
    int xcds;   // verified round-robin XCD count (0: unknown), for the recomputed router
};
hipError_t launch_layer_backward(const BackwardArgs &b, void *ws, hipStream_t stream);

}  // namespace blockffn
