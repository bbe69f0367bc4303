// Per-chunk union of active experts and its compaction into an ascending list.
//
// Skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
// Deployment", "Core Concept": the accelerator evaluates only the union of the
// experts activated by the n tokens of a chunk. Expert e is active for token t when
// its router score s[t,e] is non-zero; chunks are aligned, ceil(T/n) of them, the
// last one possibly partial ("Chunk Sparsification Loss").
//
// One wavefront per chunk, lane = expert within a 64-expert word: each lane ORs its
// expert's activity over the chunk's tokens (a coalesced row read per token, 16
// tokens in flight at a time), a wave ballot turns the 64 flags into the mask word,
// and the position of every member in the list is the popcount of the mask bits
// below its lane plus the members of earlier words, so the list comes out in
// ascending expert id. (The bf16 kernels compute the same union inside each
// workgroup instead; this kernel serves the fp32 path.)
#include "common.h"
#include "plan.h"

namespace blockffn {

__global__ void __launch_bounds__(kWave)
union_kernel(const float *__restrict__ scores, int64_t T, int E, int64_t n, int W,
             uint64_t *__restrict__ masks, int32_t *__restrict__ lists,
             int32_t *__restrict__ counts, uint64_t *__restrict__ masks_out,
             int32_t *__restrict__ lists_out, int32_t *__restrict__ counts_out)
{
    constexpr int kBatch = 32;    // tokens whose score loads are in flight together (one n = 32 chunk)
    const int64_t c = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t t0 = c * n;
    const int64_t t1 = t0 + n < T ? t0 + n : T;
    int members = 0;
    for (int w = 0; w < W; ++w) {
        const int e = w * kWave + lane;
        bool active = false;
        if (e < E) {
            for (int64_t tb = t0; tb < t1; tb += kBatch) {
                // every load issued (tokens past the chunk re-read its last token and are
                // masked out): a load under a branch would be waited for on its own
                float v[kBatch];
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
                    v[i] = scores[(tb + i < t1 ? tb + i : t1 - 1) * E + e];
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
                    active |= tb + i < t1 && v[i] != 0.0f;
            }
        }
        const uint64_t word = __ballot(active);
        if (active) {
            const int pos = members + __popcll(word & ((1ull << lane) - 1ull));
            lists[c * E + pos] = e;
            if (lists_out)
                lists_out[c * E + pos] = e;
        }
        if (lane == 0) {
            masks[c * W + w] = word;
            if (masks_out)
                masks_out[c * W + w] = word;
        }
        members += __popcll(word);
    }
    for (int i = members + lane; i < E; i += kWave) {
        lists[c * E + i] = -1;
        if (lists_out)
            lists_out[c * E + i] = -1;
    }
    if (lane == 0) {
        counts[c] = members;
        if (counts_out)
            counts_out[c] = members;
    }
}

hipError_t launch_union(const FfnPlan &p, const float *scores, void *ws,
                        uint64_t *masks_out, int32_t *lists_out, int32_t *counts_out,
                        hipStream_t stream)
{
    char *base = static_cast<char *>(ws);
    hipLaunchKernelGGL(union_kernel, dim3((unsigned)p.C), dim3(kWave), 0, stream, scores,
                       p.T, (int)p.E, p.n, (int)p.W,
                       reinterpret_cast<uint64_t *>(base + p.off_masks),
                       reinterpret_cast<int32_t *>(base + p.off_lists),
                       reinterpret_cast<int32_t *>(base + p.off_counts), masks_out,
                       lists_out, counts_out);
    return hipGetLastError();
}

}  // namespace blockffn
