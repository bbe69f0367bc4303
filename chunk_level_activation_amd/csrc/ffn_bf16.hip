// bf16 chunk FFN on the gfx950 matrix cores: per-chunk union, gathered up-projection
// with Swish and score scaling, and the down-projection summed over the chunk's union.
//
// Skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
// Deployment": "Architecture Overview" (experts are non-gated MLPs with Swish,
// d_e << d_h; the pages' kernel takes n = 32 tokens at once and computes only the
// union of activated experts) and "Core Concept" (unneeded activations are masked
// after the computation). For each chunk tile (32 token rows) and each expert e of
// the chunk's union U_c:
//     Ht_e[t,:] = bf16( s[t,e] * swish(W1_e x_t) )          (up work items)
//     y[t,:]    = bf16( sum_{e in U_c} W2_e Ht_e[t,:] )        (down work items)
// Scaling the hidden row by s before W2 equals scaling the expert output after it
// (the map is linear); a token whose score is 0 gets an all-zero hidden row, which is
// the masking. Experts outside U_c are never read.
//
// This file holds the general schedule, used whenever the chunk tiles alone give
// every CU work (prefill-sized inputs): two launches, all up items, then all down
// items, with no handoff inside a kernel. A single 32-token chunk tile (decode) runs
// as one launch instead; see ffn_bf16_chunk.hip.
//
// Every workgroup recomputes its chunk's union from the n x E scores (16-byte loads,
// all in flight together), so no separate union pass exists.
//   up item   (chunk tile, union slot, 16 hidden units): streams the slot's W1 rows,
//             reads the tile's x rows, writes 32 x 16 hidden values;
//   down item (chunk tile, 32 output columns): streams W2 rows of every union slot
//             for those columns and sums the hidden rows into the 32 x 32 y tile.
//
// Data layout (row-major): x [T, d_h], W1 [E, d_e, d_h], W2 [E, d_h, d_e], hidden
// [chunk tile][union slot][32][d_e] bf16.
#include "common.h"
#include "plan.h"

namespace blockffn {

constexpr int kThreads = 512;      // 8 waves per workgroup
constexpr int kWaves = kThreads / kWave;
constexpr int kUpRows = 16;        // hidden units per up work item
constexpr int kUpBatch = 8;        // k steps whose loads are in flight together (up)
constexpr int kDownBatch = 8;      // k steps whose loads are in flight together (down)
constexpr int kMaxWords = 4;       // 64-expert mask words, E <= 256

struct FfnArgs {
    const uint16_t *x;
    const float *scores;
    const uint16_t *w1;
    const uint16_t *w2;
    uint16_t *y;
    uint16_t *hidden;
    uint64_t *masks_out;
    int32_t *lists_out;
    int32_t *counts_out;
    int64_t T, n, CT, up_items;
    int d_h, E, d_e, MPC, RT, JT;
};

// Union of the experts active in chunk c, and its ascending list, in LDS. Returns
// |U_c|. The chunk's scores are contiguous (n x E floats); each thread reads four at
// a time with one 16-byte load where alignment allows, all in flight together.
__device__ int chunk_union(const FfnArgs &a, int64_t c, uint64_t *s_mask, int *s_list)
{
    const int tid = threadIdx.x;
    if (tid < kMaxWords)
        s_mask[tid] = 0;
    __syncthreads();
    const int64_t t0 = c * a.n;
    const int64_t t1 = t0 + a.n < a.T ? t0 + a.n : a.T;
    const int64_t total = (t1 - t0) * a.E;
    const float *sc = a.scores + t0 * a.E;
    const bool vec = (a.E % 4) == 0 && (reinterpret_cast<uintptr_t>(sc) % 16) == 0;
    if (vec) {
        for (int64_t base = 0; base < total; base += 4 * 4 * kThreads) {
            float4 v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t idx = base + 4 * ((int64_t)i * kThreads + tid);
                v[i] = idx < total ? *reinterpret_cast<const float4 *>(sc + idx)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t idx = base + 4 * ((int64_t)i * kThreads + tid);
                const float f[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (f[q] != 0.0f) {
                        const int e = (int)((idx + q) % a.E);
                        atomicOr(reinterpret_cast<unsigned long long *>(&s_mask[e >> 6]),
                                 1ull << (e & 63));
                    }
            }
        }
    } else {
        for (int64_t idx = tid; idx < total; idx += kThreads)
            if (sc[idx] != 0.0f) {
                const int e = (int)(idx % a.E);
                atomicOr(reinterpret_cast<unsigned long long *>(&s_mask[e >> 6]),
                         1ull << (e & 63));
            }
    }
    __syncthreads();
    const int W = (a.E + 63) >> 6;
    int cnt = 0;
    for (int w = 0; w < W; ++w)
        cnt += __popcll(s_mask[w]);
    if (tid < a.E) {
        const int w = tid >> 6, bit = tid & 63;
        const uint64_t word = s_mask[w];
        if ((word >> bit) & 1ull) {
            int pos = __popcll(word & ((1ull << bit) - 1ull));
            for (int v = 0; v < w; ++v)
                pos += __popcll(s_mask[v]);
            s_list[pos] = tid;
        }
    }
    __syncthreads();
    return cnt;
}

// ------------------------------------------------------------------ up item
// 16x16x32 MFMA: A = x rows (16 tokens x 32 k), B = W1 rows transposed (32 k x 16
// hidden units); the two token halves share every W1 fragment. The eight waves take
// k steps round robin; their sums are added in wave order through LDS.
__device__ void up_item(const FfnArgs &a, int64_t item, const int *s_list, int cnt)
{
    const int64_t ct = item / ((int64_t)a.E * a.RT);
    const int li = (int)(item % ((int64_t)a.E * a.RT));
    const int rt = li % a.RT;
    const int slot = li / a.RT;
    if (slot >= cnt)
        return;
    const int64_t c = ct / a.MPC;
    const int m = (int)(ct % a.MPC);
    const int e = s_list[slot];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int r = lane & 15, kg = lane >> 4;
    const int64_t tile_t0 = c * a.n + (int64_t)m * kTileM;
    const int64_t chunk_end = c * a.n + a.n < a.T ? c * a.n + a.n : a.T;
    const int64_t ta = tile_t0 + r, tb = tile_t0 + 16 + r;
    const bool va = ta < chunk_end, vb = tb < chunk_end;
    const int d_h = a.d_h;
    const uint16_t *xa = a.x + (va ? ta : 0) * d_h + kg * 8;
    const uint16_t *xb = a.x + (vb ? tb : 0) * d_h + kg * 8;
    const uint16_t *wr = a.w1 + ((int64_t)e * a.d_e + rt * kUpRows + r) * d_h + kg * 8;

    // this tile's scores of expert e, fetched alongside the operands
    __shared__ float s_col[kTileM];
    if (tid < kTileM) {
        const int64_t t = tile_t0 + tid;
        s_col[tid] = t < chunk_end ? a.scores[t * a.E + e] : 0.0f;
    }

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const int KS = d_h / 32;
    for (int kb = wave; kb < KS; kb += kWaves * kUpBatch) {
        bf16x8 bw[kUpBatch], a0[kUpBatch], a1[kUpBatch];
#pragma unroll
        for (int i = 0; i < kUpBatch; ++i) {
            const int ks = kb + i * kWaves;
            const bool ok = ks < KS;
            bw[i] = ok ? load_bf16x8_stream(wr + ks * 32) : zero_bf16x8();
            a0[i] = ok && va ? load_bf16x8(xa + ks * 32) : zero_bf16x8();
            a1[i] = ok && vb ? load_bf16x8(xb + ks * 32) : zero_bf16x8();
        }
#pragma unroll
        for (int i = 0; i < kUpBatch; ++i) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], bw[i], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[i], bw[i], acc1, 0, 0, 0);
        }
    }

    // 16x16 accumulator layout: lane holds rows (lane/16)*4 + i of column lane%16.
    __shared__ float red[kWaves][kTileM][kUpRows + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        red[wave][kg * 4 + i][r] = acc0[i];
        red[wave][16 + kg * 4 + i][r] = acc1[i];
    }
    __syncthreads();
    // 128 threads finish 4 hidden units each and store them as one 8-byte word.
    if (tid < kTileM * kUpRows / 4) {
        const int tt = tid >> 2, r0 = (tid & 3) * 4;
        uint64_t packed = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                sum += red[w][tt][r0 + q];
            const float h = swish_fast(sum) * s_col[tt];
            packed |= (uint64_t)f32_to_bf16(h) << (16 * q);
        }
        uint16_t *dst = a.hidden + ((ct * a.E + slot) * kTileM + tt) * a.d_e + rt * kUpRows + r0;
        *reinterpret_cast<uint64_t *>(dst) = packed;
    }
}

// ------------------------------------------------------------------ down item
// 32x32x16 MFMA: A = hidden rows (32 tokens x 16 k), B = W2 rows transposed (16 k x
// 32 output columns). The union's (slot, k step) units go round robin to the waves,
// so the eight waves together read whole W2 rows.
__device__ void down_item(const FfnArgs &a, int64_t item, const int *s_list, int cnt)
{
    const int64_t ct = item / a.JT;
    const int jt = (int)(item % a.JT);
    const int64_t c = ct / a.MPC;
    const int m = (int)(ct % a.MPC);
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 31, kg = lane >> 5;
    const int s0 = 0, s1 = cnt;
    const int KSe = a.d_e / 16;
    const int units = (s1 - s0) * KSe;

    // The first down item of each chunk reports the union it used.
    if (m == 0 && jt == 0) {
        const int W = (a.E + 63) >> 6;
        if (a.counts_out && tid == 0)
            a.counts_out[c] = cnt;
        if (a.lists_out)
            for (int i = tid; i < a.E; i += kThreads)
                a.lists_out[c * a.E + i] = i < cnt ? s_list[i] : -1;
        if (a.masks_out && tid < W) {
            uint64_t word = 0;
            for (int i = 0; i < cnt; ++i)
                if ((s_list[i] >> 6) == tid)
                    word |= 1ull << (s_list[i] & 63);
            a.masks_out[c * W + tid] = word;
        }
    }

    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        acc[i] = 0.0f;

    // Unit u of this group is (slot s0 + u / KSe, k step u % KSe); wave w takes units
    // w, w + 8, ... in batches of kDownBatch.
    bf16x8 bw[kDownBatch];
    auto load_w2 = [&](int ub) {
#pragma unroll
        for (int i = 0; i < kDownBatch; ++i) {
            const int u = ub + i * kWaves;
            if (u < units) {
                const int e = s_list[s0 + u / KSe];
                bw[i] = load_bf16x8_stream(a.w2 + ((int64_t)e * a.d_h + jt * 32 + col) * a.d_e +
                                           (u % KSe) * 16 + kg * 8);
            } else {
                bw[i] = zero_bf16x8();
            }
        }
    };
    load_w2(wave);

    for (int ub = wave; ub < units; ub += kWaves * kDownBatch) {
        bf16x8 ha[kDownBatch];
#pragma unroll
        for (int i = 0; i < kDownBatch; ++i) {
            const int u = ub + i * kWaves;
            if (u < units) {
                const uint16_t *hp = a.hidden +
                                     ((ct * a.E + s0 + u / KSe) * kTileM + col) * a.d_e +
                                     (u % KSe) * 16 + kg * 8;
                ha[i] = load_bf16x8(hp);
            } else {
                ha[i] = zero_bf16x8();
            }
        }
#pragma unroll
        for (int i = 0; i < kDownBatch; ++i)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha[i], bw[i], acc, 0, 0, 0);
        if (ub + kWaves * kDownBatch < units)
            load_w2(ub + kWaves * kDownBatch);
    }

    // 32x32 accumulator layout: element i of a lane is row (i/4)*8 + (lane/32)*4 + i%4
    // of column lane%32.
    __shared__ float red[kWaves][kTileM][33];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        red[wave][(i / 4) * 8 + kg * 4 + (i % 4)][col] = acc[i];
    __syncthreads();
    // 512 threads x 2 adjacent columns
    const int tt = tid >> 4, jj = (tid & 15) * 2;
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        o0 += red[w][tt][jj];
        o1 += red[w][tt][jj + 1];
    }
    const int64_t tile_t0 = c * a.n + (int64_t)m * kTileM;
    const int64_t chunk_end = c * a.n + a.n < a.T ? c * a.n + a.n : a.T;
    const int64_t t = tile_t0 + tt;
    if (t < chunk_end) {
        const uint32_t packed = (uint32_t)f32_to_bf16(o0) | ((uint32_t)f32_to_bf16(o1) << 16);
        *reinterpret_cast<uint32_t *>(a.y + t * a.d_h + jt * 32 + jj) = packed;
    }
}

__global__ void __launch_bounds__(kThreads, 4)
ffn_bf16_up_kernel(FfnArgs a)
{
    __shared__ uint64_t s_mask[kMaxWords];
    __shared__ int s_list[256];
    const int64_t item = blockIdx.x;
    const int cnt = chunk_union(a, item / ((int64_t)a.E * a.RT) / a.MPC, s_mask, s_list);
    up_item(a, item, s_list, cnt);
}

__global__ void __launch_bounds__(kThreads, 4)
ffn_bf16_down_kernel(FfnArgs a)
{
    __shared__ uint64_t s_mask[kMaxWords];
    __shared__ int s_list[256];
    const int64_t item = blockIdx.x;
    const int cnt = chunk_union(a, item / a.JT / a.MPC, s_mask, s_list);
    down_item(a, item, s_list, cnt);
}

// Workgroup-to-XCD placement probe: records the XCD each workgroup ran on, into a
// static device array (each device holds its own copy for the life of the process; the
// library allocates nothing for it).
constexpr int kProbeBlocks = 4096;
__device__ uint32_t g_xcd_probe[kProbeBlocks];

__global__ void xcd_probe_kernel(uint32_t *out)
{
    if (threadIdx.x == 0)
        out[blockIdx.x] = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // HW_REG_XCC_ID
}

hipError_t probe_xcd_placement(int nxcd, hipStream_t stream, bool *round_robin)
{
    *round_robin = false;
    uint32_t *buf = nullptr;
    hipError_t err = hipGetSymbolAddress(reinterpret_cast<void **>(&buf), HIP_SYMBOL(g_xcd_probe));
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(xcd_probe_kernel, dim3(kProbeBlocks), dim3(64), 0, stream, buf);
    err = hipGetLastError();
    static uint32_t host[kProbeBlocks];
    if (err == hipSuccess)
        err = hipMemcpyAsync(host, buf, sizeof(host), hipMemcpyDeviceToHost, stream);
    if (err == hipSuccess)
        err = hipStreamSynchronize(stream);
    if (err != hipSuccess)
        return err;
    bool ok = nxcd > 0;
    for (int b = 0; b < kProbeBlocks && ok; ++b)
        ok = (int)(host[b] & 0xF) == b % nxcd;
    *round_robin = ok;
    return hipSuccess;
}

hipError_t launch_ffn_bf16(const FfnPlan &p, const uint16_t *x, const float *scores,
                           const uint16_t *w1, const uint16_t *w2, uint16_t *y, void *ws,
                           uint64_t *masks_out, int32_t *lists_out, int32_t *counts_out,
                           hipStream_t stream)
{
    char *base = static_cast<char *>(ws);
    FfnArgs a;
    a.x = x;
    a.scores = scores;
    a.w1 = w1;
    a.w2 = w2;
    a.y = y;
    a.hidden = reinterpret_cast<uint16_t *>(base + p.off_hidden);
    a.masks_out = masks_out;
    a.lists_out = lists_out;
    a.counts_out = counts_out;
    a.T = p.T;
    a.n = p.n;
    a.CT = p.CT;
    a.d_h = (int)p.d_h;
    a.E = (int)p.E;
    a.d_e = (int)p.d_e;
    a.MPC = (int)p.MPC;
    a.RT = (int)(p.d_e / kUpRows);
    a.JT = (int)p.JT;
    a.up_items = p.CT * p.E * a.RT;
    hipLaunchKernelGGL(ffn_bf16_up_kernel, dim3((unsigned)a.up_items), dim3(kThreads), 0,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(ffn_bf16_down_kernel, dim3((unsigned)(p.CT * p.JT)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace blockffn
