// Sparsity training losses of BlockFFN and their gradient with respect to the
// activation probabilities, in one pass over p [B, S, E] (skill page, "Activation
// Locality Loss" and "Chunk Sparsification Loss"):
//
//   q = sigmoid(alpha (2p - 1))                          sharpened patterns
//   AL = 1/max(S-1,1) sum_{i<S-1} mean_{b,e} BCE(target q_i, input q_{i+1}),
//        BCE(c, n) = -(c log(n + 1e-8) + (1 - c) log(1 - n + 1e-8))
//   CS = 1/ceil(S/L) sum_c mean_{b,e} (1 - prod_{k in chunk c} (1 - p_k))
//
//   dAL/dp_t = 2 alpha q_t (1 - q_t) [ dBCE(q_t, q_{t+1})/dq_t + dBCE(q_{t-1}, q_t)/dq_t ]
//              / (B E max(S-1,1))
//   dCS/dp_t = prod_{j != t in t's chunk} (1 - p_j) / (B E ceil(S/L))
//
// HBM-bound: p is read once (plus one neighbouring row at each chunk edge, which the
// caches serve) and the gradient written once. Thread <-> (b, chunk, e): consecutive
// threads take consecutive experts, so every row access of a wavefront is a
// contiguous run of floats. With L <= 32 the chunk's values sit in registers and the
// products over the other tokens come from prefix and suffix products; longer chunks
// keep the suffix products in the gradient array between two passes.
//
// The two loss sums are deterministic: fp32 terms per thread, fp64 wavefront and
// workgroup trees, per-workgroup partials in the workspace, and the last workgroup
// to arrive adds the partials in index order.
#include "plan.h"
#include "sync.h"

namespace blockffn {
namespace {

constexpr int kLossThreads = 256;
typedef double f64x2 __attribute__((ext_vector_type(2)));
constexpr float kLogEps = 1e-8f;
constexpr uint32_t kLossGroups = 64;          // arrival counters of the first level
constexpr uint32_t kLossCounterStride = 32;   // uint32 words: one 128-byte line each

// The hardware's exp2, log2 and reciprocal (about 1 ulp each) carry every
// transcendental step: the per-element arithmetic stays within a few 1e-7 relative of
// the exact values, and the kernel stays memory-bound.
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_ln(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// q = sigmoid(alpha (2p - 1))
__device__ __forceinline__ float sharpen(float p, float alpha)
{
    return fast_rcp(1.0f + __builtin_amdgcn_exp2f(-alpha * kLog2e * (2.0f * p - 1.0f)));
}

struct LossArgs {
    const float *p;
    float *grad;                 // NULL: losses only
    int B, S, E, L, nc;
    uint32_t columns;            // B * nc * E / VW
    float alpha;
    float g_al, g_cs;            // lambda / (B E max(S-1,1)), lambda / (B E nc)
    double al_scale, cs_scale;   // 1 / (B E max(S-1,1)), 1 / (B E nc)
    double *part;                // [gridDim.x][2]
    uint32_t *arrive;
    float *losses;
};

// The pair term of the locality loss for (t, t+1) and the pieces of its gradient:
// d/dq_t and d/dq_{t+1} of BCE(q_t, q_{t+1}).
struct PairTerm {
    float bce, d_cur, d_next;
};
__device__ __forceinline__ PairTerm pair_term(float c, float n)
{
    const float a = n + kLogEps, b = 1.0f - n + kLogEps;
    const float ln = fast_ln(a), l1n = fast_ln(b);
    PairTerm r;
    r.bce = -(c * ln + (1.0f - c) * l1n);
    r.d_cur = -(ln - l1n);
    r.d_next = -(c * fast_rcp(a) - (1.0f - c) * fast_rcp(b));
    return r;
}

// Loads VW consecutive floats (VW = 4: one 16-byte access).
template <int VW>
__device__ __forceinline__ void load_vec(const float *p, float *v)
{
    if constexpr (VW == 4) {
        const float4 f = *reinterpret_cast<const float4 *>(p);
        v[0] = f.x, v[1] = f.y, v[2] = f.z, v[3] = f.w;
    } else {
        v[0] = *p;
    }
}
template <int VW>
__device__ __forceinline__ void store_vec(float *p, const float *v)
{
    if constexpr (VW == 4)
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else
        *p = v[0];
}

// One column: VW consecutive experts of one chunk of one sequence.
//
// MAXL > 0 keeps the chunk (at most MAXL tokens) and its two neighbouring tokens in
// registers. Window slot k holds token t0 - 1 + k; the loads are clamped into the
// window's valid tokens, so every load is unconditional and all of them are in
// flight together, and the slots outside the chunk are masked by selects. MAXL == 0
// handles any L with two passes, parking the suffix products in the gradient array.
// All index arithmetic is 32-bit (the entry point keeps B * S * E below 2^31).
template <int MAXL, int VW>
__device__ __forceinline__ void column(const LossArgs &a, uint32_t col, float &al, float &cs)
{
    const uint32_t E4 = (uint32_t)a.E / VW;
    const uint32_t e0 = (col % E4) * VW;
    const uint32_t bc = col / E4;
    const uint32_t c = bc % (uint32_t)a.nc, b = bc / (uint32_t)a.nc;
    const int t0 = (int)c * a.L, t1 = min(t0 + a.L, a.S), len = t1 - t0;
    const uint32_t E = (uint32_t)a.E;
    const float *pc = a.p + b * (uint32_t)a.S * E + e0;   // p[b, t, e0 + i] = pc[t E + i]
    float *gc = a.grad ? a.grad + b * (uint32_t)a.S * E + e0 : nullptr;
    al = 0.0f;
    cs = 0.0f;

    if constexpr (MAXL > 0) {
        const int lo = t0 > 0 ? t0 - 1 : 0, hi = t1 < a.S ? t1 : a.S - 1;
        float pv[MAXL + 2][VW];
#pragma unroll
        for (int k = 0; k < MAXL + 2; ++k)
            load_vec<VW>(pc + (uint32_t)min(max(t0 - 1 + k, lo), hi) * E, pv[k]);
        // suffix products over the chunk: suf[k] = prod_{j = k .. len} (1 - p[slot j])
        float suf[MAXL + 2][VW];
#pragma unroll
        for (int i = 0; i < VW; ++i)
            suf[MAXL + 1][i] = 1.0f;
#pragma unroll
        for (int k = MAXL; k >= 1; --k)
#pragma unroll
            for (int i = 0; i < VW; ++i)
                suf[k][i] = k <= len ? suf[k + 1][i] * (1.0f - pv[k][i]) : 1.0f;
        float qc[VW], pre[VW], dn[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) {
            cs += 1.0f - suf[1][i];
            qc[i] = sharpen(pv[1][i], a.alpha);
            pre[i] = 1.0f;
            // the pair (t0 - 1, t0) contributes to t0's gradient
            dn[i] = t0 > 0 ? pair_term(sharpen(pv[0][i], a.alpha), qc[i]).d_next : 0.0f;
        }
#pragma unroll
        for (int k = 1; k <= MAXL; ++k) {
            const bool in_chunk = k <= len;
            const bool pair = in_chunk && t0 + k < a.S;     // (t, t + 1), t = t0 - 1 + k
            float g[VW];
#pragma unroll
            for (int i = 0; i < VW; ++i) {
                const float qn = sharpen(pv[k + 1][i], a.alpha);
                const PairTerm pt = pair_term(qc[i], qn);
                al += pair ? pt.bce : 0.0f;
                const float dq = dn[i] + (pair ? pt.d_cur : 0.0f);
                dn[i] = pair ? pt.d_next : 0.0f;
                const float slope = 2.0f * a.alpha * qc[i] * (1.0f - qc[i]);
                g[i] = a.g_al * slope * dq + a.g_cs * (pre[i] * suf[k + 1][i]);
                pre[i] *= in_chunk ? 1.0f - pv[k][i] : 1.0f;
                qc[i] = qn;
            }
            if (gc && in_chunk)
                store_vec<VW>(gc + (uint32_t)(t0 - 1 + k) * E, g);
        }
    } else {
        static_assert(VW == 1, "the any-L path takes one expert per thread");
        // pass 1, backwards: product of the chunk, and (with a gradient) the suffix
        // product of the tokens after t parked in grad[t]
        float suf = 1.0f;
        for (int t = t1 - 1; t >= t0; --t) {
            if (gc)
                gc[(uint32_t)t * E] = suf;
            suf *= 1.0f - pc[(uint32_t)t * E];
        }
        cs = 1.0f - suf;
        // pass 2, forwards: locality terms and the gradient
        float pre = 1.0f, prev_dn = 0.0f;
        float qc = sharpen(pc[(uint32_t)t0 * E], a.alpha);
        if (t0 > 0)
            prev_dn = pair_term(sharpen(pc[(uint32_t)(t0 - 1) * E], a.alpha), qc).d_next;
        for (int t = t0; t < t1; ++t) {
            float dq = prev_dn;
            prev_dn = 0.0f;
            float qn = 0.0f;
            if (t + 1 < a.S) {
                qn = sharpen(pc[(uint32_t)(t + 1) * E], a.alpha);
                const PairTerm pt = pair_term(qc, qn);
                al += pt.bce;
                dq += pt.d_cur;
                prev_dn = pt.d_next;
            }
            const float pt_ = pc[(uint32_t)t * E];
            if (gc) {
                const float slope = 2.0f * a.alpha * qc * (1.0f - qc);
                gc[(uint32_t)t * E] = a.g_al * slope * dq + a.g_cs * (pre * gc[(uint32_t)t * E]);
            }
            pre *= 1.0f - pt_;
            qc = qn;
        }
    }
}

// Workgroups of kLossWaves wavefronts at most (blockDim.x = 64 for small problems, so
// that they spread over more CUs).
template <int MAXL, int VW>
__global__ void __launch_bounds__(kLossThreads) sparsity_losses_kernel(LossArgs a)
{
    __shared__ double red[kLossThreads / kWave][2];
    __shared__ int last;
    const int tid = threadIdx.x, nwaves = blockDim.x / kWave;
    double al_sum = 0.0, cs_sum = 0.0;
    for (uint32_t col = blockIdx.x * blockDim.x + tid; col < a.columns;
         col += gridDim.x * blockDim.x) {
        float al, cs;
        column<MAXL, VW>(a, col, al, cs);
        al_sum += (double)al;
        cs_sum += (double)cs;
    }
    al_sum = wave_sum_f64(al_sum);
    cs_sum = wave_sum_f64(cs_sum);
    if (tid % kWave == 0) {
        red[tid / kWave][0] = al_sum;
        red[tid / kWave][1] = cs_sum;
    }
    __syncthreads();
    // the partial pair of this workgroup, 16 bytes
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.part, (uint64_t)gridDim.x * 16);
    if (tid == 0) {
        double s0 = 0.0, s1 = 0.0;
        for (int w = 0; w < nwaves; ++w) {
            s0 += red[w][0];
            s1 += red[w][1];
        }
        // device-scope store (sc1): the last workgroup may sit on another XCD
        const f64x2 pair = {s0, s1};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pair), rp,
                                               (int)(blockIdx.x * 16u), 0, kSC1);
        drain_memory();
        // Two-level arrival: workgroup b counts in group b % G (its own 128-byte line),
        // the last of a group counts at the top, the last at the top reduces. Each
        // counter then sees about 1/G of the arrivals: arrivals on one address are
        // serialised by the memory system (some 10 ns each).
        const uint32_t G = gridDim.x < kLossGroups ? gridDim.x : kLossGroups;
        const uint32_t g = blockIdx.x % G;
        const uint32_t in_group = gridDim.x / G + (g < gridDim.x % G ? 1u : 0u);
        uint32_t *gc = a.arrive + (1 + g) * kLossCounterStride;
        bool top = false;
        if (add_counter(gc, 1u) == in_group - 1) {
            st_counter(gc, 0u);
            top = add_counter(a.arrive, 1u) == G - 1;
            if (top)
                st_counter(a.arrive, 0u);
        }
        last = top;
    }
    __syncthreads();
    if (!last)
        return;
    // the last workgroup: thread i adds partials i, i + blockDim, ... in that order,
    // eight loads in flight at a time (offsets past the grid read zero), then a fixed
    // tree
    double s0 = 0.0, s1 = 0.0;
    for (uint32_t base = 0; base < gridDim.x; base += 8 * blockDim.x) {
        u32x4 pv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            pv[k] = __builtin_amdgcn_raw_buffer_load_b128(
                rp, (int)((base + tid + k * blockDim.x) * 16u), 0, kSC1);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const f64x2 d = __builtin_bit_cast(f64x2, pv[k]);
            s0 += d[0];
            s1 += d[1];
        }
    }
    s0 = wave_sum_f64(s0);
    s1 = wave_sum_f64(s1);
    __syncthreads();
    if (tid % kWave == 0) {
        red[tid / kWave][0] = s0;
        red[tid / kWave][1] = s1;
    }
    __syncthreads();
    if (tid == 0) {
        double t0 = 0.0, t1 = 0.0;
        for (int w = 0; w < nwaves; ++w) {
            t0 += red[w][0];
            t1 += red[w][1];
        }
        a.losses[0] = (float)(t0 * a.al_scale);
        a.losses[1] = (float)(t1 * a.cs_scale);
    }
}

}  // namespace

namespace {

// Launch shape: the four-expert variant (16-byte accesses, a quarter of the threads)
// when chunks are at most 8 tokens, E % 4 == 0, the arrays are 16-byte aligned and
// there are still at least 64K threads; 64-thread workgroups when there are fewer
// than 64K threads, so that the workgroups spread over the CUs.
struct LossPlan {
    int maxl, vw, threads;
    uint32_t columns;
    int64_t blocks;
};
LossPlan loss_plan(int64_t B, int64_t S, int64_t E, int64_t L, bool aligned16)
{
    LossPlan pl;
    const int64_t Lc = L < S ? L : S, nc = (S + L - 1) / L, cols1 = B * nc * E;
    pl.maxl = Lc <= 8 ? 8 : (Lc <= 32 ? 32 : 0);
    pl.vw = (pl.maxl == 8 && E % 4 == 0 && aligned16 && cols1 >= 4 * 65536) ? 4 : 1;
    pl.columns = (uint32_t)(cols1 / pl.vw);
    pl.threads = pl.columns >= 65536 ? kLossThreads : kWave;
    const int64_t blocks = ((int64_t)pl.columns + pl.threads - 1) / pl.threads;
    pl.blocks = blocks < kLossMaxBlocks ? blocks : kLossMaxBlocks;
    return pl;
}

}  // namespace

int64_t sparsity_losses_blocks(int64_t B, int64_t S, int64_t E, int64_t L)
{
    // the most workgroups any launch shape of these sizes uses
    const int64_t nc = (S + L - 1) / L, cols1 = B * nc * E;
    const int64_t blocks = (cols1 + kWave - 1) / kWave;
    return blocks < kLossMaxBlocks ? blocks : kLossMaxBlocks;
}

size_t sparsity_losses_workspace_bytes(int64_t B, int64_t S, int64_t E, int64_t L)
{
    return kLossControlBytes + (size_t)sparsity_losses_blocks(B, S, E, L) * 2 * sizeof(double);
}

hipError_t launch_sparsity_losses(const float *p, int64_t B, int64_t S, int64_t E, float alpha,
                                  int64_t L, float lambda_al, float lambda_cs, float *losses,
                                  float *grad, void *ws, hipStream_t stream)
{
    const bool aligned16 = (reinterpret_cast<uintptr_t>(p) % 16 == 0) &&
                           (reinterpret_cast<uintptr_t>(grad) % 16 == 0);
    const LossPlan pl = loss_plan(B, S, E, L, aligned16);
    LossArgs a;
    a.p = p;
    a.grad = grad;
    a.B = (int)B;
    a.S = (int)S;
    a.E = (int)E;
    a.L = (int)(L < S ? L : S);
    a.nc = (int)((S + L - 1) / L);
    a.columns = pl.columns;
    a.alpha = alpha;
    const double den_al = (double)B * (double)E * (double)(S - 1 > 1 ? S - 1 : 1);
    const double den_cs = (double)B * (double)E * (double)a.nc;
    a.al_scale = 1.0 / den_al;
    a.cs_scale = 1.0 / den_cs;
    a.g_al = (float)(lambda_al / den_al);
    a.g_cs = (float)(lambda_cs / den_cs);
    a.arrive = static_cast<uint32_t *>(ws);
    a.part = reinterpret_cast<double *>(static_cast<char *>(ws) + kLossControlBytes);
    a.losses = losses;
    const dim3 grid((unsigned)pl.blocks), block((unsigned)pl.threads);
    if (pl.maxl == 8 && pl.vw == 4)
        hipLaunchKernelGGL((sparsity_losses_kernel<8, 4>), grid, block, 0, stream, a);
    else if (pl.maxl == 8)
        hipLaunchKernelGGL((sparsity_losses_kernel<8, 1>), grid, block, 0, stream, a);
    else if (pl.maxl == 32)
        hipLaunchKernelGGL((sparsity_losses_kernel<32, 1>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((sparsity_losses_kernel<0, 1>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace blockffn
