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
//     hidden units (|U| * d_e of them, slot-major) are split into X contiguous ranges
//     of equal size (to 32 units), group g on XCD g, so the hidden rows a group
//     produces and consumes stay in that XCD's L2 and every CU streams the same share
//     of the weights whatever |U| mod X is.
//   * Every workgroup computes the union itself from the scores. The scores are
//     loaded first, then x (which does not depend on the union) with contiguous 1 KB
//     accesses, staged whole in LDS (XOR-swizzled 16-byte chunks, so the MFMA operand
//     reads are conflict-free). A CU's load pipe handles contiguous accesses several
//     times faster than the row-strided ones of MFMA operand layouts, and x is the
//     one operand every CU reads whole.
//   * Up: member k owns an even-sized piece of its group's range (up to 32 units per
//     pass, up to 3 passes for wide experts, at most 2 slots per pass) over the whole
//     of d_h, so no split-k partial ever leaves the workgroup. Wave w = (16-row half
//     rh, quarter kq of d_h): A = the W1 rows (16 x 32 k, straight from memory into
//     registers: 16 rows x 64 bytes per access), B = x from LDS, 16x16x32 MFMAs for
//     both 16-token halves; the 4 k quarters meet in LDS and are added in order, then
//     Swish and the score.
//   * Down: member k owns the 64 output columns [64k, 64k + 64) over its group's
//     range. The waves of the second row half issue their W2 share right after their
//     last W1 pass, so both halves of the weight stream are in flight at once, and
//     compute every down product: wave kq takes the 16-column quarter kq over all of
//     the range's 32-unit steps. After the group's barrier (per-member flags all P
//     members set once their hidden rows are in L2) the first-half waves copy the
//     group's hidden block into LDS (in chunks of 2048 units for the widest ranges)
//     and the down waves run their MFMAs from it.
//   * The X group tiles of an output tile come from different XCDs: they go to
//     memory with device-scope stores, and the last of the X to arrive (an atomic
//     counter) adds them in group order and writes y.
// Every wait is bounded: on time-out the affected outputs become NaN and the
// workspace's status word is set. Waits are on the
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
static_assert(kWaves == 8, "the fused router splits d_h into eighths, one per wave");
constexpr int kMaxXLoads = 16;       // 16-byte x chunks per thread: d_h <= 2048
constexpr int kMaxScoreLoads = 8;    // scores per thread (token tid/16, experts tid%16 + 16 i): E <= 128
constexpr int kMaxKSteps = 16;       // 32-wide k steps per up wave: d_h / 4 <= 512
constexpr int kGroupUnitsMax = 4096; // hidden units of the union per group (<= 128 32-unit steps)
constexpr int kHidChunk = 64;        // 32-unit steps of the hidden block in LDS at once (fills the x tile)
constexpr int kMaxRows = 96;         // W1 rows (hidden units) per member: up to three passes of 32
constexpr int kDnCols = 64;          // output columns per member
constexpr int kDnSlots = 24;         // W2 steps a down wave holds in registers at once
constexpr int kMaxWords = 4;
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kMaxDh = 2048;
constexpr int kDecodeMaxJT = kMaxDh / kDnCols;
constexpr int kMaxMembers = 64;
constexpr int kMaxLayerE = 64;       // fused router: experts (2 per member at most)
constexpr int kRedPitch = kTileM + 1;     // LDS pitch of the partials [part][row][token]
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset past every range: reads zero

struct DecodeArgs {
    const uint16_t *x;
    const float *scores;
    const uint16_t *w1;
    const uint16_t *w2;
    uint16_t *y;
    uint16_t *hidden;       // [X][gfrag] fragments of 1 KB (bf16)
    float *dn_part;         // [JT][X][32][64] fp32 group tiles
    uint32_t *flags;        // [X][P] per member: calls whose hidden rows it has stored
    uint32_t *rflags;       // [X][P] per member: calls whose router logits it has stored
    float *logits;          // [X][32 tokens][16][4] router logits (expert 16 i + j at [j][i]), one copy per group
    uint32_t *dn_arrive;    // [JT] group tiles stored per output tile
    uint32_t *status;       // the workspace's status word: set when a wait times out
    // fused epilogue (LN = true): ln_out = LayerNorm(bf16(y) + x) over d_h with ln_gamma,
    // ln_beta (NULL = 1, 0) and ln_eps; y itself is written only when y != NULL
    const float *ln_gamma, *ln_beta;
    float ln_eps;
    uint16_t *ln_out;
    uint32_t *ln_arrive;    // group tiles stored (all output tiles, all groups)
    uint32_t *ln_depart;    // row owners done reading them (the last resets both to zero)
    // router probabilities (ROUTER = true): probs_out [T][E] = sigmoid(sharpness * s)
    float sharpness;
    float *probs_out;
    uint64_t *masks_out;
    int32_t *lists_out;
    int32_t *counts_out;
    // fused router (ROUTER = true): W_r [E][d_h], optional gain/bias [E], eps; the
    // scores are written to scores_out [T][E] when it is given
    const uint16_t *w_r;
    const float *gain, *bias;
    float eps;
    float *scores_out;
    int T, d_h, E, d_e;
    int X, P;               // groups (XCDs), members per group
    int gfrag;              // hidden fragments per group: 2 per 32 units of the largest group range
    int JT;                 // d_h / 64 output tiles
};

struct Shared {
    alignas(16) uint64_t wmask[kMaxWords][kWaves];   // per-wave union bits, word-major
    int list[256];
    int flag;
    int rflag;
    int last;
    float s_col[2][kTileM];   // scores of the member's (at most 2) union slots
    // router partials [8 d_h eighths][2 experts][32 tokens], then the scores
    // [E][32 tokens]; up partials [4 k quarters][32 rows][32 tokens]; down partials
    // [2 step halves][64 columns][32 tokens]
    alignas(16) float red[2 * kDnCols * kRedPitch];
    alignas(16) uint16_t xs[kTileM * kMaxDh];   // x, 16-byte chunk c of token t at chunk c ^ (t & 15)
    // the member's (at most 2) W_r rows for the router products; after the router, the
    // chunk's scores [E][32 tokens] (fp32, the same bytes: kMaxLayerE * 32 * 4)
    alignas(16) uint16_t wr[2 * kMaxDh];
};

// Workgroup barrier that waits for this wave's LDS accesses only, not for its loads
// from memory still in flight (which __syncthreads would wait for).
__device__ __forceinline__ void lds_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt left alone
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Union of the experts active in the chunk, ascending list in LDS; returns |U| and
// leaves the mask words in wm. Thread tid holds in sv[i] the score of token tid / 16
// and expert tid % 16 + 16 i (zero past T and past E), so a wave covers 4 tokens:
// one ballot per i and an OR of its four 16-bit token groups give the wave's bits of
// experts 16 i .. 16 i + 15; the 8 waves meet in LDS.
__device__ int union_of_tile(const DecodeArgs &a, Shared &sh, const float (&sv)[kMaxScoreLoads],
                             uint64_t (&wm)[kMaxWords])
{
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w)
        wm[w] = 0;
#pragma unroll
    for (int i = 0; i < kMaxScoreLoads; ++i) {
        const uint64_t b = __ballot(sv[i] != 0.0f);
        const uint64_t m16 = (b | (b >> 16) | (b >> 32) | (b >> 48)) & 0xffffull;
        wm[i / 4] |= m16 << (16 * (i % 4));
    }
    if (lane < kMaxWords)
        sh.wmask[lane][wave] = wm[lane];
    __syncthreads();
    // word w of the 8 waves: 64 contiguous bytes, four 16-byte reads
    const int W = (a.E + 63) >> 6;
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w) {
        uint64_t m = 0;
        if (w < W) {
            typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int v = 0; v < kWaves; v += 2) {
                const u64x2 p = *reinterpret_cast<const u64x2 *>(&sh.wmask[w][v]);
                m |= p[0] | p[1];
            }
        }
        wm[w] = m;
        cnt += __popcll(m);
    }
    if (tid < a.E) {
        const int w = tid >> 6, bit = tid & 63;
        uint64_t word = 0;
        int pos = 0;
#pragma unroll
        for (int v = 0; v < kMaxWords; ++v) {
            if (v < w)
                pos += __popcll(wm[v]);
            if (v == w)
                word = wm[v];
        }
        if ((word >> bit) & 1ull)
            sh.list[pos + __popcll(word & ((1ull << bit) - 1ull))] = tid;
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

// Byte offset of the hidden value of local unit lu (of the group's range) and token t
// of group g. The block is kept in the order the down products read it: fragment
// (lu / 32, t / 16) of 1 KB holds, at lane kgrp*16 + t%16, the 8 units 8*kgrp .. +8 of
// its 32 (kgrp = (lu % 32) / 8), so each operand load of a down wave is one contiguous
// access.
__device__ __forceinline__ uint32_t hid_offset(int g, int gfrag, int lu, int t)
{
    const int frag = (lu >> 5) * 2 + (t >> 4);
    const int ln = ((lu & 31) >> 3) * 16 + (t & 15);
    return (uint32_t)((((g * gfrag + frag) * kWave + ln) * 8 + (lu & 7)) * 2);
}

// Residual + LayerNorm of the layer output fused into the final sum (skill page, "Full
// BlockFFN Layer with Combined Losses": the layer returns LayerNorm(output + x) over
// d_h). Once every member has stored its group tile (a device-scope arrival count over
// all JT x X of them), the owner of token row t adds up the row's X group partials over
// all d_h columns itself (thread -> 4 columns, the groups in order, as the per-tile sum
// does), rounds y to bf16 (as the unfused layer stores it), adds x, and normalises the
// row with its own exact two-pass mean and variance (wave sums, then the 8 waves in
// order through LDS): the statistics never leave the workgroup. y is written only when
// it is asked for.
__device__ void layernorm_row(const DecodeArgs &a, __amdgpu_buffer_rsrc_t rdnp, float *red, int t,
                              bool bad)
{
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int c = tid * 4;
    const bool act = c < a.d_h;
    const int jt = c / kDnCols, cc = c % kDnCols;
    float4 pv[kMaxGroups];
#pragma unroll
    for (int q = 0; q < kMaxGroups; ++q)
        if (q < a.X)
            pv[q] = bload_f4<kSC1>(rdnp, act ? (uint32_t)((((jt * a.X + q) * kTileM + t) * kDnCols + cc) * 4)
                                             : kOOB);
    uint2 xw = make_uint2(0u, 0u);
    if (act && t < a.T)
        xw = *reinterpret_cast<const uint2 *>(a.x + (int64_t)t * a.d_h + c);
    float4 sum = pv[0];
#pragma unroll
    for (int q = 1; q < kMaxGroups; ++q)
        if (q < a.X) {
            sum.x += pv[q].x;
            sum.y += pv[q].y;
            sum.z += pv[q].z;
            sum.w += pv[q].w;
        }
    const uint16_t yb[4] = {f32_to_bf16(sum.x), f32_to_bf16(sum.y), f32_to_bf16(sum.z),
                            f32_to_bf16(sum.w)};
    float v[4];
    v[0] = bf16_to_f32(yb[0]) + bf16_to_f32((uint16_t)(xw.x & 0xffffu));
    v[1] = bf16_to_f32(yb[1]) + bf16_to_f32((uint16_t)(xw.x >> 16));
    v[2] = bf16_to_f32(yb[2]) + bf16_to_f32((uint16_t)(xw.y & 0xffffu));
    v[3] = bf16_to_f32(yb[3]) + bf16_to_f32((uint16_t)(xw.y >> 16));
    // mean, then the squared deviations from it, over the row
    float ps = act ? (v[0] + v[1]) + (v[2] + v[3]) : 0.0f;
    ps = wave_sum_f32(ps);
    if (lane == 0)
        red[wave] = ps;
    lds_barrier();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
        tot += red[w];
    const float mean = tot / (float)a.d_h;
    float pd = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        pd = fmaf(v[i] - mean, v[i] - mean, pd);
    pd = wave_sum_f32(act ? pd : 0.0f);
    if (lane == 0)
        red[kWaves + wave] = pd;
    lds_barrier();
    float dev = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
        dev += red[kWaves + w];
    const float inv = 1.0f / sqrtf(dev / (float)a.d_h + a.ln_eps);
    if (act && t < a.T) {
        uint16_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float gm = a.ln_gamma ? a.ln_gamma[c + i] : 1.0f;
            const float bt = a.ln_beta ? a.ln_beta[c + i] : 0.0f;
            o[i] = f32_to_bf16(bad ? __builtin_nanf("") : (v[i] - mean) * inv * gm + bt);
        }
        *reinterpret_cast<uint64_t *>(a.ln_out + (int64_t)t * a.d_h + c) =
            (uint64_t)o[0] | ((uint64_t)o[1] << 16) | ((uint64_t)o[2] << 32) | ((uint64_t)o[3] << 48);
        if (a.y)
            *reinterpret_cast<uint64_t *>(a.y + (int64_t)t * a.d_h + c) =
                (uint64_t)yb[0] | ((uint64_t)yb[1] << 16) | ((uint64_t)yb[2] << 32) | ((uint64_t)yb[3] << 48);
    }
    lds_barrier();    // red is reused by the next row
}

// ROUTER = false: the scores are an input. ROUTER = true: the launch first computes
// the router for the chunk itself (skill page, "Architecture Overview" and "Router
// Architecture Setup": l = W_r x, s = RMSNorm_E(ReLU(l)) * gain), from the x every
// workgroup stages in LDS anyway. The logits are split over the P members of a group:
// member k takes experts [k*c, k*c + c), c = ceil(E / P) <= 2; wave w adds up the
// d_h eighth w (A = the member's W_r rows from memory, B = x from LDS, 16x16x32
// MFMA), the eighths meet in LDS in order, and the member's logits go to the group's
// copy in L2. After a second per-member flag barrier every workgroup reads the E x 32
// logits back and applies bias, ReLU, RMSNorm over the E experts and the gain itself
// (tokens past T get zero scores). The union and the score columns then come from LDS,
// and the separate router launch and the scores' round trip through memory disappear.
//
// PACKED = true: W1 and W2 are in the tiled layout blockffn_pack_weights writes (each
// matrix as 16 x 32 tiles of 1 KB, rows and columns in order), so a wave's operand
// load of 16 rows x 32 k is one contiguous 1 KB access (two runs when a piece's rows
// do not start on a tile) instead of 16 separate 64-byte pieces.
//
// WC (width class, for wide experts): 0 = pieces of at most 32 rows, group ranges of at
// most 2048 units (one pass, the hidden block in LDS at once); 1 = pieces of up to 64
// rows (a second pass); 2 = pieces of up to 96 rows and ranges of up to 4096 units (the
// hidden block in LDS chunks of 2048 units). The lower classes keep the shorter code.
template <bool ROUTER, bool PACKED, bool LN, int WC>
__global__ void __launch_bounds__(kThreads, 1) ffn_bf16_decode_kernel(DecodeArgs a)
{
    __shared__ Shared sh;
    static_assert(kMaxLayerE * kTileM * 4 <= (int)sizeof(sh.wr), "the scores fit the W_r rows' region");
    float *const scol_lds = reinterpret_cast<float *>(sh.wr);
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane & 15, kgrp = lane >> 4;
    const int g = blockIdx.x % a.X;      // group = XCD
    const int k = blockIdx.x / a.X;      // member within the group

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint64_t)a.T * a.d_h * 2);
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(a.w1, (uint64_t)a.E * a.d_e * a.d_h * 2);
    const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(a.w2, (uint64_t)a.E * a.d_h * a.d_e * 2);
    const __amdgpu_buffer_rsrc_t rhid =
        make_rsrc(a.hidden, (uint64_t)a.X * a.gfrag * 1024);
    const __amdgpu_buffer_rsrc_t rdnp =
        make_rsrc(a.dn_part, (uint64_t)a.JT * a.X * kTileM * kDnCols * 4);
    const __amdgpu_buffer_rsrc_t rflag = make_rsrc(a.flags, (uint64_t)a.X * a.P * 4);
    // this call's epoch: one more than the member's flag, which (like every flag of
    // the group) holds the number of calls so far
    const uint32_t epoch = 1u + ld_counter(&a.flags[g * a.P + k]);

    const int cpr = a.d_h / 8;
    const int nxl = kTileM * cpr / kThreads;
    // x goes to LDS without registers: LDS chunk slot q = i * 512 + tid (token q / cpr,
    // slot q % cpr) takes the chunk the swizzled order puts there, (q % cpr) ^ (token &
    // 15); tokens past T read as zero. The (token, slot) of q steps by 512 slots per
    // load without a division.
    auto stage_x = [&]() {
        const int dt = kThreads / cpr, dp = kThreads % cpr;
        int t = tid / cpr, p = tid % cpr;
#pragma unroll
        for (int i = 0; i < kMaxXLoads; ++i) {
            if (i < nxl)
                bload_lds16<0>(rx, &sh.xs[(i * kThreads + wave * kWave) * 8],
                               (uint32_t)((t * cpr + (p ^ (t & 15))) * 16));
            p += dp;
            t += dt;
            if (p >= cpr) {
                p -= cpr;
                ++t;
            }
        }
    };
    bf16x8 xv[kMaxXLoads];
    int cnt;
    uint64_t wm[kMaxWords];
    if constexpr (!ROUTER) {
        // Prologue loads, all unconditional (entries past a buffer's end read as zero) so
        // the compiler can wait for the scores alone: the union's scores first, then x.
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scores, (uint64_t)a.T * a.E * 4);
        float sv[kMaxScoreLoads];
        {
            const int tt = tid >> 4, sub = tid & 15;
#pragma unroll
            for (int i = 0; i < kMaxScoreLoads; ++i) {
                const int e = sub + 16 * i;
                sv[i] = bload_f1<0>(rs, tt < a.T && e < a.E ? (uint32_t)((tt * a.E + e) * 4) : kOOB);
            }
        }
        // x, contiguous, through registers (staged in LDS after the union: loads straight
        // into LDS would make the union's barriers wait for them): 16-byte chunk q = i *
        // 512 + tid of the 32 x d_h tile (token q / cpr, chunk q % cpr); tokens past T
        // read as zero.
#pragma unroll
        for (int i = 0; i < kMaxXLoads; ++i)
            xv[i] = bload<0>(rx, (uint32_t)((i * kThreads + tid) * 16));
        cnt = union_of_tile(a, sh, sv, wm);
    } else {
        // x (every member stages all of it for the up phase) and this member's share of
        // the router: experts e0 .. e0 + EPM (EPM = ceil(E / P) <= 2). Wave w takes the
        // d_h eighth [w * d_h / 8, +d_h / 8): A = the member's W_r rows (16-row block,
        // rows past EPM read zero) straight from memory, B = x from LDS, 16x16x32 MFMA.
        stage_x();
        const int EPM = (a.E + a.P - 1) / a.P;
        const int e0 = k * EPM;
        const int KS8 = a.d_h / 256;              // 32-wide k steps per eighth (<= 8)
        // the member's W_r rows, contiguous: thread -> one 16-byte chunk of the (at most
        // 2) rows, rows past E read zero; staged in LDS with x
        bf16x8 wrc;
        {
            const __amdgpu_buffer_rsrc_t rwr = make_rsrc(a.w_r, (uint64_t)a.E * a.d_h * 2);
            wrc = bload<0>(rwr, tid < EPM * cpr ? (uint32_t)((e0 * a.d_h + tid * 8) * 2) : kOOB);
        }
        // this thread's epilogue entries: token tt, experts sub + 16 i
        const int tt = tid >> 4, sub = tid & 15;
        float gv[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = sub + 16 * i;
            gv[i] = (a.gain && e < a.E) ? a.gain[e] : 1.0f;
            bv[i] = (a.bias && e < a.E) ? a.bias[e] : 0.0f;
        }
        const uint32_t repoch = 1u + ld_counter(&a.rflags[g * a.P + k]);
        if (tid < 2 * cpr)
            *reinterpret_cast<bf16x8 *>(&sh.wr[tid * 8]) = wrc;
        __syncthreads();
        float *part = sh.red;                     // [8 k eighths][2 experts][32 tokens]
        {
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            // branch-free, so that all the LDS reads go out before the first MFMA: steps
            // past KS8 (d_h < 2048) re-read the last step with a zero A operand
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int jc = j < KS8 ? j : KS8 - 1;
                const int c = (wave * (a.d_h / 8) + jc * 32) / 8 + kgrp;
                const bf16x8 b0 = *reinterpret_cast<const bf16x8 *>(&sh.xs[xs_chunk(l16, c, cpr) * 8]);
                const bf16x8 b1 = *reinterpret_cast<const bf16x8 *>(&sh.xs[xs_chunk(l16 + 16, c, cpr) * 8]);
                // A: rows 0 and 1 of the 16-row block are the member's W_r rows
                const bf16x8 wr = *reinterpret_cast<const bf16x8 *>(&sh.wr[(l16 & 1) * a.d_h + c * 8]);
                const bf16x8 wa_r = (l16 < 2 && j < KS8) ? wr : zero_bf16x8();
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa_r, b0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa_r, b1, acc1, 0, 0, 0);
            }
            // element i: row (expert) kgrp*4 + i, token l16 (+16); rows 0 and 1 are kept
            if (kgrp == 0) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    part[(wave * 2 + i) * kTileM + l16] = acc0[i];
                    part[(wave * 2 + i) * kTileM + l16 + 16] = acc1[i];
                }
            }
        }
        __syncthreads();
        // the group's logits in L2 as [token][e % 16][e / 16] (E <= 64): the 4 logits a
        // thread needs below are one 16-byte piece
        const __amdgpu_buffer_rsrc_t rlg = make_rsrc(a.logits, (uint64_t)a.X * kTileM * kMaxLayerE * 4);
        if (tid < 64) {
            const int el = tid >> 5, tok = tid & 31, e = e0 + el;
            float l = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                l += part[(q * 2 + el) * kTileM + tok];
            if (el < EPM && e < a.E)
                bstore_f1<kSC0>(rlg, (uint32_t)(((g * kTileM + tok) * kMaxLayerE + (e & 15) * 4 + (e >> 4)) * 4), l);
        }
        drain_memory();
        __syncthreads();
        // router barrier of the group: every member's logits are in the XCD's L2
        {
            const __amdgpu_buffer_rsrc_t rrf = make_rsrc(a.rflags, (uint64_t)a.X * a.P * 4);
            if (tid == 0)
                xcd_flag_store(rrf, (uint32_t)((g * a.P + k) * 4), repoch);
            if (wave == 0) {
                const uint32_t *flag = &a.rflags[g * a.P + (lane < a.P ? lane : 0)];
                uint32_t spins = 0;
                bool ready = false;
                while (!ready && spins < kSpinLimit) {
                    const uint32_t v = ld_counter(flag);
                    ready = __all(lane >= a.P || v == repoch);
                    if (!ready) {
                        ++spins;
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                if (lane == 0)
                    sh.rflag = !ready;
            }
        }
        __syncthreads();
        float sv[kMaxScoreLoads];
        {
            // this thread's 4 logits from L2, then bias, ReLU, RMSNorm over the E experts,
            // gain; the scores go to LDS [e][token] (pitch kRedPitch) and to sv for the
            // union; tokens past T get 0
            const float4 l4 = bload_f4<kSC0>(rlg, (uint32_t)(((g * kTileM + tt) * kMaxLayerE + sub * 4) * 4));
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            float rv[4], sumsq = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = sub + 16 * i;
                const float l = lv[i] + bv[i];
                rv[i] = (e < a.E && l > 0.0f) ? l : 0.0f;
                sumsq = fmaf(rv[i], rv[i], sumsq);
            }
            sumsq = row16_sum_f32(sumsq);     // the 16 threads of token tt
            const float inv = 1.0f / sqrtf(sumsq / (float)a.E + a.eps);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = sub + 16 * i;
                const float sc = tt < a.T && e < a.E ? rv[i] * inv * gv[i] : 0.0f;
                sv[i] = sc;
                if (e < a.E) {
                    scol_lds[e * kTileM + tt] = sc;
                    if (blockIdx.x == 0 && a.scores_out && tt < a.T)
                        a.scores_out[tt * a.E + e] = sc;
                    if (blockIdx.x == 0 && a.probs_out && tt < a.T)
                        a.probs_out[tt * a.E + e] = 1.0f / (1.0f + expf(-a.sharpness * sc));
                }
            }
#pragma unroll
            for (int i = 4; i < kMaxScoreLoads; ++i)
                sv[i] = 0.0f;
        }
        cnt = union_of_tile(a, sh, sv, wm);
    }

    if (blockIdx.x == 0) {
        const int W = (a.E + 63) >> 6;
        if (a.masks_out && tid < W) {
            uint64_t m = wm[0];
#pragma unroll
            for (int w = 1; w < kMaxWords; ++w)
                m = tid == w ? wm[w] : m;
            a.masks_out[tid] = m;
        }
        if (a.lists_out)
            for (int i = tid; i < a.E; i += kThreads)
                a.lists_out[i] = i < cnt ? sh.list[i] : -1;
        if (a.counts_out && tid == 0)
            a.counts_out[0] = cnt;
    }
    // The N = |U| * d_e hidden units of the union (slot-major) are split evenly: group
    // g takes the 32-unit-aligned range [G0, G1), member k of it the even-sized piece
    // [M0, M0 + nrows). A member's piece spans at most 2 slots (nrows <= 64 <= d_e).
    const int nblk = cnt * (a.d_e / 32);     // <= 1024 blocks: 32-bit products suffice
    const int G0 = 32 * (g * nblk / a.X);
    const int ng = 32 * ((g + 1) * nblk / a.X) - G0;
    const int M0 = G0 + 2 * (k * (ng / 2) / a.P);
    const int nrows = G0 + 2 * ((k + 1) * (ng / 2) / a.P) - M0;
    const int fs = M0 / a.d_e;              // the member's first slot
    const int fsu = (fs + 1) * a.d_e;       // first unit of the next slot

    // the member's score columns, zero past T: requested before W1 (so that scores given
    // as an input do not arrive behind W1) and put in LDS after the up products (by then
    // they have arrived; the Swish epilogue reads them after the next barrier)
    float scv = 0.0f;
    {
        const int j = (tid / kTileM) & 1, t = tid % kTileM;
        const bool ok = tid < 2 * kTileM && nrows > 0 && fs + j < cnt;
        const int e = sh.list[ok ? fs + j : 0];
        if constexpr (ROUTER) {
            if (ok)
                scv = scol_lds[e * kTileM + t];
        } else {
            // every thread issues the load (past T or outside the columns it reads zero),
            // so the loads that follow keep exact wait counts
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scores, (uint64_t)a.T * a.E * 4);
            scv = bload_f1<0>(rs, ok && t < a.T ? (uint32_t)((t * a.E + e) * 4) : kOOB);
        }
    }
    // W1 as the A operand (16 rows x 32 k): wave (row half rh, k quarter kq); lane
    // (row l16, k group kgrp) holds row rh*16 + l16 of the member's piece (unit
    // M0 + row of the union) at k = kq*d_h/4 + 32 ks + 8 kgrp .. +8.
    const int rh = wave & 1, kq = wave >> 1;
    const int KSU = a.d_h / 128;          // 32-wide k steps per quarter
    const int kq0 = kq * (a.d_h / 4);
    bf16x8 wa[kMaxKSteps];
    // rows [32 pass, 32 pass + 32) of the piece: a piece of more than 32 rows (large
    // unions of wide experts) takes a second pass
    auto issue_w1 = [&](int pass) {
        const int row = pass * 32 + rh * 16 + l16;
        const bool vr = row < nrows;
        const int gu = M0 + row;
        const int sl = fs + (gu >= fsu ? 1 : 0);
        const int e = vr ? sh.list[sl] : 0;
        const int unit = gu - sl * a.d_e;
        // element (unit u, k) of the expert's W1: row-major, or in the tiled layout
        // tile (u / 16, k / 32) of 16 x 32, row-major inside
        const uint32_t base =
            PACKED ? (uint32_t)((e * a.d_e * a.d_h + ((unit >> 4) * (a.d_h >> 5) + (kq0 >> 5)) * 512 +
                                 (unit & 15) * 32 + kgrp * 8) *
                                2)
                   : (uint32_t)(((e * a.d_e + unit) * a.d_h + kq0 + kgrp * 8) * 2);
        const uint32_t kstride = PACKED ? 1024u : 64u;
        // Only the lanes of rows inside the piece issue loads (lanes of absent rows are
        // switched off and keep zeros), so a block with a few rows costs the CU's load
        // path only those rows; steps past d_h read zero without touching memory.
#pragma unroll
        for (int ks = 0; ks < kMaxKSteps; ++ks)
            wa[ks] = zero_bf16x8();
        if (pass * 32 + rh * 16 < nrows && vr) {
#pragma unroll
            for (int ks = 0; ks < kMaxKSteps; ++ks)
                wa[ks] = bload<kNT>(rw1, ks < KSU ? base + ks * kstride : kOOB);
        }
    };
    issue_w1(0);

    // The waves split into two roles after the up products. The up waves of the first
    // row half (rh = 0: waves 0, 2, 4, 6) hold the piece's first 16 rows, which are
    // always full; they apply Swish and the score, store the hidden rows, take part in
    // the group barrier and copy the group's hidden block into LDS. The waves of the
    // second row half (rh = 1), whose rows are few or none whenever |U| * d_e is not
    // much more than 16 units per member, stream the member's whole W2 share right
    // after their own (short) up products and compute all the down products: wave kq
    // takes output-column quarter ct = kq over all of the group's 32-unit steps.
    // Vector memory completes in order per wave, so W2 in flight on the rh = 1 waves
    // never delays the hidden rows' drain or the barrier's polls on the rh = 0 waves.
    // Lane (column l16, k group kgrp) of a down wave holds
    // W2[e][64 jt + 16 ct + l16][u + 8 kgrp .. +8] for each step (slot e, first unit u;
    // a step never crosses a slot since 32 divides d_e).
    const int jt = k;
    const bool has_dn = jt < a.JT;
    const bool dn_wave = rh == 1;
    const int ct = kq;
    const int nst = ng / 32;                       // <= kGroupUnitsMax / 32 = 128
    const int n0 = nst < kDnSlots ? nst : kDnSlots;
    // lane i finds step i's (sbase) and step 64 + i's (sbase2) expert and first unit
    int sbase = 0, sbase2 = 0;
    {
        auto step_base = [&](int st) {
            const int gu = G0 + st * 32;
            const int sl = gu / a.d_e;
            const int unit = gu - sl * a.d_e;
            return sh.list[sl] * a.d_h * a.d_e + (PACKED ? (unit >> 5) * 512 : unit);
        };
        if (lane < nst)
            sbase = step_base(lane);
        if (WC == 2 && lane + 64 < nst)
            sbase2 = step_base(lane + 64);
    }
    // (wave-uniform st)
    auto step_off = [&](int st) {
        if constexpr (WC < 2)
            return __builtin_amdgcn_readlane(sbase, st);
        const int b1 = __builtin_amdgcn_readlane(sbase, st & 63);
        const int b2 = __builtin_amdgcn_readlane(sbase2, st & 63);
        return st < 64 ? b1 : b2;
    };
    // element (column j, unit u) of the expert's W2: row-major, or tile (j / 16, u / 32)
    // of the tiled layout (columns come in 16-aligned groups here)
    const int lo = PACKED ? ((jt * 4 + ct) * (a.d_e >> 5)) * 512 + l16 * 32 + kgrp * 8
                          : (jt * kDnCols + ct * 16 + l16) * a.d_e + kgrp * 8;

    if constexpr (!ROUTER) {
#pragma unroll
        for (int i = 0; i < kMaxXLoads; ++i)
            if (i < nxl) {
                const int q = i * kThreads + tid;
                *reinterpret_cast<bf16x8 *>(&sh.xs[xs_chunk(q / cpr, q % cpr, cpr) * 8]) = xv[i];
            }
    }

    // ---- up: pre-activations of the member's rows over this wave's k quarter.
    // B = x^T (32 k x 16 tokens): lane (token l16 (+16), k group kgrp).
    // x in LDS: staged from registers above when the scores are an input (the fused
    // router staged it long ago); the score columns are read only after the next barrier
    if constexpr (!ROUTER)
        lds_barrier();
    // a down wave is done with its W1: its W2 share (the first kDnSlots steps) follows
    bf16x8 wb[kDnSlots];
    auto issue_w2 = [&]() {
#pragma unroll
        for (int i = 0; i < kDnSlots; ++i) {
            wb[i] = zero_bf16x8();
            if (dn_wave && has_dn && i < n0)
                wb[i] = bload<kNT>(rw2, (uint32_t)((step_off(i) + lo) * 2));
        }
    };
    // The products of one 32-row block of the piece (rows [pb, pb + 32)) from the W1 in
    // wa, its k quarters added in order, Swish, score, bf16 hidden rows (rh = 0 waves).
    // Thread u -> (token tt, rows r0 .. r0 + 3 of the block as two pairs, each pair of
    // one slot: pieces start at even units and d_e is even).
    auto up_block = [&](int pb, bool last) {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
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
        if (pb == 0 && tid < 2 * kTileM)
            sh.s_col[tid / kTileM][tid % kTileM] = scv;
        if (last)
            issue_w2();
        // 16x16 accumulator layout: element i of a lane is row (lane/16)*4 + i of column
        // lane%16 (here: W1 row, token)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = rh * 16 + kgrp * 4 + i;
            sh.red[(kq * kTileM + row) * kRedPitch + l16] = acc0[i];
            sh.red[(kq * kTileM + row) * kRedPitch + l16 + 16] = acc1[i];
        }
        lds_barrier();
        if (!dn_wave) {
            const int u = (wave >> 1) * kWave + lane;
            const int tt = u >> 3, r0 = (u & 7) * 4;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const int r = r0 + 2 * pr;
                if (pb + r < nrows) {
                    const int j = M0 + pb + r >= fsu ? 1 : 0;
                    float h[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        float sum = 0.0f;
#pragma unroll
                        for (int p = 0; p < 4; ++p)
                            sum += sh.red[(p * kTileM + r + q) * kRedPitch + tt];
                        h[q] = swish_fast(sum) * sh.s_col[j][tt];
                    }
                    const uint32_t off = hid_offset(g, a.gfrag, M0 + pb + r - G0, tt);
                    const uint32_t packed = (uint32_t)f32_to_bf16(h[0]) | ((uint32_t)f32_to_bf16(h[1]) << 16);
                    __builtin_amdgcn_raw_buffer_store_b32(packed, rhid, (int)off, 0, kSC0);
                }
            }
            if (last)
                drain_memory();   // this wave's hidden rows are in the XCD's L2
        }
        lds_barrier();
    };
    // a piece of more than 32 rows (large unions of wide experts) takes passes over its
    // rows 0-31 (and 32-63), each followed by the W1 of the next 32 rows; the last pass
    // issues W2 as above
    int pb = 0;
    if constexpr (WC == 1) {
        if (nrows > 32) {
            up_block(0, false);
            issue_w1(1);
            pb = 32;
        }
    } else if constexpr (WC == 2) {
        while (nrows - pb > 32) {
            up_block(pb, false);
            issue_w1((pb >> 5) + 1);
            pb += 32;
        }
    }
    up_block(pb, true);

    // ---- group barrier: every member's hidden rows are in the XCD's L2. Each member
    // publishes the call's epoch in its own flag; the first wave (rh = 0) polls all P.
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
    lds_barrier();
    const bool timed_out = sh.flag != 0 || (ROUTER && sh.rflag != 0);
    if (timed_out && tid == 0)
        __hip_atomic_fetch_or(a.status, kStatusTimedOut, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!has_dn)
        return;

    // ---- down: B = the hidden rows (32 units x 16 tokens): lane (token l16 (+16),
    // k group kgrp) holds units 32 i + 8 kgrp .. +8 of the group's range for step i. In
    // the fragment order the group's block is ng / 16 fragments of 1 KB, each
    // lane-contiguous: the rh = 0 waves copy it into LDS over the x tile (which the up
    // products are done with) by loads that write LDS, up to 64 steps (128 KB) at a
    // time, and the four down waves read it from there.
    char *hs = reinterpret_cast<char *>(sh.xs);
    static_assert(kHidChunk * 2 * 1024 <= (int)sizeof(sh.xs), "a chunk of the hidden block fits the x tile");
    const uint32_t gb = (uint32_t)(g * a.gfrag) * 1024u;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (WC == 2) {
        // the group's steps in LDS chunks of kHidChunk (one chunk unless the group range
        // exceeds 2048 units)
        for (int c0 = 0; c0 < nst; c0 += kHidChunk) {
            const int cend = nst < c0 + kHidChunk ? nst : c0 + kHidChunk;
            if (c0 > 0)
                lds_barrier();   // the down waves are done with the previous chunk
            if (!dn_wave) {
                const int nfrag = (cend - c0) * 2;
    #pragma unroll
                for (int jj = 0; jj < kHidChunk * 2 / (kWaves / 2); ++jj) {
                    const int f = jj * (kWaves / 2) + (wave >> 1);
                    if (f < nfrag)
                        bload_lds16<kSC0>(rhid, hs + f * 1024, gb + (uint32_t)(2 * c0 + f) * 1024u + lane * 16u);
                }
                drain_memory();
            }
            lds_barrier();
            if (dn_wave) {
                for (int s0 = c0; s0 < cend; s0 += kDnSlots) {
                    // the first kDnSlots steps were requested with the up products; the
                    // steps past them (unions of more than about 3/4 of E) come here
                    if (s0 > 0) {
    #pragma unroll
                        for (int i = 0; i < kDnSlots; ++i) {
                            wb[i] = zero_bf16x8();
                            if (s0 + i < cend)
                                wb[i] = bload<kNT>(rw2, (uint32_t)((step_off(s0 + i) + lo) * 2));
                        }
                    }
    #pragma unroll
                    for (int i = 0; i < kDnSlots; ++i)
                        if (s0 + i < cend) {
                            const int f = (s0 + i - c0) * 2;
                            const bf16x8 h0 = *reinterpret_cast<const bf16x8 *>(hs + f * 1024 + lane * 16);
                            const bf16x8 h1 = *reinterpret_cast<const bf16x8 *>(hs + (f + 1) * 1024 + lane * 16);
                            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i], h0, acc0, 0, 0, 0);
                            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i], h1, acc1, 0, 0, 0);
                        }
                }
            }
        }
    } else {
        // the whole block at once (at most 2048 units)
        if (!dn_wave) {
            const int nfrag = nst * 2;
#pragma unroll
            for (int jj = 0; jj < kHidChunk * 2 / (kWaves / 2); ++jj) {
                const int f = jj * (kWaves / 2) + (wave >> 1);
                if (f < nfrag)
                    bload_lds16<kSC0>(rhid, hs + f * 1024, gb + (uint32_t)f * 1024u + lane * 16u);
            }
            drain_memory();
        }
        lds_barrier();
        if (dn_wave) {
#pragma unroll
            for (int i = 0; i < kDnSlots; ++i)
                if (i < n0) {
                    const bf16x8 h0 = *reinterpret_cast<const bf16x8 *>(hs + (i * 2) * 1024 + lane * 16);
                    const bf16x8 h1 = *reinterpret_cast<const bf16x8 *>(hs + (i * 2 + 1) * 1024 + lane * 16);
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i], h0, acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i], h1, acc1, 0, 0, 0);
                }
            // the steps past the first kDnSlots (unions of more than about 3/4 of E)
            for (int i0 = kDnSlots; i0 < nst; i0 += kDnSlots) {
#pragma unroll
                for (int i = 0; i < kDnSlots; ++i) {
                    wb[i] = zero_bf16x8();
                    if (i0 + i < nst)
                        wb[i] = bload<kNT>(rw2, (uint32_t)((step_off(i0 + i) + lo) * 2));
                }
#pragma unroll
                for (int i = 0; i < kDnSlots; ++i)
                    if (i0 + i < nst) {
                        const bf16x8 h0 =
                            *reinterpret_cast<const bf16x8 *>(hs + ((i0 + i) * 2) * 1024 + lane * 16);
                        const bf16x8 h1 =
                            *reinterpret_cast<const bf16x8 *>(hs + ((i0 + i) * 2 + 1) * 1024 + lane * 16);
                        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i], h0, acc0, 0, 0, 0);
                        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i], h1, acc1, 0, 0, 0);
                    }
            }
        }
    }
    if (dn_wave) {
        // group tile: element i of a lane is column ct*16 + kgrp*4 + i of token l16 (+16)
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            const f32x4 v = th ? acc1 : acc0;
            const float4 o = timed_out ? make_float4(__builtin_nanf(""), __builtin_nanf(""),
                                                     __builtin_nanf(""), __builtin_nanf(""))
                                       : make_float4(v[0], v[1], v[2], v[3]);
            bstore_f4<kSC1>(rdnp,
                            (uint32_t)((((jt * a.X + g) * kTileM + l16 + 16 * th) * kDnCols + ct * 16 +
                                        kgrp * 4) * 4),
                            o);
        }
    }
    drain_memory();
    __syncthreads();
    if constexpr (LN) {
        // every member's group tile, then the token rows: member mid = k * X + g owns rows
        // mid, mid + JT * X, ... (the first 32 members own one each at the decode shape)
        const int NM = a.JT * a.X, mid = k * a.X + g;
        const int owners = NM < kTileM ? NM : kTileM;
        if (tid == 0)
            add_counter(a.ln_arrive, 1u);
        if (mid >= kTileM)
            return;
        if (tid == 0) {
            uint32_t spins = 0;
            bool ready = false;
            while (!ready && spins < kSpinLimit) {
                ready = ld_counter(a.ln_arrive) >= (uint32_t)NM;
                if (!ready) {
                    ++spins;
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            sh.last = !ready;
            if (!ready)
                __hip_atomic_fetch_or(a.status, kStatusTimedOut, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const bool bad = timed_out || sh.last != 0;
        for (int t = mid; t < kTileM; t += NM)
            layernorm_row(a, rdnp, sh.red, t, bad);
        // this owner has read the tiles: the last of the owners returns both counters to zero
        if (tid == 0 && !bad) {
            const uint32_t prev = add_counter(a.ln_depart, 1u);
            if (prev == (uint32_t)(owners - 1)) {
                st_counter(a.ln_arrive, 0u);
                st_counter(a.ln_depart, 0u);
            }
        }
        return;
    }
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
    const int tt = tid >> 4, c0 = (tid & 15) * 4;
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
    const uint16_t yb[4] = {f32_to_bf16(sum.x), f32_to_bf16(sum.y), f32_to_bf16(sum.z),
                            f32_to_bf16(sum.w)};
    if (tt < a.T) {
        const uint64_t packed = (uint64_t)yb[0] | ((uint64_t)yb[1] << 16) | ((uint64_t)yb[2] << 32) |
                                ((uint64_t)yb[3] << 48);
        *reinterpret_cast<uint64_t *>(a.y + (int64_t)tt * a.d_h + jt * kDnCols + c0) = packed;
    }
}

// The tiled weight layout: a row-major R x C bf16 matrix as (R/16) x (C/32) tiles of
// 16 rows x 32 columns, tiles in row-major order, each tile row-major (1 KB). Thread
// -> one 16-byte piece of the output (8 columns of one tile row); the source piece is
// contiguous too. E matrices per launch, R % 16 == 0, C % 32 == 0.
__global__ void __launch_bounds__(256) pack_tiles_kernel(const uint16_t *__restrict__ src,
                                                          uint16_t *__restrict__ dst,
                                                          int64_t pieces, int R, int C)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= pieces)
        return;
    const int64_t per = (int64_t)R * C / 8;           // pieces per matrix
    const int64_t m = q / per;
    const int r8 = (int)(q - m * per);                // piece within the matrix
    const int tile = r8 >> 6, in = r8 & 63;           // 64 pieces per 16 x 32 tile
    const int tr = tile / (C >> 5), tc = tile - tr * (C >> 5);
    const int row = tr * 16 + (in >> 2), col = tc * 32 + (in & 3) * 8;
    const uint16_t *s = src + m * R * C + (int64_t)row * C + col;
    uint16_t *d = dst + m * R * C + (int64_t)r8 * 8;
    *reinterpret_cast<u32x4 *>(d) = *reinterpret_cast<const u32x4 *>(s);
}

}  // namespace

hipError_t launch_pack_weights(const uint16_t *w1, const uint16_t *w2, int64_t E, int64_t d_h,
                               int64_t d_e, uint16_t *packed, hipStream_t stream)
{
    const int64_t pieces = E * d_e * d_h / 8;
    const unsigned blocks = (unsigned)((pieces + 255) / 256);
    hipLaunchKernelGGL(pack_tiles_kernel, dim3(blocks), dim3(256), 0, stream, w1, packed, pieces,
                       (int)d_e, (int)d_h);
    hipLaunchKernelGGL(pack_tiles_kernel, dim3(blocks), dim3(256), 0, stream, w2,
                       packed + E * d_e * d_h, pieces, (int)d_h, (int)d_e);
    return hipGetLastError();
}

// Hidden units of the largest group range: every expert in the union, split over the
// xcds groups in 32-unit blocks.
static int64_t decode_group_units(int64_t E, int64_t d_e, int xcds)
{
    return 32 * ((E * (d_e / 32) + xcds - 1) / xcds);
}

bool decode_supported(int64_t CT, int64_t d_h, int64_t E, int64_t d_e, int xcds, int members)
{
    if (CT != 1 || xcds < 1 || xcds > kMaxGroups || members < 1 || members > kMaxMembers)
        return false;
    if (d_h % 128 != 0 || d_h > kMaxDh || d_h / kDnCols > members)
        return false;
    if (d_e % 32 != 0)
        return false;
    if (E * kTileM > kMaxScoreLoads * kThreads)
        return false;
    // the largest group range (all E experts in the union) and its largest member piece,
    // which must span at most two slots (rows <= d_e)
    const int64_t ng = decode_group_units(E, d_e, xcds);
    const int64_t rows = 2 * ((ng / 2 + members - 1) / members);
    return ng <= kGroupUnitsMax && rows <= kMaxRows && rows <= d_e;
}

size_t decode_scratch_bytes(int64_t d_h, int64_t E, int64_t d_e)
{
    // X groups of at most ceil(E d_e / 32 / X) 32-unit blocks: X * ng <= E d_e + 32 X
    const size_t hidden = (size_t)(E * d_e + 32 * kMaxGroups) * kTileM * 2;
    const size_t part = (size_t)(d_h / kDnCols) * kMaxGroups * kTileM * kDnCols * 4;
    const size_t logits = (size_t)kMaxGroups * kMaxLayerE * kTileM * 4;
    return align_up(hidden, 256) + align_up(part, 256) + logits;
}

template <bool ROUTER, bool PACKED, bool LN, int WC>
static int occupancy_of()
{
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, ffn_bf16_decode_kernel<ROUTER, PACKED, LN, WC>,
                                                     kThreads, 0) != hipSuccess)
        return 0;
    return occ;
}
template <bool ROUTER, bool PACKED, bool LN>
static int occupancy_min3()
{
    const int a = occupancy_of<ROUTER, PACKED, LN, 0>(), b = occupancy_of<ROUTER, PACKED, LN, 1>(),
              c = occupancy_of<ROUTER, PACKED, LN, 2>();
    return a < b ? (a < c ? a : c) : (b < c ? b : c);
}

int decode_blocks_per_cu()
{
    // every variant must fit one workgroup per CU
    const int occ[5] = {occupancy_min3<false, false, false>(), occupancy_min3<true, false, false>(),
                        occupancy_min3<true, true, false>(), occupancy_min3<true, false, true>(),
                        occupancy_min3<true, true, true>()};
    int m = occ[0];
    for (int i = 1; i < 5; ++i)
        m = occ[i] < m ? occ[i] : m;
    return m;
}

bool layer_decode_supported(int64_t E, int64_t d_h, int members)
{
    return E >= 1 && E <= kMaxLayerE && E <= 2 * (int64_t)members && d_h % 256 == 0 && d_h <= 2048;
}

namespace {

// The width class a launch needs: its worst-case piece rows and group range.
int decode_width(const FfnPlan &p, int xcds, int members)
{
    const int64_t ng = decode_group_units(p.E, p.d_e, xcds);
    const int64_t rows = 2 * ((ng / 2 + members - 1) / members);
    if (ng > (int64_t)kHidChunk * 32 || rows > 64)
        return 2;
    return rows > 32 ? 1 : 0;
}

DecodeArgs decode_args(const FfnPlan &p, int xcds, int members, const uint16_t *x,
                       const uint16_t *w1, const uint16_t *w2, uint16_t *y, void *ws)
{
    char *base = static_cast<char *>(ws);
    uint32_t *ctrl = reinterpret_cast<uint32_t *>(base) + kDecodeControlWord;
    DecodeArgs a{};
    a.x = x;
    a.w1 = w1;
    a.w2 = w2;
    a.y = y;
    a.hidden = reinterpret_cast<uint16_t *>(base + p.off_partials);
    const size_t hidden = align_up((size_t)(p.E * p.d_e + 32 * kMaxGroups) * kTileM * 2, 256);
    a.gfrag = (int)(2 * decode_group_units(p.E, p.d_e, xcds) / 32);
    a.dn_part = reinterpret_cast<float *>(base + p.off_partials + hidden);
    a.dn_arrive = ctrl;
    a.flags = ctrl + kDecodeMaxJT;
    a.rflags = a.flags + kMaxGroups * kMaxMembers;
    a.ln_arrive = a.rflags + kMaxGroups * kMaxMembers;
    a.ln_depart = a.ln_arrive + 1;
    static_assert(kDecodeMaxJT + 2 * kMaxGroups * kMaxMembers + 2 == kDecodeControlEnd - kDecodeControlWord,
                  "the control-block layout in plan.h");
    a.status = reinterpret_cast<uint32_t *>(base) + kStatusWord;
    const size_t part = align_up((size_t)(p.d_h / kDnCols) * kMaxGroups * kTileM * kDnCols * 4, 256);
    a.logits = reinterpret_cast<float *>(base + p.off_partials + hidden + part);
    a.T = (int)p.T;
    a.d_h = (int)p.d_h;
    a.E = (int)p.E;
    a.d_e = (int)p.d_e;
    a.X = xcds;
    a.P = members;
    a.JT = (int)(p.d_h / kDnCols);
    return a;
}

}  // namespace

hipError_t launch_ffn_bf16_decode(const FfnPlan &p, int xcds, int members, const uint16_t *x,
                                  const float *scores, const uint16_t *w1, const uint16_t *w2,
                                  uint16_t *y, void *ws, uint64_t *masks_out,
                                  int32_t *lists_out, int32_t *counts_out, hipStream_t stream)
{
    DecodeArgs a = decode_args(p, xcds, members, x, w1, w2, y, ws);
    a.scores = scores;
    a.masks_out = masks_out;
    a.lists_out = lists_out;
    a.counts_out = counts_out;
    const dim3 grid((unsigned)(xcds * members)), block(kThreads);
    switch (decode_width(p, xcds, members)) {
    case 0: hipLaunchKernelGGL((ffn_bf16_decode_kernel<false, false, false, 0>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((ffn_bf16_decode_kernel<false, false, false, 1>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((ffn_bf16_decode_kernel<false, false, false, 2>), grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_layer_bf16_decode(const FfnPlan &p, int xcds, int members, const uint16_t *x,
                                    const uint16_t *w_r, const float *gain, const float *bias,
                                    float eps, const uint16_t *w1, const uint16_t *w2,
                                    bool packed, uint16_t *y, float *scores_out, void *ws,
                                    const LayerEpilogue *ep, hipStream_t stream)
{
    DecodeArgs a = decode_args(p, xcds, members, x, w1, w2, y, ws);
    a.w_r = w_r;
    a.gain = gain;
    a.bias = bias;
    a.eps = eps;
    a.scores_out = scores_out;
    const bool ln = ep && ep->ln_out;
    if (ep) {
        a.ln_gamma = ep->ln_gamma;
        a.ln_beta = ep->ln_beta;
        a.ln_eps = ep->ln_eps;
        a.ln_out = ep->ln_out;
        a.sharpness = ep->sharpness;
        a.probs_out = ep->probs;
    }
    const dim3 grid((unsigned)(xcds * members)), block(kThreads);
    const int width = decode_width(p, xcds, members);
#define BLOCKFFN_LAYER_LAUNCH(PK, L)                                                                 \
    do {                                                                                           \
        if (width == 0)                                                                            \
            hipLaunchKernelGGL((ffn_bf16_decode_kernel<true, PK, L, 0>), grid, block, 0, stream, a);  \
        else if (width == 1)                                                                       \
            hipLaunchKernelGGL((ffn_bf16_decode_kernel<true, PK, L, 1>), grid, block, 0, stream, a);  \
        else                                                                                       \
            hipLaunchKernelGGL((ffn_bf16_decode_kernel<true, PK, L, 2>), grid, block, 0, stream, a);  \
    } while (0)
    if (packed && ln)
        BLOCKFFN_LAYER_LAUNCH(true, true);
    else if (packed)
        BLOCKFFN_LAYER_LAUNCH(true, false);
    else if (ln)
        BLOCKFFN_LAYER_LAUNCH(false, true);
    else
        BLOCKFFN_LAYER_LAUNCH(false, false);
#undef BLOCKFFN_LAYER_LAUNCH
    return hipGetLastError();
}

}  // namespace blockffn
