// Layer epilogue: residual + LayerNorm over the hidden axis (skill page, "Full
// BlockFFN Layer with Combined Losses": the layer's output is nn.LayerNorm(d_h)
// applied to the expert output plus the layer input).
//
//   v = y[t,:] + x[t,:],  mu = mean_j v_j,  var = mean_j (v_j - mu)^2   (biased)
//   out[t,j] = (v_j - mu) / sqrt(var + eps) * gamma[j] + beta[j]
//
// HBM-bound: each row is read once from y and x and written once. One wavefront owns
// a row; lane l holds the 16-byte vectors l, l + 64, ... of it in registers, so the
// two row reductions (mean, then the centred sum of squares, both DPP trees) cost no
// extra memory traffic. A workgroup of R rows stages gamma and beta in LDS once,
// while its rows' loads are in flight, instead of every wavefront reading them again
// after its reductions. Rows longer than the register window (64 lanes x 8 vectors)
// are read three times instead (sum, centred squares, output); the re-reads mostly
// hit L2.
#include "common.h"
#include "plan.h"
#include "sync.h"

namespace blockffn {
namespace {

constexpr int kLnMaxVec = 8;                 // register window: vectors per lane
constexpr int kLnMaxWaves = 16;              // rows per workgroup, at most

// Element access for the two dtypes: a "vector" is 16 bytes (8 bf16 or 4 float).
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
    static constexpr int W = 8;
    __device__ static void unpack(u32x4 u, float *v)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    __device__ static u32x4 pack(const float *v)
    {
        u32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
        return u;
    }
    __device__ static void load(const uint16_t *p, float *v)
    {
        const u32x4 u = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    __device__ static void store(uint16_t *p, const float *v)
    {
        u32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
        *reinterpret_cast<u32x4 *>(p) = u;
    }
};
template <> struct Vec<float> {
    static constexpr int W = 4;
    __device__ static void unpack(u32x4 u, float *v)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = __uint_as_float(u[i]);
    }
    __device__ static u32x4 pack(const float *v)
    {
        return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3])};
    }
    __device__ static void load(const float *p, float *v)
    {
        const float4 f = *reinterpret_cast<const float4 *>(p);
        v[0] = f.x, v[1] = f.y, v[2] = f.z, v[3] = f.w;
    }
    __device__ static void store(float *p, const float *v)
    {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

// out = (v - mu) * inv * gamma + beta for the W elements at j0. gamma and beta are
// 16-byte aligned (global or LDS) and j0 is a multiple of W, so they are read four
// floats at a time; NULL means 1 and 0.
template <typename T>
__device__ __forceinline__ void affine_store(T *o, const float *gamma, const float *beta,
                                             int j0, float *v, float mu, float inv)
{
    constexpr int W = Vec<T>::W;
#pragma unroll
    for (int q = 0; q < W; q += 4) {
        const float4 g = gamma ? *reinterpret_cast<const float4 *>(gamma + j0 + q)
                               : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        const float4 b = beta ? *reinterpret_cast<const float4 *>(beta + j0 + q)
                              : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        v[q] = fmaf((v[q] - mu) * inv, g.x, b.x);
        v[q + 1] = fmaf((v[q + 1] - mu) * inv, g.y, b.y);
        v[q + 2] = fmaf((v[q + 2] - mu) * inv, g.z, b.z);
        v[q + 3] = fmaf((v[q + 3] - mu) * inv, g.w, b.w);
    }
    Vec<T>::store(o, v);
}

// NV > 0: the row (d / W vectors, at most 64 * NV) stays in registers, and gamma and
// beta are staged in dynamic LDS: [gamma d floats][beta d floats] (1 and 0 if absent).
// NV == 0: any row length, three passes, gamma and beta read from global memory.
// d is a multiple of the vector width W. The workgroup holds blockDim.x / 64 rows.
// The early return of rows past the end is per wavefront, and only the NV == 0 path
// (which has no barrier) takes it before the staging barrier.
template <typename T, int NV>
__global__ void __launch_bounds__(kLnMaxWaves * kWave)
add_layernorm_kernel(const T *y, const T *x, const float *__restrict__ gamma,
                     const float *__restrict__ beta, float eps, int64_t rows, int d, T *out)
{
    constexpr int W = Vec<T>::W;
    extern __shared__ float4 ln_lds[];
    const int lane = threadIdx.x % kWave;
    const int waves = blockDim.x / kWave;
    // the wavefront's row, wave-uniform in a scalar register (buffer descriptors built
    // from it stay scalar)
    const int64_t row =
        (int64_t)blockIdx.x * waves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const bool live = row < rows;
    const int nvec = d / W;
    const T *yr = y + row * d;
    const T *xr = x + row * d;
    T *orow = out + row * d;
    const float rd = 1.0f / (float)d;

    if constexpr (NV > 0) {
        // Every load is unconditional: buffer loads over the row, where vectors past
        // its end (and every vector of a row past the last) read as zero, so all of a
        // row's loads are in flight before the first use.
        const uint32_t row_bytes = live ? (uint32_t)d * (uint32_t)sizeof(T) : 0u;
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(yr, row_bytes);
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xr, row_bytes);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(orow, row_bytes);
        u32x4 ya[NV], xa[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int off = (lane + k * kWave) * 16;
            ya[k] = __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, 0);
            xa[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
        }
        // stage gamma and beta (ones and zeros when absent) while the rows load
        float4 *sg = ln_lds;
        float4 *sb = ln_lds + d / 4;
        for (int j = threadIdx.x; j < d / 4; j += blockDim.x) {
            sg[j] = gamma ? reinterpret_cast<const float4 *>(gamma)[j]
                          : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            sb[j] = beta ? reinterpret_cast<const float4 *>(beta)[j]
                         : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        __syncthreads();
        if (!live)
            return;
        float v[NV][W];
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            float a[W], b[W];
            Vec<T>::unpack(ya[k], a);
            Vec<T>::unpack(xa[k], b);
#pragma unroll
            for (int i = 0; i < W; ++i) {
                v[k][i] = a[i] + b[i];
                sum += v[k][i];
            }
        }
        const float mu = wave_sum_f32(sum) * rd;
        float sq = 0.0f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const float valid = lane + k * kWave < nvec ? 1.0f : 0.0f;
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const float c = (v[k][i] - mu) * valid;
                sq = fmaf(c, c, sq);
            }
        }
        const float inv = 1.0f / sqrtf(wave_sum_f32(sq) * rd + eps);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            // vectors past the row end index LDS inside the 2 d floats (d >= W) and are
            // dropped by the store
            const int vi = lane + k * kWave;
            const int j = (vi < nvec ? vi : 0) * W;
            float o[W];
#pragma unroll
            for (int q = 0; q < W; q += 4) {
                const float4 g = sg[(j + q) / 4], bb = sb[(j + q) / 4];
                o[q] = fmaf((v[k][q] - mu) * inv, g.x, bb.x);
                o[q + 1] = fmaf((v[k][q + 1] - mu) * inv, g.y, bb.y);
                o[q + 2] = fmaf((v[k][q + 2] - mu) * inv, g.z, bb.z);
                o[q + 3] = fmaf((v[k][q + 3] - mu) * inv, g.w, bb.w);
            }
            __builtin_amdgcn_raw_buffer_store_b128(Vec<T>::pack(o), ro, vi * 16, 0, 0);
        }
    } else {
        if (!live)
            return;
        float sum = 0.0f;
        for (int vi = lane; vi < nvec; vi += kWave) {
            float a[W], b[W];
            Vec<T>::load(yr + vi * W, a);
            Vec<T>::load(xr + vi * W, b);
#pragma unroll
            for (int i = 0; i < W; ++i)
                sum += a[i] + b[i];
        }
        const float mu = wave_sum_f32(sum) * rd;
        float sq = 0.0f;
        for (int vi = lane; vi < nvec; vi += kWave) {
            float a[W], b[W];
            Vec<T>::load(yr + vi * W, a);
            Vec<T>::load(xr + vi * W, b);
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const float c = a[i] + b[i] - mu;
                sq = fmaf(c, c, sq);
            }
        }
        const float inv = 1.0f / sqrtf(wave_sum_f32(sq) * rd + eps);
        // In place (out == y or out == x) is safe: a lane reads its vector of both
        // inputs before it writes that vector, and no vector is read after it has
        // been written.
        for (int vi = lane; vi < nvec; vi += kWave) {
            float a[W], b[W];
            Vec<T>::load(yr + vi * W, a);
            Vec<T>::load(xr + vi * W, b);
#pragma unroll
            for (int i = 0; i < W; ++i)
                a[i] += b[i];
            affine_store(orow + vi * W, gamma, beta, vi * W, a, mu, inv);
        }
    }
}

// Rows per workgroup: enough workgroups to spread over the chip (about two per CU
// for large T), up to 16 rows sharing one staged copy of gamma and beta, and - on the
// register path - at least as many threads as gamma has float4s, so that staging is
// one load per thread, in flight together with the rows' loads.
int ln_rows_per_block(int64_t rows, int d, bool staged)
{
    int r = 1;
    while (r < kLnMaxWaves && rows >= (int64_t)r * 2 * 512)
        r *= 2;
    while (staged && r < kLnMaxWaves && r * kWave < d / 4)
        r *= 2;
    return r;
}

template <typename T>
hipError_t launch_ln(const T *y, const T *x, const float *gamma, const float *beta, float eps,
                     int64_t rows, int d, T *out, hipStream_t stream)
{
    const int nvec = d / Vec<T>::W;
    const int R = ln_rows_per_block(rows, d, nvec <= kLnMaxVec * kWave);
    const dim3 grid((unsigned)((rows + R - 1) / R)), block(R * kWave);
    const size_t lds = 2 * (size_t)d * sizeof(float);
#define LN_LAUNCH(NV, LDS)                                                                 \
    hipLaunchKernelGGL((add_layernorm_kernel<T, NV>), grid, block, LDS, stream, y, x,      \
                       gamma, beta, eps, rows, d, out)
    if (nvec <= kWave)
        LN_LAUNCH(1, lds);
    else if (nvec <= 2 * kWave)
        LN_LAUNCH(2, lds);
    else if (nvec <= 4 * kWave)
        LN_LAUNCH(4, lds);
    else if (nvec <= kLnMaxVec * kWave)
        LN_LAUNCH(kLnMaxVec, lds);
    else
        LN_LAUNCH(0, 0);
#undef LN_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_add_layernorm(int dtype_bf16, const void *y, const void *x, const float *gamma,
                                const float *beta, float eps, int64_t T, int64_t d_h, void *out,
                                hipStream_t stream)
{
    if (dtype_bf16)
        return launch_ln(static_cast<const uint16_t *>(y), static_cast<const uint16_t *>(x),
                         gamma, beta, eps, T, (int)d_h, static_cast<uint16_t *>(out), stream);
    return launch_ln(static_cast<const float *>(y), static_cast<const float *>(x), gamma, beta,
                     eps, T, (int)d_h, static_cast<float *>(out), stream);
}

}  // namespace blockffn
