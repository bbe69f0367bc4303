// C ABI of the BlockFFN layer forward: argument validation, workspace layout and
// kernel launches. The declarations and their contracts are in include/blockffn.h.
//
// Nothing here touches the device before every argument has been checked, so an
// invalid call returns an error and enqueues nothing; this also lets the checks run
// on a machine without a GPU.
#include <cmath>
#include <mutex>
#include <string>

#include "../../include/blockffn.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

// Per-device facts some schedules depend on, found on first use (or by blockffn_init).
struct DeviceInfo {
    bool probed = false;
    int xcds = 0;          // XCDs, when round-robin workgroup placement was verified
    int cus = 0;           // compute units
};
constexpr int kMaxDevices = 64;
std::mutex g_device_mutex;
DeviceInfo g_devices[kMaxDevices];

// Probes the current device on `stream` (one small launch into a static device array,
// then a synchronisation of `stream`). Caller holds g_device_mutex.
hipError_t probe_device(int dev, hipStream_t stream, DeviceInfo &d)
{
    int nxcd = 0, cus = 0;
    bool round_robin = false;
    hipError_t err = hipDeviceGetAttribute(&nxcd, hipDeviceAttributeNumberOfXccs, dev);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess)
        return err;
    if (nxcd > 1 && nxcd <= blockffn::kMaxGroups && cus % nxcd == 0) {
        err = blockffn::probe_xcd_placement(nxcd, stream, &round_robin);
        if (err != hipSuccess)
            return err;
        if (round_robin) {
            d.xcds = nxcd;
            d.cus = cus;
        }
    }
    d.probed = true;
    return hipSuccess;
}

// The allocation-free entry point's scratch: one file-scope device array (each device
// holds its own copy until the process ends). Host code uses only the per-device
// address hipGetSymbolAddress returns for it, never the array's name. It starts
// zero-filled (a static device array), which is the state the workspace protocol needs.
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
void *g_scratch_ptr[kMaxDevices];

// Resolves `scratch` on device `dev` (which must be current); once per device. Caller
// holds g_device_mutex.
hipError_t noalloc_scratch_init(int dev)
{
    if (g_scratch_ptr[dev])
        return hipSuccess;
    void *p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err == hipSuccess)
        g_scratch_ptr[dev] = p;
    return err;
}

// Before each allocation-free call: if an earlier call's bounded wait timed out (status
// word set), the control block's flags are inconsistent, so it is zero-filled again
// (counters, flags and status word). One workgroup; the word is read before any thread
// writes.
__global__ void __launch_bounds__(1024) scratch_recover_kernel(uint32_t *control)
{
    const uint32_t status = __hip_atomic_load(control + blockffn::kStatusWord, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (status == 0)
        return;
    for (int i = threadIdx.x; i < (int)blockffn::kControlWords; i += blockDim.x)
        control[i] = 0u;
}

// Number of XCDs X of the current device if workgroup b of a launch is verified to
// run on XCD b % X, else 0. The first call on a device probes it on the caller's
// stream (see probe_device) unless blockffn_init did; the probe synchronises, so it
// is skipped (and retried on a later call) while the stream is being captured into a
// graph, and the call answers 0 meanwhile.
const DeviceInfo *device_info(hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_device_mutex);
    DeviceInfo &d = g_devices[dev];
    if (!d.probed) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess ||
            cs != hipStreamCaptureStatusNone)
            return nullptr;
        (void)probe_device(dev, stream, d);
    }
    return &d;
}

int placement_xcds(hipStream_t stream)
{
    const DeviceInfo *d = device_info(stream);
    return d ? d->xcds : 0;
}

// The one-launch schedule's grid on the current device: fills *xcds and *wg_per_xcd
// and returns true when it may be used (verified placement, enough resident
// workgroups).
bool chunk1_grid(hipStream_t stream, int *xcds, int *wg_per_xcd)
{
    const DeviceInfo *d = device_info(stream);
    if (!d || d->xcds <= 1)
        return false;
    const int per_cu = blockffn::chunk1_blocks_per_cu();
    if (per_cu < 1)
        return false;
    *xcds = d->xcds;
    *wg_per_xcd = (per_cu >= 2 ? 2 : 1) * (d->cus / d->xcds);
    return true;
}

// The decode schedule's grid: xcds groups of `members` workgroups (one per CU).
bool decode_grid(hipStream_t stream, const blockffn::FfnPlan &p, int *xcds, int *members)
{
    const DeviceInfo *d = device_info(stream);
    if (!d || d->xcds <= 1 || blockffn::decode_blocks_per_cu() < 1)
        return false;
    const int m = d->cus / d->xcds;
    if (!blockffn::decode_supported(p.CT, p.d_h, p.E, p.d_e, d->xcds, m))
        return false;
    *xcds = d->xcds;
    *members = m;
    return true;
}

blockffn_status_t fail(blockffn_status_t code, const std::string &msg)
{
    g_last_error = msg;
    return code;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

blockffn_status_t check_dtype(int dtype)
{
    if (dtype != BLOCKFFN_F32 && dtype != BLOCKFFN_BF16)
        return fail(BLOCKFFN_EINVAL, "dtype must be BLOCKFFN_F32 (0) or BLOCKFFN_BF16 (1), got " +
                                         std::to_string(dtype));
    return BLOCKFFN_OK;
}

// Sizes shared by both calls.
blockffn_status_t check_sizes(int64_t T, int64_t d_h, int64_t E, int dtype)
{
    if (T <= 0 || d_h <= 0 || E <= 0)
        return fail(BLOCKFFN_EINVAL, "T, d_h and E must be positive (T=" + std::to_string(T) +
                                         ", d_h=" + std::to_string(d_h) +
                                         ", E=" + std::to_string(E) + ")");
    if (E > 256)
        return fail(BLOCKFFN_EUNSUPPORTED,
                    "E=" + std::to_string(E) + " experts: at most 256 are supported");
    if (T > (int64_t)1 << 30 || d_h > (int64_t)1 << 20)
        return fail(BLOCKFFN_EUNSUPPORTED, "T or d_h too large");
    if (dtype == BLOCKFFN_BF16 && d_h % 32 != 0)
        return fail(BLOCKFFN_EUNSUPPORTED,
                    "bf16 needs d_h % 32 == 0, got d_h=" + std::to_string(d_h));
    return BLOCKFFN_OK;
}

blockffn_status_t check_ffn_sizes(int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                  int64_t n, int dtype)
{
    blockffn_status_t st = check_dtype(dtype);
    if (st != BLOCKFFN_OK)
        return st;
    if ((st = check_sizes(T, d_h, E, dtype)) != BLOCKFFN_OK)
        return st;
    if (d_e <= 0 || n <= 0)
        return fail(BLOCKFFN_EINVAL, "d_e and n must be positive (d_e=" + std::to_string(d_e) +
                                         ", n=" + std::to_string(n) + ")");
    if (d_e > 65536)
        return fail(BLOCKFFN_EUNSUPPORTED, "d_e too large");
    if (dtype == BLOCKFFN_BF16 && d_e % 16 != 0)
        return fail(BLOCKFFN_EUNSUPPORTED,
                    "bf16 needs d_e % 16 == 0, got d_e=" + std::to_string(d_e));
    // Grid sizes of the widest launch must fit a 32-bit grid dimension.
    const blockffn::FfnPlan p = blockffn::make_plan(T, d_h, E, d_e, n, dtype);
    if (p.CT * p.E * (d_e / 16 + 1) * 2 >= ((int64_t)1 << 31) ||
        p.CT * p.JT >= ((int64_t)1 << 31))
        return fail(BLOCKFFN_EUNSUPPORTED, "problem too large for one launch");
    return BLOCKFFN_OK;
}

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

blockffn_status_t check_loss_sizes(int64_t B, int64_t S, int64_t E, int64_t L)
{
    if (B <= 0 || S <= 0 || E <= 0 || L <= 0)
        return fail(BLOCKFFN_EINVAL, "B, S, E and L must be positive (B=" + std::to_string(B) +
                                         ", S=" + std::to_string(S) + ", E=" +
                                         std::to_string(E) + ", L=" + std::to_string(L) + ")");
    if (S > ((int64_t)1 << 30) || E > ((int64_t)1 << 20) || B > ((int64_t)1 << 30) ||
        (double)B * (double)S * (double)E >= 2147483648.0)
        return fail(BLOCKFFN_EUNSUPPORTED, "B * S * E must stay below 2^31");
    return BLOCKFFN_OK;
}

}  // namespace

extern "C" {

const char *blockffn_last_error(void) { return g_last_error.c_str(); }

const char *blockffn_version(void) { return "blockffn-gfx950 0.2.0"; }

blockffn_status_t blockffn_init(void *stream)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("no current device: ") + hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(BLOCKFFN_EUNSUPPORTED, "device index beyond the library's table");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return fail(BLOCKFFN_EINVAL, "blockffn_init synchronises its stream: call it outside "
                                     "graph capture");
    {
        std::lock_guard<std::mutex> lock(g_device_mutex);
        DeviceInfo &d = g_devices[dev];
        if (!d.probed && (err = probe_device(dev, s, d)) != hipSuccess)
            return fail(BLOCKFFN_EHIP, std::string("placement probe failed: ") +
                                           hipGetErrorString(err));
        if ((err = noalloc_scratch_init(dev)) != hipSuccess)
            return fail(BLOCKFFN_EHIP, std::string("scratch array address: ") +
                                           hipGetErrorString(err));
    }
    g_last_error.clear();
    return BLOCKFFN_OK;
}

blockffn_status_t blockffn_workspace_check(const void *workspace, size_t workspace_bytes,
                                           void *stream)
{
    if (!workspace)
        return fail(BLOCKFFN_EINVAL, "workspace must not be NULL");
    if (!aligned(workspace, 256))
        return fail(BLOCKFFN_EUNSUPPORTED, "workspace needs 256-byte alignment");
    if (workspace_bytes < blockffn::kControlBytes)
        return fail(BLOCKFFN_EWORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                             " bytes, less than its control block (" +
                                             std::to_string(blockffn::kControlBytes) + ")");
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t word = 0;
    const uint32_t *src = static_cast<const uint32_t *>(workspace) + blockffn::kStatusWord;
    hipError_t err = hipMemcpyAsync(&word, src, sizeof(word), hipMemcpyDeviceToHost, s);
    if (err == hipSuccess)
        err = hipStreamSynchronize(s);
    if (err != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("reading the status word: ") + hipGetErrorString(err));
    if (word != 0)
        return fail(BLOCKFFN_ETIMEOUT,
                    "a kernel that used this workspace timed out waiting for other workgroups "
                    "(its outputs are NaN); zero-fill the workspace before using it again");
    g_last_error.clear();
    return BLOCKFFN_OK;
}

size_t blockffn_router_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int dtype)
{
    if (check_dtype(dtype) != BLOCKFFN_OK || check_sizes(T, d_h, E, dtype) != BLOCKFFN_OK)
        return 0;
    const size_t need = dtype == BLOCKFFN_BF16 ? blockffn::router_workspace_bytes(T, d_h, E) : 0;
    return need > 256 ? need : 256;
}

blockffn_status_t blockffn_router(const void *x, const void *w_r, const float *gain,
                                  const float *bias, float eps, int64_t T, int64_t d_h,
                                  int64_t E, int dtype, float *scores, float *logits,
                                  float sharpness, float *probs, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    blockffn_status_t st = check_dtype(dtype);
    if (st != BLOCKFFN_OK)
        return st;
    if (!x || !w_r || !scores)
        return fail(BLOCKFFN_EINVAL, "x, w_r and scores must not be NULL");
    if ((st = check_sizes(T, d_h, E, dtype)) != BLOCKFFN_OK)
        return st;
    if (!(eps >= 0.0f))
        return fail(BLOCKFFN_EINVAL, "eps must be >= 0");
    const size_t ea = dtype == BLOCKFFN_BF16 ? 16 : 4;
    if (!aligned(x, ea) || !aligned(w_r, ea))
        return fail(BLOCKFFN_EUNSUPPORTED, "x and w_r must be " + std::to_string(ea) +
                                               "-byte aligned");
    if (probs && !std::isfinite(sharpness))
        return fail(BLOCKFFN_EINVAL, "sharpness must be finite");
    if (!aligned(scores, 4) || (logits && !aligned(logits, 4)) || (gain && !aligned(gain, 4)) ||
        (bias && !aligned(bias, 4)) || (probs && !aligned(probs, 4)))
        return fail(BLOCKFFN_EUNSUPPORTED, "float arrays must be 4-byte aligned");
    if (workspace) {
        if (!aligned(workspace, 256))
            return fail(BLOCKFFN_EUNSUPPORTED, "workspace needs 256-byte alignment");
        const size_t need = blockffn_router_workspace_bytes(T, d_h, E, dtype);
        if (workspace_bytes < need)
            return fail(BLOCKFFN_EWORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                                 " bytes, needs " + std::to_string(need));
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (dtype == BLOCKFFN_BF16)
        err = blockffn::launch_router_bf16(static_cast<const uint16_t *>(x),
                                           static_cast<const uint16_t *>(w_r), gain, bias, eps,
                                           T, d_h, E, scores, logits, sharpness, probs,
                                           workspace,
                                           workspace ? placement_xcds(s) : 0, s);
    else
        err = blockffn::launch_router_f32(static_cast<const float *>(x),
                                          static_cast<const float *>(w_r), gain, bias, eps, T,
                                          d_h, E, scores, logits, sharpness, probs, s);
    if (err != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("router launch failed: ") + hipGetErrorString(err));
    g_last_error.clear();
    return BLOCKFFN_OK;
}

size_t blockffn_chunk_ffn_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                          int64_t n, int dtype)
{
    if (check_ffn_sizes(T, d_h, E, d_e, n, dtype) != BLOCKFFN_OK)
        return 0;
    return blockffn::make_plan(T, d_h, E, d_e, n, dtype).total_bytes;
}

blockffn_status_t blockffn_chunk_ffn(const void *x, const float *scores, const void *w1,
                                     const void *w2, int64_t T, int64_t d_h, int64_t E,
                                     int64_t d_e, int64_t n, int dtype, void *y,
                                     void *workspace, size_t workspace_bytes,
                                     uint64_t *union_masks_out, int32_t *expert_lists_out,
                                     int32_t *union_counts_out, void *stream)
{
    if (!x || !scores || !w1 || !w2 || !y || !workspace)
        return fail(BLOCKFFN_EINVAL, "x, scores, w1, w2, y and workspace must not be NULL");
    blockffn_status_t st = check_ffn_sizes(T, d_h, E, d_e, n, dtype);
    if (st != BLOCKFFN_OK)
        return st;
    const size_t ea = dtype == BLOCKFFN_BF16 ? 16 : 4;
    if (!aligned(x, ea) || !aligned(w1, ea) || !aligned(w2, ea) || !aligned(y, ea))
        return fail(BLOCKFFN_EUNSUPPORTED, "x, w1, w2 and y must be " + std::to_string(ea) +
                                               "-byte aligned");
    if (!aligned(scores, 4) || !aligned(workspace, 256) ||
        (union_masks_out && !aligned(union_masks_out, 8)) ||
        (expert_lists_out && !aligned(expert_lists_out, 4)) ||
        (union_counts_out && !aligned(union_counts_out, 4)))
        return fail(BLOCKFFN_EUNSUPPORTED,
                    "scores/lists/counts need 4-byte, masks 8-byte, workspace 256-byte alignment");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t needed = blockffn::make_plan(T, d_h, E, d_e, n, dtype).total_bytes;
    if (workspace_bytes < needed)
        return fail(BLOCKFFN_EWORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                             " bytes, needs " + std::to_string(needed));
    const blockffn::FfnPlan p = blockffn::make_plan(T, d_h, E, d_e, n, dtype);

    hipError_t err;
    int xcds = 0, wg_per_xcd = 0, members = 0;
    if (p.decode && decode_grid(s, p, &xcds, &members)) {
        // one launch, one workgroup per CU: union, up- and down-projection
        err = blockffn::launch_ffn_bf16_decode(
            p, xcds, members, static_cast<const uint16_t *>(x), scores,
            static_cast<const uint16_t *>(w1), static_cast<const uint16_t *>(w2),
            static_cast<uint16_t *>(y), workspace, union_masks_out, expert_lists_out,
            union_counts_out, s);
    } else if (dtype == BLOCKFFN_BF16 && p.chunk1 && chunk1_grid(s, &xcds, &wg_per_xcd)) {
        // one launch: union, up- and down-projection of a single chunk tile
        err = blockffn::launch_ffn_bf16_chunk1(
            p, xcds, wg_per_xcd, static_cast<const uint16_t *>(x), scores,
            static_cast<const uint16_t *>(w1), static_cast<const uint16_t *>(w2),
            static_cast<uint16_t *>(y), workspace, union_masks_out, expert_lists_out,
            union_counts_out, s);
    } else if (p.grouped) {
        // several chunk tiles: each union expert's weights read once per launch
        err = blockffn::launch_ffn_bf16_grouped(
            p, static_cast<const uint16_t *>(x), scores, static_cast<const uint16_t *>(w1),
            static_cast<const uint16_t *>(w2), static_cast<uint16_t *>(y), workspace,
            union_masks_out, expert_lists_out, union_counts_out, s);
    } else if (dtype == BLOCKFFN_BF16) {
        err = blockffn::launch_ffn_bf16(p, static_cast<const uint16_t *>(x), scores,
                                        static_cast<const uint16_t *>(w1),
                                        static_cast<const uint16_t *>(w2),
                                        static_cast<uint16_t *>(y), workspace, union_masks_out,
                                        expert_lists_out, union_counts_out, s);
    } else {
        err = blockffn::launch_union(p, scores, workspace, union_masks_out, expert_lists_out,
                                     union_counts_out, s);
        if (err == hipSuccess)
            err = blockffn::launch_ffn_f32(p, static_cast<const float *>(x), scores,
                                           static_cast<const float *>(w1),
                                           static_cast<const float *>(w2),
                                           static_cast<float *>(y), workspace, s);
    }
    if (err != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("chunk FFN launch failed: ") + hipGetErrorString(err));
    g_last_error.clear();
    return BLOCKFFN_OK;
}

blockffn_status_t blockffn_add_layernorm(const void *y, const void *x, const float *gamma,
                                         const float *beta, float eps, int64_t T, int64_t d_h,
                                         int dtype, void *out, void *stream)
{
    blockffn_status_t st = check_dtype(dtype);
    if (st != BLOCKFFN_OK)
        return st;
    if (!y || !x || !out)
        return fail(BLOCKFFN_EINVAL, "y, x and out must not be NULL");
    if (T <= 0 || d_h <= 0)
        return fail(BLOCKFFN_EINVAL, "T and d_h must be positive (T=" + std::to_string(T) +
                                         ", d_h=" + std::to_string(d_h) + ")");
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return fail(BLOCKFFN_EINVAL, "eps must be finite and >= 0");
    const int64_t vec = dtype == BLOCKFFN_BF16 ? 8 : 4;
    if (d_h % vec != 0 || d_h > ((int64_t)1 << 20) || T > ((int64_t)1 << 31) - 4)
        return fail(BLOCKFFN_EUNSUPPORTED, "d_h must be a multiple of " + std::to_string(vec) +
                                               " and at most 2^20, T below 2^31");
    if (!aligned(y, 16) || !aligned(x, 16) || !aligned(out, 16) ||
        (gamma && !aligned(gamma, 16)) || (beta && !aligned(beta, 16)))
        return fail(BLOCKFFN_EUNSUPPORTED, "y, x, out, gamma and beta must be 16-byte aligned");
    const size_t bytes = (size_t)T * (size_t)d_h * (dtype == BLOCKFFN_BF16 ? 2 : 4);
    if ((out != y && overlap(out, bytes, y, bytes)) || (out != x && overlap(out, bytes, x, bytes)))
        return fail(BLOCKFFN_EINVAL, "out must be y, x, or not overlap them");
    const hipError_t err = blockffn::launch_add_layernorm(
        dtype == BLOCKFFN_BF16, y, x, gamma, beta, eps, T, d_h, out,
        static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("layernorm launch failed: ") + hipGetErrorString(err));
    g_last_error.clear();
    return BLOCKFFN_OK;
}

size_t blockffn_sparsity_losses_workspace_bytes(int64_t B, int64_t S, int64_t E, int64_t L)
{
    if (check_loss_sizes(B, S, E, L) != BLOCKFFN_OK)
        return 0;
    return blockffn::sparsity_losses_workspace_bytes(B, S, E, L);
}

blockffn_status_t blockffn_sparsity_losses(const float *probs, int64_t B, int64_t S, int64_t E,
                                           float alpha, int64_t L, float lambda_al,
                                           float lambda_cs, float *losses, float *grad,
                                           void *workspace, size_t workspace_bytes, void *stream)
{
    if (!probs || !losses || !workspace)
        return fail(BLOCKFFN_EINVAL, "probs, losses and workspace must not be NULL");
    blockffn_status_t st = check_loss_sizes(B, S, E, L);
    if (st != BLOCKFFN_OK)
        return st;
    if (!std::isfinite(alpha) || !std::isfinite(lambda_al) || !std::isfinite(lambda_cs))
        return fail(BLOCKFFN_EINVAL, "alpha, lambda_al and lambda_cs must be finite");
    if (!aligned(probs, 4) || !aligned(losses, 4) || (grad && !aligned(grad, 4)))
        return fail(BLOCKFFN_EUNSUPPORTED, "probs, losses and grad must be 4-byte aligned");
    if (!aligned(workspace, 256))
        return fail(BLOCKFFN_EUNSUPPORTED, "workspace needs 256-byte alignment");
    const size_t need = blockffn::sparsity_losses_workspace_bytes(B, S, E, L);
    if (workspace_bytes < need)
        return fail(BLOCKFFN_EWORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                             " bytes, needs " + std::to_string(need));
    const size_t pbytes = (size_t)B * S * E * sizeof(float);
    if ((grad && overlap(grad, pbytes, probs, pbytes)) ||
        overlap(losses, 2 * sizeof(float), probs, pbytes) ||
        (grad && overlap(losses, 2 * sizeof(float), grad, pbytes)) ||
        overlap(workspace, need, probs, pbytes) || overlap(workspace, need, losses, 8) ||
        (grad && overlap(workspace, need, grad, pbytes)))
        return fail(BLOCKFFN_EINVAL, "probs, grad, losses and workspace must not overlap");
    const hipError_t err = blockffn::launch_sparsity_losses(
        probs, B, S, E, alpha, L, lambda_al, lambda_cs, losses, grad, workspace,
        static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("loss launch failed: ") + hipGetErrorString(err));
    g_last_error.clear();
    return BLOCKFFN_OK;
}

size_t blockffn_layer_backward_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                               int64_t n, int dtype)
{
    if (check_dtype(dtype) != BLOCKFFN_OK)
        return 0;
    if (dtype != BLOCKFFN_BF16) {
        fail(BLOCKFFN_EUNSUPPORTED, "the layer backward takes bf16 inputs only");
        return 0;
    }
    if (!blockffn::backward_supported(T, d_h, E, d_e, n)) {
        fail(BLOCKFFN_EUNSUPPORTED, "layer backward needs T, n >= 1, 1 <= E <= 256, "
                                    "d_h % 256 == 0 and d_e % 128 == 0 (and 32-bit offsets)");
        return 0;
    }
    return blockffn::backward_workspace_bytes(T, d_h, E, d_e, n);
}

blockffn_status_t blockffn_layer_backward(const void *x, const void *w_r, const float *gain,
                                          const float *bias, float eps, const void *w1,
                                          const void *w2, int64_t T, int64_t d_h, int64_t E,
                                          int64_t d_e, int64_t n, int dtype, const void *dy,
                                          const float *dprobs, float sharpness, float *dx,
                                          float *dw_r, float *dgain, float *dbias, float *dw1,
                                          float *dw2, void *workspace, size_t workspace_bytes,
                                          void *stream)
{
    blockffn_status_t st = check_dtype(dtype);
    if (st != BLOCKFFN_OK)
        return st;
    if (!x || !w_r || !w1 || !w2 || !dy || !dx || !dw_r || !dw1 || !dw2 || !workspace)
        return fail(BLOCKFFN_EINVAL,
                    "x, w_r, w1, w2, dy, dx, dw_r, dw1, dw2 and workspace must not be NULL");
    if (T <= 0 || d_h <= 0 || E <= 0 || d_e <= 0 || n <= 0)
        return fail(BLOCKFFN_EINVAL, "T, d_h, E, d_e and n must be positive");
    if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(sharpness))
        return fail(BLOCKFFN_EINVAL, "eps must be finite and >= 0, sharpness finite");
    if (dtype != BLOCKFFN_BF16)
        return fail(BLOCKFFN_EUNSUPPORTED, "the layer backward takes bf16 inputs only");
    if (!blockffn::backward_supported(T, d_h, E, d_e, n))
        return fail(BLOCKFFN_EUNSUPPORTED, "layer backward needs 1 <= E <= 256, d_h % 256 == 0 "
                                           "and d_e % 128 == 0 (and 32-bit offsets)");
    if (!aligned(x, 16) || !aligned(w_r, 16) || !aligned(w1, 16) || !aligned(w2, 16) ||
        !aligned(dy, 16) || !aligned(dx, 16) || !aligned(dw_r, 4) || !aligned(dw1, 4) ||
        !aligned(dw2, 4) || (gain && !aligned(gain, 4)) || (bias && !aligned(bias, 4)) ||
        (dgain && !aligned(dgain, 4)) || (dbias && !aligned(dbias, 4)) ||
        (dprobs && !aligned(dprobs, 4)))
        return fail(BLOCKFFN_EUNSUPPORTED, "x, w_r, w1, w2, dy and dx must be 16-byte aligned, "
                                           "float arrays 4-byte aligned");
    if (!aligned(workspace, 256))
        return fail(BLOCKFFN_EUNSUPPORTED, "workspace needs 256-byte alignment");
    const size_t need = blockffn::backward_workspace_bytes(T, d_h, E, d_e, n);
    if (workspace_bytes < need)
        return fail(BLOCKFFN_EWORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                             " bytes, needs " + std::to_string(need));
    blockffn::BackwardArgs b;
    b.x = static_cast<const uint16_t *>(x);
    b.w_r = static_cast<const uint16_t *>(w_r);
    b.w1 = static_cast<const uint16_t *>(w1);
    b.w2 = static_cast<const uint16_t *>(w2);
    b.dy = static_cast<const uint16_t *>(dy);
    b.gain = gain;
    b.bias = bias;
    b.dprobs = dprobs;
    b.eps = eps;
    b.sharpness = sharpness;
    b.T = T;
    b.d_h = d_h;
    b.E = E;
    b.d_e = d_e;
    b.n = n;
    b.dx = dx;
    b.dw_r = dw_r;
    b.dgain = dgain;
    b.dbias = dbias;
    b.dw1 = dw1;
    b.dw2 = dw2;
    b.xcds = placement_xcds(static_cast<hipStream_t>(stream));
    const hipError_t err =
        blockffn::launch_layer_backward(b, workspace, static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("backward launch failed: ") + hipGetErrorString(err));
    g_last_error.clear();
    return BLOCKFFN_OK;
}

// Layer workspace: [chunk-FFN workspace][scores T x E fp32][router workspace].
namespace {
struct LayerWs {
    size_t ffn, scores, router, total;
};
LayerWs layer_ws(int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n, int dtype)
{
    LayerWs w{};
    w.ffn = blockffn_chunk_ffn_workspace_bytes(T, d_h, E, d_e, n, dtype);
    w.router = blockffn_router_workspace_bytes(T, d_h, E, dtype);
    if (w.ffn == 0 || w.router == 0)
        return w;
    w.scores = blockffn::align_up(w.ffn, 256);
    const size_t router_off = blockffn::align_up(w.scores + (size_t)T * E * 4, 256);
    w.total = router_off + w.router;
    w.router = router_off;
    return w;
}
}  // namespace

namespace {
// The full layer's y region (after the layer workspace) when the caller does not keep y.
size_t layer_y_bytes(int64_t T, int64_t d_h, int dtype)
{
    return blockffn::align_up((size_t)T * (size_t)d_h * (dtype == BLOCKFFN_BF16 ? 2 : 4), 256);
}
}  // namespace

size_t blockffn_layer_forward_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                              int64_t n, int dtype)
{
    if (check_ffn_sizes(T, d_h, E, d_e, n, dtype) != BLOCKFFN_OK)
        return 0;
    return layer_ws(T, d_h, E, d_e, n, dtype).total;
}

int blockffn_layer_forward_fused(int64_t T, int64_t d_h, int64_t E, int64_t d_e, int64_t n,
                                 int dtype, void *stream)
{
    if (check_ffn_sizes(T, d_h, E, d_e, n, dtype) != BLOCKFFN_OK)
        return 0;
    const blockffn::FfnPlan p = blockffn::make_plan(T, d_h, E, d_e, n, dtype);
    int xcds = 0, members = 0;
    return p.decode && decode_grid(static_cast<hipStream_t>(stream), p, &xcds, &members) &&
                   blockffn::layer_decode_supported(E, d_h, members)
               ? 1
               : 0;
}

namespace {
// Shared by blockffn_layer_forward (w1, w2 row-major; packed = NULL),
// blockffn_layer_forward_packed (w1 = w2 = NULL; packed in the tiled layout) and
// blockffn_layer_forward_full (ep != NULL: the epilogue, validated by the caller; y may
// then be NULL, and the workspace holds a y region after the layer's own part).
blockffn_status_t layer_forward(const void *x, const void *w_r, const float *gain,
                                const float *bias, float eps, const void *w1, const void *w2,
                                const void *packed, int64_t T, int64_t d_h, int64_t E,
                                int64_t d_e, int64_t n, int dtype, void *y, float *scores,
                                void *workspace, size_t workspace_bytes, void *stream,
                                const blockffn::LayerEpilogue *ep = nullptr)
{
    blockffn_status_t st = check_ffn_sizes(T, d_h, E, d_e, n, dtype);
    if (st != BLOCKFFN_OK)
        return st;
    if (!x || !w_r || !(packed || (w1 && w2)) || !(y || ep) || !workspace)
        return fail(BLOCKFFN_EINVAL, packed ? "x, w_r, packed, y and workspace must not be NULL"
                                            : "x, w_r, w1, w2, y and workspace must not be NULL");
    if (!(eps >= 0.0f))
        return fail(BLOCKFFN_EINVAL, "eps must be >= 0");
    const size_t ea = dtype == BLOCKFFN_BF16 ? 16 : 4;
    if (!aligned(x, ea) || !aligned(w_r, ea) || (w1 && !aligned(w1, ea)) ||
        (w2 && !aligned(w2, ea)) || (packed && !aligned(packed, ea)) || (y && !aligned(y, ea)))
        return fail(BLOCKFFN_EUNSUPPORTED, "x, w_r, the weights and y must be " +
                                               std::to_string(ea) + "-byte aligned");
    if ((scores && !aligned(scores, 4)) || (gain && !aligned(gain, 4)) || (bias && !aligned(bias, 4)))
        return fail(BLOCKFFN_EUNSUPPORTED, "float arrays must be 4-byte aligned");
    if (!aligned(workspace, 256))
        return fail(BLOCKFFN_EUNSUPPORTED, "workspace needs 256-byte alignment");
    const LayerWs L = layer_ws(T, d_h, E, d_e, n, dtype);
    const size_t need = ep ? L.total + layer_y_bytes(T, d_h, dtype) : L.total;
    if (workspace_bytes < need)
        return fail(BLOCKFFN_EWORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                             " bytes, needs " + std::to_string(need));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const blockffn::FfnPlan p = blockffn::make_plan(T, d_h, E, d_e, n, dtype);
    int xcds = 0, members = 0;
    if (p.decode && decode_grid(s, p, &xcds, &members) &&
        blockffn::layer_decode_supported(E, d_h, members)) {
        // one launch: the router computed by every workgroup from its staged x
        const uint16_t *pw = static_cast<const uint16_t *>(packed);
        const hipError_t err = blockffn::launch_layer_bf16_decode(
            p, xcds, members, static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w_r),
            gain, bias, eps, packed ? pw : static_cast<const uint16_t *>(w1),
            packed ? pw + E * d_e * d_h : static_cast<const uint16_t *>(w2), packed != nullptr,
            static_cast<uint16_t *>(y), scores, workspace, ep, s);
        if (err != hipSuccess)
            return fail(BLOCKFFN_EHIP, std::string("layer launch failed: ") + hipGetErrorString(err));
        g_last_error.clear();
        return BLOCKFFN_OK;
    }
    if (packed)
        return fail(BLOCKFFN_EUNSUPPORTED,
                    "packed weights need the one-launch layer (blockffn_layer_forward_fused)");
    char *base = static_cast<char *>(workspace);
    float *sc = scores ? scores : reinterpret_cast<float *>(base + L.scores);
    st = blockffn_router(x, w_r, gain, bias, eps, T, d_h, E, dtype, sc, nullptr,
                         ep ? ep->sharpness : 1.0f, ep ? ep->probs : nullptr, base + L.router,
                         L.total - L.router, stream);
    if (st != BLOCKFFN_OK)
        return st;
    void *yb = y ? y : base + L.total;
    st = blockffn_chunk_ffn(x, sc, w1, w2, T, d_h, E, d_e, n, dtype, yb, workspace, L.scores,
                            nullptr, nullptr, nullptr, stream);
    if (st != BLOCKFFN_OK || !ep)
        return st;
    return blockffn_add_layernorm(yb, x, ep->ln_gamma, ep->ln_beta, ep->ln_eps, T, d_h, dtype,
                                  ep->ln_out, stream);
}
}  // namespace

blockffn_status_t blockffn_layer_forward(const void *x, const void *w_r, const float *gain,
                                         const float *bias, float eps, const void *w1,
                                         const void *w2, int64_t T, int64_t d_h, int64_t E,
                                         int64_t d_e, int64_t n, int dtype, void *y, float *scores,
                                         void *workspace, size_t workspace_bytes, void *stream)
{
    if (!w1 || !w2)
        return fail(BLOCKFFN_EINVAL, "x, w_r, w1, w2, y and workspace must not be NULL");
    return layer_forward(x, w_r, gain, bias, eps, w1, w2, nullptr, T, d_h, E, d_e, n, dtype, y,
                         scores, workspace, workspace_bytes, stream);
}

size_t blockffn_pack_weights_bytes(int64_t E, int64_t d_h, int64_t d_e, int dtype)
{
    if (dtype != BLOCKFFN_BF16 || E < 1 || E > 256 || d_h < 32 || d_h % 32 != 0 || d_e < 32 ||
        d_e % 32 != 0 || E * d_h * d_e > ((int64_t)1 << 30))
        return 0;
    return (size_t)(2 * E * d_h * d_e * 2);
}

blockffn_status_t blockffn_pack_weights(const void *w1, const void *w2, int64_t E, int64_t d_h,
                                        int64_t d_e, int dtype, void *packed, void *stream)
{
    if (blockffn_pack_weights_bytes(E, d_h, d_e, dtype) == 0)
        return fail(BLOCKFFN_EINVAL, "pack_weights: bf16 only, 1 <= E <= 256, d_h and d_e "
                                     "positive multiples of 32, E*d_h*d_e <= 2^30");
    if (!w1 || !w2 || !packed)
        return fail(BLOCKFFN_EINVAL, "w1, w2 and packed must not be NULL");
    if (!aligned(w1, 16) || !aligned(w2, 16) || !aligned(packed, 16))
        return fail(BLOCKFFN_EUNSUPPORTED, "w1, w2 and packed must be 16-byte aligned");
    const hipError_t err = blockffn::launch_pack_weights(
        static_cast<const uint16_t *>(w1), static_cast<const uint16_t *>(w2), E, d_h, d_e,
        static_cast<uint16_t *>(packed), static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("pack launch failed: ") + hipGetErrorString(err));
    g_last_error.clear();
    return BLOCKFFN_OK;
}

blockffn_status_t blockffn_layer_forward_packed(const void *x, const void *w_r, const float *gain,
                                                const float *bias, float eps, const void *packed,
                                                int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                                int64_t n, int dtype, void *y, float *scores,
                                                void *workspace, size_t workspace_bytes,
                                                void *stream)
{
    if (!packed)
        return fail(BLOCKFFN_EINVAL, "x, w_r, packed, y and workspace must not be NULL");
    return layer_forward(x, w_r, gain, bias, eps, nullptr, nullptr, packed, T, d_h, E, d_e, n,
                         dtype, y, scores, workspace, workspace_bytes, stream);
}

size_t blockffn_layer_forward_full_workspace_bytes(int64_t T, int64_t d_h, int64_t E, int64_t d_e,
                                                   int64_t n, int dtype)
{
    if (check_ffn_sizes(T, d_h, E, d_e, n, dtype) != BLOCKFFN_OK)
        return 0;
    return layer_ws(T, d_h, E, d_e, n, dtype).total + layer_y_bytes(T, d_h, dtype);
}

blockffn_status_t blockffn_layer_forward_full(const void *x, const void *w_r, const float *gain,
                                              const float *bias, float eps, const void *w1,
                                              const void *w2, const void *packed, int64_t T,
                                              int64_t d_h, int64_t E, int64_t d_e, int64_t n,
                                              int dtype, const float *ln_gamma,
                                              const float *ln_beta, float ln_eps, void *out,
                                              float sharpness, float *probs, void *y,
                                              float *scores, void *workspace,
                                              size_t workspace_bytes, void *stream)
{
    blockffn_status_t st = check_ffn_sizes(T, d_h, E, d_e, n, dtype);
    if (st != BLOCKFFN_OK)
        return st;
    if (!out)
        return fail(BLOCKFFN_EINVAL, "out must not be NULL");
    if ((packed != nullptr) == (w1 != nullptr || w2 != nullptr))
        return fail(BLOCKFFN_EINVAL, "give either w1 and w2 (row-major) or packed, not both");
    if (!(ln_eps >= 0.0f) || !std::isfinite(ln_eps))
        return fail(BLOCKFFN_EINVAL, "ln_eps must be finite and >= 0");
    if (probs && !std::isfinite(sharpness))
        return fail(BLOCKFFN_EINVAL, "sharpness must be finite");
    const int64_t vec = dtype == BLOCKFFN_BF16 ? 8 : 4;
    if (d_h % vec != 0)
        return fail(BLOCKFFN_EUNSUPPORTED, "d_h must be a multiple of " + std::to_string(vec));
    if (!aligned(out, 16) || (ln_gamma && !aligned(ln_gamma, 16)) ||
        (ln_beta && !aligned(ln_beta, 16)) || (probs && !aligned(probs, 4)) ||
        !aligned(x, 16) || (y && !aligned(y, 16)))
        return fail(BLOCKFFN_EUNSUPPORTED, "x, y, out, ln_gamma and ln_beta must be 16-byte "
                                           "aligned, probs 4-byte aligned");
    const size_t elem = dtype == BLOCKFFN_BF16 ? 2 : 4;
    const size_t obytes = (size_t)T * (size_t)d_h * elem, pbytes = (size_t)T * (size_t)E * 4;
    if (overlap(out, obytes, x, obytes) || (y && overlap(out, obytes, y, obytes)) ||
        (scores && overlap(out, obytes, scores, pbytes)) ||
        (probs && overlap(out, obytes, probs, pbytes)) ||
        (probs && scores && overlap(probs, pbytes, scores, pbytes)))
        return fail(BLOCKFFN_EINVAL, "out, probs and scores must not overlap x, y or each other");
    blockffn::LayerEpilogue ep{ln_gamma, ln_beta, ln_eps, static_cast<uint16_t *>(out),
                               sharpness, probs};
    if (packed) {
        hipStream_t s = static_cast<hipStream_t>(stream);
        const blockffn::FfnPlan p = blockffn::make_plan(T, d_h, E, d_e, n, dtype);
        int xcds = 0, members = 0;
        if (!(p.decode && decode_grid(s, p, &xcds, &members) &&
              blockffn::layer_decode_supported(E, d_h, members)))
            return fail(BLOCKFFN_EUNSUPPORTED,
                        "packed weights need the one-launch layer (blockffn_layer_forward_fused)");
    }
    return layer_forward(x, w_r, gain, bias, eps, w1, w2, packed, T, d_h, E, d_e, n, dtype, y,
                         scores, workspace, workspace_bytes, stream, &ep);
}

blockffn_status_t blockffn_layer_forward_noalloc(const void *x, const void *w_r, const float *gain,
                                                 const float *bias, float eps, const void *w1,
                                                 const void *w2, int64_t T, int64_t d_h, int64_t E,
                                                 int64_t d_e, int64_t n, int dtype, void *y,
                                                 float *scores, void *stream)
{
    if (!w1 || !w2)
        return fail(BLOCKFFN_EINVAL, "x, w_r, w1, w2 and y must not be NULL");
    blockffn_status_t st = check_ffn_sizes(T, d_h, E, d_e, n, dtype);
    if (st != BLOCKFFN_OK)
        return st;
    const size_t need = layer_ws(T, d_h, E, d_e, n, dtype).total;
    if (need > kNoallocScratchBytes)
        return fail(BLOCKFFN_EUNSUPPORTED,
                    "these sizes need " + std::to_string(need) + " bytes of scratch, more than "
                    "the library's array of " + std::to_string(kNoallocScratchBytes) +
                    " bytes; use blockffn_layer_forward with a workspace");
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("no current device: ") + hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(BLOCKFFN_EUNSUPPORTED, "device index beyond the library's table");
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_device_mutex);
        if ((err = noalloc_scratch_init(dev)) != hipSuccess)
            return fail(BLOCKFFN_EHIP, std::string("scratch array address: ") +
                                           hipGetErrorString(err));
        ptr = g_scratch_ptr[dev];
    }
    // validate everything the workspace call checks before enqueueing anything
    if (!x || !w_r || !y)
        return fail(BLOCKFFN_EINVAL, "x, w_r, w1, w2 and y must not be NULL");
    if (!(eps >= 0.0f))
        return fail(BLOCKFFN_EINVAL, "eps must be >= 0");
    const size_t ea = dtype == BLOCKFFN_BF16 ? 16 : 4;
    if (!aligned(x, ea) || !aligned(w_r, ea) || !aligned(w1, ea) || !aligned(w2, ea) ||
        !aligned(y, ea))
        return fail(BLOCKFFN_EUNSUPPORTED, "x, w_r, the weights and y must be " +
                                               std::to_string(ea) + "-byte aligned");
    if ((scores && !aligned(scores, 4)) || (gain && !aligned(gain, 4)) || (bias && !aligned(bias, 4)))
        return fail(BLOCKFFN_EUNSUPPORTED, "float arrays must be 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(scratch_recover_kernel, dim3(1), dim3(1024), 0, s,
                       static_cast<uint32_t *>(ptr));
    if ((err = hipGetLastError()) != hipSuccess)
        return fail(BLOCKFFN_EHIP, std::string("scratch check launch failed: ") + hipGetErrorString(err));
    return layer_forward(x, w_r, gain, bias, eps, w1, w2, nullptr, T, d_h, E, d_e, n, dtype, y,
                         scores, ptr, kNoallocScratchBytes, stream);
}

}  // extern "C"
