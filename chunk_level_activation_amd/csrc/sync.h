// Device helpers for kernels whose workgroups hand data to one another inside a
// launch: buffer-resource loads and stores with explicit cache-policy bits, and
// relaxed device-scope counters.
//
// On gfx950 each XCD has its own L2. A store with sc0 bypasses the CU's L1 and lands
// in the XCD's L2, where other workgroups of that XCD read it with sc0 loads; sc1
// makes the access coherent across XCDs (it goes to memory / the Infinity Cache).
// A producer drains its stores (s_waitcnt covers stores on this family) before it
// bumps a counter; a consumer that has seen the counter then loads with the matching
// bit, so it cannot be served a stale line.
#pragma once

#include "common.h"

namespace blockffn {

// Cache policy bits of buffer accesses: nt = streamed once, sc0 = XCD-coherent
// (bypasses L1), sc1 = device-coherent.
constexpr int kNT = 2, kSC0 = 1, kSC1 = 16;

// 128-bit buffer descriptor (raw buffer, no swizzle) over [base, base + bytes); loads
// beyond the range return zero and stores beyond it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint64_t bytes)
{
    const int n = bytes < 0x7fffffffull ? (int)bytes : 0x7fffffff;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
template <int AUX>
__device__ __forceinline__ bf16x8 bload(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
}
// 16 bytes per lane from buffer offset off straight into LDS, without registers: lane
// l's bytes land at dst + 16 l (dst must be the same for the whole wave); an offset past
// the range stores zeros. The data is in LDS once the wave's vector-memory count covers
// the load.
typedef __attribute__((address_space(3))) void lds_void;
template <int AUX>
__device__ __forceinline__ void bload_lds16(__amdgpu_buffer_rsrc_t r, void *dst, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, off, 0, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ float4 bload_f4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ float bload_f1(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ void bstore_f4(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ void bstore_f1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, (int)off, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ void bstore_u64(__amdgpu_buffer_rsrc_t r, uint32_t off, uint64_t v)
{
    __builtin_amdgcn_raw_buffer_store_b64(
        __builtin_bit_cast(unsigned int __attribute__((ext_vector_type(2))), v), r, (int)off, 0, AUX);
}

__device__ __forceinline__ uint32_t ld_counter(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_counter(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_counter(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Flags shared only by workgroups of one XCD: the producer stores with sc0 (the value
// lands in the XCD's L2) and consumers read with a device-scope load (sc1), which is
// answered from that L2 in about 0.3 us. A plain or sc0 load may instead be served by
// a stale L1 copy of the line indefinitely, and a device-scope (write-through) store
// takes several times longer to become visible (measured on MI355X).
__device__ __forceinline__ void xcd_flag_store(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kSC0);
}

// Wait until every memory access this wave issued has completed.
__device__ __forceinline__ void drain_memory()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace blockffn
