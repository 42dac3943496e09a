// Shared device helpers for the gfx950 kernels of libbd.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define BD_LOG2E 1.4426950408889634f

__device__ __forceinline__ float bd_bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t bd_f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bd_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine each lane's value with that of lane (lane ^ 32) using
// v_permlane32_swap (a VALU lane exchange, no LDS round trip).  Both lanes of
// a pair see the same two operands, so they get bitwise-identical results.
__device__ __forceinline__ float bd_max_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float bd_sum_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void bd_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that waits only for this wave's LDS operations, not for
// its outstanding global loads (unlike __syncthreads, whose fence drains
// vmcnt).  Callers order global->LDS copies with bd_wait_vmcnt first.
__device__ __forceinline__ void bd_barrier_lds() {
    asm volatile("" ::: "memory");  // compiler-only fence: no access moves across
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ bool bd_wave_any(bool p) {
    return __builtin_amdgcn_ballot_w64(p) != 0;
}

// Cross-workgroup hand-off without whole-cache maintenance.  Partial results
// are written with agent-scope relaxed atomic stores, which gfx950 performs
// at the agent's coherence point (through the L2, not kept only in one XCD's
// L2), and read back with agent-scope relaxed atomic loads, which read from
// that point.  The writer waits until its stores are acknowledged
// (s_waitcnt 0) before its workgroup takes a ticket, and the ticket is an
// agent-scope atomic performed at the same point.  The workgroup whose ticket
// completes the count therefore comes after every other workgroup's ticket,
// each of which came after that workgroup's stores had completed; its
// coherent loads, issued after it has seen the count, observe them.  Only the
// hand-off locations need ordering, so no release / acquire fence (which on
// gfx950 writes back or invalidates the whole L2 at agent scope) is used.
__device__ __forceinline__ void bd_coherent_store2(float *p, float a, float b) {
    const uint64_t v = ((uint64_t)__float_as_uint(b) << 32) | (uint64_t)__float_as_uint(a);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 bd_coherent_load2(const float *p) {
    const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ __forceinline__ void bd_coherent_store(float *p, float a) {
    __hip_atomic_store(p, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void bd_coherent_store(int *p, int a) {
    __hip_atomic_store(p, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float bd_coherent_load(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int bd_coherent_load(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void bd_coherent_store_u2(uint2 *p, uint2 v) {
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), ((uint64_t)v.y << 32) | v.x, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 bd_coherent_load_u2(const uint2 *p) {
    const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}
__device__ __forceinline__ void bd_coherent_store64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t bd_coherent_load64(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Non-temporal stores for data the next kernel consumes: the lines are not
// kept dirty in L2, so the write-back that ends a kernel has little left to
// do and the next kernel on the stream starts sooner.
typedef float floatx2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void bd_store_nt(void *p, uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void bd_store_nt(void *p, float2 v) {
    __builtin_nontemporal_store(floatx2_nt{v.x, v.y}, reinterpret_cast<floatx2_nt *>(p));
}
__device__ __forceinline__ void bd_store_nt(void *p, uint2 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2 *>(p));
}
// Write-through stores (cache policy sc1) of 16 or 8 bytes at byte offset
// `off` of a region of `bytes` bytes at `base`, through a raw buffer
// resource (stores past the region are dropped by the range check).  The
// lines do not stay dirty in L2 for the kernel-end write-back, and unlike
// non-temporal stores they stay in the last-level cache, where the next
// kernel on the stream reads them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bd_region(void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
constexpr int kPolicySc1 = 16;  // buffer-op cache policy bits: sc1
__device__ __forceinline__ void bd_store_wt(__amdgpu_buffer_rsrc_t r, unsigned off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, (int)off, 0, kPolicySc1);
}
__device__ __forceinline__ void bd_store_wt(__amdgpu_buffer_rsrc_t r, unsigned off, float2 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v.x), __float_as_uint(v.y)}, r, (int)off, 0,
                                          kPolicySc1);
}
// Wait until every memory operation this thread issued has completed (for a
// store: acknowledged by the memory side).  The empty asm statements keep the
// compiler from moving any memory access across the wait.
__device__ __forceinline__ void bd_wait_all_memory() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
}
// Relaxed agent-scope ticket: returns the previous count.
__device__ __forceinline__ int bd_ticket(int *counter) {
    return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
