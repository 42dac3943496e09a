// Shared device helpers for the gfx950 kernels of libbd.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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

// Value of lane (lane ^ 32): exchanges the two 32-lane halves of a wave.
__device__ __forceinline__ float bd_swap_halves(float v) { return __shfl_xor(v, 32, 64); }

__device__ __forceinline__ bool bd_wave_any(bool p) {
    return __builtin_amdgcn_ballot_w64(p) != 0;
}
