// Device helpers shared by the liboscar kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

namespace oscar {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Nearest bfloat16 (ties to even) of a finite or infinite fp32 value, as bits.
__device__ __forceinline__ uint16_t bf16_bits_rn(float x) {
    const uint32_t u = __float_as_uint(x);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ __bf16 bits_to_bf16(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

// MFMA 16x16x32 wrappers.  Operand layout used throughout: lane l holds row
// (A) or column (B) l % 16 and eight k-slots selected by l / 16; the output
// lane l holds column l % 16, rows 4 (l / 16) + i in element i.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace oscar
