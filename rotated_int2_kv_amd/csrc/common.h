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


// E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; the all-ones
// exponent still holds numbers, largest finite 448): the 8-bit scale/zero
// format.  Value of a code (codes 0x7F / 0xFF, NaN, are never written).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    const uint32_t e = (code >> 3) & 15u, m = code & 7u;
    const float mag = e == 0 ? float(m) * 0x1p-9f : __builtin_ldexpf(float(8u + m), int(e) - 10);
    return (code & 0x80u) ? -mag : mag;
}

// Code of the E4M3 value nearest to x (ties to the even code), magnitudes
// above 448 saturating to 448; a zero result keeps the sign of x.  The scaled
// magnitude is exact in fp32 (a power-of-two scaling) and rounded once to an
// integer with the current round-to-nearest-even mode.
__device__ __forceinline__ uint32_t e4m3_code_rn(float x) {
    const float a = fminf(fabsf(x), 448.0f);
    uint32_t mag;
    if (a < 0x1p-6f) {
        mag = uint32_t(__builtin_rintf(a * 512.0f));        // subnormal steps of 2^-9; 8 is 2^-6 (code 8)
    } else {
        int e2 = 0;
        (void)__builtin_frexpf(a, &e2);                     // a in [2^(e2 - 1), 2^e2)
        const uint32_t q = uint32_t(__builtin_rintf(__builtin_ldexpf(a, 4 - e2)));   // 8 .. 16
        mag = (uint32_t(e2 - 1 + 7) << 3) + (q - 8u);     // q = 16 carries into the exponent
    }
    return mag | (__builtin_signbitf(x) ? 0x80u : 0u);
}

// Two E4M3 codes (bytes 0 and 1 of w) as an fp16 pair (low half = byte 0),
// exact: the code's exponent and mantissa fields moved into the fp16 fields
// give the value times 2^-8 (fp16's exponent bias is 15, E4M3's 7; code
// exponent 0 lands on fp16 subnormals the same way), and one fp16 multiply
// by 2^8 restores it.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    const uint32_t x = __builtin_amdgcn_perm(0u, w, 0x0C010C00u);      // byte 0 -> bits 0..7, byte 1 -> 16..23
    const uint32_t h = ((x << 7) & 0x3F803F80u) | ((x << 8) & 0x80008000u);
    const f16x2 v = __builtin_bit_cast(f16x2, h) * f16x2{_Float16(256.0f), _Float16(256.0f)};
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace oscar
