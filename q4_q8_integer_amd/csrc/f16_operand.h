// f16_operand.h - packed binary16 helpers of the binary16-MFMA kernels
// (mmq_f16.hip, mmq_q6k_f16.hip): exact integer operands built from bit
// patterns, two values per register.
//
//   * A nibble or small code n placed under the exponent bits 0x6400 is the
//     binary16 value 1024 + n (the exponent's unit is 1 there), so
//     (x & mask) | 0x64006400 turns two bytes' fields into two binary16
//     values in one instruction; a fused multiply-add with exact constants
//     then removes the 1024 and applies a scale, rounding nothing when the
//     result is an integer (or a multiple of a power of two) below 2048.
//   * An int8 code q: byte ^ 0x80 = q + 128, under 0x64 that is 1152 + q,
//     minus 1152.
//   * Pairs are (byte 0, byte 2) and (byte 1, byte 3) of a dword, on the
//     weight side and the activation side alike, so both sides agree on k.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmq {

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

__device__ __forceinline__ uint32_t pk_fma_f16(uint32_t a, uint32_t b, uint32_t c) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, a),
                                                                   __builtin_bit_cast(h2, b),
                                                                   __builtin_bit_cast(h2, c)));
}

__device__ __forceinline__ uint32_t pk_add_f16(uint32_t a, uint32_t b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) + __builtin_bit_cast(h2, b));
}

__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) * __builtin_bit_cast(h2, b));
}

// (x & mask) | bits in one vector instruction (the compiler otherwise emits two).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(mask), "v"(bits));
    return r;
}

// Both binary16 halves set to v.
__device__ __forceinline__ uint32_t f16x2_splat(float v) {
    const unsigned short h = __builtin_bit_cast(unsigned short, (_Float16)v);
    return (uint32_t)h | ((uint32_t)h << 16);
}

// 4 int8 codes -> binary16 pairs [b0, b2], [b1, b3], exactly.
__device__ __forceinline__ void q8_word(uint32_t y, uint32_t& p02, uint32_t& p13) {
    const uint32_t z = y ^ 0x80808080u;
    const uint32_t m1152 = 0xE480E480u;  // (-1152, -1152)
    p02 = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, z, 0x04020400u), m1152);
    p13 = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, z, 0x04030401u), m1152);
}

}  // namespace mmq
