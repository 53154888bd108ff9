// f16_operand.h - shared pieces of the binary16-MFMA kernels (mmq_f16.hip,
// mmq_q6k_f16.hip): packed binary16 helpers that build exact integer
// operands from bit patterns, two values per register, and the
// direct-to-LDS copy of operand-tile blocks.
//
//   * A nibble or small code n placed under the exponent bits 0x6400 is the
//     binary16 value 1024 + n (the exponent's unit is 1 there), so
//     (x & mask) | 0x64006400 turns two bytes' fields into two binary16
//     values in one instruction; a fused multiply-add with exact constants
//     then removes the 1024 and applies a scale, rounding nothing when the
//     result is an integer (or a multiple of a power of two) below 2048.
//   * An int8 code q: the vector unit's sub-dword operand select picks one
//     byte, sign-extends it and converts it to binary16 (exact, |q| <= 128),
//     writing either half of the destination and keeping the other, so four
//     codes become two pairs in four instructions.
//   * Pairs are (byte 0, byte 2) and (byte 1, byte 3) of a dword, on the
//     weight side and the activation side alike, so both sides agree on k.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmq {

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
    uint32_t a, b;
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_2"
        : "=&v"(a) : "v"(y));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_1\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
        : "=&v"(b) : "v"(y));
    p02 = a; p13 = b;
}

// One 16-byte direct-to-LDS copy per lane (buffer_load_dwordx4 ... lds):
// lane i writes 16 bytes at LDS address lds + 16 i, from byte voff of the
// buffer rsrc.  Inline asm, outside the compiler's wait bookkeeping: the
// callers place the vmcnt waits that complete these copies themselves.
// M0 is a reserved register; in the kernels using this nothing else sets or
// reads it, so the clobber only tells the compiler what the asm does.  A
// load that writes LDS reads M0 and needs one wait state after an SALU
// write of it (the compiler inserts the same s_nop 0 before its own such
// loads; inside asm it does not).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(u32x4 rsrc, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace mmq
