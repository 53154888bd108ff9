// q6k_device.h - reading q6_K super-blocks on the device (shared by the q6_K
// kernels).
//
// q6_K (the second k-quant weight format; named in the r31 page's closing
// notes of the yusiwen.cn "minfer" pages, layout from the GGUF k-quants):
// 256 weights in 210 bytes, ql[128] low nibbles at 0, qh[64] high bit pairs at
// 128, sixteen int8 scales at 192 (one per 16 weights), binary16 d at 208.
// Weight 128h + 32g + l has the code q = nibble (g >> 1) of ql[64h + 32(g & 1) + l]
// | (bits 2g..2g+1 of qh[32h + l]) << 4 and the value d * sc[(128h + 32g + l) / 16] * (q - 32).
//
// A block starts at byte 210*(row*(k/256) + b) of the matrix: always even,
// every other block not a multiple of 4.  A 16-byte field at a multiple-of-4
// offset x of a block is read as the five aligned dwords from (start + x) & ~3
// and shifted into place with v_alignbyte (shift 0 or 2 bytes).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmq {

constexpr int kQ6kBlockBytes = 210;

namespace q6k {

__device__ __forceinline__ uint32_t ld32(const uint8_t* p) {
    return *reinterpret_cast<const uint32_t*>(p);
}

// The dwords covering bytes [B + x, B + x + 16) of the weights, B the block's
// byte offset, sh = B & 3 (0 or 2).  The fifth dword is needed only when
// sh == 2; with sh == 0 it would end 4 bytes past the field, which for the
// scale field (x = 192) is past the block, so it is then read from
// `fifth_if_aligned` bytes after the start instead (a dword of the field).
__device__ __forceinline__ void load_run(const uint8_t* w, int64_t B, int x, uint32_t sh,
                                         uint32_t (&v)[5], int fifth_if_aligned = 16) {
    const uint8_t* a = w + B + x - sh;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld32(a + 4 * i);
    v[4] = ld32(a + (sh ? 16 : fifth_if_aligned));
}

// Dword i of the 16-byte field held in v (see load_run).
__device__ __forceinline__ uint32_t run_word(const uint32_t (&v)[5], int i, uint32_t sh) {
    return __builtin_amdgcn_alignbyte(v[i + 1], v[i], sh);
}

// Signed codes q - 32 of four weights as int8 bytes.  lo holds the low
// nibbles in bits 0-3 of each byte, hi the 2-bit high parts in bits 0-1.
// q - 32 = nibble + 16*(hi2 - 2): the second term, 0xE0 0xF0 0x00 0x10 for
// hi2 = 0..3, has a zero low nibble, so the byte is nibble | table[hi2], the
// table lookup being one v_perm_b32 with the table in its low source.
__device__ __forceinline__ uint32_t signed_codes(uint32_t lo, uint32_t hi) {
    return (lo & 0x0F0F0F0Fu) | __builtin_amdgcn_perm(0u, 0x1000F0E0u, hi & 0x03030303u);
}

// Quarter p = 2h + e of a block covers, for g = 0..3, the 16 weights
// 128h + 32g + 16e + [0, 16) (scale group 8h + 2g + e).  Its bytes: ql0 =
// ql[64h + 16e ..] (groups g = 0, 2), ql1 = ql[64h + 32 + 16e ..] (g = 1, 3),
// qh = qh[32h + 16e ..].  Block offsets of the three 16-byte fields:
__device__ __forceinline__ int ql0_off(int h, int e) { return 64 * h + 16 * e; }
__device__ __forceinline__ int ql1_off(int h, int e) { return 64 * h + 32 + 16 * e; }
__device__ __forceinline__ int qh_off(int h, int e) { return 128 + 32 * h + 16 * e; }

// cw[g][i] = signed codes of weights 128h + 32g + 16e + 4i .. +3.
__device__ __forceinline__ void quarter_codes(const uint32_t (&ql0)[5], const uint32_t (&ql1)[5],
                                              const uint32_t (&qh)[5], uint32_t sh,
                                              uint32_t (&cw)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a = run_word(ql0, i, sh), b = run_word(ql1, i, sh), h = run_word(qh, i, sh);
        cw[0][i] = signed_codes(a, h);
        cw[1][i] = signed_codes(b, h >> 2);
        cw[2][i] = signed_codes(a >> 4, h >> 4);
        cw[3][i] = signed_codes(b >> 4, h >> 6);
    }
}

}  // namespace q6k
}  // namespace mmq
