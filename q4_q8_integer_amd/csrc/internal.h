// internal.h - launchers shared between the kernel translation units and the
// C-ABI entry points.  Arguments are validated by the caller (mmq_api.hip);
// each launcher only enqueues work and returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmq {

// Bytes of one q4_K super-block (256 weights).
constexpr int kBlockBytes = 144;
// Bytes of one record (16 rows x one super-block) of the repacked q4_K layout.
constexpr int kRepackRecordBytes = 2368;

hipError_t launch_q8_quantize(const float* x, int64_t nblocks, int8_t* q, uint32_t* ds,
                              hipStream_t stream);

// q8 quantize with the codes written as binary16 operand tiles (token tiles
// of 128, k stages of 128, 32 KiB per tile and stage; k % 256 == 0).
hipError_t launch_q8_quantize_tiled(const float* x, int n, int k, uint16_t* qt, uint32_t* ds,
                                    hipStream_t stream);

// The same, with the codes written as operand tiles.
hipError_t launch_q8_quantize_silu_mul_tiled(const float* g, const float* u, int n, int k, uint16_t* qt,
                                             uint32_t* ds, hipStream_t stream);

// q8 quantize of h = float32(g*u / (1 + exp(-g))) (float64 evaluation).
hipError_t launch_q8_quantize_silu_mul(const float* g, const float* u, int64_t nblocks, int8_t* q,
                                       uint32_t* ds, hipStream_t stream);

// Exact int32 block dots, dots[t][o][c].
hipError_t launch_mmq_dots(const uint8_t* w, int m, int k, const int8_t* q, int n,
                           int32_t* dots, hipStream_t stream);

// Output element of the fold kernels: float32, or binary16 rounded to
// nearest-even from the same float32 value (half_out).
template <bool H>
struct OutElem {
    typedef float T;
};
template <>
struct OutElem<true> {
    typedef _Float16 T;
};

// The low 16 bits of h as a binary16 value, widened to float32 (exact).
__device__ __forceinline__ float half_lo(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

template <bool H>
__device__ __forceinline__ void store_out(void* out, int64_t i, float v) {
    reinterpret_cast<typename OutElem<H>::T*>(out)[i] = (typename OutElem<H>::T)v;
}

// Four consecutive outputs from index i (16-byte aligned for float32, 8 for binary16).
template <bool H>
__device__ __forceinline__ void store_out4(void* out, int64_t i, float a, float b, float c, float d) {
    if (H) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<h4*>(reinterpret_cast<_Float16*>(out) + i) =
            h4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + i) = make_float4(a, b, c, d);
    }
}

// Two-term fold, out[t][o] (float32 or binary16), int8 MFMA + three-operation epilogue.
hipError_t launch_mmq_fp32(const uint8_t* w, int m, int k, const int8_t* q,
                           const uint32_t* ds, int n, void* out, bool half_out, hipStream_t stream);

// Two-term fold, out[t][o], binary16 MFMA on exact sc*q4 and q8 operands +
// float32 MFMA for the min term (above 64 tokens).
hipError_t launch_mmq_fp32_f16(const uint8_t* w, int m, int k, const int8_t* q,
                               const uint32_t* ds, int n, void* out, bool half_out,
                               hipStream_t stream);

// The binary16-MFMA kernel on q4k_repack records (same arithmetic and order
// as launch_mmq_fp32_f16, so the same float32 result bit for bit).
hipError_t launch_mmq_fp32_f16_repacked(const uint8_t* wr, int m, int k, const int8_t* q,
                                        const uint32_t* ds, int n, float* out, hipStream_t stream);

// The binary16-MFMA kernel with the activations as q8 operand tiles (from
// launch_q8_quantize_tiled), on q4_K rows or q4k_repack records; the same
// float32 result bit for bit as the int8-activation kernel.
hipError_t launch_mmq_fp32_f16_tiles(const uint8_t* w, bool repacked, int m, int k, const uint16_t* qt,
                                     const uint32_t* ds, int n, float* out, hipStream_t stream);

// Two-term fold, out[t][o], for n <= 64 tokens: weight-streaming int8-MFMA
// kernel (8 waves per 16 rows, each over a slice of k).
hipError_t launch_mmq_fp32_small(const uint8_t* w, int m, int k, const int8_t* q,
                                 const uint32_t* ds, int n, void* out, bool half_out,
                                 hipStream_t stream);

// Two-term fold, out[t][o], for 1 <= n <= kGemvMaxN tokens: 4-way int8 dot
// products on the vector ALU, no token padding.
hipError_t launch_mmq_fp32_gemv(const uint8_t* w, int m, int k, const int8_t* q,
                                const uint32_t* ds, int n, void* out, bool half_out,
                                hipStream_t stream);
constexpr int kGemvMaxN = 8;

// Load-time repack of q4_K into 16-row records (repack.hip), and the dot4
// kernel on that layout (1 <= n <= kGemvMaxN; w is the repacked buffer).
hipError_t launch_q4k_repack(const uint8_t* w, int m, int k, uint8_t* wr, hipStream_t stream);
hipError_t launch_mmq_fp32_gemv_repacked(const uint8_t* wr, int m, int k, const int8_t* q,
                                         const uint32_t* ds, int n, void* out, bool half_out,
                                         hipStream_t stream);

// Largest token count the few-token kernel takes.
constexpr int kSmallMaxN = 64;

// Two-term fold, out[t][o], for 1 <= n <= kNarrowMaxN tokens: 4x4x4 int8
// MFMA on weights and tokens staged through LDS, one (row, super-block,
// chunk half) per lane (mmq_narrow.hip).
hipError_t launch_mmq_fp32_narrow(const uint8_t* w, int m, int k, const int8_t* q,
                                  const uint32_t* ds, int n, void* out, bool half_out,
                                  hipStream_t stream);
constexpr int kNarrowMaxN = 16;

// The narrow kernel's layout for an m x k weight: 32-row tiles where they
// fill the 256 CUs (at least 256 tiles) with at least 8 super-blocks per
// wave, run by 4 waves per workgroup from 512 tiles on (two workgroups per
// CU) and by 8 below; the return value is that wave count, or 0 for 16-row
// tiles.
inline int narrow_waves32(int64_t m, int64_t k) {
    const int64_t tiles = (m + 31) / 32, w = tiles >= 512 ? 4 : 8;
    return tiles >= 256 && (k >> 8) >= 8 * w ? (int)w : 0;
}

// q6_K weights (210-byte super-blocks, one int8 scale per 16 weights).
// Exact int32 group dots, dots[t][o][g] (g = k/16 groups).
hipError_t launch_q6k_dots(const uint8_t* w, int m, int k, const int8_t* q, int n,
                           int32_t* dots, hipStream_t stream);

// out[t][o] (float32 or binary16) for any n: int8 MFMA per scale group.
hipError_t launch_q6k_i8(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                         int n, void* out, bool half_out, hipStream_t stream);

// out[t][o] for any n: binary16 MFMA on the split exact operands sc*nibble/64
// and sc*(hi2 - 2)/4 (one FMA per output and chunk).
hipError_t launch_q6k_f16(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
                          void* out, bool half_out, hipStream_t stream);

// launch_q6k_f16 with the activations as q8 operand tiles (float32 output).
hipError_t launch_q6k_f16_tiles(const uint8_t* w, int m, int k, const uint16_t* qt, const uint32_t* ds,
                                int n, float* out, hipStream_t stream);

// out[t][o] for 1 <= n <= kQ6kGemvMaxN: 4-way int8 dots on the vector ALU.
hipError_t launch_q6k_gemv(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                           int n, void* out, bool half_out, hipStream_t stream);
constexpr int kQ6kGemvMaxN = 8;

}  // namespace mmq
