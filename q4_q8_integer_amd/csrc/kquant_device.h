// kquant_device.h - device helpers shared by the k-quant kernels: the 6-bit
// scale decode of the q4_K super-block header (one definition for every
// kernel that reads GGUF rows), and the buffer-resource and wait-count
// constants of the gfx950 loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmq {

// Word 3 of a raw (unformatted, stride 0) buffer resource on gfx950.
constexpr int kBufferFlags = 0x00020000;

// s_waitcnt operand: at most n vector-memory operations outstanding, the
// other counters unconstrained.
constexpr int kWaitVmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// The q4_K scale packing (the GGUF k-quant super-block header): twelve bytes
// after d and dmin hold eight 6-bit scales sc[j] and mins m[j].  For j < 4,
// sc[j] is the low 6 bits of byte j and m[j] the low 6 bits of byte j + 4.
// For j >= 4, sc[j] is the low nibble of byte j + 4 with the top 2 bits of
// byte j - 4 above it, and m[j] the high nibble of byte j + 4 with the top 2
// bits of byte j above it.  The bytes arrive as three dwords: s03 = bytes
// 0-3, s47 = bytes 4-7, s811 = bytes 8-11.

// (sc, m) of sub-block j (0..7).  Register bit-field extracts only (a byte
// array here would live in scratch).
__device__ __forceinline__ void scale_min(uint32_t s03, uint32_t s47, uint32_t s811, int j, int& sc, int& mn) {
    const int sh = 8 * (j & 3);
    const int by = (s03 >> sh) & 0xFF, bz = (s47 >> sh) & 0xFF, bw = (s811 >> sh) & 0xFF;
    const bool hi = j >= 4;
    sc = hi ? ((bw & 15) | ((by >> 6) << 4)) : (by & 63);
    mn = hi ? ((bw >> 4) | ((bz >> 6) << 4)) : (bz & 63);
}

// (sc, m) of the chunk pair 2p, 2p + 1 (p = 0..3), for kernels where p
// differs between lanes: both halves of the packing read as a 4-bit field
// plus a 2-bit field from lane-selected dwords and shifts, so no lane takes
// a branch.  Same values as scale_min(.., 2p, ..) and scale_min(.., 2p + 1, ..).
__device__ __forceinline__ void scale_min_pair(uint32_t s03, uint32_t s47, uint32_t s811, int p, uint32_t& sc0,
                                               uint32_t& sc1, uint32_t& m0, uint32_t& m1) {
    const bool lo4 = p < 2;
    const int sh = 16 * (p & 1);
    const uint32_t xs = lo4 ? s03 : s811, xm = lo4 ? s47 : s811;
    const int oh = lo4 ? 4 : 6, om = lo4 ? 0 : 4;
    sc0 = __builtin_amdgcn_ubfe(xs, sh, 4) | (__builtin_amdgcn_ubfe(s03, sh + oh, 2) << 4);
    sc1 = __builtin_amdgcn_ubfe(xs, sh + 8, 4) | (__builtin_amdgcn_ubfe(s03, sh + 8 + oh, 2) << 4);
    m0 = __builtin_amdgcn_ubfe(xm, sh + om, 4) | (__builtin_amdgcn_ubfe(s47, sh + oh, 2) << 4);
    m1 = __builtin_amdgcn_ubfe(xm, sh + 8 + om, 4) | (__builtin_amdgcn_ubfe(s47, sh + 8 + oh, 2) << 4);
}

}  // namespace mmq
