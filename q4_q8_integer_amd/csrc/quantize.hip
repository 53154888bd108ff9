// quantize.hip - q8 activation quantizer for gfx950.
//
// Per token and 32-element block (the q8 activation definition: da =
// max|x|/127, q = round(x/da), ssum = sum q; the packed scale word of the
// r31 page, section 3.2: binary16 da low, signed 16-bit ssum high).
//
// The input rows are contiguous and k % 32 == 0, so the n*k/32 blocks are
// simply consecutive 128-byte runs of x: the kernel maps over blocks, not
// rows.  A DPP quad (4 lanes) owns one block, 8 floats per lane (two 16-byte
// loads); the block max and the sum are reduced inside the quad with
// quad_perm DPP moves (no LDS).  A wave reads 2 KiB contiguously and writes
// 512 contiguous bytes of q; the quantizer is HBM-bound (4 B read + 1.125 B
// written per element).
//
// The same kernel quantizes h = SiLU(gate) * up without writing h (the fused
// input of an FFN's down projection): the block's values are computed from
// the two inputs as they are loaded.
//
// Tiled output (q8_quantize_rows_tiled): the same codes and words, the codes
// written as the binary16 operands of the binary16-MFMA matmul, in its LDS
// stage order (token tiles of 128, k stages of 128, 32 KiB per tile and
// stage; a quantize-transpose pass ahead of the matmul).  A lane's 8 codes
// are exactly one 16-byte operand slot (k = 32c + 8 part .. +7, in the pair
// order 0,2,1,3,4,6,5,7), so the wave takes 16 consecutive tokens of one
// block index and its lanes of one part write 256 contiguous bytes.  Tokens
// past n (up to the tile's 128) get zero slots and no scale word.
//
// Numerics: x/da is the IEEE fp32 division (hipcc's default correctly
// rounded divide; never built with fast-math), roundf rounds ties away from
// zero, and v_cvt_f16_f32 rounds to nearest even keeping subnormals.
#include "internal.h"

namespace mmq {
namespace {

// quad_perm controls: lane i of each quad reads lane i^1, or lane i^2.
constexpr int kQuadXor1 = 0xB1;  // [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // [2,3,0,1]

__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                                __builtin_bit_cast(int, v), kQuadXor1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                                __builtin_bit_cast(int, v), kQuadXor2, 0xF, 0xF, false)));
    return v;
}

__device__ __forceinline__ int quad_sum(int v) {
    v += __builtin_amdgcn_mov_dpp(v, kQuadXor1, 0xF, 0xF, false);
    v += __builtin_amdgcn_mov_dpp(v, kQuadXor2, 0xF, 0xF, false);
    return v;
}

typedef float v4f __attribute__((ext_vector_type(4)));

// The 8 values of lane `part` of block `blk`: the activations themselves.
struct PlainSrc {
    const float* x;
    __device__ __forceinline__ void load(int64_t blk, int part, float (&v)[8]) const {
        const v4f* src = reinterpret_cast<const v4f*>(x + blk * 32 + part * 8);
        const v4f lo = __builtin_nontemporal_load(src);      // read once: do not keep in cache
        const v4f hi = __builtin_nontemporal_load(src + 1);
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    }
};

// h = SiLU(g) * u of the FFN's gate and up outputs, as the float32 rounding
// of the float64 value g*u / (1 + exp(-g)): g*u is exact in float64, then an
// IEEE add, an IEEE divide and the round to float32 (one function, exp, is
// the device library's), so h is the correctly rounded value but for a
// float64 ulp of exp.
struct SiluMulSrc {
    const float* g;
    const float* u;
    __device__ __forceinline__ void load(int64_t blk, int part, float (&v)[8]) const {
        const v4f* gs = reinterpret_cast<const v4f*>(g + blk * 32 + part * 8);
        const v4f* us = reinterpret_cast<const v4f*>(u + blk * 32 + part * 8);
        const v4f g0 = __builtin_nontemporal_load(gs), g1 = __builtin_nontemporal_load(gs + 1);
        const v4f u0 = __builtin_nontemporal_load(us), u1 = __builtin_nontemporal_load(us + 1);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double gd = (double)gv[i];
            const double den = 1.0 + exp(-gd);
            v[i] = (float)(gd * (double)uv[i] / den);
        }
    }
};

// TILES = false: quad i takes block i (row-major blocks), codes to q.
// TILES = true:  wave w takes block c = w % C of tokens 16 (w / C) .. +15
//                (one per quad), codes to the operand tiles qt.
template <class Src, bool TILES>
__global__ __launch_bounds__(256) void q8_quantize_kernel(Src src, int64_t nblocks, int n, int C,
                                                          int8_t* __restrict__ q,
                                                          uint16_t* __restrict__ qt,
                                                          uint32_t* __restrict__ ds) {
    const int64_t lane_id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int part = threadIdx.x & 3;
    int64_t blk = lane_id >> 2;  // quads are aligned, so a quad is all in or all out
    int tok = 0, c = 0;
    bool pad = false;
    if (TILES) {
        const int64_t w = lane_id >> 6;
        const int64_t tg = w / C;
        c = (int)(w - tg * C);
        tok = (int)(tg * 16 + ((lane_id >> 2) & 15));
        if (tok >= ((n + 127) & ~127)) return;   // past the last tile (whole waves)
        pad = tok >= n;
        blk = (int64_t)tok * C + c;
    } else if (blk >= nblocks) {
        return;
    }

    float v[8];
    if (TILES && pad) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    } else {
        src.load(blk, part, v);
    }

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = quad_max(amax);

    uint32_t packed[2] = {0u, 0u};
    int sum = 0;
    uint32_t word = 0u;
    if (amax > 0.0f) {
        const float da = amax / 127.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float r = roundf(v[i] / da);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            const int qi = (int)r;
            sum += qi;
            packed[i >> 2] |= (uint32_t)(qi & 0xFF) << (8 * (i & 3));
        }
        word = (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)da);
    }
    sum = quad_sum(sum);
    word |= (uint32_t)(uint16_t)(int16_t)sum << 16;

    if (TILES) {
        // slot ((cl * 2 + h) * 2 + g) * 128 + tt of block (tile, stage), part = 2 g + h
        const int cl = c & 3, g = part >> 1, h = part & 1;
        const int64_t stage = c >> 2, stages = C >> 2;
        const int64_t slot = (((int64_t)(tok >> 7) * stages + stage) * 16 + (cl * 2 + h) * 2 + g) * 128 +
                             (tok & 127);
        uint32_t hv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int qi = (int8_t)(uint8_t)(packed[i >> 2] >> (8 * (i & 3)));
            hv[i] = __builtin_bit_cast(unsigned short, (_Float16)(float)qi);   // exact
        }
        *reinterpret_cast<uint4*>(qt + slot * 8) =
            make_uint4(hv[0] | (hv[2] << 16), hv[1] | (hv[3] << 16), hv[4] | (hv[6] << 16),
                       hv[5] | (hv[7] << 16));
        if (part == 0 && !pad) ds[blk] = word;
    } else {
        *reinterpret_cast<uint2*>(q + blk * 32 + part * 8) = make_uint2(packed[0], packed[1]);
        if (part == 0) ds[blk] = word;
    }
}

template <class Src>
hipError_t launch(Src src, int64_t nblocks, int8_t* q, uint32_t* ds, hipStream_t stream) {
    const int64_t lanes = nblocks * 4;
    const unsigned grid = (unsigned)((lanes + 255) / 256);
    hipLaunchKernelGGL((q8_quantize_kernel<Src, false>), dim3(grid), dim3(256), 0, stream, src, nblocks,
                       0, 0, q, (uint16_t*)nullptr, ds);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_q8_quantize(const float* x, int64_t nblocks, int8_t* q, uint32_t* ds,
                              hipStream_t stream) {
    return launch(PlainSrc{x}, nblocks, q, ds, stream);
}

// 16 tokens x one block per wave, over whole tiles of 128 tokens.
template <class Src>
hipError_t launch_tiled(Src src, int n, int k, uint16_t* qt, uint32_t* ds, hipStream_t stream) {
    const int C = k / 32;
    const int64_t waves = (int64_t)((n + 127) / 128) * 8 * C;
    const unsigned grid = (unsigned)((waves * 64 + 255) / 256);
    hipLaunchKernelGGL((q8_quantize_kernel<Src, true>), dim3(grid), dim3(256), 0, stream, src,
                       (int64_t)n * C, n, C, (int8_t*)nullptr, qt, ds);
    return hipGetLastError();
}

hipError_t launch_q8_quantize_tiled(const float* x, int n, int k, uint16_t* qt, uint32_t* ds,
                                    hipStream_t stream) {
    return launch_tiled(PlainSrc{x}, n, k, qt, ds, stream);
}

hipError_t launch_q8_quantize_silu_mul_tiled(const float* g, const float* u, int n, int k, uint16_t* qt,
                                             uint32_t* ds, hipStream_t stream) {
    return launch_tiled(SiluMulSrc{g, u}, n, k, qt, ds, stream);
}

hipError_t launch_q8_quantize_silu_mul(const float* g, const float* u, int64_t nblocks, int8_t* q,
                                       uint32_t* ds, hipStream_t stream) {
    return launch(SiluMulSrc{g, u}, nblocks, q, ds, stream);
}

}  // namespace mmq
