// mmq_q6k_i8.hip - q6_K x q8 quantized matmul on gfx950 int8 MFMA (any n).
//
// The q6_K weight format (the second k-quant, named in the r31 page's
// closing notes of the yusiwen.cn "minfer" pages) carries one signed 8-bit
// scale per 16 weights and no min term, so the method becomes: per 16-weight
// group g an exact integer dot D = sum (q - 32) * q8, then
//   out[t][o] = sum_g d[o] * sc[o,g] * da[t, g/2] * D[t][o][g].
//
// gfx950 mapping
//   * One v_mfma_i32_32x32x16_i8 is exactly one scale group (k = 16) of a
//     32-row x 32-token tile: its i32 result is D itself.
//   * The weights are decoded once per workgroup and super-block into LDS as
//     signed codes q - 32 in weight order (int8: -32..31), so the A operand
//     is 8 plain bytes like the q8 B operand.
//   * Per 32-element chunk (two groups, one da):
//         I = sc[g0] * D0 + sc[g1] * D1      (24-bit integer multiply-adds;
//                                              |I| < 2^24, exact in float32)
//         acc_b += da * float(I)
//     and per super-block out += d * acc_b.
//   * Workgroup tile 128 rows x 128 tokens, 4 waves of 64x64 (2x2 MFMA tiles),
//     one super-block (256 k) staged per step.  LDS rows are 272 bytes
//     (256 + 16 pad) for both operands; with the scales as 16-bit values a
//     workgroup takes under 80 KB, so two share a CU.
//
// Epilogues: kDots (exact int32 group dots[t][o][g], the parity entry), kFp32
// (float32 out[t][o]), kF16 (the same float32 value stored as binary16).
#include "internal.h"
#include "q6k_device.h"

namespace mmq {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;            // weight rows per workgroup
constexpr int BN = 128;            // tokens per workgroup
constexpr int NT = 256;            // threads per workgroup (4 waves)
constexpr int STRIDE = 272;        // LDS bytes per row of either operand

enum { kDots = 0, kFp32 = 1, kF16 = 2 };

template <int EPI>
__global__ __launch_bounds__(NT, 2) void mmq_q6k_i8_kernel(const uint8_t* __restrict__ w,
                                                        const int8_t* __restrict__ q,
                                                        const uint32_t* __restrict__ ds,
                                                        int M, int N, int K, int tiles_m,
                                                        void* __restrict__ outp) {
    __shared__ __attribute__((aligned(16))) uint8_t sW[BM * STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t sX[BN * STRIDE];
    __shared__ __attribute__((aligned(16))) short sSc[16][BM];   // scale per (group, row)
    __shared__ __attribute__((aligned(16))) float sD[BM];        // d per row
    __shared__ __attribute__((aligned(16))) float sDa[8][BN];    // da per (chunk, token)

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int g = lane >> 5, l32 = lane & 31;
    const int bm = blockIdx.x % tiles_m, bn = blockIdx.x / tiles_m;
    const int row0 = bm * BM, tok0 = bn * BN;
    const int S = K >> 8, C = K >> 5, G = K >> 4;

    float acc[2][2][16], accb[2][2][16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = accb[a][b][v] = 0.0f;

    for (int sb = 0; sb < S; ++sb) {
        __syncthreads();  // every wave is done reading the previous stage
        // ---- weights: BM rows x 4 quarters, each 64 signed codes
        for (int i = tid; i < BM * 4; i += NT) {
            const int r = i >> 2, p = i & 3, h = p >> 1, e = p & 1;
            const int row = min(row0 + r, M - 1);
            const int64_t B = ((int64_t)row * S + sb) * kQ6kBlockBytes;
            const uint32_t sh = (uint32_t)B & 3u;
            uint32_t ql0[5], ql1[5], qh[5], cw[4][4];
            q6k::load_run(w, B, q6k::ql0_off(h, e), sh, ql0);
            q6k::load_run(w, B, q6k::ql1_off(h, e), sh, ql1);
            q6k::load_run(w, B, q6k::qh_off(h, e), sh, qh);
            q6k::quarter_codes(ql0, ql1, qh, sh, cw);
#pragma unroll
            for (int gg = 0; gg < 4; ++gg)
                *reinterpret_cast<uint4*>(sW + r * STRIDE + 128 * h + 32 * gg + 16 * e) =
                    make_uint4(cw[gg][0], cw[gg][1], cw[gg][2], cw[gg][3]);
        }
        if (EPI != kDots) {
            for (int r = tid; r < BM; r += NT) {
                const int row = min(row0 + r, M - 1);
                const int64_t B = ((int64_t)row * S + sb) * kQ6kBlockBytes;
                const uint32_t sh = (uint32_t)B & 3u;
                uint32_t sv[5];
                q6k::load_run(w, B, 192, sh, sv, 12);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t word = q6k::run_word(sv, j, sh);
#pragma unroll
                    for (int b = 0; b < 4; ++b) sSc[4 * j + b][r] = (short)(int8_t)(word >> (8 * b));
                }
                sD[r] = half_lo(*reinterpret_cast<const uint16_t*>(w + B + 208));
            }
        }
        // ---- q8 tile: BN tokens x 16 x 16 B
        for (int i = tid; i < BN * 16; i += NT) {
            const int t = i >> 4, p = i & 15;
            const int tok = min(tok0 + t, N - 1);
            *reinterpret_cast<uint4*>(sX + t * STRIDE + p * 16) =
                *reinterpret_cast<const uint4*>(q + (int64_t)tok * K + sb * 256 + p * 16);
        }
        if (EPI != kDots) {
            for (int i = tid; i < BN * 8; i += NT) {
                const int t = i >> 3, j = i & 7;
                const int tok = min(tok0 + t, N - 1);
                sDa[j][t] = half_lo(ds[(int64_t)tok * C + sb * 8 + j]);
            }
        }
        __syncthreads();

        // ---- contract: 8 chunks of two scale groups
#pragma unroll 2
        for (int c = 0; c < 8; ++c) {
            int64_t aop[2][2], bop[2][2];  // [group half][tile]
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    aop[hh][mt] = *reinterpret_cast<const int64_t*>(
                        sW + (wm * 64 + mt * 32 + l32) * STRIDE + 32 * c + 16 * hh + 8 * g);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    bop[hh][nt] = *reinterpret_cast<const int64_t*>(
                        sX + (wn * 64 + nt * 32 + l32) * STRIDE + 32 * c + 16 * hh + 8 * g);
            }
            if (EPI == kDots) {
                int32_t* dots = reinterpret_cast<int32_t*>(outp);
                const v16i zero = {};
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            const v16i D = __builtin_amdgcn_mfma_i32_32x32x16_i8(aop[hh][mt], bop[hh][nt],
                                                                                 zero, 0, 0, 0);
                            const int tok = tok0 + wn * 64 + nt * 32 + l32;
                            if (tok >= N) continue;
                            const int gi = sb * 16 + 2 * c + hh;
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const int o = row0 + wm * 64 + mt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
                                if (o < M) dots[((int64_t)tok * M + o) * G + gi] = D[v];
                            }
                        }
            } else {
                float da[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) da[nt] = sDa[c][wn * 64 + nt * 32 + l32];
                const v16i zero = {};
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    int s0[16], s1[16];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r = wm * 64 + mt * 32 + 8 * jj + 4 * g;
                        const uint2 a = *reinterpret_cast<const uint2*>(&sSc[2 * c][r]);
                        const uint2 b = *reinterpret_cast<const uint2*>(&sSc[2 * c + 1][r]);
                        s0[4 * jj] = (short)a.x; s0[4 * jj + 1] = (int)a.x >> 16;
                        s0[4 * jj + 2] = (short)a.y; s0[4 * jj + 3] = (int)a.y >> 16;
                        s1[4 * jj] = (short)b.x; s1[4 * jj + 1] = (int)b.x >> 16;
                        s1[4 * jj + 2] = (short)b.y; s1[4 * jj + 3] = (int)b.y >> 16;
                    }
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const v16i D0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(aop[0][mt], bop[0][nt], zero, 0, 0, 0);
                        const v16i D1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(aop[1][mt], bop[1][nt], zero, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int I = __mul24(D0[v], s0[v]) + __mul24(D1[v], s1[v]);
                            accb[mt][nt][v] = fmaf(da[nt], (float)I, accb[mt][nt][v]);
                        }
                    }
                }
            }
        }
        if (EPI != kDots) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float4 d4 = *reinterpret_cast<const float4*>(&sD[wm * 64 + mt * 32 + 8 * jj + 4 * g]);
                    const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int v = 4 * jj + i;
                            acc[mt][nt][v] = fmaf(dv[i], accb[mt][nt][v], acc[mt][nt][v]);
                            accb[mt][nt][v] = 0.0f;
                        }
                }
        }
    }

    if (EPI != kDots) {
        constexpr bool H = EPI == kF16;
        const bool vec = (M & 3) == 0;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int tok = tok0 + wn * 64 + nt * 32 + l32;
                if (tok >= N) continue;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int o = row0 + wm * 64 + mt * 32 + 8 * jj + 4 * g;
                    const int64_t idx = (int64_t)tok * M + o;
                    if (vec && o + 3 < M) {
                        store_out4<H>(outp, idx, acc[mt][nt][4 * jj], acc[mt][nt][4 * jj + 1],
                                      acc[mt][nt][4 * jj + 2], acc[mt][nt][4 * jj + 3]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (o + i < M) store_out<H>(outp, idx + i, acc[mt][nt][4 * jj + i]);
                    }
                }
            }
    }
}

template <int EPI>
hipError_t launch(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
                  void* out, hipStream_t stream) {
    int tiles_m = (m + BM - 1) / BM;
    const int64_t tiles = (int64_t)tiles_m * ((n + BN - 1) / BN);
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k,
                    (void*)&tiles_m, (void*)&out};
    return hipLaunchKernel((const void*)mmq_q6k_i8_kernel<EPI>, dim3((unsigned)tiles), dim3(NT),
                           args, 0, stream);
}

}  // namespace

hipError_t launch_q6k_dots(const uint8_t* w, int m, int k, const int8_t* q, int n,
                           int32_t* dots, hipStream_t stream) {
    return launch<kDots>(w, m, k, q, nullptr, n, dots, stream);
}

hipError_t launch_q6k_i8(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                         int n, void* out, bool half_out, hipStream_t stream) {
    return half_out ? launch<kF16>(w, m, k, q, ds, n, out, stream)
                    : launch<kFp32>(w, m, k, q, ds, n, out, stream);
}

}  // namespace mmq
