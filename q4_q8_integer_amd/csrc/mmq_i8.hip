// mmq_i8.hip - q4_K x q8 quantized matmul on gfx950 int8 MFMA.
//
// Method (the yusiwen.cn "minfer" r31 page, sections 1-2): per 32-element
// chunk c an exact integer dot product D = sum q4*q8, then the two-term
// rank-1 fold  out += (d*sc)[o,c]*da[t,c]*D - (dmin*m)[o,c]*da[t,c]*ssum[t,c].
//
// gfx950 mapping
//   * One v_mfma_i32_32x32x32_i8 is exactly one chunk (K = 32) of a 32-row x
//     32-token tile, so the i32 result of each MFMA is D itself (C = 0): no
//     reformulation of the method is needed.
//   * Weights are the MFMA A operand (rows), tokens the B operand (columns).
//     In the 32x32 accumulator layout a lane holds one column (token) and 16
//     rows, so the activation scale da is a per-lane scalar in the epilogue.
//   * A lane's 16 A bytes are the nibbles of 16 consecutive q4_K qs bytes:
//     one 16-byte LDS read feeds chunk 2p (low nibbles, AND 0x0F0F0F0F) and
//     chunk 2p+1 (high nibbles, shift + AND).  The B operand takes the q8
//     bytes of the same 16 k positions, so A and B agree on k.
//   * Workgroup tile 128 rows x 128 tokens, 4 waves of 64x64 (2x2 MFMA
//     tiles); one q4_K super-block (256 k) is staged per step.
//   * LDS row strides are 144 B (one whole q4_K block) and 272 B (256 q8 +
//     16 pad): both advance 4 banks per row, so the 16-byte operand reads of
//     8 consecutive rows touch 32 distinct banks.
//
// Epilogues (template parameter):
//   kDots  exact int32 dots[t][o][c] (parity / inspection entry point);
//   kFp32  float32 out[t][o] with the two-term fold applied per chunk;
//   kF16   the same, stored as binary16 (nearest-even from the float32 value).
#include "internal.h"
#include "kquant_device.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;            // weight rows per workgroup
constexpr int BN = 128;            // tokens per workgroup
constexpr int NT = 256;            // threads per workgroup (4 waves)
constexpr int W_STRIDE = 144;      // LDS bytes per weight row (one q4_K block)
constexpr int X_STRIDE = 272;      // LDS bytes per token row (256 q8 + pad)

enum { kDots = 0, kFp32 = 1, kF16 = 2 };

template <int EPI>
__global__ __launch_bounds__(NT) void mmq_i8_kernel(const uint8_t* __restrict__ w,
                                                    const int8_t* __restrict__ q,
                                                    const uint32_t* __restrict__ ds,
                                                    int M, int N, int K, int tiles_m,
                                                    void* __restrict__ outp) {
    __shared__ __attribute__((aligned(16))) uint8_t sW[BM * W_STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t sX[BN * X_STRIDE];
    __shared__ __attribute__((aligned(16))) float sDsc[8][BM];   // d*sc per (chunk, row)
    __shared__ __attribute__((aligned(16))) float sNdm[8][BM];   // -dmin*m per (chunk, row)
    __shared__ __attribute__((aligned(16))) float2 sXs[8][BN];   // (da, da*ssum) per (chunk, token)

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int g = lane >> 5, l32 = lane & 31;
    const int bm = blockIdx.x % tiles_m, bn = blockIdx.x / tiles_m;
    const int row0 = bm * BM, tok0 = bn * BN;
    const int S = K >> 8, C = K >> 5;

    float acc[2][2][16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

    for (int sb = 0; sb < S; ++sb) {
        __syncthreads();  // every wave is done reading the previous stage
        // ---- stage the weight blocks: BM rows x 9 x 16 B
        for (int i = tid; i < BM * 9; i += NT) {
            const int r = i / 9, p = i - r * 9;
            const int row = min(row0 + r, M - 1);
            const uint4 v = *reinterpret_cast<const uint4*>(
                w + ((int64_t)row * S + sb) * kBlockBytes + p * 16);
            *reinterpret_cast<uint4*>(sW + r * W_STRIDE + p * 16) = v;
            if (EPI != kDots && p == 0) {
                const float d = half_lo(v.x);
                const float dmin = half_lo(v.x >> 16);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    int sc, mn;
                    scale_min(v.y, v.z, v.w, j, sc, mn);
                    sDsc[j][r] = d * (float)sc;
                    sNdm[j][r] = -(dmin * (float)mn);
                }
            }
        }
        // ---- stage the q8 tile: BN tokens x 16 x 16 B
        for (int i = tid; i < BN * 16; i += NT) {
            const int t = i >> 4, p = i & 15;
            const int tok = min(tok0 + t, N - 1);
            const uint4 v = *reinterpret_cast<const uint4*>(q + (int64_t)tok * K + sb * 256 + p * 16);
            *reinterpret_cast<uint4*>(sX + t * X_STRIDE + p * 16) = v;
        }
        if (EPI != kDots) {
            for (int i = tid; i < BN * 8; i += NT) {
                const int t = i >> 3, j = i & 7;
                const int tok = min(tok0 + t, N - 1);
                const uint32_t word = ds[(int64_t)tok * C + sb * 8 + j];
                const float da = half_lo(word);
                const float ss = (float)(int16_t)(uint16_t)(word >> 16);
                sXs[j][t] = make_float2(da, da * ss);  // exact: 11 x 13 significant bits
            }
        }
        __syncthreads();

        // ---- contract: 4 pairs of chunks per super-block
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            v4i araw[2], bop[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                araw[mt] = *reinterpret_cast<const v4i*>(
                    sW + (wm * 64 + mt * 32 + l32) * W_STRIDE + 16 + 32 * p + 16 * g);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    bop[nt][h] = *reinterpret_cast<const v4i*>(
                        sX + (wn * 64 + nt * 32 + l32) * X_STRIDE + 64 * p + 32 * h + 16 * g);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j = 2 * p + h;  // chunk within the super-block
                v4i aop[2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    aop[mt] = h ? ((araw[mt] >> 4) & 0x0F0F0F0F) : (araw[mt] & 0x0F0F0F0F);
                v16i D[2][2];
                const v16i zero = {};
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        D[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[mt], bop[nt][h], zero, 0, 0, 0);

                if (EPI == kDots) {
                    int32_t* dots = reinterpret_cast<int32_t*>(outp);
                    const int c = sb * 8 + j;
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            const int tok = tok0 + wn * 64 + nt * 32 + l32;
                            if (tok >= N) continue;
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const int o = row0 + wm * 64 + mt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
                                if (o < M) dots[((int64_t)tok * M + o) * C + c] = D[mt][nt][v];
                            }
                        }
                } else {
                    float2 xs[2];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) xs[nt] = sXs[j][wn * 64 + nt * 32 + l32];
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int r = wm * 64 + mt * 32 + 8 * jj + 4 * g;
                            const float4 dsc = *reinterpret_cast<const float4*>(&sDsc[j][r]);
                            const float4 ndm = *reinterpret_cast<const float4*>(&sNdm[j][r]);
                            const float dscv[4] = {dsc.x, dsc.y, dsc.z, dsc.w};
                            const float ndmv[4] = {ndm.x, ndm.y, ndm.z, ndm.w};
#pragma unroll
                            for (int i = 0; i < 4; ++i)
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    const int v = 4 * jj + i;
                                    float a = acc[mt][nt][v];
                                    a = fmaf(dscv[i] * xs[nt].x, (float)D[mt][nt][v], a);
                                    a = fmaf(ndmv[i], xs[nt].y, a);
                                    acc[mt][nt][v] = a;
                                }
                        }
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
    return hipLaunchKernel((const void*)mmq_i8_kernel<EPI>, dim3((unsigned)tiles), dim3(NT),
                           args, 0, stream);
}

}  // namespace

hipError_t launch_mmq_dots(const uint8_t* w, int m, int k, const int8_t* q, int n,
                           int32_t* dots, hipStream_t stream) {
    return launch<kDots>(w, m, k, q, nullptr, n, dots, stream);
}

hipError_t launch_mmq_fp32(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                           int n, void* out, bool half_out, hipStream_t stream) {
    return half_out ? launch<kF16>(w, m, k, q, ds, n, out, stream)
                    : launch<kFp32>(w, m, k, q, ds, n, out, stream);
}

}  // namespace mmq
