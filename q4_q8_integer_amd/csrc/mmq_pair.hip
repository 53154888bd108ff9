// mmq_pair.hip - q4_K x q8 matmul for 9..16 tokens, float32 or binary16
// result: weights streamed once from HBM, one int8 matrix-core instruction
// per chunk pair, 8 tokens and 16 weight rows.
//
// The method is the one of the other kernels (the yusiwen.cn "minfer" r31
// page, sections 1-2: an exact integer dot per 32-weight chunk, then the
// two-term fold d*sc*da*D - dmin*m*da*ssum).  What is particular here is how
// the chunks meet v_mfma_i32_16x16x64_i8 (16 bytes of k per lane):
//
//   * The 16 B columns are 16 weight rows.  Lane (row r, k-group g) holds the
//     16 qs bytes 32p + 16(g & 1) .. +15 of chunk pair p, as low nibbles for
//     g < 2 (chunk 2p) and high nibbles for g >= 2 (chunk 2p+1): one 16-byte
//     load per lane and pair, no shuffling.
//   * The 16 A rows are 8 tokens x 2 chunk halves: row (t, h) carries token
//     t's bytes of chunk 2p + h in the k-groups of half h and zeros in the
//     other half, so one instruction returns the two chunks' dots apart:
//     D[(t, h)][r] = chunk (2p + h) dot of token t and row r.  The zeros come
//     from buffer loads with an offset past the end (a buffer resource reads 0
//     there), not from instructions.
//   * Per value: acc += (da*d*sc) * D + (-dmin*m) * (da*ssum), four VALU
//     operations for 8 tokens x 16 rows x 2 chunks per instruction.
//   * A wave step covers 16 rows x 2 consecutive super-blocks; all of a
//     step's loads are issued before its math.  The waves of a workgroup
//     split the super-blocks and their partial sums are added in a fixed order
//     (the two chunk halves of a lane pair, then the waves in index order).
#include "internal.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;        // waves per workgroup (split of the super-blocks)
constexpr int SW = 2;            // super-blocks per wave step
constexpr int kBufferFlags = 0x00020000;  // word 3 of a raw buffer resource on gfx950
constexpr uint32_t kPastEnd = 0x80000000u;  // an offset beyond any q extent: reads 0

__device__ __forceinline__ float half_lo(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

// 6-bit (sc, m) of chunk j (GGUF k-quant scale packing): chunks 0-3 keep the
// low 6 bits of scale bytes j (sc) and j+4 (m); chunks 4-7 take a nibble of
// byte j+4 (low: sc, high: m) topped with the 2 high bits of byte j-4 (sc) or
// j (m).
__device__ __forceinline__ void scale_min(const v4u h, int j, uint32_t& sc, uint32_t& mn) {
    const int sh = 8 * (j & 3);
    if (j < 4) {
        sc = __builtin_amdgcn_ubfe(h[1], sh, 6);
        mn = __builtin_amdgcn_ubfe(h[2], sh, 6);
    } else {
        sc = __builtin_amdgcn_ubfe(h[3], sh, 4) | (__builtin_amdgcn_ubfe(h[1], sh + 6, 2) << 4);
        mn = __builtin_amdgcn_ubfe(h[3], sh + 4, 4) | (__builtin_amdgcn_ubfe(h[2], sh + 6, 2) << 4);
    }
}

template <int G>
struct Step {
    v4u hdr[SW];
    v4u qsp[SW][4];        // [super-block][pair]: this lane's 16 qs bytes
    v4u tok[SW][G][4];     // [super-block][token group][pair]: A operand (zeros off-half)
    uint2 words[G];        // two scale words of (token, super-block, chunk pair)
};

template <int G, bool H>
__global__ __launch_bounds__(64 * kWaves) void mmq_pair_kernel(const uint8_t* __restrict__ w,
                                                               const int8_t* __restrict__ q,
                                                               const uint32_t* __restrict__ ds,
                                                               int M, int N, int K,
                                                               void* __restrict__ out) {
    constexpr int NTOK = 8 * G;
    // decoded scales of the current step: [super-block][chunk][token]
    __shared__ float sDa[kWaves][SW][8][NTOK];
    __shared__ float sDass[kWaves][SW][8][NTOK];
    __shared__ float red[kWaves][NTOK][16];

    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane & 15, kg = lane >> 4;
    const int t8 = lane & 7, ah = (lane >> 3) & 1;  // A row (token, half) of this lane
    const int row0 = blockIdx.x * 16;
    const int S = K >> 8, C = K >> 5;
    const int sb0 = (int)((int64_t)S * wv / W), sb1 = (int)((int64_t)S * (wv + 1) / W);
    const int last = sb1 - 1;
    const uint8_t* wrow = w + (int64_t)min(row0 + r, M - 1) * S * kBlockBytes;

    const __amdgpu_buffer_rsrc_t qr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(q), 0, N * K, kBufferFlags);
    // A-operand byte offset of token group g in super-block 0, pair 0 (past
    // the end where this lane's half is not the k-group's half, or for
    // padded tokens)
    uint32_t aoff[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int t = 8 * g + t8;
        aoff[g] = (ah == (kg >> 1) && t < N) ? (uint32_t)(t * K + 16 * kg) : kPastEnd;
    }
    // scale words: lane -> token (lane >> 3) + 8g, super-block (lane >> 2) & 1
    // of the step, chunk pair lane & 3
    const int wt = lane >> 3, wj = (lane >> 2) & 1, wp = lane & 3;

    float acc[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g][i] = 0.0f;

    for (int s = sb0; s < sb1; s += SW) {
        const int ns = min(SW, sb1 - s);
        // ---- every load of the step, unconditional (slots past the wave's
        // last super-block re-read it and are computed with d = dmin = 0)
        Step<G> st;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = min(8 * g + wt, N - 1);
            st.words[g] = *reinterpret_cast<const uint2*>(ds + (int64_t)t * C + min(s + wj, last) * 8 + 2 * wp);
        }
#pragma unroll
        for (int j = 0; j < SW; ++j) {
            const int sb = min(s + j, last);
            const uint8_t* b = wrow + (int64_t)sb * kBlockBytes;
            st.hdr[j] = *reinterpret_cast<const v4u*>(b);
#pragma unroll
            for (int p = 0; p < 4; ++p)
                st.qsp[j][p] = *reinterpret_cast<const v4u*>(b + 16 + 32 * p + 16 * (kg & 1));
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t o = aoff[g] == kPastEnd ? kPastEnd : aoff[g] + sb * 256 + 64 * p;
                    st.tok[j][g][p] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(qr, o, 0, 0));
                }
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- decoded scales to the wave's LDS table (LDS accesses of one
        // wave are in order: these writes precede the reads below, and the
        // previous step's reads precede them)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t wd[2] = {st.words[g].x, st.words[g].y};
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float da = half_lo(wd[e]);
                sDa[wv][wj][2 * wp + e][8 * g + wt] = da;
                sDass[wv][wj][2 * wp + e][8 * g + wt] = da * (float)(int16_t)(uint16_t)(wd[e] >> 16);
            }
        }

        // ---- compute
#pragma unroll
        for (int j = 0; j < SW; ++j) {
            const bool live = j < ns;
            const v4u h = st.hdr[j];
            const float d = live ? half_lo(h[0]) : 0.0f, dmin = live ? half_lo(h[0] >> 16) : 0.0f;
            const int nshift = 4 * (kg >> 1);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                // this lane's output chunk: 2p + (kg >> 1)
                uint32_t sc0, mn0, sc1, mn1;
                scale_min(h, 2 * p, sc0, mn0);
                scale_min(h, 2 * p + 1, sc1, mn1);
                const bool odd = (kg >> 1) != 0;
                const float dsc = d * (float)(odd ? sc1 : sc0);
                const float dmm = -(dmin * (float)(odd ? mn1 : mn0));
                const int ch = 2 * p + (kg >> 1);
                v4i bop;
#pragma unroll
                for (int i = 0; i < 4; ++i) bop[i] = (int)((st.qsp[j][p][i] >> nshift) & 0x0F0F0F0Fu);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        __builtin_bit_cast(v4i, st.tok[j][g][p]), bop, v4i{0, 0, 0, 0}, 0, 0, 0);
                    const int t0 = 8 * g + 4 * (kg & 1);
                    const float4 da4 = *reinterpret_cast<const float4*>(&sDa[wv][j][ch][t0]);
                    const float4 ds4 = *reinterpret_cast<const float4*>(&sDass[wv][j][ch][t0]);
                    const float dav[4] = {da4.x, da4.y, da4.z, da4.w};
                    const float dsv[4] = {ds4.x, ds4.y, ds4.z, ds4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[g][i] = fmaf(dav[i] * dsc, (float)D[i], acc[g][i]);
                        acc[g][i] = fmaf(dmm, dsv[i], acc[g][i]);
                    }
                }
            }
        }
    }

    // a lane holds tokens 8g + 4(kg & 1) + i for chunk half kg >> 1: add the
    // two halves (lanes kg and kg ^ 2), then the waves in index order
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[g][i] += __shfl_xor(acc[g][i], 32);
            if (kg < 2) red[wv][8 * g + 4 * kg + i][r] = acc[g][i];
        }
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * NTOK; e += blockDim.x) {
        const int t = e >> 4, rr = e & 15;
        if (t >= N || row0 + rr >= M) continue;
        float sum = red[0][t][rr];
        for (int v = 1; v < W; ++v) sum += red[v][t][rr];
        store_out<H>(out, (int64_t)t * M + row0 + rr, sum);
    }
}

template <int G>
hipError_t launch_g(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
                    void* out, bool half_out, hipStream_t stream) {
    const int S = k / 256;
    const int rows = (m + 15) / 16;
    const int waves = S < kWaves ? S : kWaves;
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k, (void*)&out};
    const void* f = half_out ? (const void*)mmq_pair_kernel<G, true> : (const void*)mmq_pair_kernel<G, false>;
    return hipLaunchKernel(f, dim3((unsigned)rows), dim3(64 * waves), args, 0, stream);
}

}  // namespace

hipError_t launch_mmq_fp32_pair(const uint8_t* w, int m, int k, const int8_t* q,
                                const uint32_t* ds, int n, void* out, bool half_out,
                                hipStream_t stream) {
    if (n <= 8) return launch_g<1>(w, m, k, q, ds, n, out, half_out, stream);
    if (n <= 16) return launch_g<2>(w, m, k, q, ds, n, out, half_out, stream);
    return hipErrorInvalidValue;
}

}  // namespace mmq
