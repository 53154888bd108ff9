// mmq_gemv.hip - q4_K x q8 matmul for very few tokens (1 <= n <= 8), float32
// result, on the vector ALU's 4-way int8 dot product instead of the matrix
// cores.
//
// The method is the one of the other kernels (the yusiwen.cn "minfer" r31
// page, sections 1-2: an exact integer dot per 32-weight chunk, then the
// two-term fold d*sc*da*D - dmin*m*da*ssum).  With a handful of tokens a
// matrix-core tile of 16 tokens is mostly padding, and its fp32 fold costs
// the same for padding as for real tokens; here every instruction serves a
// real (row, token) pair:
//
//   * A wave owns 16 weight rows.  Lane 16p + r takes row r and chunk pair p
//     of every super-block: qs bytes 32p..32p+31, whose low nibbles are chunk
//     2p and high nibbles chunk 2p+1.  Per token, a chunk's dot is 8 v_dot4
//     over nibble words (x & 0x0F0F0F0F, (x >> 4) & 0x0F0F0F0F) and the
//     token's q8 bytes 64p..64p+63 of the super-block.
//   * The 16 lanes of a DPP row share p, so they need the same token bytes:
//     each lane loads one 16-byte piece (together one coalesced KiB per token
//     and step) and v_dot4c reads the piece of the lane that holds it through
//     a row_newbcast DPP operand.  Token data never goes through LDS.  The
//     decoded scales (da, da*ssum) are broadcast the same way into v_fmac.
//   * A wave step covers 16 rows x 4 consecutive super-blocks (16 runs of
//     576 contiguous bytes): reading q4_K in runs of several blocks per row
//     keeps HBM close to its streaming rate, where one block from each of
//     many rows does not.
//   * A workgroup is 16 rows; its waves split the super-blocks, and the
//     partial sums are added in a fixed order (a butterfly over the four
//     chunk-pair lanes of a row, then the waves in index order): results do
//     not depend on timing.
#include "internal.h"

namespace mmq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kMaxWaves = 4;   // waves per workgroup (split of the super-blocks)
constexpr int kStepSb = 4;     // super-blocks per wave step

__device__ __forceinline__ float half_lo(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

__device__ __forceinline__ v4u ld16(const void* p) { return *reinterpret_cast<const v4u*>(p); }

// The two chunk dots of pair p in super-block J of the step, for one token:
//   D0 = sum_i dot4(lo[i], token word i),  D1 = sum_i dot4(hi[i], word 8 + i)
// where token words 4c..4c+3 sit in lane 4J + c of the DPP row (row_newbcast).
// Inline asm hides the instructions from the compiler's hazard checks, so
// the block carries its own: s_nop 1 before (a DPP read needs 2 wait states
// after a VALU write of its source) and s_nop 2 after (a VALU other than
// another dot reading a v_dot4 result needs 3).  The two chains interleave.
template <int J>
__device__ __forceinline__ void dot_pair_bcast(int& D0, int& D1, v4u t, const int* lo,
                                               const int* hi) {
    D0 = 0;
    D1 = 0;
    asm("s_nop 1\n\t"
        "v_dot4c_i32_i8_dpp %0, %2, %6 row_newbcast:%c22 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %2, %14 row_newbcast:%c24 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %3, %7 row_newbcast:%c22 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %3, %15 row_newbcast:%c24 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %4, %8 row_newbcast:%c22 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %4, %16 row_newbcast:%c24 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %5, %9 row_newbcast:%c22 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %5, %17 row_newbcast:%c24 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %2, %10 row_newbcast:%c23 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %2, %18 row_newbcast:%c25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %3, %11 row_newbcast:%c23 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %3, %19 row_newbcast:%c25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %4, %12 row_newbcast:%c23 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %4, %20 row_newbcast:%c25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %5, %13 row_newbcast:%c23 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %5, %21 row_newbcast:%c25 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 2"
        : "+v"(D0), "+v"(D1)
        : "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]),
          "v"(lo[0]), "v"(lo[1]), "v"(lo[2]), "v"(lo[3]), "v"(lo[4]), "v"(lo[5]), "v"(lo[6]), "v"(lo[7]),
          "v"(hi[0]), "v"(hi[1]), "v"(hi[2]), "v"(hi[3]), "v"(hi[4]), "v"(hi[5]), "v"(hi[6]), "v"(hi[7]),
          "n"(4 * J), "n"(4 * J + 1), "n"(4 * J + 2), "n"(4 * J + 3));
}

// acc + a * (b of lane L of the DPP row)
template <int L>
__device__ __forceinline__ float fma_bcast(float acc, float b, float a) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %1, %2 row_newbcast:%c3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(b), "v"(a), "n"(L));
    return acc;
}

// One super-block J of the step for every token.  A slot past the wave's
// last super-block (live false) runs with d = dmin = 0 and adds exactly 0:
// no branch, so the compiler keeps all of the step's loads ahead of the math.
template <int N, int J>
__device__ __forceinline__ void gemv_sb(const v4u h, const v4u qa, const v4u qb, int p, bool live,
                                        const v4u* tq, const float* tda, const float* tdass,
                                        float* acc) {
    const float d = live ? half_lo(h[0]) : 0.0f, dmin = live ? half_lo(h[0] >> 16) : 0.0f;
    // 6-bit (sc, m) of chunks 2p and 2p+1 (GGUF k-quant scale packing).
    // Chunks 0-3: low 6 bits of scale bytes j (sc) and j+4 (m).  Chunks 4-7:
    // a nibble of byte j+4 (low: sc, high: m) topped with the 2 high bits of
    // byte j-4 (sc) or j (m).  Both cases as a 4-bit field plus a 2-bit
    // field, so no lane branches.
    const bool lo4 = p < 2;
    const int sh = 16 * (p & 1);
    const uint32_t xs = lo4 ? h[1] : h[3], xm = lo4 ? h[2] : h[3];
    const int oh = lo4 ? 4 : 6, om = lo4 ? 0 : 4;
    const uint32_t sc0 = __builtin_amdgcn_ubfe(xs, sh, 4) | (__builtin_amdgcn_ubfe(h[1], sh + oh, 2) << 4);
    const uint32_t sc1 = __builtin_amdgcn_ubfe(xs, sh + 8, 4) | (__builtin_amdgcn_ubfe(h[1], sh + 8 + oh, 2) << 4);
    const uint32_t m0 = __builtin_amdgcn_ubfe(xm, sh + om, 4) | (__builtin_amdgcn_ubfe(h[2], sh + oh, 2) << 4);
    const uint32_t m1 = __builtin_amdgcn_ubfe(xm, sh + 8 + om, 4) | (__builtin_amdgcn_ubfe(h[2], sh + 8 + oh, 2) << 4);
    const float dsc0 = d * (float)sc0, dsc1 = d * (float)sc1;
    const float dmm0 = -(dmin * (float)m0), dmm1 = -(dmin * (float)m1);
    int lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = (int)(qa[i] & 0x0F0F0F0Fu);
        lo[4 + i] = (int)(qb[i] & 0x0F0F0F0Fu);
        hi[i] = (int)((qa[i] >> 4) & 0x0F0F0F0Fu);
        hi[4 + i] = (int)((qb[i] >> 4) & 0x0F0F0F0Fu);
    }
#pragma unroll
    for (int t = 0; t < N; ++t) {
        int D0, D1;
        dot_pair_bcast<J>(D0, D1, tq[t], lo, hi);
        float a = acc[t];
        a = fma_bcast<2 * J>(a, tda[t], dsc0 * (float)D0);
        a = fma_bcast<2 * J + 1>(a, tda[t], dsc1 * (float)D1);
        a = fma_bcast<2 * J>(a, tdass[t], dmm0);
        a = fma_bcast<2 * J + 1>(a, tdass[t], dmm1);
        acc[t] = a;
    }
}

template <int N>
__global__ __launch_bounds__(64 * kMaxWaves) void mmq_gemv_kernel(const uint8_t* __restrict__ w,
                                                                  const int8_t* __restrict__ q,
                                                                  const uint32_t* __restrict__ ds,
                                                                  int M, int K,
                                                                  float* __restrict__ out) {
    __shared__ float red[kMaxWaves][N][16];

    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int p = lane >> 4, r = lane & 15;
    const int row0 = blockIdx.x * 16;
    const int S = K >> 8, C = K >> 5;
    const int sb0 = (int)((int64_t)S * wv / W), sb1 = (int)((int64_t)S * (wv + 1) / W);
    const uint8_t* wrow = w + (int64_t)min(row0 + r, M - 1) * S * kBlockBytes;

    float acc[N];
#pragma unroll
    for (int t = 0; t < N; ++t) acc[t] = 0.0f;

    for (int s = sb0; s < sb1; s += kStepSb) {
        const int ns = min(kStepSb, sb1 - s);  // wave-uniform

        // Every load is issued unconditionally (slots past the wave's last
        // super-block re-read that block and are not used), so that all of a
        // step's loads are in flight before the first wait.
        // q8: lane (p, r) holds piece r&3 of pair p of super-block s + (r>>2)
        // (the wave reads the step's q8 bytes of a token as one KiB)
        v4u tq[N];
        const int64_t qoff = (int64_t)min(s + (r >> 2), sb1 - 1) * 256 + 64 * p + 16 * (r & 3);
#pragma unroll
        for (int t = 0; t < N; ++t) tq[t] = ld16(q + (int64_t)t * K + qoff);
        // scale word of chunk 2p + (r&1) of super-block s + ((r>>1)&3)
        uint32_t tw[N];
        const int64_t woff = (int64_t)min(s + ((r >> 1) & 3), sb1 - 1) * 8 + 2 * p + (r & 1);
#pragma unroll
        for (int t = 0; t < N; ++t) tw[t] = ds[(int64_t)t * C + woff];
        v4u hdr[kStepSb], qa[kStepSb], qb[kStepSb];
#pragma unroll
        for (int j = 0; j < kStepSb; ++j) {
            const uint8_t* b = wrow + (int64_t)min(s + j, sb1 - 1) * kBlockBytes;
            hdr[j] = ld16(b);
            qa[j] = ld16(b + 16 + 32 * p);
            qb[j] = ld16(b + 32 + 32 * p);
        }
        // keep every load of the step above the math (the scheduler would
        // otherwise trade the overlap for registers)
        __builtin_amdgcn_sched_barrier(0);
        float tda[N], tdass[N];
#pragma unroll
        for (int t = 0; t < N; ++t) {
            tda[t] = half_lo(tw[t]);
            tdass[t] = tda[t] * (float)(int16_t)(uint16_t)(tw[t] >> 16);
        }
        gemv_sb<N, 0>(hdr[0], qa[0], qb[0], p, true, tq, tda, tdass, acc);
        gemv_sb<N, 1>(hdr[1], qa[1], qb[1], p, ns > 1, tq, tda, tdass, acc);
        gemv_sb<N, 2>(hdr[2], qa[2], qb[2], p, ns > 2, tq, tda, tdass, acc);
        gemv_sb<N, 3>(hdr[3], qa[3], qb[3], p, ns > 3, tq, tda, tdass, acc);
    }

    // the four chunk-pair lanes of a row (every lane ends with the same
    // bits), then the waves in index order
#pragma unroll
    for (int t = 0; t < N; ++t) {
        acc[t] += __shfl_xor(acc[t], 16);
        acc[t] += __shfl_xor(acc[t], 32);
        if (p == 0) red[wv][t][r] = acc[t];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * N; e += blockDim.x) {
        const int t = e >> 4, rr = e & 15;
        float sum = red[0][t][rr];
        for (int v = 1; v < W; ++v) sum += red[v][t][rr];
        if (row0 + rr < M) out[(int64_t)t * M + row0 + rr] = sum;
    }
}

template <int N>
hipError_t launch_n(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                    float* out, hipStream_t stream) {
    const int S = k / 256;
    const int rows = (m + 15) / 16;
    // the super-blocks of a row are split over up to 4 waves, so that about
    // 4096 waves (16 per CU) cover the matrix at once
    int waves = 4096 / rows;
    waves = waves < 1 ? 1 : waves > kMaxWaves ? kMaxWaves : waves;
    waves = waves > S ? S : waves;
    hipLaunchKernelGGL(mmq_gemv_kernel<N>, dim3(rows), dim3(64 * waves), 0, stream, w, q, ds, m, k,
                       out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mmq_fp32_gemv(const uint8_t* w, int m, int k, const int8_t* q,
                                const uint32_t* ds, int n, float* out, hipStream_t stream) {
    switch (n) {
        case 1: return launch_n<1>(w, m, k, q, ds, out, stream);
        case 2: return launch_n<2>(w, m, k, q, ds, out, stream);
        case 3: return launch_n<3>(w, m, k, q, ds, out, stream);
        case 4: return launch_n<4>(w, m, k, q, ds, out, stream);
        case 5: return launch_n<5>(w, m, k, q, ds, out, stream);
        case 6: return launch_n<6>(w, m, k, q, ds, out, stream);
        case 7: return launch_n<7>(w, m, k, q, ds, out, stream);
        case 8: return launch_n<8>(w, m, k, q, ds, out, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mmq
