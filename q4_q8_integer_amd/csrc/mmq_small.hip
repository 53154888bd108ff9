// mmq_small.hip - q4_K x q8 matmul for few tokens (n <= 64), float32 result.
//
// Same method as the other kernels (the yusiwen.cn "minfer" r31 page, sections
// 1-2: exact per-32 integer dots, then the two-term rank-1 fold).  With few
// tokens the weights (0.5625 B each) are read once and used by at most 64
// tokens, so the kernel is built to stream W at HBM speed:
//
//   * One v_mfma_i32_16x16x32_i8 is one chunk (k = 32) of 16 tokens x 16
//     weight rows.  Weights are the B operand: a lane's 8 bytes are the
//     nibbles of 8 consecutive qs bytes, & 0x0F0F0F0F for chunk 2p and
//     >> 4 for chunk 2p+1 (no conversion beyond that), and the lane's output
//     column is its own weight row, so sc, d and dmin are per-lane scalars.
//   * Tokens are the A operand (q8 bytes at the same k), read straight from
//     L2; their scale words are decoded per super-block into a small
//     wave-private LDS table (da and da*ssum per token and chunk).
//   * Per chunk: acc_b += da[t] * float(sc * D)   (int multiply, convert, FMA)
//     Per super-block: out += d * acc_b;  min term on v_mfma_f32_16x16x4_f32
//     (4 chunks per instruction) with A = da*ssum, B = -dmin*m.
//   * A workgroup is 8 waves on the same 16 rows, each wave one eighth of the
//     super-blocks (so even 8192-row matrices give 512 workgroups).  The 8
//     partial sums are added in LDS in a fixed order: results do not depend
//     on timing, and nothing outside the output is written.
//   * T token tiles of 16 (n <= 16*T) reuse each unpacked weight operand,
//     and RB row tiles of 16 per wave reuse each token operand read from LDS
//     (halving the token bytes fetched per weight byte; measured: 8192 x
//     28672 at 33 tokens 129 -> 120 us, 28672 x 8192 140 -> 139 us).
//   * After the main loop the staging LDS is reused for the partial sums.
#include "internal.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int WAVES = 8;
constexpr int NT = 64 * WAVES;

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

// 6-bit (sc, m) of sub-block j from the scale bytes in three dwords (GGUF
// k-quant packing; see mmq_f16.hip).
__device__ __forceinline__ void scale_min(uint32_t s03, uint32_t s47, uint32_t s811, int j,
                                          int& sc, int& mn) {
    const int sh = 8 * (j & 3);
    const int by = (s03 >> sh) & 0xFF, bz = (s47 >> sh) & 0xFF, bw = (s811 >> sh) & 0xFF;
    const bool hi = j >= 4;
    sc = hi ? ((bw & 15) | ((by >> 6) << 4)) : (by & 63);
    mn = hi ? ((bw >> 4) | ((bz >> 6) << 4)) : (bz & 63);
}

// LDS of a workgroup: the staging areas of the main loop, reused after it
// for the partial sums of the 8 waves (reduced in a fixed order).
template <int T, int RB>
struct SmallLds {
    struct Main {
        float da[WAVES][8][16 * T];     // per wave: da of its super-block, [chunk][token]
        float dass[WAVES][8][16 * T];   // per wave: da*ssum, [chunk][token]
        // per wave: one 16-token tile of the super-block's q8 bytes, rows
        // padded to 272 B so that the 16 lanes reading one chunk slot of 16
        // rows hit distinct banks
        uint4 tok[WAVES][16][17];
    };
    union {
        Main m;
        v4f red[WAVES][T][RB][64];
    };
};

template <int T, int RB, bool PF, bool H>
__global__ __launch_bounds__(NT) void mmq_small_kernel(const uint8_t* __restrict__ w,
                                                       const int8_t* __restrict__ q,
                                                       const uint32_t* __restrict__ ds,
                                                       int M, int N, int K,
                                                       void* __restrict__ out) {
    __shared__ SmallLds<T, RB> L;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane & 15, kg = lane >> 4;
    const int row0 = blockIdx.x * 16 * RB;
    const int S = K >> 8, C = K >> 5;
    const int sb0 = (int)((int64_t)S * wv / WAVES), sb1 = (int)((int64_t)S * (wv + 1) / WAVES);

    // lane's weight row in each of the RB row tiles (rows past m repeat the last)
    const uint8_t* blk[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) blk[rb] = w + (int64_t)min(row0 + 16 * rb + r, M - 1) * S * kBlockBytes;
    // q8 staging loads: piece j of a tile is tokens 4j .. 4j+3, lane -> token
    // 4j + (lane >> 4), bytes 16*(lane & 15) of the super-block (one
    // contiguous 256-byte run per token).  Padded tokens repeat the last real
    // one and are never stored.
    const int8_t* qpiece[T][4];
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            qpiece[tt][j] = q + (int64_t)min(16 * tt + 4 * j + (lane >> 4), N - 1) * K + 16 * (lane & 15);

    v4f acc[RB][T], accb[RB][T];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            acc[rb][tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            accb[rb][tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }

    // Global data of one super-block step, as this lane loads it.  Two sets
    // alternate: the loads of step sb+1 are in flight while sb is computed.
    struct Fetch {
        uint4 hdr[RB];
        uint2 qs[RB][4];
        uint4 tq[T][4];
        uint32_t word[T][2];
    };
    auto fetch = [&](Fetch& f, int sb) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const uint8_t* b = blk[rb] + (int64_t)sb * kBlockBytes;
            f.hdr[rb] = *reinterpret_cast<const uint4*>(b);
#pragma unroll
            for (int p = 0; p < 4; ++p) f.qs[rb][p] = *reinterpret_cast<const uint2*>(b + 16 + 32 * p + 8 * kg);
        }
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) f.tq[tt][j] = *reinterpret_cast<const uint4*>(qpiece[tt][j] + sb * 256);
            const int tok = min(16 * tt + r, N - 1);
#pragma unroll
            for (int h = 0; h < 2; ++h) f.word[tt][h] = ds[(int64_t)tok * C + sb * 8 + kg + 4 * h];
        }
    };
    auto compute = [&](const Fetch& f) {
        // scale words of this super-block: lane handles (token 16tt + r, chunks kg and kg + 4)
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t word = f.word[tt][h];
                const float da = half_bits_to_float(word);
                L.m.da[wv][kg + 4 * h][16 * tt + r] = da;
                L.m.dass[wv][kg + 4 * h][16 * tt + r] = da * (float)(int16_t)(uint16_t)(word >> 16);
            }
        // The LDS areas are wave-private: LDS accesses of one wave complete in
        // order, so each write below is seen by the reads after it, and a tile's
        // reads finish before the next tile overwrites the area.
        int64_t bw[RB][8];
        float scf[RB][8];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                int sc, mn;
                scale_min(f.hdr[rb].y, f.hdr[rb].z, f.hdr[rb].w, c, sc, mn);
                scf[rb][c] = (float)sc;
                const uint2 x = f.qs[rb][c >> 1];
                bw[rb][c] = (c & 1) ? (int64_t)(((uint64_t)((x.y >> 4) & 0x0F0F0F0Fu) << 32) | ((x.x >> 4) & 0x0F0F0F0Fu))
                                    : (int64_t)(((uint64_t)(x.y & 0x0F0F0F0Fu) << 32) | (x.x & 0x0F0F0F0Fu));
            }
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) L.m.tok[wv][4 * j + (lane >> 4)][lane & 15] = f.tq[tt][j];
            const uint8_t* arow = reinterpret_cast<const uint8_t*>(L.m.tok[wv][r]) + 8 * kg;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int64_t a = *reinterpret_cast<const int64_t*>(arow + 32 * c);
                const float4 da4 = *reinterpret_cast<const float4*>(&L.m.da[wv][c][16 * tt + 4 * kg]);
                const float dav[4] = {da4.x, da4.y, da4.z, da4.w};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const v4i D = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bw[rb][c], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        accb[rb][tt][i] = fmaf(dav[i] * scf[rb][c], (float)D[i], accb[rb][tt][i]);
                }
            }
        }
        // min term, 4 chunks per MFMA: A = da*ssum (token x chunk), B = -dmin*m (chunk x row)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float dmin = half_bits_to_float(f.hdr[rb].x >> 16);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                int sc, mn;
                scale_min(f.hdr[rb].y, f.hdr[rb].z, f.hdr[rb].w, 4 * j + kg, sc, mn);
                const float bneg = -(dmin * (float)mn);
#pragma unroll
                for (int tt = 0; tt < T; ++tt)
                    acc[rb][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(L.m.dass[wv][4 * j + kg][16 * tt + r], bneg,
                                                                       acc[rb][tt], 0, 0, 0);
            }
            const float d = half_bits_to_float(f.hdr[rb].x);
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[rb][tt][i] = fmaf(d, accb[rb][tt][i], acc[rb][tt][i]);
                accb[rb][tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    };

    if constexpr (PF) {
        // Every fetch is unconditional (a fetch past the last step re-reads it).
        Fetch fa, fb;
        if (sb0 < sb1) fetch(fa, sb0);
        for (int sb = sb0; sb < sb1; sb += 2) {
            fetch(fb, min(sb + 1, sb1 - 1));
            compute(fa);
            if (sb + 1 >= sb1) break;
            fetch(fa, min(sb + 2, sb1 - 1));
            compute(fb);
        }
    } else {
        // one step at a time: the step's loads are all issued before its math
        for (int sb = sb0; sb < sb1; ++sb) {
            Fetch f;
            fetch(f, sb);
            compute(f);
        }
    }

    __syncthreads();  // every wave is done with the staging areas the sums reuse
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) L.red[wv][tt][rb][lane] = acc[rb][tt];
    __syncthreads();
    // 64*T*RB output values of 4 floats; the 8 waves share them, each summing
    // the 8 partials in wave order.
    for (int e = threadIdx.x; e < 64 * T * RB; e += NT) {
        const int l = e & 63, rb = (e >> 6) % RB, tt = (e >> 6) / RB;
        v4f sum = L.red[0][tt][rb][l];
#pragma unroll
        for (int v = 1; v < WAVES; ++v) sum += L.red[v][tt][rb][l];
        const int row = row0 + 16 * rb + (l & 15);
        if (row >= M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 16 * tt + 4 * (l >> 4) + i;
            if (tok < N) store_out<H>(out, (int64_t)tok * M + row, sum[i]);
        }
    }
}

template <int T, bool PF>
hipError_t launch_t(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
                    void* out, bool half_out, hipStream_t stream) {
    constexpr int RB = 2;
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k, (void*)&out};
    const void* f = half_out ? (const void*)mmq_small_kernel<T, RB, PF, true>
                             : (const void*)mmq_small_kernel<T, RB, PF, false>;
    return hipLaunchKernel(f, dim3((unsigned)((m + 16 * RB - 1) / (16 * RB))), dim3(NT), args, 0, stream);
}

}  // namespace

hipError_t launch_mmq_fp32_small(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                                 int n, void* out, bool half_out, hipStream_t stream) {
    // Prefetching the next super-block into a second register set pays when
    // each wave has many steps (8192 x 28672: 14 per wave, 16 tokens 67 ->
    // 56 us) and costs occupancy when it has few (28672 x 8192: 4 per wave,
    // 63 -> 73 us); with 3-4 token tiles the second set does not fit.
    const bool pf = (k / 256) / WAVES >= 8;
    if (n <= 16) return pf ? launch_t<1, true>(w, m, k, q, ds, n, out, half_out, stream)
                           : launch_t<1, false>(w, m, k, q, ds, n, out, half_out, stream);
    if (n <= 32) return pf ? launch_t<2, true>(w, m, k, q, ds, n, out, half_out, stream)
                           : launch_t<2, false>(w, m, k, q, ds, n, out, half_out, stream);
    if (n <= 48) return launch_t<3, false>(w, m, k, q, ds, n, out, half_out, stream);
    return launch_t<4, false>(w, m, k, q, ds, n, out, half_out, stream);
}

}  // namespace mmq
