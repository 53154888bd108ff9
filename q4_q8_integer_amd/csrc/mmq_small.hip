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
//   * Up to 16 tokens (one tile) a second kernel, mmq_few_kernel, makes the
//     same contraction from copies that bypass registers: each wave copies
//     its weight rows and token tile per super-block into its own LDS area
//     with buffer loads that write LDS directly (the scattered 8-byte
//     weight loads above kept the address unit busy), in workgroups of 4
//     waves, with the next step's copies in flight where a wave has enough
//     steps (measured 28672 x 8192 / 8192 x 28672 at 16 tokens 58 / 55 ->
//     49 / 50 us).  With 2-4 tiles its per-wave token copies cost more LDS
//     than they save, so this kernel keeps 17-64 tokens.
#include "internal.h"
#include "kquant_device.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int WAVES = 8;
constexpr int NT = 64 * WAVES;

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
                const float da = half_lo(word);
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
            // Software-pipelined over the chunks: the operand reads of chunk
            // c + 1 and the MFMAs of chunk c are issued before the fold of
            // chunk c - 1, so neither the LDS nor the matrix-core latency sits
            // between dependent instructions.
            int64_t an = *reinterpret_cast<const int64_t*>(arow);
            float4 dn = *reinterpret_cast<const float4*>(&L.m.da[wv][0][16 * tt + 4 * kg]);
            v4i Dp[RB];
            float4 dp;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int64_t a = an;
                const float4 da4 = dn;
                if (c < 7) {
                    an = *reinterpret_cast<const int64_t*>(arow + 32 * (c + 1));
                    dn = *reinterpret_cast<const float4*>(&L.m.da[wv][c + 1][16 * tt + 4 * kg]);
                }
                v4i Dc[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    Dc[rb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bw[rb][c], v4i{0, 0, 0, 0}, 0, 0, 0);
                if (c > 0) {
                    const float dav[4] = {dp.x, dp.y, dp.z, dp.w};
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            accb[rb][tt][i] = fmaf(dav[i] * scf[rb][c - 1], (float)Dp[rb][i], accb[rb][tt][i]);
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) Dp[rb] = Dc[rb];
                dp = da4;
            }
            {
                const float dav[4] = {dp.x, dp.y, dp.z, dp.w};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        accb[rb][tt][i] = fmaf(dav[i] * scf[rb][7], (float)Dp[rb][i], accb[rb][tt][i]);
            }
        }
        // min term, 4 chunks per MFMA: A = da*ssum (token x chunk), B = -dmin*m (chunk x row)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float dmin = half_lo(f.hdr[rb].x >> 16);
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
            const float d = half_lo(f.hdr[rb].x);
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

// ---------------------------------------------------------------------------
// Up to 16 tokens: the copies bypass registers.  A workgroup is 16 rows and
// 4 waves that split the super-blocks; per super-block a wave copies its 16
// weight rows and the 16-token tile into its own LDS area with buffer loads
// that write LDS directly, then runs the same MFMA and fold as above from
// there.  The weight rows are read as 144-byte runs per row and step, but
// with no register cost a second area can take the next step's copies while
// a step computes.
constexpr int kFewWaves = 4;
constexpr int kFewNT = 64 * kFewWaves;
constexpr int kWaitVmcnt0 = 0x0F70;        // s_waitcnt vmcnt(0), other counters untouched

// Copies are made by buffer loads that write LDS directly: lane i of a load
// instruction writes 16 bytes at 16*i from its base, so every instruction
// fills 64 consecutive 16-byte slots.  Every instruction is issued with all
// lanes active (a load under a lane mask is not kept in place by the
// compiler relative to the loads after it), so areas are whole instructions.
//
// A wave's copy of one super-block of its 16 weight rows: slot i holds
// piece i % 11 of row i / 11 (pieces 9 and 10, and rows 16+, padding), so
// rows sit 176 bytes apart and the 16 rows' reads of one field hit distinct
// banks; 3 instructions.
constexpr int kWSlots = 11;
constexpr int kWLoads = 3;
constexpr int kWBytes = 1024 * kWLoads;
// A wave's copy of one super-block of a 16-token tile: slot 16t + s holds
// piece s ^ t of token t (an XOR swizzle instead of padding, so the 16
// tokens' reads of one piece hit distinct banks); 4 instructions.
constexpr int kTLoads = 4;
constexpr int kTBytes = 1024 * kTLoads;

// A wave's LDS: the copies (two sets with PF, the next step's in flight
// while a step computes) and the decoded activation scales of the step.
template <int T, bool PF>
struct alignas(16) FewWaveLds {
    uint8_t w[PF ? 2 : 1][kWBytes];
    uint8_t tok[PF ? 2 : 1][T][kTBytes];
    float da[8][16 * T];     // [chunk][token]
    float dass[8][16 * T];   // da*ssum, [chunk][token]
};

// LDS of a workgroup: the waves' areas, reused after the main loop for the
// partial sums of the 4 waves (reduced in a fixed order).
template <int T, bool PF>
struct FewLds {
    union {
        FewWaveLds<T, PF> wave[kFewWaves];
        v4f red[kFewWaves][T][64];
    };
};

// Buffer resources over the tile's weight rows and all token rows.
struct Sources {
    __amdgpu_buffer_rsrc_t w, q;
};

// Issue the copies of super-block sb into a wave's set: the weights to
// wdst, token tile tt to tdst + tt * kTBytes.
template <int T>
__device__ __forceinline__ void issue_copies(uint8_t* wdst, uint8_t* tdst, const Sources& src,
                                             const int* woff, const int* toff, int sb) {
#pragma unroll
    for (int c = 0; c < kWLoads; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.w, (__attribute__((address_space(3))) void*)(wdst + 1024 * c),
                                                 16, woff[c] + sb * kBlockBytes, 0, 0, 0);
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
#pragma unroll
        for (int c = 0; c < kTLoads; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                src.q, (__attribute__((address_space(3))) void*)(tdst + tt * kTBytes + 1024 * c), 16,
                toff[tt * kTLoads + c] + sb * 256, 0, 0, 0);
}

template <int T, bool PF, bool H>
__global__ __launch_bounds__(kFewNT) void mmq_few_kernel(const uint8_t* __restrict__ w,
                                                       const int8_t* __restrict__ q,
                                                       const uint32_t* __restrict__ ds,
                                                       int M, int N, int K,
                                                       void* __restrict__ out) {
    __shared__ FewLds<T, PF> L;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane & 15, kg = lane >> 4;
    const int row0 = blockIdx.x * 16;
    const int S = K >> 8, C = K >> 5;
    const int sb0 = (int)((int64_t)S * wv / kFewWaves), sb1 = (int)((int64_t)S * (wv + 1) / kFewWaves);
    FewWaveLds<T, PF>& my = L.wave[wv];

    // The tile's weight rows (rows past m, and the padding rows, read as
    // zeros; the former are never stored) and all n token rows, as buffer
    // resources; each lane's copy offsets without the super-block term
    // (padded tokens repeat the last real one and are never stored).
    Sources src;
    src.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + (int64_t)row0 * S * kBlockBytes), 0,
                                              min(16, M - row0) * S * kBlockBytes, kBufferFlags);
    src.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(q), 0, N * K, kBufferFlags);
    int woff[kWLoads], toff[T * kTLoads];
#pragma unroll
    for (int c = 0; c < kWLoads; ++c) {
        const int i = lane + 64 * c, rr = i / kWSlots, ch = min(i - rr * kWSlots, 8);
        woff[c] = rr * S * kBlockBytes + 16 * ch;   // rr = 16 (the last 16 slots): past the tile
    }
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
#pragma unroll
        for (int c = 0; c < kTLoads; ++c) {
            const int tk = 4 * c + (lane >> 4), ch = (lane & 15) ^ tk;
            toff[tt * kTLoads + c] = min(16 * tt + tk, N - 1) * K + 16 * ch;
        }
    // scale words of a step: lane handles (token 16tt + r, chunks kg and kg + 4)
    auto words = [&](uint32_t (&wd)[T][2], int sb) {
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            const int tok = min(16 * tt + r, N - 1);
#pragma unroll
            for (int h = 0; h < 2; ++h) wd[tt][h] = ds[(int64_t)tok * C + sb * 8 + kg + 4 * h];
        }
    };

    v4f acc[T], accb[T];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        acc[tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        accb[tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // One super-block from the copies in set b.  LDS accesses of one wave
    // complete in order: the table writes are seen by the reads after them,
    // and a step's reads finish before later writes to the same bytes.
    auto compute = [&](const uint32_t (&wd)[T][2], int b) {
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float da = half_lo(wd[tt][h]);
                my.da[kg + 4 * h][16 * tt + r] = da;
                my.dass[kg + 4 * h][16 * tt + r] = da * (float)(int16_t)(uint16_t)(wd[tt][h] >> 16);
            }
        const uint8_t* wrow = my.w[b] + r * (16 * kWSlots);
        const uint4 hdr = *reinterpret_cast<const uint4*>(wrow);
        int64_t bw[8];
        float scf[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            int sc, mn;
            scale_min(hdr.y, hdr.z, hdr.w, c, sc, mn);
            scf[c] = (float)sc;
            const uint2 x = *reinterpret_cast<const uint2*>(wrow + 16 + 32 * (c >> 1) + 8 * kg);
            bw[c] = (c & 1) ? (int64_t)(((uint64_t)((x.y >> 4) & 0x0F0F0F0Fu) << 32) | ((x.x >> 4) & 0x0F0F0F0Fu))
                            : (int64_t)(((uint64_t)(x.y & 0x0F0F0F0Fu) << 32) | (x.x & 0x0F0F0F0Fu));
        }
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            // token r's bytes 32c + 8kg: piece 2c + (kg >> 1), swizzled
            const uint8_t* arow = my.tok[b][tt] + 256 * r + 8 * (kg & 1);
            // software-pipelined over the chunks as in mmq_small_kernel
            int64_t an = *reinterpret_cast<const int64_t*>(arow + 16 * ((kg >> 1) ^ r));
            float4 dn = *reinterpret_cast<const float4*>(&my.da[0][16 * tt + 4 * kg]);
            v4i Dp;
            float4 dp;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int64_t a = an;
                const float4 da4 = dn;
                if (c < 7) {
                    an = *reinterpret_cast<const int64_t*>(arow + 16 * ((2 * (c + 1) + (kg >> 1)) ^ r));
                    dn = *reinterpret_cast<const float4*>(&my.da[c + 1][16 * tt + 4 * kg]);
                }
                const v4i Dc = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bw[c], v4i{0, 0, 0, 0}, 0, 0, 0);
                if (c > 0) {
                    const float dav[4] = {dp.x, dp.y, dp.z, dp.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) accb[tt][i] = fmaf(dav[i] * scf[c - 1], (float)Dp[i], accb[tt][i]);
                }
                Dp = Dc;
                dp = da4;
            }
            {
                const float dav[4] = {dp.x, dp.y, dp.z, dp.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) accb[tt][i] = fmaf(dav[i] * scf[7], (float)Dp[i], accb[tt][i]);
            }
        }
        // min term, 4 chunks per MFMA: A = da*ssum (token x chunk), B = -dmin*m (chunk x row)
        const float dmin = half_lo(hdr.x >> 16);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int sc, mn;
            scale_min(hdr.y, hdr.z, hdr.w, 4 * j + kg, sc, mn);
            const float bneg = -(dmin * (float)mn);
#pragma unroll
            for (int tt = 0; tt < T; ++tt)
                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(my.dass[4 * j + kg][16 * tt + r], bneg, acc[tt], 0, 0, 0);
        }
        const float d = half_lo(hdr.x);
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[tt][i] = fmaf(d, accb[tt][i], acc[tt][i]);
            accb[tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    if constexpr (PF) {
        uint32_t nx[T][2];
        if (sb0 < sb1) {
            words(nx, sb0);
            issue_copies<T>(my.w[0], my.tok[0][0], src, woff, toff, sb0);
        }
        for (int sb = sb0, b = 0; sb < sb1; ++sb, b ^= 1) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __builtin_amdgcn_sched_barrier(0);
            uint32_t wd[T][2];
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
                wd[tt][0] = nx[tt][0];
                wd[tt][1] = nx[tt][1];
            }
            if (sb + 1 < sb1) {
                words(nx, sb + 1);
                issue_copies<T>(my.w[b ^ 1], my.tok[b ^ 1][0], src, woff, toff, sb + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            compute(wd, b);
        }
    } else {
        for (int sb = sb0; sb < sb1; ++sb) {
            uint32_t wd[T][2];
            words(wd, sb);
            issue_copies<T>(my.w[0], my.tok[0][0], src, woff, toff, sb);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __builtin_amdgcn_sched_barrier(0);
            compute(wd, 0);
        }
    }

    __syncthreads();  // every wave is done with the areas the sums reuse
#pragma unroll
    for (int tt = 0; tt < T; ++tt) L.red[wv][tt][lane] = acc[tt];
    __syncthreads();
    // 64*T output values of 4 floats; the 4 waves share them, each summing
    // the 4 partials in wave order.
    for (int e = threadIdx.x; e < 64 * T; e += kFewNT) {
        const int l = e & 63, tt = e >> 6;
        v4f sum = L.red[0][tt][l];
#pragma unroll
        for (int v = 1; v < kFewWaves; ++v) sum += L.red[v][tt][l];
        const int row = row0 + (l & 15);
        if (row >= M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 16 * tt + 4 * (l >> 4) + i;
            if (tok < N) store_out<H>(out, (int64_t)tok * M + row, sum[i]);
        }
    }
}

template <int T, bool PF>
hipError_t launch_few(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
                    void* out, bool half_out, hipStream_t stream) {
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k, (void*)&out};
    const void* f = half_out ? (const void*)mmq_few_kernel<T, PF, true>
                             : (const void*)mmq_few_kernel<T, PF, false>;
    return hipLaunchKernel(f, dim3((unsigned)((m + 15) / 16)), dim3(kFewNT), args, 0, stream);
}

}  // namespace

hipError_t launch_mmq_fp32_small(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                                 int n, void* out, bool half_out, hipStream_t stream) {
    // Prefetching the next super-block into a second register set pays when
    // each wave has many steps (8192 x 28672: 14 per wave, 16 tokens 67 ->
    // 56 us) and costs occupancy when it has few (28672 x 8192: 4 per wave,
    // 63 -> 73 us); with 3-4 token tiles the second set does not fit.
    if (n <= 16) {
        // the second copy area pays from 16 super-blocks per wave (8192 x
        // 28672: 28 per wave, 52 -> 50 us; 28672 x 8192: 8 per wave, 49 -> 59 us)
        return (k / 256) / kFewWaves >= 16 ? launch_few<1, true>(w, m, k, q, ds, n, out, half_out, stream)
                                           : launch_few<1, false>(w, m, k, q, ds, n, out, half_out, stream);
    }
    const bool pf = (k / 256) / WAVES >= 8;
    if (n <= 32) return pf ? launch_t<2, true>(w, m, k, q, ds, n, out, half_out, stream)
                           : launch_t<2, false>(w, m, k, q, ds, n, out, half_out, stream);
    if (n <= 48) return launch_t<3, false>(w, m, k, q, ds, n, out, half_out, stream);
    return launch_t<4, false>(w, m, k, q, ds, n, out, half_out, stream);
}

}  // namespace mmq
