// mmq_stream.hip - q4_K x q8 matmul for a few tokens (1 <= n <= 16), float32
// or binary16 result: weights streamed in long runs past token operands that
// a workgroup holds in LDS.
//
// The method is the one of the other kernels (the yusiwen.cn "minfer" r31
// page, sections 1-2: an exact integer dot per 32-weight chunk, then the
// two-term fold d*sc*da*D - dmin*m*da*ssum), with the arithmetic of the
// narrow kernel (mmq_narrow.hip): v_mfma_i32_4x4x4i8 on unpacked nibbles,
// acc += (da * d*sc) * float(D) per chunk and token, the min term on
// v_mfma_f32_4x4x1f32.  What differs is the memory side.
//
//   * Token operands are shared.  A workgroup owns many 8-row tiles (one
//     workgroup per CU), and its waves read the tokens' q8 rows and scale
//     words from one copy in LDS: k is cut into phases of 16 super-blocks (8
//     with more than 8 tokens), the workgroup copies a phase's token rows and
//     words once,
//     double-buffered, with one workgroup barrier per phase.  Each token byte
//     is then read from L2 once per workgroup instead of once per few rows.
//   * Weights stream in long runs.  A wave's step is 8 rows x 4 consecutive
//     super-blocks: eight 576-byte runs, copied into the wave's LDS area with
//     five 1 KiB direct-to-LDS loads (two areas, the next step's copies in
//     flight while a step computes).  Lane l takes row l % 8, super-block
//     slot (l / 8) % 4 and chunk half l / 32; the four lanes of an MFMA block
//     share slot and half, i.e. k.
//   * A wave owns whole tiles (one or two, accumulated side by side) and a
//     fixed share of each phase's steps (WPT waves per tile take every WPT-th
//     step).  Steps past k or tiles past m compute on clamped, valid data
//     with d = dmin = 0 (adding exactly 0) or are never stored.  At the end
//     the partial sums of a row (8 lanes per wave, WPT waves) are added in
//     LDS in an order fixed by m and k alone.  Float32 partials move into a
//     second accumulator every 32 super-blocks of a tile (the max-k bar).
//
// LDS layout (16-byte slots):
//   * weight area of a step: row r's 36 pieces (4 blocks x 9) in slots
//     40r .. 40r + 39, piece p at slot 40r + (p ^ r): the 16 lanes of a
//     half-wave (8 rows, 2 slots, one piece) read 16 distinct 4-bank groups;
//   * token phase: token t's kP super-blocks in slots 16 kP t + 16u + .., piece
//     q of super-block u at 16u + (q ^ x), x = 2 (t & 3) + (u & 1): the
//     eight (token, super-block) pairs that a half-wave's read touches fall
//     in eight different 4-bank groups;
//   * scale words of a phase: token t's 8 kP words at dword (8 kP + 1) t + 8u + c
//     as copied; after the phase barrier the workgroup converts them once to
//     (da, da*ssum) float pairs at the same index (a second barrier), so the
//     arithmetic reads one pair per chunk and group instead of a word and
//     three conversions.  The odd row length keeps a read's pairs in
//     distinct banks.
#include <algorithm>

#include "internal.h"
#include "stream.h"
#include "kquant_device.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kRT = 8;                      // rows per tile
constexpr int kSlots = 4;                   // super-blocks per step
constexpr int kRowSlots = 40;               // 36 weight pieces of a row's run, padded
constexpr int kAreaBytes = kRT * kRowSlots * 16;   // 5 KiB: five copy instructions
constexpr int kMaxWaves = 8;
constexpr int kFlushSteps = 32 / kSlots;    // a tile's steps between accumulator moves

// A token phase for G groups of 4 tokens: kP super-blocks (16 with one or
// two groups, 8 with three or four, so that the two buffers stay within
// 64 KiB of token rows).
template <int G>
struct Phase {
    static constexpr int kP = G <= 2 ? 16 : 8;                // super-blocks per phase
    static constexpr int kTok = 4 * G;                       // token rows (4 per group)
    static constexpr int kTokSlots = kTok * 16 * kP;         // 16-byte slots
    static constexpr int kTokLoads = kTokSlots / 64;         // 1 KiB copies (kP / 4 per token)
    static constexpr int kWordRow = 8 * kP + 1;              // dwords per token's words (odd)
    static constexpr int kWords = kTok * kWordRow;           // dwords
    static constexpr int kWordLoads = kTok * kP * 8 / 64;    // 256-byte copies (kP / 8 per token)
    static constexpr int kGroupBytes = 4 * 16 * kP * 16;     // token rows of one group
    static constexpr int kGroupWordBytes = 4 * kWordRow * 8;  // (da, da*ssum) pairs of one group
};

// One 16-byte direct-to-LDS copy per lane (the weight steps): lane i writes
// bytes [16i, 16i + 16) at dst, from byte voff of src.  Non-temporal: each
// weight byte is read once (cache policy 2, as the dot4 kernel's staged
// copies).
#ifndef STREAM_WAUX
#define STREAM_WAUX 2
#endif
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t src, uint32_t voff, void* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0,
                                             STREAM_WAUX);
}

// Direct-to-LDS copies in inline asm, outside the compiler's wait
// bookkeeping (buffer_load_dword[x4] ... lds: lane i writes 4 or 16 bytes at
// LDS address lds + 4i or 16i).  The token copies of a phase use these, so
// that the token reads of the phase being computed do not wait for the next
// phase's copies (the compiler cannot tell the two buffers of one array
// apart); the kernel completes them itself, with the vmcnt(0) at each step's
// top and before each phase barrier.  The compiler's own waits for the
// weight copies can then only be stricter than needed, never looser.  M0 is
// set here and by the compiler before its own copies (the clobber tells it);
// an LDS-writing load needs one wait state after an SALU write of M0.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void asm_copy16(u32x4 rsrc, uint32_t lds, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
__device__ __forceinline__ void asm_copy4(u32x4 rsrc, uint32_t lds, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ u32x4 raw_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, (uint32_t)kBufferFlags};
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T*)p;
}

// Copy the token rows and scale words of phase ph (super-blocks kP ph ..)
// into one phase buffer.  The copy instructions are dealt to the W waves;
// every instruction runs on a whole wave.
template <int G>
__device__ __forceinline__ void issue_phase(u32x4 qr, u32x4 dr, int ph, int S, int N, int K, int wv, int W,
                                            int lane, const uint4* tok, const uint32_t* word) {
    typedef Phase<G> P;
    const int C = S * 8;
    for (int c = wv; c < P::kTokLoads + P::kWordLoads; c += W) {
        if (c < P::kTokLoads) {
            // token t = c / (kP / 4), super-blocks 4 (c % (kP / 4)) .. +3 of the phase
            constexpr int kQ = P::kP / 4;
            const int t = c / kQ, cq = c % kQ, u = 4 * cq + (lane >> 4), qp = lane & 15;
            const int x = 2 * (t & 3) + (u & 1);
            const int sb = min(P::kP * ph + u, S - 1);
            const uint32_t src = (uint32_t)min(t, N - 1) * (uint32_t)K + (uint32_t)sb * 256u + 16u * (uint32_t)(qp ^ x);
            asm_copy16(qr, lds_addr(tok + 16 * P::kP * t + 64 * cq), src);
        } else {
            // words: token t = c' / (kP / 8), part c' % (kP / 8) (64 words = 8 super-blocks)
            constexpr int kH = P::kP / 8;
            const int cw = c - P::kTokLoads, t = cw / kH, ch = cw % kH;
            const int wi = min(8 * P::kP * ph + 64 * ch + lane, C - 1);
            const uint32_t src = ((uint32_t)min(t, N - 1) * (uint32_t)C + (uint32_t)wi) * 4u;
            asm_copy4(dr, lds_addr(word + P::kWordRow * t + 64 * ch), src);
        }
    }
}

// The lane's share of a weight step: instruction c, lane u fills slot
// i = 64c + u of row i / 40, whose piece (i % 40) ^ row is block p / 9, piece
// p % 9 of the run (slots past the 36 pieces re-read piece 0).  base[c] is
// that piece's byte offset from the tile's first row at the step's first
// super-block.  Rows past m and blocks past the end of the last row lie
// beyond the tile's buffer range and read as zeros (their slots compute with
// d = dmin = 0 or are never stored); blocks past k in other rows read the
// next row's bytes, which the same d = dmin = 0 slots ignore.
__device__ __forceinline__ void init_wcopy(uint32_t (&base)[5], int lane, uint32_t row_bytes) {
#pragma unroll
    for (int c = 0; c < 5; ++c) {
        const int i = 64 * c + lane, r = i / kRowSlots, p = (i % kRowSlots) ^ r;
        const bool v = p < 9 * kSlots;
        base[c] = (uint32_t)r * row_bytes + (v ? (uint32_t)(p / 9) * kBlockBytes + 16u * (uint32_t)(p % 9) : 0u);
    }
}

// Copies of the step (tile rows row0 .., super-blocks st .. st + 3) into area.
__device__ __forceinline__ void issue_step(const uint8_t* w, const uint32_t (&base)[5], int row0, int st, int M,
                                           int64_t row_bytes, uint8_t* area) {
    const int r0 = min(row0, M - 1), rows = min(kRT, M - r0);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(w) + r0 * row_bytes, 0, (int)(rows * row_bytes), kBufferFlags);
    const uint32_t so = (uint32_t)st * (uint32_t)kBlockBytes;
#pragma unroll
    for (int c = 0; c < 5; ++c) copy16_to_lds(wr, base[c] + so, area + 1024 * c);
}

// Per-lane LDS offsets of the token operands and scale words, fixed for the
// whole kernel: lane (row r, slot s, half h, token ti) reads chunk
// c = 4h + 2pp + e of its slot's super-block: token slots
// 16 kP ti + 16 s + ((2c + part) ^ x), x = 2 ti + (s & 1) (phase-local
// super-blocks of a step start at a multiple of 4, so the parity of the
// lane's super-block is s & 1), and word (8 kP + 1) ti + 8 s + c.  Token
// group g adds 4 token rows of slots and of words.
struct TokOff {
    uint32_t tok[2][2][2];   // [pp][e][part], bytes
    uint32_t word[2][2];     // [pp][e], bytes into the (da, da*ssum) pairs
};

template <int G>
__device__ __forceinline__ void init_tokoff(TokOff& to, int s, int h, int ti) {
    typedef Phase<G> P;
    const int x = 2 * ti + (s & 1);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = 4 * h + 2 * pp + e;
#pragma unroll
            for (int part = 0; part < 2; ++part)
                to.tok[pp][e][part] = 16u * (uint32_t)(16 * P::kP * ti + 16 * s + ((2 * c + part) ^ x));
            to.word[pp][e] = 8u * (uint32_t)(P::kWordRow * ti + 8 * s + c);
        }
}

// The bits of 1.5 * 2^23 as a float32 and as an int32.  An int8 dot chain
// started from these bits ends at the bits of the float32 1.5 * 2^23 + D
// exactly while |D| < 2^22, so fma(x, that float, -1.5 * 2^23 * x) is x * D
// rounded once (the product and the constant are exact in the FMA).
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

// acc[v] += (da of the quad's lane v) * t[v], v = 0..3: the broadcast is the
// FMA's own DPP operand (quad_perm), where a separate v_mov_b32_dpp per value
// would cost as much again.  A DPP operand written by a vector instruction
// needs two wait states before it is read (the leading s_nop 1: the asm is
// outside the compiler's hazard bookkeeping).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void fold_quad(float (&acc)[4], float da, float t0, float t1, float t2, float t3) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %5 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %4, %6 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %4, %7 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %4, %8 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(da), "v"(t0), "v"(t1), "v"(t2), "v"(t3));
}
#pragma clang diagnostic pop

// The float32 with the bits of x.  (By value: __builtin_bit_cast of an
// element of an ext_vector_type lvalue reads the vector's first element,
// whatever the index.)
__device__ __forceinline__ float as_float(int x) { return __builtin_bit_cast(float, x); }

// The arithmetic of one step: lane (row r, slot s, half h, token ti of each
// group); tb / wb = the phase buffers at the step's first super-block.
//   Low nibbles (chunk 2p): B = x & 0x0F0F0F0F, the dot D itself.
//   High nibbles (2p + 1):  B = (x & 0xF0F0F0F0) ^ 0x80808080 = 16n - 128 as
//     int8 (one bitwise op), so the chain gives 16 D - 128 ssum: the fold
//     takes d*sc/16 (exact) and the min term's row factor becomes
//     8 d*sc - dmin*m (the -128 ssum part, moved there), rounded once.
//   Per chunk and token: t = d*sc*D (one FMA on the chain's bits, above),
//   acc += da * t, with da from the token's lane (quad broadcast).
template <int G>
__device__ __forceinline__ void compute_step(const uint8_t* area, const uint8_t* tb, const uint8_t* wb,
                                             const TokOff& to, bool live, int r, int s, int h,
                                             float (*acc)[4], v4f* accm) {
    const v4u* wp = reinterpret_cast<const v4u*>(area) + r * kRowSlots;
    const v4u hdr = wp[(9 * s) ^ r];
    v4u qv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) qv[j] = wp[(9 * s + 1 + 4 * h + j) ^ r];
    const float d = live ? half_lo(hdr.x) : 0.0f, dmin = live ? half_lo(hdr.x >> 16) : 0.0f;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        uint32_t sc2[2], mn2[2];
        scale_min_pair(hdr.y, hdr.z, hdr.w, 2 * h + pp, sc2[0], sc2[1], mn2[0], mn2[1]);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float dsc = d * (float)sc2[e], mneg = -(dmin * (float)mn2[e]);
            const float dsce = e ? dsc * 0.0625f : dsc;
            const float mrow = e ? fmaf(8.0f, dsc, mneg) : mneg;
            const float nk = -kMagic * dsce;
            int b[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const uint32_t xw = qv[2 * pp + (kk >> 2)][kk & 3];
                b[kk] = (int)(e ? (xw & 0xF0F0F0F0u) ^ 0x80808080u : xw & 0x0F0F0F0Fu);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const v4u a0 = *reinterpret_cast<const v4u*>(tb + to.tok[pp][e][0] + Phase<G>::kGroupBytes * g);
                const v4u a1 = *reinterpret_cast<const v4u*>(tb + to.tok[pp][e][1] + Phase<G>::kGroupBytes * g);
                v4i D = v4i{kMagicBits, kMagicBits, kMagicBits, kMagicBits};
                D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a0[0], b[0], D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a0[1], b[1], D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a0[2], b[2], D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a0[3], b[3], D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a1[0], b[4], D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a1[1], b[5], D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a1[2], b[6], D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a1[3], b[7], D, 0, 0, 0);
                const float2 dd = *reinterpret_cast<const float2*>(wb + to.word[pp][e] + Phase<G>::kGroupWordBytes * g);
                const float da = dd.x, dass = dd.y;
                accm[g] = __builtin_amdgcn_mfma_f32_4x4x1f32(dass, mrow, accm[g], 0, 0, 0);
                fold_quad(acc[g], da, fmaf(dsce, as_float(D[0]), nk), fmaf(dsce, as_float(D[1]), nk),
                          fmaf(dsce, as_float(D[2]), nk), fmaf(dsce, as_float(D[3]), nk));
            }
        }
    }
}

// Workgroup: tiles TG = TQ * TPW (8 rows each) from tile blockIdx.x * TG;
// W = TQ * WPT waves; wave w owns local tiles w % TQ + j TQ (j < TPW) and
// takes the steps o, o + WPT, .. (o = w / TQ) of each phase's four.
template <int G, bool H, int TPW>
__global__ __launch_bounds__(64 * kMaxWaves) void mmq_stream_kernel(const uint8_t* __restrict__ w,
                                                                     const int8_t* __restrict__ q,
                                                                     const uint32_t* __restrict__ ds, int M, int N,
                                                                     int K, void* __restrict__ out, int TQ, int WPT) {
    typedef Phase<G> P;
    // Token phases (two buffers, one array each for rows and words, indexed
    // by phase parity) and two weight areas per wave, as separate arrays:
    // copies into one area are in flight while the other is read, and the
    // compiler can tell the arrays apart (a pointer selected between two
    // arrays would make it wait for every copy before a token read).
    __shared__ __attribute__((aligned(16))) uint4 tok[2][P::kTokSlots];
    __shared__ __attribute__((aligned(16))) uint32_t word[P::kWords];    // the next phase's words, as copied
    __shared__ __attribute__((aligned(16))) float2 wpair[P::kWords];     // this phase's (da, da*ssum)
    __shared__ __attribute__((aligned(16))) uint8_t area0[kMaxWaves][kAreaBytes];
    __shared__ __attribute__((aligned(16))) uint8_t area1[kMaxWaves][kAreaBytes];

    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 7, s = (lane >> 3) & 3, h = lane >> 5, ti = lane & 3;   // ti: the lane's token of a group
    const int S = K >> 8, C = K >> 5;
    const int TG = TQ * TPW, tile0 = blockIdx.x * TG;
    const int js = wv % TQ, o = wv / TQ;
    constexpr int kP = P::kP;
    const int NJ = kP / kSlots / WPT;            // steps per phase per tile and wave
    const int NS = NJ * TPW;                     // steps per phase per wave
    const int nph = (S + kP - 1) / kP;
    const int E = nph * NS;

    const u32x4 qr = raw_rsrc(q, (uint32_t)N * (uint32_t)K);
    const u32x4 dr = raw_rsrc(ds, (uint32_t)N * (uint32_t)C * 4u);
    const int64_t row_bytes = (int64_t)S * kBlockBytes;
    uint32_t wbase[5];
    init_wcopy(wbase, lane, (uint32_t)row_bytes);
    TokOff to;
    init_tokoff<G>(to, s, h, ti);

    // Step e of this wave: phase e / NS; within it step j = o + WPT (rem / TPW)
    // of tile js + TQ (rem % TPW).
    auto step_row0 = [&](int e) { return (tile0 + js + TQ * ((e % NS) % TPW)) * kRT; };
    auto step_sb = [&](int e) { return kP * (e / NS) + kSlots * (o + WPT * ((e % NS) / TPW)); };

    // acc: the chunk folds (plain floats: the fold's asm takes them one by
    // one); accm: the min-term MFMA accumulator; acc2: both, moved every 32
    // super-blocks.
    float acc[TPW][G][4];
    v4f accm[TPW][G], acc2[TPW][G];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[j][g][v] = 0.0f;
            accm[j][g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            acc2[j][g] = accm[j][g];
        }
    auto flush = [&](int j, int e) {
        if ((((e % NS) / TPW + NJ * (e / NS)) & (kFlushSteps - 1)) == kFlushSteps - 1) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    acc2[j][g][v] += acc[j][g][v];
                    acc2[j][g][v] += accm[j][g][v];
                    acc[j][g][v] = 0.0f;
                }
                accm[j][g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    };
    // The words of a phase as (da, da*ssum) pairs, each thread a share.
    auto convert_words = [&]() {
        for (int i = threadIdx.x; i < P::kWords; i += blockDim.x) {
            const uint32_t wd = word[i];
            const float da = half_lo(wd);
            wpair[i] = make_float2(da, da * (float)(int16_t)(uint16_t)(wd >> 16));   // exact
        }
    };
    // End of phase ph (after this wave's last step of it): every wave's copies
    // of phase ph + 1 are complete and phase ph's buffers are free; the words
    // of phase ph + 1 are converted (a second barrier before their use).
    auto phase_end = [&](int ph) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
        __syncthreads();
        if (ph + 1 < nph) {
            convert_words();
            __syncthreads();
        }
    };
    // At the top of the first step of phase p (after its wait): the copies of
    // phase p + 1, token rows into the buffer of phase p - 1, words into the
    // copy buffer (phase p's were converted at the last phase end).  They
    // have the step's compute to land; the next step's wait completes them.
    auto next_phase = [&](int e) {
        const int p = e / NS;
        if (e == p * NS && p + 1 < nph)
            issue_phase<G>(qr, dr, p + 1, S, N, K, wv, W, lane, tok[(p + 1) & 1], word);
    };
    auto run = [&](int e, int j, const uint8_t* area) {
        const int ph = e / NS, st = step_sb(e);
        const int u0 = st - kP * ph;   // the step's first phase-local super-block (a multiple of 4)
        compute_step<G>(area, reinterpret_cast<const uint8_t*>(tok[ph & 1] + 16 * u0),
                        reinterpret_cast<const uint8_t*>(wpair + 8 * u0), to, st + s < S, r, s, h, acc[j],
                        accm[j]);
        flush(j, e);
        if ((e + 1) % NS == 0) phase_end(ph);
    };

    issue_phase<G>(qr, dr, 0, S, N, K, wv, W, lane, tok[0], word);
    issue_step(w, wbase, step_row0(0), step_sb(0), M, row_bytes, area0[wv]);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
    __syncthreads();
    convert_words();
    __syncthreads();
    // Steps in pairs (areas 0 and 1); with TPW = 2 the pair is one step of
    // each tile at the same k.
    for (int e = 0; e < E; e += 2) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
        __builtin_amdgcn_sched_barrier(0);
        next_phase(e);
        if (e + 1 < E) issue_step(w, wbase, step_row0(e + 1), step_sb(e + 1), M, row_bytes, area1[wv]);
        __builtin_amdgcn_sched_barrier(0);
        run(e, 0, area0[wv]);
        if (e + 1 >= E) break;
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
        __builtin_amdgcn_sched_barrier(0);
        next_phase(e + 1);
        if (e + 2 < E) issue_step(w, wbase, step_row0(e + 2), step_sb(e + 2), M, row_bytes, area0[wv]);
        __builtin_amdgcn_sched_barrier(0);
        run(e + 1, TPW - 1, area1[wv]);
    }

    // Partial sums red[(wave * TPW + j) * G + g][v][lane] over the token
    // buffers (every wave is past its last phase barrier).  Output
    // (tile js + TQ j, row rr, token 4g + v) adds, for o = 0 .. WPT - 1 in
    // order, the lanes rr + 8 s + 32 h of wave js + TQ o, h then s in order.
    float* red = reinterpret_cast<float*>(&tok[0][0]);
    static_assert(sizeof(tok) >= kMaxWaves * TPW * G * 4 * 64 * 4, "reduction fits");
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[(((wv * TPW + j) * G + g) * 4 + v) * 64 + lane] = (acc2[j][g][v] + acc[j][g][v]) + accm[j][g][v];
    __syncthreads();
    for (int e = threadIdx.x; e < TG * kRT * 4 * G; e += blockDim.x) {
        const int rr = e & 7, lt = (e >> 3) % TG, gv = (e >> 3) / TG;   // gv = 4g + v, the token
        const int j = lt / TQ, jw = lt % TQ;
        float sum = 0.0f;
        for (int oo = 0; oo < WPT; ++oo) {
            const float* rp = red + (((jw + TQ * oo) * TPW + j) * G * 4 + gv) * 64 + rr;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int ss = 0; ss < 4; ++ss) sum += rp[32 * hh + 8 * ss];
        }
        const int row = (tile0 + lt) * kRT + rr;
        if (gv < N && row < M) store_out<H>(out, (int64_t)gv * M + row, sum);
    }
}

template <int G, int TPW>
hipError_t launch_t(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n, void* out,
                    bool half_out, int tq, int wpt, hipStream_t stream) {
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k, (void*)&out,
                    (void*)&tq, (void*)&wpt};
    const void* f = half_out ? (const void*)mmq_stream_kernel<G, true, TPW>
                             : (const void*)mmq_stream_kernel<G, false, TPW>;
    const int tiles = (m + kRT - 1) / kRT, tg = tq * TPW;
    return hipLaunchKernel(f, dim3((unsigned)((tiles + tg - 1) / tg)), dim3(64 * tq * wpt), args, 0, stream);
}

template <int G>
hipError_t launch_g(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n, void* out,
                    bool half_out, hipStream_t stream) {
    int tq, tpw, wpt;
    stream_layout(m, tq, tpw, wpt);
    wpt = std::min(wpt, Phase<G>::kP / kSlots);   // the steps of a phase per tile
    return tpw == 2 ? launch_t<G, 2>(w, m, k, q, ds, n, out, half_out, tq, wpt, stream)
                    : launch_t<G, 1>(w, m, k, q, ds, n, out, half_out, tq, wpt, stream);
}

}  // namespace

hipError_t launch_mmq_fp32_stream(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
                                  void* out, bool half_out, hipStream_t stream) {
    switch ((n + 3) / 4) {
        case 1: return launch_g<1>(w, m, k, q, ds, n, out, half_out, stream);
        case 2: return launch_g<2>(w, m, k, q, ds, n, out, half_out, stream);
        case 3: return launch_g<3>(w, m, k, q, ds, n, out, half_out, stream);
        case 4: return launch_g<4>(w, m, k, q, ds, n, out, half_out, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mmq
