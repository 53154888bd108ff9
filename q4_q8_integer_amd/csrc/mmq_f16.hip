// mmq_f16.hip - q4_K x q8 quantized matmul, float32 result, on gfx950 f16 MFMA.
//
// Same method as mmq_i8.hip (the yusiwen.cn "minfer" r31 page, sections 1-2:
// exact per-32 dot products, then the two-term rank-1 fold), re-associated so
// that the per-chunk work left for the vector ALU is one FMA per output:
//
//   * A operand = sc*q4 as binary16.  sc*q4 <= 63*15 = 945 is an integer
//     below 2048, so it is exact; the B operand q8 in [-127, 127] is exact as
//     well.  Every partial sum of a chunk's 32 products is an integer below
//     945*127*32 < 2^22, so the two chained v_mfma_f32_32x32x16_f16 of a chunk
//     return P = sc*D exactly, in float32.
//   * Per chunk:       acc_b += da[t,c] * P          (da is a per-lane scalar)
//     Per super-block: out   += d[o] * acc_b         (8 chunks share d)
//   * The min term  -(dmin*m)[o,c] * (da*ssum)[t,c]  is a rank-1 update per
//     chunk; over the chunks it is a float32 GEMM of depth k/32, done on
//     v_mfma_f32_32x32x2_f32 (two chunks per instruction) straight into out.
//
// The int8 alternative needs three VALU operations per output and chunk
// (int multiply by sc, convert, FMA) against one here; the vector ALU, not the
// matrix core, is what bounds this operation on gfx950.
//
// Tiling: workgroup 128 rows x 128 tokens (x 64 tokens where 128-token
// tiles would leave CUs idle); 8 consumer waves of 64 rows x 32 tokens (32 x
// 32 with 64-token tiles) and 8 producer waves; k is staged 128 at a time
// (half a super-block, 4 chunks) in two alternating LDS stages (~141 KB, one
// workgroup per CU).  Producers convert each weight and each activation once
// per workgroup into binary16 operand slots laid out
// [chunk][k-half][lane-half][row or token][8 halves], so that the 32 lanes of
// a half-wave read 32 consecutive 16-byte slots (conflict-free) and each
// staging store is a run of consecutive slots.
//
// The same kernel reads q4k_repack records (REP): per stage and piece the
// producers load the row's d | dmin dword and its chunk pair's scale dword
// (sc and m as bytes) in place of the 16-byte block header, and skip the
// 6-bit scale decode; everything after the scales is the same arithmetic, so
// the two layouts give the same result bit for bit.
//
// With QT the activations arrive as q8_quantize_rows_tiled's operand tiles,
// already binary16 and already in the B slot order: the producers copy each
// stage's 32 KiB block into LDS with buffer_load ... lds and convert weights
// only.
#include "f16_operand.h"
#include "internal.h"
#include "kquant_device.h"

namespace mmq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128;
constexpr int CT = 512;          // consumer threads (8 waves of 64 rows x 32 tokens)
constexpr int PT = 512;          // producer threads (8 waves)
constexpr int NT = CT + PT;
constexpr int WPC = 512 / PT;    // weight pieces per producer thread (128 rows x 4)
constexpr int APC = 1024 / PT;   // q8 pieces per producer thread (128 tokens x 8)
constexpr int SPC = 512 / PT;    // scale words per producer thread (128 tokens x 4)
constexpr int CS = 4;  // chunks per stage (128 k)
constexpr int NTW = 1;  // 32-token tiles per consumer wave
// One (token tile, stage) block of the q8 operand tiles: 16 slot rows x 128
// tokens x 8 binary16 values.
constexpr int kQtBlockBytes = 16 * BN * 16;

// 4 qs bytes x = [b0 b1 b2 b3] -> binary16 pairs of sc*nibble, exactly:
//   low nibbles (chunk 2p):   (x & 0x000F000F) | 0x64006400 = (1024 + n, 1024 + n')
//                             fma(1024 + n, sc, -1024 sc) = sc*n
//   high nibbles (2p+1):      (x & 0x00F000F0) | 0x64006400 = (1024 + 16n, ...)
//                             fma(1024 + 16n, sc/16, -64 sc) = sc*n
// and the same on x >> 8 for bytes b1, b3.  Pair order: [b0,b2], [b1,b3].
// sc, sc/16, -1024 sc and -64 sc are exact binary16 for sc <= 63.
__device__ __forceinline__ void unpack_word(uint32_t x, uint32_t sclo, uint32_t nblo, uint32_t schi,
                                            uint32_t nbhi, uint32_t& lo02, uint32_t& lo13,
                                            uint32_t& hi02, uint32_t& hi13) {
    const uint32_t y = x >> 8;
    lo02 = pk_fma_f16(and_or(x, 0x000F000Fu, 0x64006400u), sclo, nblo);
    lo13 = pk_fma_f16(and_or(y, 0x000F000Fu, 0x64006400u), sclo, nblo);
    hi02 = pk_fma_f16(and_or(x, 0x00F000F0u, 0x64006400u), schi, nbhi);
    hi13 = pk_fma_f16(and_or(y, 0x00F000F0u, 0x64006400u), schi, nbhi);
}

// One stage of operands (128 k = 4 chunks) in LDS.  The q8 operands are an
// LDS array of their own (StageB), so that the compiler can tell the
// direct-to-LDS copies into it from the weight stores (it would otherwise
// wait for the copies, and with them for the next stage's loads, before
// every store).
struct StageB {
    uint4 B[CS][2][2][BN];   // q8 binary16 operand slots [chunk][k-half][lane-half][token]
};
struct Stage {
    uint4 A[CS][2][2][BM];   // sc*q4 binary16 operand slots [chunk][k-half][lane-half][row]
    float D[BM];             // d of the stage's super-block
    float CA[CS][BM];        // -dmin*m per (chunk, row)
    // da and da*ssum per (chunk, token).  Rows padded by 8 floats: the
    // producers store a token's 4 chunks from 4 neighbouring lanes, which
    // rows 128 floats apart would put in one bank.
    float Da[CS][BN + 8];
    float Dass[CS][BN + 8];
};

// Raw global data of one stage, as one producer thread loads it.
struct Raw {
    uint4 hdr[WPC], qs[WPC]; // weight pieces: block header + 16 nibble bytes (repacked
                             // records: hdr.x = d | dmin << 16, hdr.y = the scale dword)
    uint4 y[APC];            // activation pieces of 16 q8 bytes
    uint32_t word[SPC];      // activation scale words
};

// Producer loads go through buffer resources: one resource per operand,
// based at the workgroup's first row / token, with the per-lane byte offset
// fixed for the whole k loop and the per-stage advance in the scalar offset
// (no vector address arithmetic in the loop).  The resource's record count is
// the extent the workgroup may read, so an out-of-range offset would read
// zeros instead of faulting.
struct Src {
    __amdgpu_buffer_rsrc_t w, q, ds;
    const uint16_t* qt;      // operand tiles (QT): the workgroup's 128-token tile
    int qhalf;               // QT with 64-token tiles: which half of it
    int wh[WPC], wq[WPC];    // weight piece offsets: block header (repacked: d | dmin), nibbles
    int wsc[WPC];            // repacked records: scale dword
    int y[APC];              // q8 piece offsets
    int word[SPC];           // scale-word offsets
};

// TB: tokens of the workgroup tile (BN, or BN / 2 where full tiles would
// leave CUs idle); the LDS stage keeps its BN-token size.
// REP: w holds q4k_repack records (16-row tiles, one 2368-byte record per
// tile and super-block) instead of q4_K rows.
template <int TB, bool REP, bool QT>
__device__ __forceinline__ void init_src(Src& p, const uint8_t* __restrict__ w,
                                         const int8_t* __restrict__ q,
                                         const uint32_t* __restrict__ ds, int pt, int row0,
                                         int tok0, int M, int N, int K) {
    const int S = K >> 8, C = K >> 5;
    const int rows = min(BM, M - row0), toks = min(TB, N - tok0);
    const int row_bytes = S * kBlockBytes;
    // repacked: the workgroup's 16-row tiles (up to 8), S records each
    const int tile_bytes = S * kRepackRecordBytes, ntile = (rows + 15) >> 4;
    if (REP)
        p.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + (int64_t)(row0 >> 4) * tile_bytes), 0,
                                                ntile * tile_bytes, kBufferFlags);
    else
        p.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + (int64_t)row0 * row_bytes), 0,
                                                rows * row_bytes, kBufferFlags);
    p.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(q + (int64_t)tok0 * K), 0,
                                            (int)((uint32_t)toks * (uint32_t)K), kBufferFlags);   // up to 2^31 bytes
    p.ds = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(ds + (int64_t)tok0 * C), 0,
                                             toks * C * 4, kBufferFlags);
    if (QT) {
        p.qt = reinterpret_cast<const uint16_t*>(q) + (int64_t)(tok0 >> 7) * (K >> 7) * (kQtBlockBytes / 2);
        p.qhalf = (tok0 >> 6) & 1;
    }
#pragma unroll
    for (int rr = 0; rr < WPC; ++rr) {
        const int i = pt + rr * PT;
        const int row = (i & 15) | ((i >> 6) << 4);
        const int j = (i >> 4) & 3, pl = j >> 1, gg = j & 1;
        if (REP) {
            // record: [0,64) d | dmin dword r; [64,320) scale dword 16p + r;
            // [320,2368) qs bytes 32p + 16h .. +15 of row r at 320 + 512p + 256h + 16r
            const int base = min(row >> 4, ntile - 1) * tile_bytes, r = row & 15;
            p.wh[rr] = base + 4 * r;
            p.wsc[rr] = base + 64 + 64 * pl + 4 * r;
            p.wq[rr] = base + 320 + 512 * pl + 256 * gg + 16 * r;
        } else {
            p.wh[rr] = min(row, rows - 1) * row_bytes;
            p.wq[rr] = p.wh[rr] + 16 + 32 * pl + 16 * gg;
        }
    }
#pragma unroll
    for (int rr = 0; rr < TB * 8 / PT; ++rr) {
        const int i = pt + rr * PT;
        const int tok = (i & 15) | ((i >> 7) << 4);
        const int j = (i >> 4) & 7, cl = j >> 1, gg = j & 1;
        p.y[rr] = min(tok, toks - 1) * K + 32 * cl + 16 * gg;
    }
#pragma unroll
    for (int rr = 0; rr < SPC; ++rr) {
        // thread i loads chunk i & 3 of token i >> 2, so that the four lanes
        // of a token read one 16-byte run (one cache line per 16 lanes rather
        // than per lane); with TB < BN only the first TB * 4 producer threads
        // hold a word (the others re-read the last one and store nothing)
        const int i = TB == BN ? pt + rr * PT : min(pt + rr * PT, TB * 4 - 1);
        const int tok = i >> 2, cl = i & 3;
        p.word[rr] = (min(tok, toks - 1) * C + cl) * 4;
    }
}

template <int TB, bool REP, bool QT>
__device__ __forceinline__ void load_stage(Raw& r, const Src& p, int st) {
    if (REP) {
        // stage st: record st / 2, chunk pairs 2 (st & 1) and 2 (st & 1) + 1
        const int roff = (st >> 1) * kRepackRecordBytes, hs = st & 1;
#pragma unroll
        for (int rr = 0; rr < WPC; ++rr) {
            r.hdr[rr].x = __builtin_amdgcn_raw_buffer_load_b32(p.w, p.wh[rr], roff, 0);
            r.hdr[rr].y = __builtin_amdgcn_raw_buffer_load_b32(p.w, p.wsc[rr], roff + 128 * hs, 0);
            r.qs[rr] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(p.w, p.wq[rr], roff + 1024 * hs, 0));
        }
    } else {
        const int boff = (st >> 1) * kBlockBytes, qoff = boff + (st & 1) * 64;
#pragma unroll
        for (int rr = 0; rr < WPC; ++rr) {
            r.hdr[rr] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(p.w, p.wh[rr], boff, 0));
            r.qs[rr] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(p.w, p.wq[rr], qoff, 0));
        }
    }
    if (!QT)
#pragma unroll
        for (int rr = 0; rr < TB * 8 / PT; ++rr)
            r.y[rr] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(p.q, p.y[rr], 128 * st, 0));
#pragma unroll
    for (int rr = 0; rr < SPC; ++rr)
        r.word[rr] = __builtin_amdgcn_raw_buffer_load_b32(p.ds, p.word[rr], 16 * st, 0);
}

template <int TB, bool REP, bool QT>
__device__ __forceinline__ void convert_stage(const Raw& r, Stage& sg, StageB& sb, int pt, int st) {
    const int hs = st & 1;
#pragma unroll
    for (int rr = 0; rr < WPC; ++rr) {
        const int i = pt + rr * PT;
        const int row = (i & 15) | ((i >> 6) << 4);
        const int j = (i >> 4) & 3, pl = j >> 1, gg = j & 1;
        const uint4 hdr = r.hdr[rr], qs = r.qs[rr];
        const int c0 = 2 * (2 * hs + pl);
        int sclo, schi, mn;
        if (REP) {
            // the scale dword of chunk pair c0/2: sc[c0] | sc[c0+1] << 8 | m[c0] << 16 | m[c0+1] << 24
            sclo = hdr.y & 0xFF;
            schi = (hdr.y >> 8) & 0xFF;
        } else {
            scale_min(hdr.y, hdr.z, hdr.w, c0, sclo, mn);
            scale_min(hdr.y, hdr.z, hdr.w, c0 + 1, schi, mn);
        }
        const uint32_t sl2 = f16x2_splat((float)sclo), nl2 = f16x2_splat(-1024.0f * sclo);
        const uint32_t sh2 = f16x2_splat(0.0625f * schi), nh2 = f16x2_splat(-64.0f * schi);
        uint32_t lo[8], hi[8];
        const uint32_t xw[4] = {qs.x, qs.y, qs.z, qs.w};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
            unpack_word(xw[k4], sl2, nl2, sh2, nh2, lo[2 * k4], lo[2 * k4 + 1], hi[2 * k4],
                        hi[2 * k4 + 1]);
        sg.A[2 * pl][0][gg][row] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        sg.A[2 * pl][1][gg][row] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
        sg.A[2 * pl + 1][0][gg][row] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        sg.A[2 * pl + 1][1][gg][row] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
        // The four pieces of a row share its header: piece j writes the min
        // scale of the stage's chunk j, and all four write d (same value).
        // No branch here, so the loop body stays straight-line.
        {
            const float d = half_lo(hdr.x);
            const float dmin = half_lo(hdr.x >> 16);
            int sc, m;
            if (REP)
                m = (hdr.y >> (16 + 8 * gg)) & 0xFF;   // chunk 4 hs + j = c0 + gg
            else
                scale_min(hdr.y, hdr.z, hdr.w, 4 * hs + j, sc, m);
            sg.D[row] = d;
            sg.CA[j][row] = -(dmin * (float)m);
        }
    }
#pragma unroll
    for (int rr = 0; rr < (QT ? 0 : TB * 8 / PT); ++rr) {   // QT: copied by dma_stage
        const int i = pt + rr * PT;
        const int tok = (i & 15) | ((i >> 7) << 4);
        const int j = (i >> 4) & 7, cl = j >> 1, gg = j & 1;
        const uint4 y = r.y[rr];
        uint32_t p[8];
        q8_word(y.x, p[0], p[1]);
        q8_word(y.y, p[2], p[3]);
        q8_word(y.z, p[4], p[5]);
        q8_word(y.w, p[6], p[7]);
        sb.B[cl][0][gg][tok] = make_uint4(p[0], p[1], p[2], p[3]);
        sb.B[cl][1][gg][tok] = make_uint4(p[4], p[5], p[6], p[7]);
    }
#pragma unroll
    for (int rr = 0; rr < SPC; ++rr) {
        const int i = pt + rr * PT;
        const int tok = i >> 2, cl = i & 3;
        const float da = half_lo(r.word[rr]);
        if (TB == BN || i < TB * 4) {
            sg.Da[cl][tok] = da;
            sg.Dass[cl][tok] = da * (float)(int16_t)(uint16_t)(r.word[rr] >> 16);  // exact
        }
    }
}

// Vector-memory operations load_stage issues (the wait that completes a
// stage's operand-tile copies leaves these in flight).
template <bool REP, bool QT>
constexpr int stage_loads() { return WPC * (REP ? 3 : 2) + SPC + (QT ? 0 : APC); }

// QT: the stage's q8 operands are one 32 KiB block of the operand tiles, in
// the order of StageB, copied with direct-to-LDS buffer loads (lane i of an
// instruction writes 16 bytes at M0 + 16 i: one KiB, 64 token slots of one
// slot row).  128-token tiles take the whole block (32 copies, 4 per producer
// wave), 64-token tiles their half of each row (16 copies).  Every copy is
// issued by a full wave.
//
// The copies are inline asm, outside the compiler's wait bookkeeping: with
// the builtin it waits for them (and with them for the next stage's register
// loads) before the first LDS store of every stage.  The producer loop
// places the waits itself: everything older is complete before the copies
// are issued, and a vmcnt that leaves only the next stage's loads in flight
// completes them before the barrier.  The compiler's own waits can then only
// be stricter than needed, never looser.

// An empty asm that reads a stage's raw registers: the compiler completes
// their loads here (nothing newer is in flight yet), so that no later use
// waits on a count that the uncounted copies would make too strict.
template <bool REP>
__device__ __forceinline__ void settle(const Raw& r) {
#pragma unroll
    for (int rr = 0; rr < WPC; ++rr) {
        if (REP)
            asm volatile("" ::"v"(r.hdr[rr].x), "v"(r.hdr[rr].y));
        else
            asm volatile("" ::"v"(r.hdr[rr].x), "v"(r.hdr[rr].y), "v"(r.hdr[rr].z), "v"(r.hdr[rr].w));
        asm volatile("" ::"v"(r.qs[rr].x), "v"(r.qs[rr].y), "v"(r.qs[rr].z), "v"(r.qs[rr].w));
    }
#pragma unroll
    for (int rr = 0; rr < SPC; ++rr) asm volatile("" ::"v"(r.word[rr]));
}

template <int TB>
__device__ __forceinline__ void dma_stage(StageB& sb, const Src& p, int st, int pw, int lane) {
    constexpr int kCopies = TB * 16 / 64 / (PT / 64);
    const uint64_t a = reinterpret_cast<uint64_t>(p.qt + (int64_t)st * (kQtBlockBytes / 2));
    const u32x4 rsrc = {(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, (uint32_t)kQtBlockBytes,
                        (uint32_t)kBufferFlags};
    const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4*)&sb.B[0][0][0][0];
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
        const int i = pw * kCopies + j;
        const int row = TB == BN ? i >> 1 : i;
        const int half = TB == BN ? (i & 1) : p.qhalf;
        const int dst = row * BN + (TB == BN ? half * 64 : 0);
        lds_copy16(rsrc, base + 16 * dst, (row * BN + half * 64 + lane) * 16);
    }
}

// One stage for one consumer wave (64 rows x 32*NTW tokens as 2 x NTW tiles of 32x32).
// HS is the stage's half of the super-block: HS = 0 starts acc_b (the first
// chunk multiplies instead of accumulating), HS = 1 ends it with the d fold.
// Per chunk all eight MFMAs are issued before any of the epilogue, so each
// tile's FMAs find their MFMA results done instead of waiting on them.
// RT: 32-row tiles per wave (2 with 128-token tiles, 1 with 64: the 8
// waves then cover 4 x 32 rows x 2 x 32 tokens); r0 = the wave's first row.
template <int HS, int RT>
__device__ __forceinline__ void consume_stage(const Stage& sg, const StageB& sb, int wm, int wn, int g, int l32,
                                              v16f (&acc)[2][NTW], v16f (&accb)[2][NTW]) {
    // min term: out += (-dmin*m) x (da*ssum), two chunks per MFMA.  First in
    // the stage: its scalar operands arrive quickly, and its MFMAs cover the
    // LDS latency of the first chunk's operand reads, which every consumer
    // wave issues at once after the stage barrier (acc sees the same updates
    // in the same order as with the min term last).
#pragma unroll
    for (int cp = 0; cp < CS / 2; ++cp) {
        float ca[2], cb[NTW];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) ca[rt] = sg.CA[2 * cp + g][wm * 32 * RT + rt * 32 + l32];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) cb[nt] = sg.Dass[2 * cp + g][wn * 32 * NTW + nt * 32 + l32];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
                acc[rt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ca[rt], cb[nt], acc[rt][nt], 0, 0, 0);
    }
#pragma unroll
    for (int cl = 0; cl < CS; ++cl) {
        v8h a0[2], a1[2], b0[NTW], b1[NTW];
        float da[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int t = wn * 32 * NTW + nt * 32 + l32;
            b0[nt] = __builtin_bit_cast(v8h, sb.B[cl][0][g][t]);
            b1[nt] = __builtin_bit_cast(v8h, sb.B[cl][1][g][t]);
            da[nt] = sg.Da[cl][t];
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int rr = wm * 32 * RT + rt * 32 + l32;
            a0[rt] = __builtin_bit_cast(v8h, sg.A[cl][0][g][rr]);
            a1[rt] = __builtin_bit_cast(v8h, sg.A[cl][1][g][rr]);
        }
        v16f pr[2][NTW];
        const v16f zero = {};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
                pr[rt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[rt], b0[nt], zero, 0, 0, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
                pr[rt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[rt], b1[nt], pr[rt][nt], 0, 0, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                if (HS == 0 && cl == 0)
                    accb[rt][nt] = pr[rt][nt] * da[nt];
                else
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        accb[rt][nt][v] = fmaf(da[nt], pr[rt][nt][v], accb[rt][nt][v]);
            }
    }
    // end of a super-block: out += d * acc_b
    if (HS == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float4 d4 = *reinterpret_cast<const float4*>(&sg.D[wm * 32 * RT + rt * 32 + 8 * jj + 4 * g]);
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        acc[rt][nt][4 * jj + i] = fmaf(dv[i], accb[rt][nt][4 * jj + i], acc[rt][nt][4 * jj + i]);
            }
        }
    }
}

// Super-blocks per float32 partial of the output (BIG kernels only, k
// above kGroup * 256): every kGroup super-blocks the consumers add their
// partial into a second accumulator and restart it, so that no float32 sum
// runs over more than kGroup super-blocks.  (Serial rounding error grows with
// the square root of the term count: at the largest k, 65536 super-blocks,
// one sum reaches 1.4e-5 relative; two levels of 256 stay near 2e-6.)
constexpr int kGroup = 256;

// Waves 0-7 consume (MFMA + fold), waves 8-15 produce (load, convert to
// binary16 operand slots, or with QT copy the tile block straight into LDS).
// Two LDS stages alternate: while the consumers
// work on stage s, the producers fill stage s+1 (their global loads run one
// stage further ahead in registers, two with int8 codes).  One workgroup
// barrier per stage.
template <int TB, bool H, bool REP, bool QT, bool BIG>
__global__ __launch_bounds__(NT) void mmq_f16_kernel(const uint8_t* __restrict__ w,
                                                     const int8_t* __restrict__ q,
                                                     const uint32_t* __restrict__ ds,
                                                     int M, int N, int K, int tiles_m, int tile_m0,
                                                     void* __restrict__ out) {
    __shared__ Stage stage[2];
    __shared__ StageB stage_b[2];

    const int tid = threadIdx.x;
    // row tiles tile_m0 .. tile_m0 + tiles_m - 1 of the M rows (a launch may
    // cover part of them), token tiles of TB
    const int bm = tile_m0 + blockIdx.x % tiles_m, bn = blockIdx.x / tiles_m;
    const int row0 = bm * BM, tok0 = bn * TB;
    const int stages = K >> 7;

    if (tid >= CT) {
        // ------------------------------------------------------- producer
        // Raw register sets rotate, so that the loads of later stages stay
        // in flight while stage s is converted (a register copy would force a
        // wait on them).  k is a multiple of 256, so the stage count is even.
        // Every load is unconditional (prefetches past the end re-read the
        // final stage), which lets the compiler wait only for the oldest set.
        const int pt = tid - CT;
        Src src;
        init_src<TB, REP, QT>(src, w, q, ds, pt, row0, tok0, M, N, K);
        Raw ra, rb;
        if constexpr (!QT) {
            // Three sets: loads run two stages ahead of the conversion (the
            // loads, not the conversions, bound the producers with one stage
            // of prefetch: measured 151 -> 132 us for the producers alone on
            // q-proj, 4-7% for the whole kernel; a fourth set gained
            // nothing).  Stage s uses set s % 3 and LDS stage s % 2, so the
            // loop body covers 6 stages.
            Raw rc;
            load_stage<TB, REP, QT>(ra, src, 0);
            load_stage<TB, REP, QT>(rb, src, min(1, stages - 1));
            for (int it = 0; it < stages; it += 6) {
                load_stage<TB, REP, QT>(rc, src, min(it + 2, stages - 1));
                convert_stage<TB, REP, QT>(ra, stage[0], stage_b[0], pt, it);
                __syncthreads();
                load_stage<TB, REP, QT>(ra, src, min(it + 3, stages - 1));
                convert_stage<TB, REP, QT>(rb, stage[1], stage_b[1], pt, it + 1);
                __syncthreads();
                if (it + 2 >= stages) break;
                load_stage<TB, REP, QT>(rb, src, min(it + 4, stages - 1));
                convert_stage<TB, REP, QT>(rc, stage[0], stage_b[0], pt, it + 2);
                __syncthreads();
                load_stage<TB, REP, QT>(rc, src, min(it + 5, stages - 1));
                convert_stage<TB, REP, QT>(ra, stage[1], stage_b[1], pt, it + 3);
                __syncthreads();
                if (it + 4 >= stages) break;
                load_stage<TB, REP, QT>(ra, src, min(it + 6, stages - 1));
                convert_stage<TB, REP, QT>(rb, stage[0], stage_b[0], pt, it + 4);
                __syncthreads();
                load_stage<TB, REP, QT>(rb, src, min(it + 7, stages - 1));
                convert_stage<TB, REP, QT>(rc, stage[1], stage_b[1], pt, it + 5);
                __syncthreads();
            }
        } else {
            // Operand tiles: two sets (the weights only; the q8 operands are
            // direct-to-LDS copies whose waits the loop places itself).
            // Everything older completes first (loads issued a half-step
            // ago), then the stage's q8 copies, so that waiting for them
            // before the barrier leaves only the next stage's loads in flight.
            const int pw = __builtin_amdgcn_readfirstlane(pt >> 6), lane = pt & 63;
            load_stage<TB, REP, QT>(ra, src, 0);
            for (int it = 0; it < stages; it += 2) {
                settle<REP>(ra);
                dma_stage<TB>(stage_b[0], src, it, pw, lane);
                load_stage<TB, REP, QT>(rb, src, it + 1);
                convert_stage<TB, REP, QT>(ra, stage[0], stage_b[0], pt, it);
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt(stage_loads<REP, QT>()));
                __syncthreads();
                settle<REP>(rb);
                dma_stage<TB>(stage_b[1], src, it + 1, pw, lane);
                load_stage<TB, REP, QT>(ra, src, min(it + 2, stages - 1));
                convert_stage<TB, REP, QT>(rb, stage[1], stage_b[1], pt, it + 1);
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt(stage_loads<REP, QT>()));
                __syncthreads();
            }
        }
        __syncthreads();  // the consumers' last stage
        return;
    }

    // ----------------------------------------------------------- consumer
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int RT = TB / 64;                 // 32-row tiles per wave
    constexpr int RW = 128 / (32 * RT);         // waves along the rows
    const int wm = wave % RW, wn = wave / RW;
    const int g = lane >> 5, l32 = lane & 31;

    v16f acc[2][NTW], accb[2][NTW], acc2[2][NTW];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NTW; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = acc2[a][b][v] = 0.0f;

    // Stages come in (first, second) half-super-block pairs: stage[0] holds
    // even stages, stage[1] odd ones.  The barriers pair with the producers'.
    __syncthreads();
    for (int st = 0; st < stages; st += 2) {
        consume_stage<0, RT>(stage[0], stage_b[0], wm, wn, g, l32, acc, accb);
        __syncthreads();
        consume_stage<1, RT>(stage[1], stage_b[1], wm, wn, g, l32, acc, accb);
        __syncthreads();
        if (BIG && (((st >> 1) + 1) & (kGroup - 1)) == 0) {
#pragma unroll
            for (int a = 0; a < RT; ++a)
#pragma unroll
                for (int b = 0; b < NTW; ++b) {
                    acc2[a][b] += acc[a][b];
                    acc[a][b] = v16f{};
                }
        }
    }
    if (BIG)
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int b = 0; b < NTW; ++b) acc[a][b] += acc2[a][b];

    const bool vec = (M & 3) == 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int tok = tok0 + wn * 32 * NTW + nt * 32 + l32;
            if (tok >= N) continue;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int o = row0 + wm * 32 * RT + rt * 32 + 8 * jj + 4 * g;
                const int64_t idx = (int64_t)tok * M + o;
                if (vec && o + 3 < M) {
                    store_out4<H>(out, idx, acc[rt][nt][4 * jj], acc[rt][nt][4 * jj + 1],
                                  acc[rt][nt][4 * jj + 2], acc[rt][nt][4 * jj + 3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (o + i < M) store_out<H>(out, idx + i, acc[rt][nt][4 * jj + i]);
                }
            }
        }
}

}  // namespace

// Token-tile width and tile count of a launch: tiles of 128 tokens, or of 64
// where 128-token tiles would not give every CU one (the 7B layer set at 512
// tokens 99 -> 88 us per projection: its 4096-row projections have 128 tiles
// of 128 tokens); with enough tiles the halved tiles lose (2630-token FFN
// 565 -> 690 us: each converts the whole weight tile for half the tokens).
//
// Where the 128-token tiles fill some rounds of 256 CUs and then part of one
// more, the launch is cut by rows (split_m): the first split_m row tiles in
// 128-token tiles, a whole number of rounds, and the remaining rows in
// 64-token tiles, at most one round of half-size tiles in place of the tail
// round (each output is the same arithmetic in either tile, bit for bit).
// The 11008-row projections of the 7B layer set: 86 x 16 tiles at 2048
// tokens = 80 x 16 + 6 x 32; 86 x 4 at 512 tokens = 64 x 4 + 22 x 8.
struct TileShape {
    int tiles_m;     // row tiles of 128
    bool half;       // the whole launch in 64-token tiles
    int split_m;     // 0, or the row tiles of the 128-token part
};

static TileShape tile_shape(int m, int n) {
    TileShape t;
    t.tiles_m = (m + BM - 1) / BM;
    const int64_t nt = (n + BN - 1) / BN, full = (int64_t)t.tiles_m * nt;
    t.half = full < 256;
    t.split_m = 0;
    if (!t.half && full % 256 != 0)
        for (int r = t.tiles_m - 1; r >= 1; --r)
            if ((int64_t)r * nt % 256 == 0) {
                if ((int64_t)(t.tiles_m - r) * ((n + BN / 2 - 1) / (BN / 2)) <= 256) t.split_m = r;
                break;
            }
    return t;
}

// The kernel instance for a launch: token tile, output type, weight layout,
// activation format, and whether k has more than kGroup super-blocks.
template <bool H, bool REP, bool QT>
static const void* pick_kernel(bool half_tiles, bool big) {
    if (half_tiles)
        return big ? (const void*)mmq_f16_kernel<BN / 2, H, REP, QT, true>
                   : (const void*)mmq_f16_kernel<BN / 2, H, REP, QT, false>;
    return big ? (const void*)mmq_f16_kernel<BN, H, REP, QT, true>
               : (const void*)mmq_f16_kernel<BN, H, REP, QT, false>;
}

static hipError_t launch_part(const void* f, const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                              int n, void* out, int tiles_m, int tile_m0, int tb, hipStream_t stream) {
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k,
                    (void*)&tiles_m, (void*)&tile_m0, (void*)&out};
    const int64_t tiles = (int64_t)tiles_m * ((n + tb - 1) / tb);
    return hipLaunchKernel(f, dim3((unsigned)tiles), dim3(NT), args, 0, stream);
}

// One launch, or the two parts of a row split, on the caller's stream.
template <bool H, bool REP, bool QT>
static hipError_t launch(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n, void* out,
                         hipStream_t stream) {
    const TileShape t = tile_shape(m, n);
    const bool big = (k >> 8) > kGroup;
    if (t.split_m == 0)
        return launch_part(pick_kernel<H, REP, QT>(t.half, big), w, m, k, q, ds, n, out, t.tiles_m, 0,
                           t.half ? BN / 2 : BN, stream);
    const hipError_t e = launch_part(pick_kernel<H, REP, QT>(false, big), w, m, k, q, ds, n, out, t.split_m, 0,
                                     BN, stream);
    if (e != hipSuccess) return e;
    return launch_part(pick_kernel<H, REP, QT>(true, big), w, m, k, q, ds, n, out, t.tiles_m - t.split_m,
                       t.split_m, BN / 2, stream);
}

hipError_t launch_mmq_fp32_f16(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                               int n, void* out, bool half_out, hipStream_t stream) {
    return half_out ? launch<true, false, false>(w, m, k, q, ds, n, out, stream)
                    : launch<false, false, false>(w, m, k, q, ds, n, out, stream);
}

hipError_t launch_mmq_fp32_f16_repacked(const uint8_t* wr, int m, int k, const int8_t* q,
                                        const uint32_t* ds, int n, float* out, hipStream_t stream) {
    return launch<false, true, false>(wr, m, k, q, ds, n, out, stream);
}

hipError_t launch_mmq_fp32_f16_tiles(const uint8_t* w, bool repacked, int m, int k, const uint16_t* qt,
                                     const uint32_t* ds, int n, float* out, hipStream_t stream) {
    const int8_t* q = reinterpret_cast<const int8_t*>(qt);
    return repacked ? launch<false, true, true>(w, m, k, q, ds, n, out, stream)
                    : launch<false, false, true>(w, m, k, q, ds, n, out, stream);
}

}  // namespace mmq
