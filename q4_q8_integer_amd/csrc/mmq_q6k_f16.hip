// mmq_q6k_f16.hip - q6_K x q8 matmul, float32 result, on gfx950 binary16
// MFMA (the path above 8 tokens).
//
// Method (q6_K, the second k-quant weight format named in the r31 page's
// closing notes of the yusiwen.cn "minfer" pages): one signed 8-bit scale per
// 16 weights, weight d*sc*(q - 32), so
//   out[t][o] = sum_c da[t,c] * d[o] * P[t][o][c],   P = sum_{32 k of chunk c} sc(k)*(q - 32)*q8.
// As in the q4_K binary16 kernel, the per-chunk work left for the vector ALU
// is one FMA per output (acc_b += da * P) once P comes out of the matrix
// core exactly.  sc*(q - 32) reaches 4096 in magnitude and is not exact in
// binary16, so the A operand is split into two exact binary16 values, both
// scaled by 1/64:
//   A1 = sc * nibble / 64          (|sc*nibble| <= 1920: 11 bits)
//   A2 = sc * (hi2 - 2) / 4        (= 16 sc (hi2 - 2) / 64, |.| <= 64)
// with q = nibble + 16*hi2, so A1 + A2 = sc*(q - 32)/64.  Each chunk runs
// four v_mfma_f32_32x32x16_f16 (A1 and A2 times the two 16-k halves of q8).
// Every partial sum is a multiple of 1/64 below 32*4096*127/64 < 2^18 in
// magnitude, so the float32 accumulation is exact in any order: P/64 is
// returned exactly, and the fold multiplies by 64*d (a power-of-2 scaling).
//
// Operand bits, exactly:
//   A1 pair: (x & 0x000F000F) | 0x64006400 = (1024 + n, 1024 + n');
//            fma(1024 + n, sc/64, -16 sc) = sc*n/64  (sc/64 and -16 sc exact)
//   A2 pair: (y & 0x00030003) | 0x64006400 = (1024 + h, ...);
//            ((1024 + h) - 1026) * (sc/4) = (h - 2)*sc/4
//   q8 pair: byte ^ 0x80 under exponent 0x64 gives 1152 + q, minus 1152.
// Pairs are (byte 0, byte 2) and (byte 1, byte 3) of a dword on both sides,
// so A and B agree on k.
//
// Tiling: workgroup 128 rows x 128 tokens; 8 consumer waves (64 rows x 32
// tokens each) and 8 producer waves; k staged 64 at a time (two chunks) in
// two alternating LDS stages, four stages per super-block.  q6_K blocks are
// only 2-byte aligned, and 16-byte loads at unaligned addresses keep the
// address unit busy, so once per super-block the producers copy each row's
// 210 bytes into LDS with aligned 16-byte loads (two raw areas alternate,
// the next super-block's copied during the current one), and take every
// field from there as aligned dwords shifted into place.
#include "f16_operand.h"
#include "internal.h"
#include "kquant_device.h"
#include "q6k_device.h"

namespace mmq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128;
constexpr int CT = 512;          // consumer threads (8 waves of 64 rows x 32 tokens)
constexpr int PT = 512;          // producer threads (8 waves)
constexpr int NT = CT + PT;
constexpr int CS = 2;            // chunks per stage (64 k)
// s_waitcnt operand: at most n vector-memory operations outstanding.
// One (token tile, 128-k stage) block of the q8 operand tiles (bytes).
constexpr int kQtBlockBytes = 16 * BN * 16;

// One stage (64 k = 2 chunks) of operands.  Slots of 8 halves laid out
// [chunk][part][j][lane-half][row or token]: MFMA j of a chunk takes, in
// lane half g, k = 16 g + 8 j .. +7 of the chunk (the q4_K kernel's order, so
// that q8 operand tiles serve both); the 32 lanes of a half-wave read 32
// consecutive 16-byte slots.  The q8 operands are an LDS array of their own
// (StageB), so that the compiler can tell direct-to-LDS copies into it from
// the weight stores.
struct StageB {
    uint4 B[CS][2][2][BN];      // q8 as binary16
};
struct Stage {
    uint4 A[CS][2][2][2][BM];   // parts A1, A2
    float D[BM];                // 64*d of the super-block, per row
    float Da[CS][BN];           // da per (chunk, token)
};

// Raw copy of one super-block's 128 blocks: row r's bytes from the 16-byte
// boundary at or below its block, 14 pieces (224 bytes), at r * kRawStride.
// The stride is an odd number of dwords, so the 64 lanes of a wave (64
// consecutive rows) reading, or writing, one dword each hit distinct banks.
// Producer thread pt copies pieces (pt >> 7) + 4j of row pt & 127: a wave
// writes the same piece of 64 consecutive rows.  (Consecutive pieces of one
// row per wave read global memory in longer runs, but their dword stores
// from rows 57 dwords apart met in the same banks: 9.7% of the kernel's
// LDS-active cycles were bank conflicts, 0.7% without them.)
constexpr int kRawPieces = 14;
constexpr int kRawStride = 228;
constexpr int kRawPiecesPerThread = (kRawPieces + PT / BM - 1) / (PT / BM);   // 4
struct Raw16 {
    uint8_t b[BM * kRawStride];
};

// Raw global data of one stage, as one producer thread loads it: its weight
// item (row, chunk of the stage gi, k-half kh) - two 16-byte code fields and
// the dword holding its scale, and d - one 16-byte q8 piece and, for the
// first 256 threads, one scale word.
struct Raw {
    uint4 y;
    uint32_t word;
};

// The aligned 16-byte pieces of the next super-block's raw copy, as one
// producer thread loads them.
struct RawPieces {
    uint4 v[kRawPiecesPerThread];
};

// Producer sources: buffer resources based at the workgroup's first row and
// token, so every offset fits 32 bits and an offset past the extent reads 0.
struct Src {
    __amdgpu_buffer_rsrc_t w, q, ds;
    const uint16_t* qt;   // operand tiles (QT): the workgroup's 128-token tile
    int extent;           // bytes of the weight resource
    int rbytes;           // bytes of one row (k/256 blocks)
    int y, word;          // q8 piece and scale-word byte offsets (stage 0)
};

// Weight item of producer thread pt: row pt & 127, chunk-in-stage gi and
// k-half kh from pt >> 7 (threads 0..127 of a half take consecutive rows).
__device__ __forceinline__ void item_of(int pt, int& row, int& gi, int& kh) {
    row = pt & (BM - 1);
    gi = (pt >> 7) & 1;
    kh = pt >> 8;
}

__device__ __forceinline__ void init_src(Src& p, const uint8_t* __restrict__ w,
                                         const int8_t* __restrict__ q,
                                         const uint32_t* __restrict__ ds, int pt, int row0,
                                         int tok0, int M, int N, int K) {
    const int S = K >> 8, C = K >> 5;
    const int rows = min(BM, M - row0), toks = min(BN, N - tok0);
    const int64_t rbytes = (int64_t)S * kQ6kBlockBytes;
    // The raw copy reads whole 16-byte pieces, up to 14 bytes past a row's
    // block: past the workgroup's last row that is the next row (16 more
    // bytes of extent), except at the end of the matrix.
    const int64_t left = ((int64_t)M - row0) * rbytes;
    p.extent = (int)min(left, rows * rbytes + 16);
    p.rbytes = (int)rbytes;
    p.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + (int64_t)row0 * rbytes), 0,
                                            p.extent, kBufferFlags);
    p.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(q + (int64_t)tok0 * K), 0,
                                            (int)((uint32_t)toks * (uint32_t)K), kBufferFlags);   // up to 2^31 bytes
    p.ds = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(ds + (int64_t)tok0 * C), 0,
                                             toks * C * 4, kBufferFlags);
    // q8 piece pt: token pt & 127, 16-byte piece pt >> 7 of the stage's 64 bytes
    p.y = min(pt & (BN - 1), toks - 1) * K + 16 * (pt >> 7);
    p.qt = reinterpret_cast<const uint16_t*>(q) + (int64_t)(tok0 >> 7) * (K >> 7) * (kQtBlockBytes / 2);
    // scale word (threads < 256): token pt & 127, chunk-in-stage pt >> 7
    p.word = (min(pt & (BN - 1), toks - 1) * C + ((pt >> 7) & 1)) * 4;
}

// Offset in the resource of row r's block of super-block sb (rows past the
// workgroup's last repeat it).
__device__ __forceinline__ int block_off(const Src& p, int r, int sb) {
    return r * p.rbytes + sb * kQ6kBlockBytes;
}

// Issue the loads of the raw copy of super-block sb: piece (pt >> 7) + 4j
// of row pt & 127 (rows past the workgroup's last repeat it).  A piece that
// would cross the end of the resource (only at the end of the matrix) is
// read as 2-byte halves within it; the rest of it is never used.
__device__ __forceinline__ void load_raw(RawPieces& rp, const Src& p, int rows, int pt, int sb) {
#pragma unroll
    for (int j = 0; j < kRawPiecesPerThread; ++j) {
        const int pc = (pt >> 7) + (PT / BM) * j;
        const int r = min(pt & (BM - 1), rows - 1);
        const int o = (block_off(p, r, sb) & ~15) + 16 * pc;
        if (pc >= kRawPieces) {
            rp.v[j] = make_uint4(0, 0, 0, 0);
        } else if (o + 16 <= p.extent) {
            rp.v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(p.w, o, 0, 0));
        } else {
            uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (o + 2 * e + 2 <= p.extent)
                    d[e >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(p.w, o + 2 * e, 0, 0) << (16 * (e & 1));
            rp.v[j] = make_uint4(d[0], d[1], d[2], d[3]);
        }
    }
}

__device__ __forceinline__ void store_raw(const RawPieces& rp, Raw16& raw, int pt) {
#pragma unroll
    for (int j = 0; j < kRawPiecesPerThread; ++j) {
        const int pc = (pt >> 7) + (PT / BM) * j, r = pt & (BM - 1);
        if (pc >= kRawPieces) continue;
        uint32_t* dst = reinterpret_cast<uint32_t*>(raw.b + r * kRawStride + 16 * pc);
        dst[0] = rp.v[j].x;
        dst[1] = rp.v[j].y;
        dst[2] = rp.v[j].z;
        dst[3] = rp.v[j].w;
    }
}

template <bool QT>
__device__ __forceinline__ void load_stage(Raw& r, const Src& p, int pt, int st) {
    if (!QT) r.y = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(p.q, p.y, 64 * st, 0));
    r.word = pt < 2 * BN ? __builtin_amdgcn_raw_buffer_load_b32(p.ds, p.word, 8 * st, 0) : 0u;
}

// The five LDS dwords covering 16 bytes at byte a (2-aligned) of a row's raw copy.
__device__ __forceinline__ void raw_run(const uint8_t* row_raw, int a, uint32_t (&v)[5]) {
    const uint32_t* q4 = reinterpret_cast<const uint32_t*>(row_raw + (a & ~3));
#pragma unroll
    for (int i = 0; i < 5; ++i) v[i] = q4[i];
}

template <bool QT>
__device__ __forceinline__ void convert_stage(const Raw& r, const Raw16& raw, Stage& sg, StageB& sgb,
                                              const Src& p, int rows, int pt, int st) {
    int row, gi, kh;
    item_of(pt, row, gi, kh);
    const int sb = st >> 2, s4 = st & 3, h = s4 >> 1, g = 2 * (s4 & 1) + gi;
    const int bo = block_off(p, min(row, rows - 1), sb);
    const int lo = bo & 15;                       // block start within the row's raw copy
    const uint32_t sh = (uint32_t)bo & 3u;
    const uint8_t* row_raw = raw.b + row * kRawStride;
    uint32_t ql[5], qh[5];
    raw_run(row_raw, lo + 64 * h + 32 * (g & 1) + 16 * kh, ql);
    raw_run(row_raw, lo + 128 + 32 * h + 16 * kh, qh);
    const int osc = lo + 192 + 8 * h + 2 * g + kh;
    const int sc = (int)(int8_t)(*reinterpret_cast<const uint32_t*>(row_raw + (osc & ~3)) >> (8 * (osc & 3)));
    const uint32_t c1 = f16x2_splat((float)sc * 0.015625f);   // sc/64
    const uint32_t n1 = f16x2_splat(-16.0f * (float)sc);      // -16 sc
    const uint32_t c2 = f16x2_splat((float)sc * 0.25f);       // sc/4
    const uint32_t m1026 = 0xE402E402u;                         // (-1026, -1026)
    const int nsh = 4 * (g >> 1), hsh = 2 * g;
    uint32_t a1[8], a2[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = q6k::run_word(ql, i, sh) >> nsh;
        const uint32_t y = q6k::run_word(qh, i, sh) >> hsh;
        a1[2 * i] = pk_fma_f16(and_or(x, 0x000F000Fu, 0x64006400u), c1, n1);
        a1[2 * i + 1] = pk_fma_f16(and_or(x >> 8, 0x000F000Fu, 0x64006400u), c1, n1);
        a2[2 * i] = pk_mul_f16(pk_add_f16(and_or(y, 0x00030003u, 0x64006400u), m1026), c2);
        a2[2 * i + 1] = pk_mul_f16(pk_add_f16(and_or(y >> 8, 0x00030003u, 0x64006400u), m1026), c2);
    }
    // the item's 16 k (16 kh .. +15 of chunk gi): its first 8 go to MFMA 0,
    // its last 8 to MFMA 1, both in lane half kh
    const int c = gi;
    sg.A[c][0][0][kh][row] = make_uint4(a1[0], a1[1], a1[2], a1[3]);
    sg.A[c][0][1][kh][row] = make_uint4(a1[4], a1[5], a1[6], a1[7]);
    sg.A[c][1][0][kh][row] = make_uint4(a2[0], a2[1], a2[2], a2[3]);
    sg.A[c][1][1][kh][row] = make_uint4(a2[4], a2[5], a2[6], a2[7]);
    if (gi == 0 && kh == 0) {
        const int od = lo + 208;   // 2-aligned: d lies in the dword at od & ~3
        const uint32_t dw = *reinterpret_cast<const uint32_t*>(row_raw + (od & ~3)) >> (8 * (od & 3));
        sg.D[row] = 64.0f * half_lo(dw);
    }
    // q8 piece: token pt & 127, k 16*(pt >> 7) .. +15 of the stage (QT: copied
    // by dma_stage instead)
    if (!QT) {
        const int tok = pt & (BN - 1), pc = pt >> 7, cc = pc >> 1, kk = pc & 1;
        uint32_t pp[8];
        q8_word(r.y.x, pp[0], pp[1]);
        q8_word(r.y.y, pp[2], pp[3]);
        q8_word(r.y.z, pp[4], pp[5]);
        q8_word(r.y.w, pp[6], pp[7]);
        sgb.B[cc][0][kk][tok] = make_uint4(pp[0], pp[1], pp[2], pp[3]);
        sgb.B[cc][1][kk][tok] = make_uint4(pp[4], pp[5], pp[6], pp[7]);
    }
    if (pt < 2 * BN) sg.Da[pt >> 7][pt & (BN - 1)] = half_lo(r.word);
}

// One stage for one consumer wave (64 rows x 32 tokens as 2 tiles of 32x32).
// FIRST: the stage opens a super-block (the first chunk sets acc_b);
// LAST: it closes one (out += 64 d * acc_b).
template <bool FIRST, bool LAST>
__device__ __forceinline__ void consume_stage(const Stage& sg, const StageB& sb, int wm, int wn, int g,
                                              int l32, v16f (&acc)[2], v16f (&accb)[2]) {
    const int t = wn * 32 + l32;
#pragma unroll
    for (int c = 0; c < CS; ++c) {
        const v8h b0 = __builtin_bit_cast(v8h, sb.B[c][0][g][t]);
        const v8h b1 = __builtin_bit_cast(v8h, sb.B[c][1][g][t]);
        const float da = sg.Da[c][t];
        v16f pr[2];
        const v16f zero = {};
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int rr = wm * 64 + rt * 32 + l32;
            pr[rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, sg.A[c][0][0][g][rr]), b0,
                                                            zero, 0, 0, 0);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int rr = wm * 64 + rt * 32 + l32;
            pr[rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, sg.A[c][0][1][g][rr]), b1,
                                                            pr[rt], 0, 0, 0);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int rr = wm * 64 + rt * 32 + l32;
            pr[rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, sg.A[c][1][0][g][rr]), b0,
                                                            pr[rt], 0, 0, 0);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int rr = wm * 64 + rt * 32 + l32;
            pr[rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, sg.A[c][1][1][g][rr]), b1,
                                                            pr[rt], 0, 0, 0);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (FIRST && c == 0)
                accb[rt] = pr[rt] * da;
            else
#pragma unroll
                for (int v = 0; v < 16; ++v) accb[rt][v] = fmaf(da, pr[rt][v], accb[rt][v]);
        }
    }
    if (LAST) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float4 d4 = *reinterpret_cast<const float4*>(&sg.D[wm * 64 + rt * 32 + 8 * jj + 4 * g]);
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[rt][4 * jj + i] = fmaf(dv[i], accb[rt][4 * jj + i], acc[rt][4 * jj + i]);
            }
    }
}

// QT: a stage's q8 operands (64 k) are the half (st & 1) of the operand-tile
// block of 128 k, slot rows 8 (st & 1) .. +7: 16 KiB, copied with 16
// direct-to-LDS loads of one KiB (64 token slots), 2 per producer wave.  As
// in the q4_K kernel, the copies are inline asm outside the compiler's wait
// bookkeeping, and the producer loop completes older loads before issuing
// them and waits for everything before the stage barrier.
__device__ __forceinline__ void dma_stage(StageB& sb, const Src& p, int st, int pw, int lane) {
    const uint64_t a = reinterpret_cast<uint64_t>(p.qt + (int64_t)(st >> 1) * (kQtBlockBytes / 2));
    const u32x4 rsrc = {(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, (uint32_t)kQtBlockBytes,
                        (uint32_t)kBufferFlags};
    const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4*)&sb.B[0][0][0][0];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int i = pw * 2 + j, row = i >> 1, half = i & 1;
        const int dst = row * BN + half * 64;
        lds_copy16(rsrc, base + 16 * dst, ((8 * (st & 1) + row) * BN + half * 64 + lane) * 16);
    }
}

// An empty asm that reads registers a producer loaded earlier: the compiler
// completes those loads here, before the uncounted copies are issued.
__device__ __forceinline__ void settle(const Raw& r) { asm volatile("" ::"v"(r.word)); }
__device__ __forceinline__ void settle(const RawPieces& rp) {
#pragma unroll
    for (int j = 0; j < kRawPiecesPerThread; ++j)
        asm volatile("" ::"v"(rp.v[j].x), "v"(rp.v[j].y), "v"(rp.v[j].z), "v"(rp.v[j].w));
}

// Super-blocks per float32 partial of the output (BIG kernels only, k above
// kGroup * 256): every kGroup super-blocks the consumers add their partial
// into a second accumulator and restart it, so that no float32 sum runs over
// more than kGroup super-blocks (the serial rounding error grows with the
// square root of the term count).
constexpr int kGroup = 256;

// Waves 0-7 consume (MFMA + fold), waves 8-15 produce (load, convert).  Two
// LDS stages alternate: while the consumers work on stage s, the producers
// fill stage s+1, their loads running one stage further ahead in registers.
// One workgroup barrier per stage.
template <bool H, bool QT, bool BIG>
__global__ __launch_bounds__(NT) void mmq_q6k_f16_kernel(const uint8_t* __restrict__ w,
                                                         const int8_t* __restrict__ q,
                                                         const uint32_t* __restrict__ ds,
                                                         int M, int N, int K, int tiles_m,
                                                         void* __restrict__ out) {
    __shared__ Stage stage[2];
    __shared__ StageB stage_b[2];
    __shared__ Raw16 raw[2];

    const int tid = threadIdx.x;
    const int bm = blockIdx.x % tiles_m, bn = blockIdx.x / tiles_m;
    const int row0 = bm * BM, tok0 = bn * BN;
    const int stages = K >> 6;   // a multiple of 4

    if (tid >= CT) {
        // Producers.  Two register sets of q8 data alternate (stage s+1's
        // loads stay in flight while stage s is converted), and the raw copy
        // of super-block sb+1 is loaded during sb and stored after its second
        // stage: the stage barriers that follow order it before its first
        // reader and after the last reader of the area it replaces.
        const int pt = tid - CT;
        const int rows = min(BM, M - row0);
        Src src;
        init_src(src, w, q, ds, pt, row0, tok0, M, N, K);
        const int S = K >> 8;
        Raw ra, rb;
        RawPieces rp;
        load_raw(rp, src, rows, pt, 0);
        store_raw(rp, raw[0], pt);
        load_stage<QT>(ra, src, pt, 0);
        const int pw = __builtin_amdgcn_readfirstlane(pt >> 6), lane = pt & 63;
        __syncthreads();   // raw copy 0 visible (the consumers meet it too)
        for (int it = 0; it < stages; it += 2) {
            const int sb = it >> 2;
            if (QT) settle(ra);
            if ((it & 3) == 0) load_raw(rp, src, rows, pt, min(sb + 1, S - 1));
            load_stage<QT>(rb, src, pt, it + 1);
            if (QT) dma_stage(stage_b[0], src, it, pw, lane);
            convert_stage<QT>(ra, raw[sb & 1], stage[0], stage_b[0], src, rows, pt, it);
            if (QT) __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
            __syncthreads();
            if (QT) {
                settle(rb);
                settle(rp);
            }
            load_stage<QT>(ra, src, pt, min(it + 2, stages - 1));
            if (QT) dma_stage(stage_b[1], src, it + 1, pw, lane);
            convert_stage<QT>(rb, raw[sb & 1], stage[1], stage_b[1], src, rows, pt, it + 1);
            if ((it & 3) == 0 && sb + 1 < S) store_raw(rp, raw[(sb + 1) & 1], pt);
            if (QT) __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
            __syncthreads();
        }
        __syncthreads();  // the consumers' last stage
        return;
    }

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int g = lane >> 5, l32 = lane & 31;

    v16f acc[2], accb[2], acc2[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][v] = accb[a][v] = acc2[a][v] = 0.0f;

    // Four stages per super-block: (first, -, -, last) on stages 0,1,0,1.
    __syncthreads();   // the producers' raw copy 0
    __syncthreads();
    for (int st = 0; st < stages; st += 4) {
        consume_stage<true, false>(stage[0], stage_b[0], wm, wn, g, l32, acc, accb);
        __syncthreads();
        consume_stage<false, false>(stage[1], stage_b[1], wm, wn, g, l32, acc, accb);
        __syncthreads();
        consume_stage<false, false>(stage[0], stage_b[0], wm, wn, g, l32, acc, accb);
        __syncthreads();
        consume_stage<false, true>(stage[1], stage_b[1], wm, wn, g, l32, acc, accb);
        __syncthreads();
        if (BIG && (((st >> 2) + 1) & (kGroup - 1)) == 0) {
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                acc2[a] += acc[a];
                acc[a] = v16f{};
            }
        }
    }
    if (BIG)
#pragma unroll
        for (int a = 0; a < 2; ++a) acc[a] += acc2[a];

    const bool vec = (M & 3) == 0;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int tok = tok0 + wn * 32 + l32;
        if (tok >= N) continue;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int o = row0 + wm * 64 + rt * 32 + 8 * jj + 4 * g;
            const int64_t idx = (int64_t)tok * M + o;
            if (vec && o + 3 < M) {
                store_out4<H>(out, idx, acc[rt][4 * jj], acc[rt][4 * jj + 1], acc[rt][4 * jj + 2],
                              acc[rt][4 * jj + 3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (o + i < M) store_out<H>(out, idx + i, acc[rt][4 * jj + i]);
            }
        }
    }
}

}  // namespace

hipError_t launch_q6k_f16(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
                          void* out, bool half_out, hipStream_t stream) {
    int tiles_m = (m + BM - 1) / BM;
    const int64_t tiles = (int64_t)tiles_m * ((n + BN - 1) / BN);
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k,
                    (void*)&tiles_m, (void*)&out};
    const bool big = (k >> 8) > kGroup;
    const void* f = half_out ? (big ? (const void*)mmq_q6k_f16_kernel<true, false, true>
                                    : (const void*)mmq_q6k_f16_kernel<true, false, false>)
                             : (big ? (const void*)mmq_q6k_f16_kernel<false, false, true>
                                    : (const void*)mmq_q6k_f16_kernel<false, false, false>);
    return hipLaunchKernel(f, dim3((unsigned)tiles), dim3(NT), args, 0, stream);
}

hipError_t launch_q6k_f16_tiles(const uint8_t* w, int m, int k, const uint16_t* qt, const uint32_t* ds,
                                int n, float* out, hipStream_t stream) {
    int tiles_m = (m + BM - 1) / BM;
    const int64_t tiles = (int64_t)tiles_m * ((n + BN - 1) / BN);
    const int8_t* q = reinterpret_cast<const int8_t*>(qt);
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k,
                    (void*)&tiles_m, (void*)&out};
    const void* f = (k >> 8) > kGroup ? (const void*)mmq_q6k_f16_kernel<false, true, true>
                                      : (const void*)mmq_q6k_f16_kernel<false, true, false>;
    return hipLaunchKernel(f, dim3((unsigned)tiles), dim3(NT), args, 0, stream);
}

}  // namespace mmq
