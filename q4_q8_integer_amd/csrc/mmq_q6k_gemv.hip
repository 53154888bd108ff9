// mmq_q6k_gemv.hip - q6_K x q8 matmul for very few tokens (1 <= n <= 8),
// float32 result, on the vector ALU's 4-way int8 dot product.
//
// Method as in mmq_q6k_i8.hip (q6_K, the second k-quant weight format named
// in the r31 page's closing notes of the yusiwen.cn "minfer" pages): per
// 16-weight group an exact integer dot D = sum (q - 32) * q8, then
// out[t][o] = sum_g d*sc[g] * da[t, g/2] * D.
//
//   * A wave owns 16 weight rows.  Lane 16p + r takes row r and quarter
//     p = 2h + e of every super-block: the weights 128h + 32g + 16e + [0, 16)
//     for g = 0..3 (four scale groups, in the four chunks 4h + g).  Its bytes
//     are three 16-byte fields of the block (two of ql, one of qh), decoded to
//     signed codes q - 32 with one v_perm_b32 table lookup per 4 weights.
//   * The 16 lanes of a DPP row share the quarter, so they need the same 64
//     token bytes: lane r loads token dword (g, i) = (r >> 2, r & 3) (the 64
//     lanes of a wave together read a token's 256-byte super-block in one
//     coalesced load), and v_dot4c reads it from lane 4g + i through a
//     row_newbcast DPP operand.  Lanes 0-3 of a row hold the scale words of
//     chunks 4h + 0..3, broadcast the same way into v_fmac.
//   * A wave step covers 16 rows x SW consecutive super-blocks.  q6_K blocks
//     (210 bytes) start only 2-byte aligned, and 16-byte loads at 4-byte
//     aligned addresses measured slow (the address unit was ~65% busy), so
//     the step's bytes of each row are first copied into the wave's LDS area
//     with aligned 16-byte buffer loads that write LDS directly, and the
//     block fields are read from LDS.  With enough steps per wave a second
//     area takes the next step's copy while a step computes (it costs no
//     registers).
//   * A workgroup is 16 rows; its waves split the super-blocks, and the
//     partial sums are added in a fixed order (the four quarter lanes of a
//     row by a butterfly, then the waves in index order).
#include "internal.h"
#include "kquant_device.h"
#include "q6k_device.h"

namespace mmq {
namespace {

constexpr int kMaxWaves = 4;   // waves per workgroup (split of the super-blocks)

// Each dot chain starts from the bits of kMagic = 1.5 * 2^23 instead of 0:
// as |D| < 2^22, the integer sum kMagic_bits + D is the float32 kMagic + D
// exactly, and fma(dsc, kMagic + D, -kMagic * dsc) rounds the exact dsc * D
// once, as dsc * float(D) does (-kMagic * dsc is exact: dsc = d * sc has at
// most 19 significant bits, times 3 * 2^22 at most 21).  One instruction in
// place of a conversion and a multiply.
constexpr float kMagic = 12582912.0f;
constexpr int kMagicBits = 0x4B400000;

// Four group dots of one token: Df[g] = kMagic + sum_i dot4(cw[g][i], token
// word 4g + i of the DPP row), exact as |D| <= 65024.  The asm keeps the
// hazard rules the compiler cannot see: 2 wait states before a DPP read of a
// VALU-written source (s_nop 1), and 3 between a v_dot4 result and a non-dot
// VALU reading it (s_nop 2 last).
__device__ __forceinline__ void group_dots(float (&Df)[4], uint32_t tok, const uint32_t (&cw)[4][4]) {
    int A0 = kMagicBits, A1 = kMagicBits, A2 = kMagicBits, A3 = kMagicBits;
    asm("s_nop 1\n\t"
        "v_dot4c_i32_i8_dpp %0, %4, %5 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %4, %9 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %4, %13 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %4, %17 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %4, %6 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %4, %10 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %4, %14 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %4, %18 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %4, %7 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %4, %11 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %4, %15 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %4, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %4, %8 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %4, %12 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %4, %16 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %4, %20 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 2"
        : "+v"(A0), "+v"(A1), "+v"(A2), "+v"(A3)
        : "v"(tok), "v"(cw[0][0]), "v"(cw[0][1]), "v"(cw[0][2]), "v"(cw[0][3]), "v"(cw[1][0]),
          "v"(cw[1][1]), "v"(cw[1][2]), "v"(cw[1][3]), "v"(cw[2][0]), "v"(cw[2][1]), "v"(cw[2][2]),
          "v"(cw[2][3]), "v"(cw[3][0]), "v"(cw[3][1]), "v"(cw[3][2]), "v"(cw[3][3]));
    Df[0] = __builtin_bit_cast(float, A0);
    Df[1] = __builtin_bit_cast(float, A1);
    Df[2] = __builtin_bit_cast(float, A2);
    Df[3] = __builtin_bit_cast(float, A3);
}

// acc += sum_g da(lane g of the DPP row) * y[g]
__device__ __forceinline__ void fold4(float& acc, float da, const float (&y)[4]) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %1, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(da), "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]));
}

// One wave step: SW super-blocks of 16 rows.  The rows' bytes are copied
// into the wave's LDS area by buffer loads that write LDS directly (no
// registers hold the copy): row r's run of SW blocks, from the 16-byte
// boundary below its first byte, in aligned 16-byte pieces.  Slot i of the
// area (16 bytes at 16*i) holds piece i % kSlots of row i / kSlots; the last
// slot of a row is padding, which spreads the 16 rows' reads over the banks.
// The 2-byte-aligned block fields are then read from LDS as aligned dwords
// and shifted into place (see q6k_device.h).
template <int SW>
struct Seg {
    static constexpr int kChunks = (SW * kQ6kBlockBytes + 14 + 15) / 16;  // pieces per row
    static constexpr int kSlots = kChunks + 1;
    static constexpr int kBytes = 16 * kSlots;                           // row stride in LDS
    static constexpr int kArea = 16 * kBytes;
    static constexpr int kLoads = (16 * kSlots + 63) / 64;               // load instructions per step
};

// s_waitcnt operand: no vector-memory operation outstanding, the other
// counters untouched
constexpr int kWaitVmcnt0 = 0x0F70;

// A 16-byte piece at byte offset a (a % 16 == 0) of the weights, reading
// nothing at or past byte `total` (its bytes past the end read as 0).
__device__ __forceinline__ uint4 load_piece(const uint8_t* __restrict__ w, int64_t a, int64_t total) {
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (a + 2 * i + 2 <= total)
            d[i >> 1] |= (uint32_t)*reinterpret_cast<const uint16_t*>(w + a + 2 * i) << (16 * (i & 1));
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// The five LDS dwords covering 16 bytes at LDS byte address `a` (2-aligned).
__device__ __forceinline__ void lds_run(const uint8_t* base, int a, uint32_t (&v)[5]) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(base + (a & ~3));
#pragma unroll
    for (int i = 0; i < 5; ++i) v[i] = p[i];
}

// The weights of a workgroup's tile of rows: a buffer resource over its
// whole 16-byte pieces, and the partial piece at its end (the tile's bytes
// need not end on a 16-byte boundary), which a buffer load would read as
// zeros and stage_patch copies in with 2-byte loads.
struct Tile {
    __amdgpu_buffer_rsrc_t rs;
    const uint8_t* base;
    int end;     // the tile's bytes
    int rows;    // rows in the tile
};

// Issue the copy of the step at super-block s into `area`.  Pieces past a
// row's end (a wave's last step may run over it) read the next row, past
// the resource they read zeros; neither is used.
template <int SW>
__device__ __forceinline__ void stage_issue(const Tile& tl, int S, int s, int lane, uint8_t* area) {
    typedef Seg<SW> G;
#pragma unroll
    for (int c = 0; c < G::kLoads; ++c) {
        const int i = lane + 64 * c;
        const int rr = i / G::kSlots, ch = min(i - rr * G::kSlots, G::kChunks - 1);
        const int off = (((rr * S + s) * kQ6kBlockBytes) & ~15) + 16 * ch;
        if (i < 16 * G::kSlots)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(tl.rs, (__attribute__((address_space(3))) void*)(area + 1024 * c),
                                                     16, off, 0, 0, 0);
    }
}

// After the copy of step s has landed: the tile's partial last piece, if
// this step's run of the tile's last row covers it.
template <int SW>
__device__ __forceinline__ void stage_patch(const Tile& tl, int S, int s, int lane, uint8_t* area) {
    typedef Seg<SW> G;
    const int end16 = tl.end & ~15;
    if (end16 == tl.end) return;
    const int rr = tl.rows - 1;
    const int ch = (end16 - (((rr * S + s) * kQ6kBlockBytes) & ~15)) >> 4;
    if (lane == 0 && ch >= 0 && ch < G::kChunks)
        *reinterpret_cast<uint4*>(area + rr * G::kBytes + 16 * ch) = load_piece(tl.base, end16, tl.end);
}

// The activations of one wave step, as one lane holds them: its token dword
// and scale word of every slot.
template <int N, int SW>
struct Fetch {
    uint32_t tq[N][SW], tw[N][SW];
};

// Issue the activation loads of the step at super-block s (slots past the
// wave's range re-read its last block and are not used).
template <int N, int SW>
__device__ __forceinline__ void fetch_step(Fetch<N, SW>& f, const int8_t* __restrict__ q,
                                           const uint32_t* __restrict__ ds, int K, int C, int s,
                                           int last, int h, int e, int r) {
#pragma unroll
    for (int j = 0; j < SW; ++j) {
        const int sb = min(s + j, last);
        const int64_t toff = (int64_t)sb * 256 + 128 * h + 32 * (r >> 2) + 16 * e + 4 * (r & 3);
        const int64_t woff = (int64_t)sb * 8 + 4 * h + (r & 3);
#pragma unroll
        for (int t = 0; t < N; ++t) {
            f.tq[t][j] = q6k::ld32(reinterpret_cast<const uint8_t*>(q) + (int64_t)t * K + toff);
            f.tw[t][j] = ds[(int64_t)t * C + woff];
        }
    }
}

// Compute the step at super-block s from the wave's LDS copy.  rowS = the
// lane's row times S (any row past the matrix reads a zero copy and is not
// stored).
template <int N, int SW>
__device__ __forceinline__ void compute_step(const Fetch<N, SW>& f, const uint8_t* __restrict__ lds,
                                             int64_t rowS, int s, int last, int h, int e, int r,
                                             float* acc) {
    typedef Seg<SW> G;
    const int64_t base0 = ((rowS + s) * kQ6kBlockBytes) & ~(int64_t)15;
    const uint8_t* row_lds = lds + r * G::kBytes;
#pragma unroll
    for (int j = 0; j < SW; ++j) {
        // byte offset of block s + j in the row's LDS copy; a slot past the
        // wave's last block reads the last block (and computes with d = 0)
        const int off = (int)((rowS + min(s + j, last)) * kQ6kBlockBytes - base0);
        const uint32_t sh = (uint32_t)off & 3u;
        uint32_t ql0[5], ql1[5], qh[5], sc[5], cw[4][4];
        lds_run(row_lds, off + q6k::ql0_off(h, e), ql0);
        lds_run(row_lds, off + q6k::ql1_off(h, e), ql1);
        lds_run(row_lds, off + q6k::qh_off(h, e), qh);
        lds_run(row_lds, off + 192, sc);
        const uint32_t dword = *reinterpret_cast<const uint32_t*>(row_lds + ((off + 208) & ~3));
        q6k::quarter_codes(ql0, ql1, qh, sh, cw);
        const float d = s + j <= last ? half_lo(dword >> (8 * sh)) : 0.0f;
        // scales of groups 8h + 2g + e: byte 2(g & 1) + e of scale word 2h + (g >> 1)
        const uint32_t w0 = q6k::run_word(sc, 0, sh), w1 = q6k::run_word(sc, 1, sh);
        const uint32_t w2 = q6k::run_word(sc, 2, sh), w3 = q6k::run_word(sc, 3, sh);
        const uint32_t lo = h ? w2 : w0, hi = h ? w3 : w1;
        float dsc[4], kn[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            dsc[g] = d * (float)(int)(int8_t)(((g >> 1) ? hi : lo) >> (8 * (2 * (g & 1) + e)));
            kn[g] = -kMagic * dsc[g];
        }
#pragma unroll
        for (int t = 0; t < N; ++t) {
            float Df[4], y[4];
            group_dots(Df, f.tq[t][j], cw);
#pragma unroll
            for (int g = 0; g < 4; ++g) y[g] = fmaf(dsc[g], Df[g], kn[g]);
            fold4(acc[t], half_lo(f.tw[t][j]), y);
        }
    }
}

// PF: two LDS areas per wave, the next step's copy (and activation loads)
// in flight while a step computes.
template <int N, int SW, bool PF, bool H>
__global__ __launch_bounds__(64 * kMaxWaves) void mmq_q6k_gemv_kernel(const uint8_t* __restrict__ w,
                                                                      const int8_t* __restrict__ q,
                                                                      const uint32_t* __restrict__ ds,
                                                                      int M, int K,
                                                                      void* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) uint8_t seg[];   // W x (PF ? 2 : 1) x Seg<SW>::kArea
    __shared__ float red[kMaxWaves][N][16];

    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int p = lane >> 4, r = lane & 15, h = p >> 1, e = p & 1;
    const int row0 = blockIdx.x * 16;
    const int S = K >> 8, C = K >> 5;
    const int sb0 = (int)((int64_t)S * wv / W), sb1 = (int)((int64_t)S * (wv + 1) / W);
    const int64_t rowS = (int64_t)(row0 + r) * S;

    Tile tl;
    tl.rows = min(16, M - row0);
    tl.end = tl.rows * S * kQ6kBlockBytes;
    tl.base = w + (int64_t)row0 * S * kQ6kBlockBytes;
    tl.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tl.base), 0, tl.end & ~15, kBufferFlags);

    float acc[N];
#pragma unroll
    for (int t = 0; t < N; ++t) acc[t] = 0.0f;

    const int last = sb1 - 1;
    constexpr int kAreas = PF ? 2 : 1;
    uint8_t* lds = seg + wv * kAreas * Seg<SW>::kArea;
    if constexpr (PF) {
        Fetch<N, SW> nx;
        if (sb0 < sb1) {
            fetch_step<N, SW>(nx, q, ds, K, C, sb0, last, h, e, r);
            stage_issue<SW>(tl, S, sb0, lane, lds);
        }
        for (int s = sb0, b = 0; s < sb1; s += SW, b ^= 1) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __builtin_amdgcn_sched_barrier(0);
            uint8_t* cur = lds + b * Seg<SW>::kArea;
            stage_patch<SW>(tl, S, s, lane, cur);
            Fetch<N, SW> f = nx;
            if (s + SW < sb1) {
                fetch_step<N, SW>(nx, q, ds, K, C, s + SW, last, h, e, r);
                stage_issue<SW>(tl, S, s + SW, lane, lds + (b ^ 1) * Seg<SW>::kArea);
            }
            __builtin_amdgcn_sched_barrier(0);
            compute_step<N, SW>(f, cur, rowS, s, last, h, e, r, acc);
        }
    } else {
        // LDS accesses of one wave complete in order: a step's reads finish
        // before the next step's copy is issued (its math needs them).
        for (int s = sb0; s < sb1; s += SW) {
            Fetch<N, SW> f;
            fetch_step<N, SW>(f, q, ds, K, C, s, last, h, e, r);
            stage_issue<SW>(tl, S, s, lane, lds);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __builtin_amdgcn_sched_barrier(0);
            stage_patch<SW>(tl, S, s, lane, lds);
            compute_step<N, SW>(f, lds, rowS, s, last, h, e, r, acc);
        }
    }

#pragma unroll
    for (int t = 0; t < N; ++t) {
        acc[t] += __shfl_xor(acc[t], 16);
        acc[t] += __shfl_xor(acc[t], 32);
        if (p == 0) red[wv][t][r] = acc[t];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 16 * N; i += blockDim.x) {
        const int t = i >> 4, rr = i & 15;
        float sum = red[0][t][rr];
        for (int v = 1; v < W; ++v) sum += red[v][t][rr];
        if (row0 + rr < M) store_out<H>(out, (int64_t)t * M + row0 + rr, sum);
    }
}

template <int N, int SW, bool PF>
hipError_t launch_sw(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                     void* out, bool half_out, hipStream_t stream, int waves) {
    const int rows = (m + 15) / 16;
    const size_t lds = (size_t)waves * (PF ? 2 : 1) * Seg<SW>::kArea;
    if (half_out)
        hipLaunchKernelGGL((mmq_q6k_gemv_kernel<N, SW, PF, true>), dim3(rows), dim3(64 * waves), lds, stream,
                           w, q, ds, m, k, out);
    else
        hipLaunchKernelGGL((mmq_q6k_gemv_kernel<N, SW, PF, false>), dim3(rows), dim3(64 * waves), lds, stream,
                           w, q, ds, m, k, out);
    return hipGetLastError();
}

template <int N>
hipError_t launch_n(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                    void* out, bool half_out, hipStream_t stream) {
    // Measured on the 28672 x 8192 q6_K matrix (1-7 tokens, steps of 1, 2
    // and 4 super-blocks, 1-4 waves, with and without the next step in
    // flight): one token streams best in steps of 2 with about 1024 waves in
    // all, more tokens (more vector work per byte) in steps of 1 with 4 waves
    // per row tile; the second LDS area pays up to 4 tokens once a wave has
    // at least 8 steps.
    const int S = k / 256, rows = (m + 15) / 16;
    int waves = N == 1 ? 1024 / rows : kMaxWaves;
    waves = waves < 1 ? 1 : waves > kMaxWaves ? kMaxWaves : waves;
    waves = waves > S ? S : waves;
    constexpr int SW = N == 1 ? 2 : 1;
    if constexpr (N <= 4)
        if (S / (waves * SW) >= 8) return launch_sw<N, SW, true>(w, m, k, q, ds, out, half_out, stream, waves);
    return launch_sw<N, SW, false>(w, m, k, q, ds, out, half_out, stream, waves);
}

}  // namespace

hipError_t launch_q6k_gemv(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                           int n, void* out, bool half_out, hipStream_t stream) {
    switch (n) {
        case 1: return launch_n<1>(w, m, k, q, ds, out, half_out, stream);
        case 2: return launch_n<2>(w, m, k, q, ds, out, half_out, stream);
        case 3: return launch_n<3>(w, m, k, q, ds, out, half_out, stream);
        case 4: return launch_n<4>(w, m, k, q, ds, out, half_out, stream);
        case 5: return launch_n<5>(w, m, k, q, ds, out, half_out, stream);
        case 6: return launch_n<6>(w, m, k, q, ds, out, half_out, stream);
        case 7: return launch_n<7>(w, m, k, q, ds, out, half_out, stream);
        case 8: return launch_n<8>(w, m, k, q, ds, out, half_out, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mmq
