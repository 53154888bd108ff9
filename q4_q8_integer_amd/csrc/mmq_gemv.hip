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
//   * Up to 6 tokens the weights go through LDS: per step the wave copies
//     its 16 runs with buffer loads that write LDS directly (consecutive
//     16-byte pieces, so each load instruction covers about one contiguous
//     KiB and no registers hold the copy), then each lane reads its three
//     16-byte fields from there.  Loading the fields straight into registers
//     costs 64 lanes x 3 scattered 16-byte reads per block column, which
//     keeps the address units, not HBM, busy; it is kept for 6-8 tokens,
//     where the vector work is the bound.  With >= 4 steps per wave, a
//     second LDS area takes the next step's copy while a step computes.
//   * A workgroup is 16 rows; its waves split the super-blocks, and the
//     partial sums are added in a fixed order (a butterfly over the four
//     chunk-pair lanes of a row, then the waves in index order): results do
//     not depend on timing.
#include "internal.h"
#include "kquant_device.h"

namespace mmq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kMaxWaves = 4;   // waves per workgroup (split of the super-blocks)

// Weight layouts the kernel reads: GGUF q4_K rows loaded straight into
// registers, the repacked 16-row records, or GGUF rows staged through LDS
// (one area per wave, or two with the next step's copy in flight).
enum { kDirect = 0, kRepacked = 1, kStaged = 2, kStagedPf = 3 };
constexpr bool staged_layout(int L) { return L == kStaged || L == kStagedPf; }
constexpr int kStagedRow = 4 * kBlockBytes + 16;   // LDS bytes per row of a 4-block step
constexpr int kStagedArea = 16 * kStagedRow;        // LDS bytes of one step's copy
// s_waitcnt operand: at most n vector-memory operations outstanding, the
// other counters untouched (vmcnt bits 3:0 and 15:14)
// Cache policy of the staged weight copies and of the repacked layout's
// loads: non-temporal (each weight byte is read once; measured at one token
// staged 24.0 -> 23.4 us and repacked 23.8 -> 21.6 us on 28672 x 8192).  Not
// for the register-loaded GGUF layout, whose lanes share cache lines within
// and across load instructions (40 -> 52 us at 7 tokens with it).
constexpr int kStreamAux = 2;

__device__ __forceinline__ v4u ld16(const void* p) { return *reinterpret_cast<const v4u*>(p); }
// repacked weight loads: non-temporal (kStreamAux)
__device__ __forceinline__ v4u ld16w(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
}
__device__ __forceinline__ uint32_t ld4w(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Chunk dots of pair p in super-block J of the step:  D0 = sum_i dot4(lo[i],
// token word i), D1 = sum_i dot4(hi[i], token word 8 + i), where token words
// 4c..4c+3 sit in lane 4J + c of the DPP row (row_newbcast).  Each chain
// starts from the bits of kMagic = 1.5 * 2^23 instead of 0: as |D| < 2^16,
// the integer sum kMagic_bits + D is the float32 kMagic + D exactly, so the
// results come back as floats with no conversion (see scaled_dot).  Inline
// asm hides these instructions from the compiler's hazard checks, so the
// blocks keep the rules themselves: a DPP read needs 2 wait states after a
// VALU write of its source (s_nop 1 first), and a VALU other than a dot that
// reads a v_dot4 result needs 3 (s_nop 2 last).
constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
constexpr int kMagicBits = 0x4B400000;

// dsc * D from a chain's result kMagic + D, rounded once as dsc * float(D)
// would be: kneg = -kMagic * dsc is exact (dsc = d * sc carries at most 17
// significant bits, times 3 * 2^22 at most 19), so the fused multiply-add
// rounds the exact dsc * D.
__device__ __forceinline__ float scaled_dot(float dsc, float kneg, float chain) {
    return fmaf(dsc, chain, kneg);
}

template <int J>
__device__ __forceinline__ void dots_two_tokens(float& a0, float& a1, float& b0, float& b1, v4u ta,
                                                v4u tb, const int* lo, const int* hi) {
    int A0 = kMagicBits, A1 = kMagicBits, B0 = kMagicBits, B1 = kMagicBits;
    asm(
        "s_nop 1\n\t"
        "v_dot4c_i32_i8_dpp %0, %4, %12 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %4, %20 row_newbcast:%c30 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %8, %12 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %8, %20 row_newbcast:%c30 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %5, %13 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %5, %21 row_newbcast:%c30 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %9, %13 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %9, %21 row_newbcast:%c30 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %6, %14 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %6, %22 row_newbcast:%c30 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %10, %14 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %10, %22 row_newbcast:%c30 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %7, %15 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %7, %23 row_newbcast:%c30 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %11, %15 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %11, %23 row_newbcast:%c30 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %4, %16 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %4, %24 row_newbcast:%c31 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %8, %16 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %8, %24 row_newbcast:%c31 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %5, %17 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %5, %25 row_newbcast:%c31 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %9, %17 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %9, %25 row_newbcast:%c31 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %6, %18 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %6, %26 row_newbcast:%c31 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %10, %18 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %10, %26 row_newbcast:%c31 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %7, %19 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %7, %27 row_newbcast:%c31 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %11, %19 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %11, %27 row_newbcast:%c31 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 2"
        : "+v"(A0), "+v"(A1), "+v"(B0), "+v"(B1)
        : "v"(ta[0]), "v"(ta[1]), "v"(ta[2]), "v"(ta[3]), "v"(tb[0]), "v"(tb[1]), "v"(tb[2]), "v"(tb[3]),
          "v"(lo[0]), "v"(lo[1]), "v"(lo[2]), "v"(lo[3]), "v"(lo[4]), "v"(lo[5]), "v"(lo[6]), "v"(lo[7]),
          "v"(hi[0]), "v"(hi[1]), "v"(hi[2]), "v"(hi[3]), "v"(hi[4]), "v"(hi[5]), "v"(hi[6]), "v"(hi[7]),
          "n"(4 * J), "n"(4 * J + 1), "n"(4 * J + 2), "n"(4 * J + 3));
    a0 = __builtin_bit_cast(float, A0);
    a1 = __builtin_bit_cast(float, A1);
    b0 = __builtin_bit_cast(float, B0);
    b1 = __builtin_bit_cast(float, B1);
}

template <int J>
__device__ __forceinline__ void dots_one_token(float& a0, float& a1, v4u ta, const int* lo,
                                               const int* hi) {
    int A0 = kMagicBits, A1 = kMagicBits;
    asm(
        "s_nop 1\n\t"
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
        : "+v"(A0), "+v"(A1)
        : "v"(ta[0]), "v"(ta[1]), "v"(ta[2]), "v"(ta[3]),
          "v"(lo[0]), "v"(lo[1]), "v"(lo[2]), "v"(lo[3]), "v"(lo[4]), "v"(lo[5]), "v"(lo[6]), "v"(lo[7]),
          "v"(hi[0]), "v"(hi[1]), "v"(hi[2]), "v"(hi[3]), "v"(hi[4]), "v"(hi[5]), "v"(hi[6]), "v"(hi[7]),
          "n"(4 * J), "n"(4 * J + 1), "n"(4 * J + 2), "n"(4 * J + 3));
    a0 = __builtin_bit_cast(float, A0);
    a1 = __builtin_bit_cast(float, A1);
}

// acc += da(2p) * x0 + da(2p+1) * x1 + dass(2p) * m0 + dass(2p+1) * m1, the
// scales taken from lanes 2J (chunk 2p) and 2J + 1 (chunk 2p+1) of the row.
template <int J>
__device__ __forceinline__ void fold_one_token(float& acc, float da, float dass, float x0, float x1,
                                               float m0, float m1) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:%c7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:%c8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %5 row_newbcast:%c7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %6 row_newbcast:%c8 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(da), "v"(dass), "v"(x0), "v"(x1), "v"(m0), "v"(m1), "n"(2 * J), "n"(2 * J + 1));
}

template <int J>
__device__ __forceinline__ void fold_two_tokens(float& acca, float& accb, float daa, float dassa,
                                                float dab, float dassb, float x0a, float x1a,
                                                float x0b, float x1b, float m0, float m1) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %2, %6 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %4, %8 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %7 row_newbcast:%c13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %4, %9 row_newbcast:%c13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %3, %10 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %10 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %3, %11 row_newbcast:%c13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %11 row_newbcast:%c13 row_mask:0xf bank_mask:0xf"
        : "+v"(acca), "+v"(accb)
        : "v"(daa), "v"(dassa), "v"(dab), "v"(dassb), "v"(x0a), "v"(x1a), "v"(x0b), "v"(x1b),
          "v"(m0), "v"(m1), "n"(2 * J), "n"(2 * J + 1));
}

// One super-block J of the step for every token.  A slot past the wave's
// last super-block (live false) runs with d = dmin = 0 and adds exactly 0:
// no branch, so the compiler keeps all of the step's loads ahead of the math.
template <int N, int J, int L>
__device__ __forceinline__ void gemv_sb(const v4u h, const v4u qa, const v4u qb, int p, bool live,
                                        const v4u* tq, const float* tda, const float* tdass,
                                        float* acc) {
    const float d = live ? half_lo(h[0]) : 0.0f, dmin = live ? half_lo(h[0] >> 16) : 0.0f;
    uint32_t sc0, sc1, m0, m1;
    if constexpr (L == kRepacked) {
        // repacked layout: the four scales as bytes of one dword
        sc0 = h[1] & 0xFF;
        sc1 = (h[1] >> 8) & 0xFF;
        m0 = (h[1] >> 16) & 0xFF;
        m1 = h[1] >> 24;
    } else {
        // 6-bit (sc, m) of chunks 2p and 2p+1 (GGUF k-quant scale packing)
        scale_min_pair(h[1], h[2], h[3], p, sc0, sc1, m0, m1);
    }
    const float dsc0 = d * (float)sc0, dsc1 = d * (float)sc1;
    const float kn0 = -kMagic * dsc0, kn1 = -kMagic * dsc1;
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
    for (int t = 0; t + 1 < N; t += 2) {
        float a0, a1, b0, b1;
        dots_two_tokens<J>(a0, a1, b0, b1, tq[t], tq[t + 1], lo, hi);
        fold_two_tokens<J>(acc[t], acc[t + 1], tda[t], tdass[t], tda[t + 1], tdass[t + 1],
                           scaled_dot(dsc0, kn0, a0), scaled_dot(dsc1, kn1, a1),
                           scaled_dot(dsc0, kn0, b0), scaled_dot(dsc1, kn1, b1), dmm0, dmm1);
    }
    if constexpr ((N & 1) != 0) {
        float a0, a1;
        dots_one_token<J>(a0, a1, tq[N - 1], lo, hi);
        fold_one_token<J>(acc[N - 1], tda[N - 1], tdass[N - 1], scaled_dot(dsc0, kn0, a0),
                          scaled_dot(dsc1, kn1, a1), dmm0, dmm1);
    }
}

// Registers of one wave step: SW super-blocks of the lane's row (header and
// its 32 qs bytes), the lane's q8 piece and scale word of every token.
template <int N, int SW>
struct Step {
    v4u hdr[SW], qa[SW], qb[SW];
    v4u tq[N];
    uint32_t tw[N];
};

// Issue the loads of the step starting at super-block s.  Every load is
// unconditional: slots past the wave's last super-block re-read that block
// (and are computed with live = false).  wrow is the lane's row (GGUF
// layout) or the workgroup's 16-row tile of records (repacked layout).  The
// staged layout loads only the activations here (its weights go through
// stage_issue / stage_read).
template <int N, int SW, int L>
__device__ __forceinline__ void load_step(Step<N, SW>& st, const uint8_t* wrow,
                                          const int8_t* __restrict__ q,
                                          const uint32_t* __restrict__ ds, int K, int C, int s,
                                          int last, int p, int r) {
    // q8: lane (p, r) holds piece r&3 of pair p of super-block s + (r>>2)
    // (the wave reads up to 4 super-blocks of a token as one KiB)
    const int64_t qoff = (int64_t)min(s + (r >> 2), last) * 256 + 64 * p + 16 * (r & 3);
#pragma unroll
    for (int t = 0; t < N; ++t) st.tq[t] = ld16(q + (int64_t)t * K + qoff);
    // scale word of chunk 2p + (r&1) of super-block s + ((r>>1)&3)
    const int64_t woff = (int64_t)min(s + ((r >> 1) & 3), last) * 8 + 2 * p + (r & 1);
#pragma unroll
    for (int t = 0; t < N; ++t) st.tw[t] = ds[(int64_t)t * C + woff];
    if constexpr (staged_layout(L)) return;   // fields come from the wave's LDS area
#pragma unroll
    for (int j = 0; j < SW; ++j) {
        if constexpr (L == kRepacked) {
            const uint8_t* b = wrow + (int64_t)min(s + j, last) * kRepackRecordBytes;
            st.hdr[j] = v4u{ld4w(b + 4 * r), ld4w(b + 64 + 4 * (16 * p + r)), 0u, 0u};
            st.qa[j] = ld16w(b + 320 + 512 * p + 16 * r);
            st.qb[j] = ld16w(b + 320 + 512 * p + 256 + 16 * r);
        } else {
            const uint8_t* b = wrow + (int64_t)min(s + j, last) * kBlockBytes;
            st.hdr[j] = ld16(b);
            st.qa[j] = ld16(b + 16 + 32 * p);
            st.qb[j] = ld16(b + 32 + 32 * p);
        }
    }
}

// Staged GGUF layout.  The wave copies the 16 runs of 4 blocks of a step
// into one of its two LDS areas with consecutive 16-byte pieces (one load
// instruction reads about one contiguous KiB and writes it to LDS without
// passing through registers), so the next step's copy is in flight while
// this step computes.  Slot i of an area (16 bytes at 16*i) holds piece
// i % 37 of row i / 37 of the tile; piece 36 is padding, which makes the row
// stride 592 bytes and the 16-row reads of stage_read free of bank
// conflicts.  wt spans the tile's rows: pieces past the end of a row (a
// wave's last step may run over it) read the next row, past the tile they
// read zeros; either way they are never used.
constexpr int kStagedSlots = 16 * kStagedRow / 16;
constexpr int kStagedLoads = (kStagedSlots + 63) / 64;   // load instructions per step

__device__ __forceinline__ void stage_issue(__amdgpu_buffer_rsrc_t wt, int S, int s, int lane,
                                            uint8_t* area) {
#pragma unroll
    for (int c = 0; c < kStagedLoads; ++c) {
        const int i = lane + 64 * c;
        const int rr = i / (kStagedRow / 16), ch = min(i - rr * (kStagedRow / 16), 4 * 9 - 1);
        const uint32_t off = (uint32_t)(rr * S + s + ch / 9) * kBlockBytes + 16 * (ch % 9);
        if (i < kStagedSlots)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wt, (__attribute__((address_space(3))) void*)(area + 1024 * c),
                                                     16, off, 0, 0, kStreamAux);
    }
}

template <int N, int SW>
__device__ __forceinline__ void stage_read(Step<N, SW>& st, const uint8_t* area, int p, int r) {
    static_assert(SW == 4, "staged rows hold four blocks");
#pragma unroll
    for (int j = 0; j < SW; ++j) {
        const uint8_t* b = area + r * kStagedRow + j * kBlockBytes;
        st.hdr[j] = *reinterpret_cast<const v4u*>(b);
        st.qa[j] = *reinterpret_cast<const v4u*>(b + 16 + 32 * p);
        st.qb[j] = *reinterpret_cast<const v4u*>(b + 32 + 32 * p);
    }
}

template <int N, int SW, int L>
__device__ __forceinline__ void compute_step(const Step<N, SW>& st, int ns, int p, float* acc) {
    float tda[N], tdass[N];
#pragma unroll
    for (int t = 0; t < N; ++t) {
        tda[t] = half_lo(st.tw[t]);
        tdass[t] = tda[t] * (float)(int16_t)(uint16_t)(st.tw[t] >> 16);
    }
    gemv_sb<N, 0, L>(st.hdr[0], st.qa[0], st.qb[0], p, ns > 0, st.tq, tda, tdass, acc);
    if constexpr (SW > 1) gemv_sb<N, 1, L>(st.hdr[1], st.qa[1], st.qb[1], p, ns > 1, st.tq, tda, tdass, acc);
    if constexpr (SW > 2) gemv_sb<N, 2, L>(st.hdr[2], st.qa[2], st.qb[2], p, ns > 2, st.tq, tda, tdass, acc);
    if constexpr (SW > 3) gemv_sb<N, 3, L>(st.hdr[3], st.qa[3], st.qb[3], p, ns > 3, st.tq, tda, tdass, acc);
}

// Waves per SIMD the register allocation is held to.  The repacked layout at
// 8 tokens takes 148 VGPRs otherwise (3 waves per SIMD); held to 128 (4
// waves, at the cost of a 16-byte spill per lane) it measured 37.8 -> 35.4 us
// on 28672 x 8192 and 39.0 -> 38.6 us on 8192 x 28672.  The GGUF layout at 7 tokens gained nothing from
// the same (146 -> 128 VGPRs, within 2%), and at 8 it spills.
template <int N, int L>
constexpr int min_waves_per_simd() {
    return L == kRepacked && N == 8 ? 4 : 1;
}

template <int N, int SW, bool H, int L>
__global__ __launch_bounds__(64 * kMaxWaves)
__attribute__((amdgpu_waves_per_eu(min_waves_per_simd<N, L>()))) void mmq_gemv_kernel(const uint8_t* __restrict__ w,
                                                                  const int8_t* __restrict__ q,
                                                                  const uint32_t* __restrict__ ds,
                                                                  int M, int K,
                                                                  void* __restrict__ out) {
    __shared__ float red[kMaxWaves][N][16];
    extern __shared__ __attribute__((aligned(16))) uint8_t staged[];   // W x 2 areas (staged layout)

    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int p = lane >> 4, r = lane & 15;
    const int row0 = blockIdx.x * 16;
    const int S = K >> 8, C = K >> 5;
    const int sb0 = (int)((int64_t)S * wv / W), sb1 = (int)((int64_t)S * (wv + 1) / W);
    const uint8_t* wrow = L == kRepacked ? w + (int64_t)blockIdx.x * S * kRepackRecordBytes
                                         : w + (int64_t)min(row0 + r, M - 1) * S * kBlockBytes;
    uint8_t* lds = staged + wv * (L == kStagedPf ? 2 : 1) * kStagedArea;
    const __amdgpu_buffer_rsrc_t wt =   // the tile's GGUF rows (used by the staged layout)
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + (int64_t)row0 * S * kBlockBytes), 0,
                                          min(16, M - row0) * S * kBlockBytes, kBufferFlags);

    float acc[N];
#pragma unroll
    for (int t = 0; t < N; ++t) acc[t] = 0.0f;

    // One step at a time: all of its loads are issued, then it is computed.
    // (Prefetching the next step into a second register set measured
    // slower: it halves the waves a CU holds, and a wave's own latency is not
    // what limits the stream.)
    const int last = sb1 - 1;
    if constexpr (L == kStaged) {
        for (int s = sb0; s < sb1; s += SW) {
            Step<N, SW> A;
            load_step<N, SW, L>(A, wrow, q, ds, K, C, s, last, p, r);
            stage_issue(wt, S, s, lane, lds);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
            __builtin_amdgcn_sched_barrier(0);
            stage_read(A, lds, p, r);
            compute_step<N, SW, L>(A, sb1 - s, p, acc);
        }
    } else if constexpr (L == kStagedPf) {
        // The next step's weights (into the other LDS area) and activations
        // (into registers) are in flight while a step computes; one wait for
        // everything at the top of the step.
        Step<N, SW> nx;
        if (sb0 < sb1) {
            load_step<N, SW, L>(nx, wrow, q, ds, K, C, sb0, last, p, r);
            stage_issue(wt, S, sb0, lane, lds);
        }
        for (int s = sb0, b = 0; s < sb1; s += SW, b ^= 1) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
            __builtin_amdgcn_sched_barrier(0);
            Step<N, SW> A;
#pragma unroll
            for (int t = 0; t < N; ++t) {
                A.tq[t] = nx.tq[t];
                A.tw[t] = nx.tw[t];
            }
            if (s + SW < sb1) {
                load_step<N, SW, L>(nx, wrow, q, ds, K, C, s + SW, last, p, r);
                stage_issue(wt, S, s + SW, lane, lds + (b ^ 1) * kStagedArea);
            }
            __builtin_amdgcn_sched_barrier(0);
            stage_read(A, lds + b * kStagedArea, p, r);
            compute_step<N, SW, L>(A, sb1 - s, p, acc);
        }
    } else {
        for (int s = sb0; s < sb1; s += SW) {
            Step<N, SW> A;
            load_step<N, SW, L>(A, wrow, q, ds, K, C, s, last, p, r);
            __builtin_amdgcn_sched_barrier(0);
            compute_step<N, SW, L>(A, sb1 - s, p, acc);
        }
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
        if (row0 + rr < M) store_out<H>(out, (int64_t)t * M + row0 + rr, sum);
    }
}

template <int N, int L>
hipError_t launch_n(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds,
                    void* out, bool half_out, hipStream_t stream) {
    const int S = k / 256;
    const int rows = (m + 15) / 16;
    // The super-blocks of a row are split over the 4 waves of a workgroup
    // (fewer when a row has fewer super-blocks).  Every layout splits the
    // same way, so every layout sums in the same order.
    int waves = S < 4 ? S : 4;
    constexpr int SW = 4;
    const size_t lds = L == kStaged ? (size_t)waves * kStagedArea
                       : L == kStagedPf ? (size_t)waves * 2 * kStagedArea : 0;
    if (half_out)
        hipLaunchKernelGGL((mmq_gemv_kernel<N, SW, true, L>), dim3(rows), dim3(64 * waves), lds, stream,
                           w, q, ds, m, k, out);
    else
        hipLaunchKernelGGL((mmq_gemv_kernel<N, SW, false, L>), dim3(rows), dim3(64 * waves), lds, stream,
                           w, q, ds, m, k, out);
    return hipGetLastError();
}

// Token counts each layout is launched for (the staged layouts up to 6
// tokens, the register-loaded GGUF layout from 6): the others are not
// instantiated.
template <int L>
constexpr bool serves(int n) {
    return staged_layout(L) ? n <= 6 : L == kDirect ? n >= 6 : true;
}

template <int L, int N>
hipError_t launch_if(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, void* out,
                     bool half_out, hipStream_t stream) {
    if constexpr (serves<L>(N)) return launch_n<N, L>(w, m, k, q, ds, out, half_out, stream);
    return hipErrorInvalidValue;
}

template <int L>
hipError_t launch_any(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
                      void* out, bool half_out, hipStream_t stream) {
    switch (n) {
        case 1: return launch_if<L, 1>(w, m, k, q, ds, out, half_out, stream);
        case 2: return launch_if<L, 2>(w, m, k, q, ds, out, half_out, stream);
        case 3: return launch_if<L, 3>(w, m, k, q, ds, out, half_out, stream);
        case 4: return launch_if<L, 4>(w, m, k, q, ds, out, half_out, stream);
        case 5: return launch_if<L, 5>(w, m, k, q, ds, out, half_out, stream);
        case 6: return launch_if<L, 6>(w, m, k, q, ds, out, half_out, stream);
        case 7: return launch_if<L, 7>(w, m, k, q, ds, out, half_out, stream);
        case 8: return launch_if<L, 8>(w, m, k, q, ds, out, half_out, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_mmq_fp32_gemv(const uint8_t* w, int m, int k, const int8_t* q,
                                const uint32_t* ds, int n, void* out, bool half_out,
                                hipStream_t stream) {
    // Staging through LDS pays while the stream, not the vector work, is the
    // bound; the next step's copy in flight pays when a wave has at least 4
    // steps (4 waves of 4-block steps: 64 super-blocks per row).  Measured
    // on the 28672 x 8192 and 8192 x 28672 matrices, 1-8 tokens.
    const bool pf = k / 256 >= 64;
    if (n <= 5 || (n == 6 && pf))
        return pf ? launch_any<kStagedPf>(w, m, k, q, ds, n, out, half_out, stream)
                  : launch_any<kStaged>(w, m, k, q, ds, n, out, half_out, stream);
    return launch_any<kDirect>(w, m, k, q, ds, n, out, half_out, stream);
}

hipError_t launch_mmq_fp32_gemv_repacked(const uint8_t* wr, int m, int k, const int8_t* q,
                                         const uint32_t* ds, int n, void* out, bool half_out,
                                         hipStream_t stream) {
    return launch_any<kRepacked>(wr, m, k, q, ds, n, out, half_out, stream);
}

}  // namespace mmq
