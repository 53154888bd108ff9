// mmq_narrow.hip - q4_K x q8 matmul for a few tokens (1 <= n <= 8), float32
// or binary16 result, on the 4x4x4 int8 matrix instruction with one weight
// row and super-block per lane.
//
// The method is the one of the other kernels (the yusiwen.cn "minfer" r31
// page, sections 1-2: an exact integer dot per 32-weight chunk, then the
// two-term fold d*sc*da*D - dmin*m*da*ssum).  With a handful of tokens the
// weights are streamed once and the cost that remains is per weight row and
// chunk: unpacking the nibbles, the scale decode, and the fold of each
// (row, token) dot.  A 16x16 matrix tile pads a 4-token product to 16 tokens
// and folds the padding too; the vector ALU's 4-way dot product needs one
// instruction per 4 weights and token.  Here:
//
//   * v_mfma_i32_4x4x4i8 is 16 independent 4 x 4 x 4 products.  Lane 4b + j
//     supplies column j of block b of the B operand and holds column j of
//     block b of the result; lane 4b + i supplies row i of block b of A.  B is
//     the weights: lane l takes weight row l % 16 of the wave's 16 rows in
//     super-block l / 16 of a step of 4 consecutive super-blocks, so a step
//     reads 16 runs of 576 contiguous bytes.  A is 4 tokens at the same k as
//     the block's weights, so a lane's 4 results are its (row, super-block)
//     against 4 tokens.  Eight instructions are one chunk (k = 32).
//   * B is the lane's qs dword & 0x0F0F0F0F (low nibbles, chunk 2p) or
//     (dword >> 4) & 0x0F0F0F0F (high nibbles, chunk 2p+1); nothing else.
//   * A is the q8 bytes of the tokens, read from a wave-private LDS copy of
//     the step's token rows (made with buffer loads that write LDS directly:
//     contiguous 256-byte runs).  Each wave has two such areas and two
//     weight register sets: a step's loads are in flight while the previous
//     step computes.
//   * Each lane owns its block's scales: d*sc and -dmin*m per chunk come from
//     the lane's own block header.  The token scales da sit in the lane of
//     their token (lane 4b + i holds token i's), and reach the other lanes
//     of the quad through a quad_perm DPP broadcast.
//   * Per chunk and token: acc += (da * d*sc) * float(D)   (3 operations);
//     the min term -(dmin*m)*(da*ssum) is a rank-1 update per chunk, done by
//     v_mfma_f32_4x4x1f32 (A = da*ssum of the 4 tokens, B = -dmin*m of the
//     lane's block) into an accumulator of its own.
//   * n <= 4G tokens run as G groups of 4; every weight operand serves all
//     groups.
//   * A workgroup is W waves on the same 16 rows, each over a contiguous
//     range of steps (16 rows x 4 super-blocks).  A step slot past the
//     wave's range computes with
//     d = dmin = 0 (adding exactly 0) on valid data.  The partial sums (W
//     waves x 4 super-block slots per row) are added in LDS in a fixed order,
//     so results do not depend on timing.  Within a wave the chunk sums are
//     added into a float32 accumulator that is moved (with the min-term
//     accumulator) into a second one every 8 steps, which keeps the rounding
//     error of very long rows (k up to 2^24) within the float32 bar.
#include <algorithm>

#include "internal.h"
#include "kquant_device.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kFlushSteps = 8;   // steps between moves into the second accumulator
constexpr int kNarrowWaves = 4;  // waves per workgroup at most

// A wave's LDS area for one step: 16G token rows of 256 bytes (row
// R = 16g + 4s + i is token 4g + i in super-block s of the step), then
// their scale words (row R's eight words at 32R).  Row R's 16-byte piece p
// sits in slot p ^ 2x with x = i + 4(s & 1): the eight rows that a
// half-wave's chunk read touches (i = 0..3, two values of s) then fall in
// eight different 32-byte bank groups, and a chunk's two pieces stay
// adjacent.  The direct-to-LDS copies fill whole instructions of 64 slots
// (one instruction is 4 rows: the token part takes 4G).
template <int G>
struct Area {
    static constexpr int kTokLoads = 4 * G;
    static constexpr int kWordLoads = (32 * G + 63) / 64;
    static constexpr int kTokBytes = 1024 * kTokLoads;
    static constexpr int kBytes = kTokBytes + 1024 * kWordLoads;
};

// One 16-byte direct-to-LDS copy per lane: lane i writes slot i of the 64
// slots at dst, from byte voff + soff of src.  (A device function of its
// own: the address-space cast is device code only.)
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t src, uint32_t voff, uint32_t soff, uint8_t* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// The value of x in lane 4*(lane/4) + v of the lane's quad.
template <int V>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), V * 0x55, 0xF, 0xF, true));
}

// The weight block a lane reads in a step: header and the 128 qs bytes.
struct Blk {
    v4u hdr;
    v4u qv[8];
};

template <int G>
struct Copy {
    __amdgpu_buffer_rsrc_t qr, dr;
    uint32_t tok[G][2];       // per group and parity of s: token row and piece offset (the step adds the super-block)
    uint32_t word[Area<G>::kWordLoads];
    int word_sl[Area<G>::kWordLoads];
};

// Issue the loads of the step at super-block st: the token rows and words
// into area, the lane's weight block into b.
template <int G>
__device__ __forceinline__ void issue_step(const Copy<G>& cp, int st, int S, const uint8_t* wrow, int sl,
                                           uint8_t* area, Blk& b) {
    typedef Area<G> A;
#pragma unroll
    for (int c = 0; c < A::kTokLoads; ++c)   // instruction c: group c / 4, super-block slot c % 4
        copy_to_lds(cp.qr, cp.tok[c >> 2][c & 1], (uint32_t)min(st + (c & 3), S - 1) * 256u, area + 1024 * c);
#pragma unroll
    for (int c = 0; c < A::kWordLoads; ++c)
        copy_to_lds(cp.dr, cp.word[c] + (uint32_t)min(st + cp.word_sl[c], S - 1) * 32u, 0,
                    area + A::kTokBytes + 1024 * c);
    const uint8_t* blk = wrow + (int64_t)min(st + sl, S - 1) * kBlockBytes;
    b.hdr = *reinterpret_cast<const v4u*>(blk);
#pragma unroll
    for (int j = 0; j < 8; ++j) b.qv[j] = *reinterpret_cast<const v4u*>(blk + 16 + 16 * j);
}

// The arithmetic of one step from its LDS area and the lane's weight block.
template <int G>
__device__ __forceinline__ void compute_step(const uint8_t* area, const Blk& bk, bool live, int sl, int ti,
                                             v4f* acc, v4f* accm) {
    typedef Area<G> A;
    const float d = live ? half_lo(bk.hdr.x) : 0.0f, dmin = live ? half_lo(bk.hdr.x >> 16) : 0.0f;
    // this lane's token's scale words: group g, chunk c at word 8*(16g + 4sl + ti) + c
    const uint32_t* wd = reinterpret_cast<const uint32_t*>(area + A::kTokBytes) + 8 * (4 * sl + ti);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        int sc, mn;
        scale_min(bk.hdr.y, bk.hdr.z, bk.hdr.w, c, sc, mn);
        const float dsc = d * (float)sc, mneg = -(dmin * (float)mn);
        int b[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const uint32_t x = bk.qv[2 * (c >> 1) + (kk >> 2)][kk & 3];
            b[kk] = (int)((c & 1) ? (x >> 4) & 0x0F0F0F0Fu : x & 0x0F0F0F0Fu);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            // chunk c of row R = 16g + 4sl + ti: slots 2(c ^ x), 2(c ^ x) + 1
            const uint8_t* tp = area + (16 * g + 4 * sl + ti) * 256 + 32 * (c ^ (ti + 4 * (sl & 1)));
            const v4u a0 = *reinterpret_cast<const v4u*>(tp), a1 = *reinterpret_cast<const v4u*>(tp + 16);
            v4i D = v4i{0, 0, 0, 0};
            D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a0[0], b[0], D, 0, 0, 0);
            D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a0[1], b[1], D, 0, 0, 0);
            D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a0[2], b[2], D, 0, 0, 0);
            D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a0[3], b[3], D, 0, 0, 0);
            D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a1[0], b[4], D, 0, 0, 0);
            D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a1[1], b[5], D, 0, 0, 0);
            D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a1[2], b[6], D, 0, 0, 0);
            D = __builtin_amdgcn_mfma_i32_4x4x4i8((int)a1[3], b[7], D, 0, 0, 0);
            const uint32_t word = wd[128 * g + c];
            const float da = half_lo(word);
            const float dass = da * (float)(int16_t)(uint16_t)(word >> 16);
            accm[g] = __builtin_amdgcn_mfma_f32_4x4x1f32(dass, mneg, accm[g], 0, 0, 0);
            acc[g][0] = fmaf(quad_bcast<0>(da) * dsc, (float)D[0], acc[g][0]);
            acc[g][1] = fmaf(quad_bcast<1>(da) * dsc, (float)D[1], acc[g][1]);
            acc[g][2] = fmaf(quad_bcast<2>(da) * dsc, (float)D[2], acc[g][2]);
            acc[g][3] = fmaf(quad_bcast<3>(da) * dsc, (float)D[3], acc[g][3]);
        }
    }
}

template <int G, bool H>
__global__ __launch_bounds__(64 * kNarrowWaves) void mmq_narrow_kernel(const uint8_t* __restrict__ w,
                                                                       const int8_t* __restrict__ q,
                                                                       const uint32_t* __restrict__ ds,
                                                                       int M, int N, int K,
                                                                       void* __restrict__ out) {
    typedef Area<G> A;
    // Two areas per wave, as two arrays: the copies into one are in flight
    // while the other is read, and the compiler can tell them apart.
    __shared__ __attribute__((aligned(16))) uint8_t area0[kNarrowWaves][A::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t area1[kNarrowWaves][A::kBytes];

    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int ti = lane & 3;     // the lane's token in a group (A operand)
    const int sl = lane >> 4;    // the lane's super-block slot in a step
    const int row0 = blockIdx.x * 16;
    const int S = K >> 8, C = K >> 5;
    const int steps = (S + 3) >> 2;
    const int sb0 = 4 * (int)((int64_t)steps * wv / W);
    const int sb1 = min(S, 4 * (int)((int64_t)steps * (wv + 1) / W));
    const uint8_t* wrow = w + (int64_t)min(row0 + (lane & 15), M - 1) * S * kBlockBytes;

    // Copy sources.  Token instruction c writes rows 4c .. 4c + 3 (group
    // c / 4, super-block slot s = c % 4): lane u takes row 4c + u / 16 (token
    // 4g + u / 16) and its slot u % 16, i.e. piece (u % 16) ^ 2x with
    // x = u / 16 + 4(s & 1).
    // Word instruction c: lane u takes half u & 1 of row 32c + u / 2.
    // Tokens past n re-read token n - 1 (their results are never stored);
    // super-blocks past k re-read the last one (computed with d = dmin = 0).
    Copy<G> cp;
    cp.qr = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(q), 0, N * K, kBufferFlags);
    cp.dr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(ds), 0, N * C * 4, kBufferFlags);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            cp.tok[g][h] = (uint32_t)min(4 * g + (lane >> 4), N - 1) * (uint32_t)K +
                           16u * ((lane & 15) ^ (2 * ((lane >> 4) + 4 * h)));
#pragma unroll
    for (int c = 0; c < A::kWordLoads; ++c) {
        const int r = min(32 * c + (lane >> 1), 16 * G - 1);
        cp.word[c] = (uint32_t)min(4 * (r >> 4) + (r & 3), N - 1) * (uint32_t)(C * 4) + 16u * (lane & 1);
        cp.word_sl[c] = (r >> 2) & 3;
    }

    v4f acc[G], accm[G], acc2[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        acc[g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        accm[g] = acc[g];
        acc2[g] = acc[g];
    }
    auto flush = [&](int n_st) {
        if ((n_st & (kFlushSteps - 1)) == kFlushSteps - 1) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                acc2[g] += acc[g];
                acc2[g] += accm[g];
                acc[g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                accm[g] = acc[g];
            }
        }
    };

    // Steps in pairs (areas 0 and 1, weight blocks ba and bb): the next
    // step's loads are issued before a step is computed; one wait for
    // everything at the top of each step.
    Blk ba, bb;
    if (sb0 < sb1) issue_step<G>(cp, sb0, S, wrow, sl, area0[wv], ba);
    for (int st = sb0, n_st = 0; st < sb1; st += 8, n_st += 2) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
        __builtin_amdgcn_sched_barrier(0);
        if (st + 4 < sb1) issue_step<G>(cp, st + 4, S, wrow, sl, area1[wv], bb);
        __builtin_amdgcn_sched_barrier(0);
        compute_step<G>(area0[wv], ba, st + sl < sb1, sl, ti, acc, accm);
        flush(n_st);
        if (st + 4 >= sb1) break;
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
        __builtin_amdgcn_sched_barrier(0);
        if (st + 8 < sb1) issue_step<G>(cp, st + 8, S, wrow, sl, area0[wv], ba);
        __builtin_amdgcn_sched_barrier(0);
        compute_step<G>(area1[wv], bb, st + 4 + sl < sb1, sl, ti, acc, accm);
        flush(n_st + 1);
    }

    // Partial sums: red[wave][g][v][lane], in area 0 once every wave is past
    // its loop.  Output (row r, token 4g + v) adds the lanes r + 16s of every
    // wave, waves in order and slots in order within a wave.
    __syncthreads();
    float* red = reinterpret_cast<float*>(&area0[0][0]);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[((wv * G + g) * 4 + v) * 64 + lane] = (acc2[g][v] + acc[g][v]) + accm[g][v];
    __syncthreads();
    for (int e = threadIdx.x; e < G * 4 * 16; e += blockDim.x) {
        const int r = e & 15, gv = e >> 4;   // gv = 4g + v, the token
        float sum = 0.0f;
        for (int u = 0; u < W; ++u)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) sum += red[(u * G * 4 + gv) * 64 + 16 * s4 + r];
        const int row = row0 + r;
        if (gv < N && row < M) store_out<H>(out, (int64_t)gv * M + row, sum);
    }
}

template <int G>
hipError_t launch_g(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n, void* out,
                    bool half_out, hipStream_t stream) {
    const int wgs = (m + 15) / 16, steps = ((k >> 8) + 3) / 4;
    // Waves per workgroup (splitting the steps): up to 4, about 8192 waves
    // in all, preferring a count that divides the steps evenly.
    const int wmax = (int)std::max<int64_t>(1, std::min<int64_t>({kNarrowWaves, steps, (8192 + wgs - 1) / wgs}));
    int W = wmax;
    for (int c = wmax; c * 2 > wmax; --c)
        if (steps % c == 0) { W = c; break; }
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k, (void*)&out};
    const void* f = half_out ? (const void*)mmq_narrow_kernel<G, true> : (const void*)mmq_narrow_kernel<G, false>;
    return hipLaunchKernel(f, dim3((unsigned)wgs), dim3(64 * W), args, 0, stream);
}

}  // namespace

hipError_t launch_mmq_fp32_narrow(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
                                  void* out, bool half_out, hipStream_t stream) {
    switch ((n + 3) / 4) {
        case 1: return launch_g<1>(w, m, k, q, ds, n, out, half_out, stream);
        case 2: return launch_g<2>(w, m, k, q, ds, n, out, half_out, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mmq
