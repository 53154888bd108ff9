// mmq_narrow.hip - q4_K x q8 matmul for a few tokens (1 <= n <= 8), float32
// or binary16 result, on the 4x4x4 int8 matrix instruction.
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
//     the weights: a step is RT rows x 32/RT consecutive super-blocks (RT = 16
//     or 32), and lane l takes row l % RT, super-block slot (l / 16) % 2 of
//     the step (RT = 16 only) and chunk half l / 32 (chunks 4h .. 4h + 3) of
//     that block.  A is 4 tokens at the same k as the block's weights, so a
//     lane's 4 results are its (row, super-block, half) against 4 tokens.
//     Eight instructions are one chunk.
//   * B is the lane's qs dword & 0x0F0F0F0F (low nibbles, chunk 2p) or
//     (dword >> 4) & 0x0F0F0F0F (high nibbles, chunk 2p+1); nothing else.
//   * Each wave copies a step's weights (RT runs of 32/RT blocks), its
//     token rows (256-byte runs) and their scale words into a wave-private
//     LDS area with buffer loads that write LDS directly: every copy
//     instruction moves one contiguous KiB or whole 256-byte runs, where
//     loading each lane's own block into registers touched a cache line per
//     lane.  Each wave has two areas: a step's copies are in flight while the
//     previous step computes.  The lanes read their header and four qs
//     pieces from the area.  32-row tiles let one token copy serve twice the
//     rows and give a wave twice the steps over the same k; 16-row tiles
//     give twice the tiles where 32-row ones cannot fill the CUs.
//   * The lane decodes the scales of its four chunks from its block header
//     (d*sc and -dmin*m per chunk).  The token scales da sit in the lane of
//     their token (lane 4b + i holds token i's), and reach the other lanes of
//     the quad through a quad_perm DPP broadcast.
//   * Per chunk and token: acc += (da * d*sc) * float(D)   (3 operations);
//     the min term -(dmin*m)*(da*ssum) is a rank-1 update per chunk, done by
//     v_mfma_f32_4x4x1f32 (A = da*ssum of the 4 tokens, B = -dmin*m of the
//     lane's block) into an accumulator of its own.
//   * n <= 4G tokens run as G groups of 4; every weight operand serves all
//     groups.
//   * A workgroup is W waves on the same RT rows, wave w taking the steps
//     w, w + W, w + 2W, ...: the waves read W adjacent blocks of every row at
//     about the same time, runs that a single wave's step is too short for
//     (contiguous step ranges per wave were 2-8% slower).  A step slot past
//     k computes with d = dmin = 0 (adding exactly 0) on valid data.  The
//     partial sums (W waves x 64/RT lanes per row) are added in LDS in a
//     fixed order, so results do not depend on timing.  Within a wave the chunk sums are
//     added into a float32 accumulator that is moved (with the min-term
//     accumulator) into a second one every 32 super-blocks, which keeps the
//     rounding error of very long rows (k up to 2^24) within the float32 bar.
#include <algorithm>

#include "internal.h"
#include "kquant_device.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// The step of an RT-row tile (RT = 16 or 32).
template <int RT>
struct Tile {
    static_assert(RT == 16 || RT == 32, "16- or 32-row tiles");
    static constexpr int kSlots = 32 / RT;                    // super-blocks per step
    static constexpr int kRowPieces = RT == 16 ? 20 : 10;      // 16-byte slots per weight row (9 per block + unused)
    static constexpr int kFlushSteps = 32 / kSlots;           // 32 super-blocks between accumulator moves
    // The slot of piece p of weight row r (see Area).
    __device__ static int wslot(int r, int p) { return p ^ (RT == 16 ? (r >> 2) & 3 : (r >> 3) & 1); }
};

// A wave's LDS area for one step.
//   * Weights: row r in slots kRowPieces * r ..; piece p of the row's run
//     (9 per block; the last one or two slots unused) sits in slot
//     Tile::wslot(r, p).  The 16 lanes that read the same piece of 16 rows
//     together then hit 16 different 4-bank groups: rows 320 (RT = 16) or
//     160 bytes (RT = 32) apart spread r & 3 or r & 7 over the bank groups,
//     and the xor spreads the rest.  RT * kRowPieces = 320 slots: five copy
//     instructions.
//   * Tokens: 4G * kSlots rows of 256 bytes (row R = 4 kSlots g + 4s + i is
//     token 4g + i in super-block slot s).  Row R's 16-byte piece p sits in
//     slot p ^ 2x with x = i + 4s: the rows that a half-wave's chunk read
//     touches fall in different 32-byte bank groups, and a chunk's two
//     pieces stay adjacent.  One instruction is 4 rows.
//   * Scale words: row R's eight words at 32R (one instruction).
template <int G, int RT>
struct Area {
    static constexpr int kWLoads = RT * Tile<RT>::kRowPieces / 64;
    static constexpr int kWBytes = 1024 * kWLoads;
    static constexpr int kTokLoads = G * Tile<RT>::kSlots;
    static constexpr int kTokBytes = 1024 * kTokLoads;
    static constexpr int kWordLoads = (8 * G * Tile<RT>::kSlots + 63) / 64;
    static constexpr int kBytes = kWBytes + kTokBytes + 1024 * kWordLoads;
    static_assert(RT * Tile<RT>::kRowPieces % 64 == 0, "weight slots fill whole copy instructions");
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

template <int G, int RT>
struct Copy {
    static constexpr int kW = Area<G, RT>::kWLoads, kS = Tile<RT>::kSlots;
    __amdgpu_buffer_rsrc_t wr, qr, dr;
    uint32_t wpiece[kW];   // per weight instruction: the lane's row and piece offset
    int wblk[kW];          // and the block of the step its piece is in
    uint32_t tok[G][kS];   // per group and slot: token row and piece offset (the step adds the super-block)
    uint32_t word;
    int word_sl;
};

// Issue the copies of the step at super-block st into area.
template <int G, int RT>
__device__ __forceinline__ void issue_step(const Copy<G, RT>& cp, int st, int S, uint8_t* area) {
    typedef Area<G, RT> A;
    constexpr int kS = Tile<RT>::kSlots;
#pragma unroll
    for (int c = 0; c < A::kWLoads; ++c)
        copy_to_lds(cp.wr, cp.wpiece[c] + (uint32_t)min(st + cp.wblk[c], S - 1) * (uint32_t)kBlockBytes, 0,
                    area + 1024 * c);
#pragma unroll
    for (int c = 0; c < A::kTokLoads; ++c)   // instruction c: group c / kS, super-block slot c % kS
        copy_to_lds(cp.qr, cp.tok[c / kS][c % kS], (uint32_t)min(st + c % kS, S - 1) * 256u,
                    area + A::kWBytes + 1024 * c);
    copy_to_lds(cp.dr, cp.word + (uint32_t)min(st + cp.word_sl, S - 1) * 32u, 0, area + A::kWBytes + A::kTokBytes);
}

// The arithmetic of one step from its LDS area: lane (row r, slot s, half h).
template <int G, int RT>
__device__ __forceinline__ void compute_step(const uint8_t* area, bool live, int r, int s, int h, int ti,
                                             v4f* acc, v4f* accm) {
    typedef Area<G, RT> A;
    typedef Tile<RT> T;
    const v4u* wp = reinterpret_cast<const v4u*>(area) + r * T::kRowPieces;
    const v4u hdr = wp[T::wslot(r, 9 * s)];
    v4u qv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) qv[j] = wp[T::wslot(r, 9 * s + 1 + 4 * h + j)];
    const float d = live ? half_lo(hdr.x) : 0.0f, dmin = live ? half_lo(hdr.x >> 16) : 0.0f;
    // this lane's token rows: group g at R = 4 kSlots g + 4s + ti; its scale
    // word for chunk c at word 8R + c
    const int R0 = 4 * s + ti, x = ti + 4 * s;
    const uint32_t* wd = reinterpret_cast<const uint32_t*>(area + A::kWBytes + A::kTokBytes) + 8 * R0;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        uint32_t sc2[2], mn2[2];
        scale_min_pair(hdr.y, hdr.z, hdr.w, 2 * h + pp, sc2[0], sc2[1], mn2[0], mn2[1]);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = 4 * h + 2 * pp + e;   // the chunk (lane-dependent through h)
            const float dsc = d * (float)sc2[e], mneg = -(dmin * (float)mn2[e]);
            int b[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const uint32_t xw = qv[2 * pp + (kk >> 2)][kk & 3];
                b[kk] = (int)(e ? (xw >> 4) & 0x0F0F0F0Fu : xw & 0x0F0F0F0Fu);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                // chunk c of row R: slots 2(c ^ x), 2(c ^ x) + 1
                const uint8_t* tp = area + A::kWBytes + (4 * T::kSlots * g + R0) * 256 + 32 * (c ^ x);
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
                const uint32_t word = wd[32 * T::kSlots * g + c];
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
}

template <int G, bool H, int RT, int WM>
__global__ __launch_bounds__(64 * WM) void mmq_narrow_kernel(const uint8_t* __restrict__ w,
                                                             const int8_t* __restrict__ q,
                                                             const uint32_t* __restrict__ ds,
                                                             int M, int N, int K,
                                                             void* __restrict__ out) {
    typedef Area<G, RT> A;
    typedef Tile<RT> T;
    constexpr int kS = T::kSlots;
    // Two areas per wave, as two arrays: the copies into one are in flight
    // while the other is read, and the compiler can tell them apart.
    __shared__ __attribute__((aligned(16))) uint8_t area0[WM][A::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t area1[WM][A::kBytes];

    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane & (RT - 1), s = (lane >> 4) & (kS - 1), h = lane >> 5;
    const int ti = lane & 3;     // the lane's token in a group (A operand)
    const int row0 = blockIdx.x * RT;
    const int rows = min(RT, M - row0);
    const int S = K >> 8, C = K >> 5;
    // Interleaved: wave wv takes the steps wv, wv + W, wv + 2W, ..., so the
    // W waves on these rows read W adjacent blocks of every row together.
    const int D = kS * W;          // super-blocks between a wave's steps
    const int sb0 = kS * wv, sb1 = S;

    // Copy sources.  Weight instruction c: lane u fills slot i = 64c + u of
    // row i / kRowPieces, whose piece p has wslot(row, p) = i % kRowPieces
    // (the xor is its own inverse; unused slots re-read piece 0).  Token
    // instruction c writes rows 4c .. 4c + 3 (group c / kSlots, slot
    // s = c % kSlots): lane u takes token 4g + u / 16 and its slot u % 16,
    // i.e. piece (u % 16) ^ 2x with x = u / 16 + 4s.  Word instruction: lane
    // u takes half u & 1 of row u / 2.  Rows past m re-read row m - 1 and
    // tokens past n token n - 1 (their results are never stored);
    // super-blocks past k re-read the last one (computed with d = dmin = 0).
    // The weight buffer starts at the tile's first row, so its offsets stay
    // within 32 bits for every k.
    Copy<G, RT> cp;
    const int64_t row_bytes = (int64_t)S * kBlockBytes;
    cp.wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w) + row0 * row_bytes, 0, (int)(rows * row_bytes),
                                              kBufferFlags);
    cp.qr = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(q), 0, N * K, kBufferFlags);
    cp.dr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(ds), 0, N * C * 4, kBufferFlags);
#pragma unroll
    for (int c = 0; c < A::kWLoads; ++c) {
        const int i = 64 * c + lane, wrow = i / T::kRowPieces;
        const int pc = T::wslot(wrow, i % T::kRowPieces);
        const int pv = pc < 9 * kS ? pc : 0;
        cp.wpiece[c] = (uint32_t)min(wrow, rows - 1) * (uint32_t)row_bytes + 16u * (uint32_t)(pv % 9);
        cp.wblk[c] = pv / 9;
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int sl = 0; sl < kS; ++sl)
            cp.tok[g][sl] = (uint32_t)min(4 * g + (lane >> 4), N - 1) * (uint32_t)K +
                            16u * ((lane & 15) ^ (2 * ((lane >> 4) + 4 * sl)));
    {
        const int wrr = min(lane >> 1, 4 * kS * G - 1);   // row R = 4 kSlots g + 4s + i
        const int tok = 4 * (wrr / (4 * kS)) + (wrr & 3);
        cp.word = (uint32_t)min(tok, N - 1) * (uint32_t)(C * 4) + 16u * (lane & 1);
        cp.word_sl = (wrr >> 2) & (kS - 1);
    }

    v4f acc[G], accm[G], acc2[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        acc[g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        accm[g] = acc[g];
        acc2[g] = acc[g];
    }
    auto flush = [&](int n_st) {
        if ((n_st & (T::kFlushSteps - 1)) == T::kFlushSteps - 1) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                acc2[g] += acc[g];
                acc2[g] += accm[g];
                acc[g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                accm[g] = acc[g];
            }
        }
    };

    // Steps in pairs (areas 0 and 1): the next step's copies are issued
    // before a step is computed; one wait for everything at the top of each
    // step.
    if (sb0 < sb1) issue_step<G, RT>(cp, sb0, S, area0[wv]);
    for (int st = sb0, n_st = 0; st < sb1; st += 2 * D, n_st += 2) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
        __builtin_amdgcn_sched_barrier(0);
        if (st + D < sb1) issue_step<G, RT>(cp, st + D, S, area1[wv]);
        __builtin_amdgcn_sched_barrier(0);
        compute_step<G, RT>(area0[wv], st + s < sb1, r, s, h, ti, acc, accm);
        flush(n_st);
        if (st + D >= sb1) break;
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt(0));
        __builtin_amdgcn_sched_barrier(0);
        if (st + 2 * D < sb1) issue_step<G, RT>(cp, st + 2 * D, S, area0[wv]);
        __builtin_amdgcn_sched_barrier(0);
        compute_step<G, RT>(area1[wv], st + D + s < sb1, r, s, h, ti, acc, accm);
        flush(n_st + 1);
    }

    // Partial sums: red[wave][g][v][lane], in area 0 once every wave is past
    // its loop.  Output (row r, token 4g + v) adds the lanes r + RT j of
    // every wave, waves in order and j in order within a wave.
    __syncthreads();
    float* red = reinterpret_cast<float*>(&area0[0][0]);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[((wv * G + g) * 4 + v) * 64 + lane] = (acc2[g][v] + acc[g][v]) + accm[g][v];
    __syncthreads();
    for (int e = threadIdx.x; e < G * 4 * RT; e += blockDim.x) {
        const int rr = e & (RT - 1), gv = e / RT;   // gv = 4g + v, the token
        float sum = 0.0f;
        for (int u = 0; u < W; ++u)
#pragma unroll
            for (int j = 0; j < 64 / RT; ++j) sum += red[(u * G * 4 + gv) * 64 + RT * j + rr];
        const int row = row0 + rr;
        if (gv < N && row < M) store_out<H>(out, (int64_t)gv * M + row, sum);
    }
}

template <int G, int RT, int WM>
hipError_t launch_t(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n, void* out,
                    bool half_out, int W, hipStream_t stream) {
    void* args[] = {(void*)&w, (void*)&q, (void*)&ds, (void*)&m, (void*)&n, (void*)&k, (void*)&out};
    const void* f = half_out ? (const void*)mmq_narrow_kernel<G, true, RT, WM>
                             : (const void*)mmq_narrow_kernel<G, false, RT, WM>;
    return hipLaunchKernel(f, dim3((unsigned)((m + RT - 1) / RT)), dim3(64 * W), args, 0, stream);
}

// Tile and waves per workgroup.  A wave's two areas take 14 to 28 KiB of
// LDS (5 KiB of weights, 1 (32-row tiles) or 2 KiB of token rows per group
// and 1 KiB of scale words, twice), so two 4-wave or one 8-wave workgroup
// fit a CU.  32-row tiles as narrow_waves32 says; otherwise 16-row tiles
// with up to 4 waves, about 8192 waves in all, preferring a count that
// divides the steps evenly.
template <int G>
hipError_t launch_g(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n, void* out,
                    bool half_out, hipStream_t stream) {
    const int w32 = narrow_waves32(m, k);
    if (w32 == 4) return launch_t<G, 32, 4>(w, m, k, q, ds, n, out, half_out, 4, stream);
    if (w32 == 8) return launch_t<G, 32, 8>(w, m, k, q, ds, n, out, half_out, 8, stream);
    const int wgs = (m + 15) / 16, steps = ((k >> 8) + 1) / 2;
    const int wmax = (int)std::max<int64_t>(1, std::min<int64_t>({4, steps, (8192 + wgs - 1) / wgs}));
    int W = wmax;
    for (int c = wmax; c * 2 > wmax; --c)
        if (steps % c == 0) { W = c; break; }
    return launch_t<G, 16, 4>(w, m, k, q, ds, n, out, half_out, W, stream);
}

}  // namespace

hipError_t launch_mmq_fp32_narrow(const uint8_t* w, int m, int k, const int8_t* q, const uint32_t* ds, int n,
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
