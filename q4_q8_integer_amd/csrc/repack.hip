// repack.hip - load-time re-layout of q4_K weights (few-token dot4 kernel,
// and the binary16-MFMA prefill kernel's producers).
//
// The pages name a "load-time B pre-expansion" round and a later scale
// "predecode" round (the r17 page's and the r31 page's neighbours), not a
// format; this layout is the library's.  Rows are taken in tiles of 16, one
// 2368-byte record per (tile, super-block), records tile-major:
//   [0, 64)      dword r:         d | dmin << 16 of row r (binary16 bits)
//   [64, 320)    dword 16p + r:   sc[2p] | sc[2p+1] << 8 | m[2p] << 16 | m[2p+1] << 24
//   [320, 2368)  16 bytes at 320 + 512p + 256h + 16r: qs bytes 32p + 16h .. +15 of row r
// Rows past m are zero.  A wave of the dot4 kernel then reads a step as one
// contiguous run, with every lane's data at a fixed offset, and takes its
// 6-bit scales as bytes (no bit-field decode); the binary16 kernel's
// producers likewise read a chunk pair's (sc, m) as one dword.  148 bytes per
// row and super-block against 144.
#include "internal.h"
#include "kquant_device.h"

namespace mmq {
namespace {

// One record per 64 lanes: lane 16p + r takes row r's header and its qs
// bytes 32p .. 32p+31.
__global__ __launch_bounds__(256) void q4k_repack_kernel(const uint8_t* __restrict__ w, int M, int S,
                                                         uint8_t* __restrict__ wr) {
    const int64_t rec = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nrec = (int64_t)((M + 15) / 16) * S;
    if (rec >= nrec) return;
    const int lane = threadIdx.x & 63, p = lane >> 4, r = lane & 15;
    const int64_t t = rec / S, b = rec - t * S;
    const int64_t row = t * 16 + r;
    uint4 hdr = make_uint4(0, 0, 0, 0), qa = hdr, qb = hdr;
    if (row < M) {
        const uint8_t* blk = w + (row * S + b) * kBlockBytes;
        hdr = *reinterpret_cast<const uint4*>(blk);
        qa = *reinterpret_cast<const uint4*>(blk + 16 + 32 * p);
        qb = *reinterpret_cast<const uint4*>(blk + 32 + 32 * p);
    }
    uint8_t* out = wr + rec * kRepackRecordBytes;
    if (p == 0) *reinterpret_cast<uint32_t*>(out + 4 * r) = hdr.x;
    int sc0, m0, sc1, m1;
    scale_min(hdr.y, hdr.z, hdr.w, 2 * p, sc0, m0);
    scale_min(hdr.y, hdr.z, hdr.w, 2 * p + 1, sc1, m1);
    *reinterpret_cast<uint32_t*>(out + 64 + 4 * (16 * p + r)) =
        (uint32_t)sc0 | ((uint32_t)sc1 << 8) | ((uint32_t)m0 << 16) | ((uint32_t)m1 << 24);
    *reinterpret_cast<uint4*>(out + 320 + 512 * p + 16 * r) = qa;
    *reinterpret_cast<uint4*>(out + 320 + 512 * p + 256 + 16 * r) = qb;
}

}  // namespace

hipError_t launch_q4k_repack(const uint8_t* w, int m, int k, uint8_t* wr, hipStream_t stream) {
    const int S = k / 256;
    const int64_t nrec = (int64_t)((m + 15) / 16) * S;
    const unsigned grid = (unsigned)((nrec + 3) / 4);
    hipLaunchKernelGGL(q4k_repack_kernel, dim3(grid), dim3(256), 0, stream, w, m, S, wr);
    return hipGetLastError();
}

}  // namespace mmq
