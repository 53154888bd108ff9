// stream.h - the stream kernel's launcher, work split and automatic range
// (mmq_stream.hip): kept out of internal.h, whose every includer is a
// kernel source.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace mmq {

// Two-term fold for 1 <= n <= kStreamMaxN tokens with the narrow kernel's
// arithmetic, token operands held in LDS by a workgroup of many 8-row tiles
// and weights streamed in 576-byte runs (mmq_stream.hip).
hipError_t launch_mmq_fp32_stream(const uint8_t* w, int m, int k, const int8_t* q,
                                  const uint32_t* ds, int n, void* out, bool half_out,
                                  hipStream_t stream);
constexpr int kStreamMaxN = 16;

// The stream kernel's work split for m rows: TG = tq * tpw tiles of 8 rows
// per workgroup, about one workgroup per CU (256), at most 16 tiles each
// (more workgroups beyond that); a wave owns tpw tiles (two from 9 tiles per
// workgroup on, the count then rounded up to even), and wpt waves share each
// tile's steps, so that tq * wpt <= 8 waves.
inline void stream_layout(int64_t m, int& tq, int& tpw, int& wpt) {
    const int64_t tiles = (m + 7) / 8;
    int tg = (int)std::min<int64_t>(16, (tiles + 255) / 256);
    tpw = tg > 8 ? 2 : 1;
    tq = (tg + tpw - 1) / tpw;
    wpt = tq == 1 ? 4 : tq == 2 ? 4 : tq <= 4 ? 2 : 1;
}

// Where the automatic choice takes the stream kernel (3-4 and 6-8 tokens):
// at least 7 x 256 tiles of 8 rows and k <= 8192 (at most two token phases).
inline bool stream_fits(int64_t m, int64_t k) { return (m + 7) / 8 >= 7 * 256 && (k >> 8) <= 32; }

}  // namespace mmq
