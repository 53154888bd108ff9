// mmq_api.hip - the C ABI declared in include/mmq.h.
//
// Every argument is checked on the host before any HIP call; only then is
// the current device checked (once per device: gfx950 or MMQ_ERR_DEVICE) and
// the kernel enqueued on the caller's stream.  Nothing here allocates.
#include <atomic>
#include <cstring>

#include "../../include/mmq.h"
#include "internal.h"
#include "stream.h"
#include "q6k_device.h"

namespace {

constexpr int64_t kMaxDim = 0x7fffffffLL;      // n, m
constexpr int64_t kMaxK = 1LL << 24;
constexpr int64_t kMaxElems = 1LL << 40;       // n*k, m*k/256*144, n*m, n*m*k/32

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 0 = not yet checked, 1 = gfx950, 2 = something else.
std::atomic<int> g_device_ok[64];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return MMQ_ERR_DEVICE;
    }
    if (dev < 64) {
        const int known = g_device_ok[dev].load(std::memory_order_relaxed);
        if (known == 1) return MMQ_OK;
        if (known == 2) return MMQ_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return MMQ_ERR_DEVICE;
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? MMQ_OK : MMQ_ERR_DEVICE;
}

// Shared checks of the MMQ calls (before any HIP call); block_bytes is the
// weight format's super-block size (144 for q4_K, 210 for q6_K).
int check_mmq(const void* w, int64_t m, int64_t k, const int8_t* q, int64_t n, const void* out,
              bool* empty, int64_t block_bytes = 144) {
    if (n < 0 || m < 0 || k <= 0 || (k & 255) != 0) return MMQ_ERR_SHAPE;
    if (n > kMaxDim || m > kMaxDim || k > kMaxK) return MMQ_ERR_OVERFLOW;
    if (n * k >= kMaxElems || m * (k / 256) * block_bytes >= kMaxElems || n * m >= kMaxElems)
        return MMQ_ERR_OVERFLOW;
    *empty = (n == 0 || m == 0);
    if (*empty) return MMQ_OK;
    if (!w || !q || !out) return MMQ_ERR_NULL;
    if (!aligned16(w) || !aligned16(q) || !aligned16(out)) return MMQ_ERR_ALIGN;
    return MMQ_OK;
}

using FoldLaunch = hipError_t (*)(const uint8_t*, int, int, const int8_t*, const uint32_t*, int, void*, bool,
                                  hipStream_t);

// HIP takes at most 2^32 - 1 work-items per grid dimension.
bool threads_ok(int64_t blocks, int64_t per_block) { return blocks * per_block < (1LL << 32); }

// Kernel behind the q4_K fold entry points for MMQ_KERNEL_AUTO, by token
// count and shape.  Set from timing sweeps of every kernel at 1-64 tokens
// over 22 matrices from 1024 x 4096 to 32768 x 4096, 28672 x 8192 and
// 8192 x 28672 (weights streamed from HBM; 478 cases): against the fastest
// named kernel per case the choice loses 0.18% in the geometric mean, 8.4% at
// most.
//   dot4 (1-2 tokens, and 5 unless the narrow kernel has long rows): its
//     workgroups of 16 rows fill the chip from about 10240 rows (8192 with
//     rows of >= 64 super-blocks), and its waves split a row's super-blocks
//     in 4-block steps, so it needs a multiple of 16 super-blocks: on
//     4096-row matrices the narrow kernel is 2-86% faster, on 13824 x 5120
//     (20 super-blocks) 23-51%;
//   stream (3-4 and 6-16 tokens): where it fits (at least 7 x 256 tiles of 8
//     rows, k <= 8192) and k is whole token phases (it computes every step
//     of the last one: 16 super-blocks up to 8 tokens, 8 above; 24576 x 6144
//     at 3-8 tokens is 8-18% slower than the narrow kernel); up to 8 tokens
//     with 7 or 8 waves per workgroup (5-6 waves, from 9-12 tiles per
//     workgroup, leave SIMDs idle: 20480 x 4096 5-13% behind), above 8
//     where k > 4096 or a workgroup holds at least 14 tiles (one phase is
//     paid back only over many rows: 14336 x 4096 at 9-16 tokens 8-24%
//     behind the few-token kernel); and at 9-12 tokens on rows of at least
//     64 super-blocks whatever the row count (6144 x 16384, 6144 x 28672 and
//     8160 x 28672: 24.2 / 39.6 / 39.1 us against 27.3 / 44.3 / 45.2 us for
//     the few-token kernel; at 13-16 tokens, or on rows of 32 super-blocks,
//     the few-token kernel leads):
//     28672 x 8192 at 4 / 7 / 12 / 16 tokens 25.9 / 30.9 / 39.3 / 45.1 us
//     against 28.3 / 34.5 / 45.1 / 47.9 us for the next kernel;
//   narrow (elsewhere up to 8 tokens; 9-16 where its 32-row tiles give each
//     wave at least 11 super-blocks, or on at most 4096 rows; 8192 x 22528,
//     11 per wave, at 12 tokens 28.9 us against 32.1 us for the stream kernel): 8192 x 28672
//     at 4 / 12 tokens 26.1 / 37.6 us against 28.7 / 45.8 us; 4096 x 14336
//     at 1 / 12 tokens 8.2 / 13.6 us against 11.4 / 20.4 us;
//   few-token int8-MFMA kernels (9-64 tokens otherwise): 11008 x 4096 at 12
//     tokens 10.1 us against 12.5 us for the stream kernel;
//   binary16-MFMA kernel: at 17-32 tokens where its 64-token tiles fill
//     224-255 CUs in one round (28672 rows: 67.1-68.4 us against 70.2-78.5
//     us; 24576 rows, 192 tiles, 8-10% behind; with 256 or more row tiles it
//     takes 128-token tiles and loses), at
//     33-64 tokens from 160 tiles (90.4 against 68.4 us at 33 tokens on
//     28672 x 8192), and above 64 tokens.
int q4k_auto_kernel(int64_t m, int64_t k, int64_t n) {
    const int64_t S = k >> 8;
    const int64_t f16_tiles = ((m + 127) / 128) * ((n + 127) / 128);
    const int w32 = mmq::narrow_waves32(m, k);
    const bool narrow_long = w32 > 0 && S / w32 >= 11;
    // the stream kernel's tiles per workgroup and its waves (two tiles each above 8)
    const int64_t tg = std::min<int64_t>(16, ((m + 7) / 8 + 255) / 256), tq = tg > 8 ? (tg + 1) / 2 : tg;
    const bool stream = mmq::stream_fits(m, k) && S % 16 == 0 && tq >= 7;               // up to 8 tokens
    const bool stream16 = mmq::stream_fits(m, k) && S % 8 == 0 && (S > 16 || tg >= 14);  // 9-16 tokens
    const bool stream12 = stream16 || (S % 8 == 0 && S >= 64);                           // 9-12 tokens
    const bool dot4 = S % 16 == 0 && (m >= 10240 || (m >= 8192 && S >= 64));
    if (n <= 2) return dot4 ? MMQ_KERNEL_DOT4 : MMQ_KERNEL_NARROW;
    if (n <= 4) return stream ? MMQ_KERNEL_STREAM : MMQ_KERNEL_NARROW;
    if (n <= 5) return dot4 && !narrow_long ? MMQ_KERNEL_DOT4 : MMQ_KERNEL_NARROW;
    if (n <= 8) return stream ? MMQ_KERNEL_STREAM : MMQ_KERNEL_NARROW;
    if (n <= mmq::kNarrowMaxN)
        return narrow_long || m <= 4096                  ? MMQ_KERNEL_NARROW
               : stream16 || (n <= 12 && stream12)       ? MMQ_KERNEL_STREAM
                                                         : MMQ_KERNEL_FEW;
    if (n <= 32) return f16_tiles >= 224 && f16_tiles < 256 ? MMQ_KERNEL_F16 : MMQ_KERNEL_FEW;
    if (n <= mmq::kSmallMaxN) return f16_tiles >= 160 ? MMQ_KERNEL_F16 : MMQ_KERNEL_FEW;
    return MMQ_KERNEL_F16;
}

// The repacked-weight entry: above 16 tokens the binary16-MFMA kernel on the
// records, where it has tiles enough for the CUs (>= 160 of 128 x 128) or the
// slices would be many (> 40 tokens); otherwise the dot4 kernel, in slices of
// 8 tokens.  Measured per call: 28672 x 8192 (224 tiles) at 9 / 16 / 24
// tokens 60 / 76 / 121 us in slices against 75 us; 8192 x 28672 (64 tiles)
// at 33 / 48 tokens 197 / 273 us in slices against 221 us.
int q4kr_auto_kernel(int64_t m, int64_t n) {
    const int64_t f16_tiles = ((m + 127) / 128) * ((n + 127) / 128);
    return n > 16 && (f16_tiles >= 160 || n > 40) ? MMQ_KERNEL_F16 : MMQ_KERNEL_DOT4;
}

// The launcher of a q4_K fold kernel choice, and whether its grid fits.
int q4k_fold_launcher(int kernel, int64_t m, int64_t k, int64_t n, FoldLaunch* f) {
    if (kernel == MMQ_KERNEL_AUTO) kernel = q4k_auto_kernel(m, k, n);
    switch (kernel) {
        case MMQ_KERNEL_DOT4:
            if (n > mmq::kGemvMaxN) return MMQ_ERR_KERNEL;
            *f = mmq::launch_mmq_fp32_gemv;
            return threads_ok((m + 15) / 16, 256) ? MMQ_OK : MMQ_ERR_OVERFLOW;
        case MMQ_KERNEL_FEW:
            if (n > mmq::kSmallMaxN) return MMQ_ERR_KERNEL;
            *f = mmq::launch_mmq_fp32_small;
            return threads_ok((m + 15) / 16, 512) ? MMQ_OK : MMQ_ERR_OVERFLOW;
        case MMQ_KERNEL_F16:
            *f = mmq::launch_mmq_fp32_f16;
            return threads_ok((m + 127) / 128 * ((n + 63) / 64), 1024) ? MMQ_OK : MMQ_ERR_OVERFLOW;
        case MMQ_KERNEL_I8:
            *f = mmq::launch_mmq_fp32;
            return threads_ok((m + 127) / 128 * ((n + 127) / 128), 256) ? MMQ_OK : MMQ_ERR_OVERFLOW;
        case MMQ_KERNEL_NARROW:
            if (n > mmq::kNarrowMaxN) return MMQ_ERR_KERNEL;
            *f = mmq::launch_mmq_fp32_narrow;
            return threads_ok((m + 15) / 16, 512) ? MMQ_OK : MMQ_ERR_OVERFLOW;
        case MMQ_KERNEL_STREAM:
            if (n > mmq::kStreamMaxN) return MMQ_ERR_KERNEL;
            *f = mmq::launch_mmq_fp32_stream;
            return threads_ok((m + 7) / 8, 512) ? MMQ_OK : MMQ_ERR_OVERFLOW;
        default:
            return MMQ_ERR_KERNEL;
    }
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return MMQ_OK;
    (void)hipGetLastError();
    return MMQ_ERR_HIP;
}

// The q4_K fold entry points: same checks, same kernels, float32 or binary16
// stores of the same float32 result.
int fold_entry(const void* w, int64_t m, int64_t k, const int8_t* q, const uint32_t* ds, int64_t n,
               void* out, bool half_out, int kernel, hipStream_t stream) {
    bool empty = false;
    int rc = check_mmq(w, m, k, q, n, out, &empty);
    if (rc != MMQ_OK || empty) return rc;
    if (!ds) return MMQ_ERR_NULL;
    if (!aligned16(ds)) return MMQ_ERR_ALIGN;
    FoldLaunch launch = nullptr;
    rc = q4k_fold_launcher(kernel, m, k, n, &launch);
    if (rc != MMQ_OK) return rc;
    rc = check_device();
    if (rc != MMQ_OK) return rc;
    return hip_status(launch(static_cast<const uint8_t*>(w), (int)m, (int)k, q, ds, (int)n, out, half_out,
                             stream));
}

// The fold entry points on q8 operand tiles: always the binary16-MFMA kernel
// (the tiles are its operand layout), on q4_K rows or repacked records.
int tiles_fold_entry(const void* w, bool repacked, int64_t m, int64_t k, const uint16_t* qt,
                     const uint32_t* ds, int64_t n, float* out, hipStream_t stream) {
    bool empty = false;
    int rc = check_mmq(w, m, k, reinterpret_cast<const int8_t*>(qt), n, out, &empty);
    if (rc != MMQ_OK || empty) return rc;
    if (n > kMaxDim - 127 || (n + 127) / 128 * 128 * k >= kMaxElems) return MMQ_ERR_OVERFLOW;
    if (repacked && (m + 15) / 16 * (k / 256) * mmq::kRepackRecordBytes >= kMaxElems)
        return MMQ_ERR_OVERFLOW;
    if (!threads_ok((m + 127) / 128 * ((n + 63) / 64), 1024)) return MMQ_ERR_OVERFLOW;
    if (!ds) return MMQ_ERR_NULL;
    if (!aligned16(ds)) return MMQ_ERR_ALIGN;
    rc = check_device();
    if (rc != MMQ_OK) return rc;
    return hip_status(mmq::launch_mmq_fp32_f16_tiles(static_cast<const uint8_t*>(w), repacked, (int)m,
                                                     (int)k, qt, ds, (int)n, out, stream));
}

// Kernel behind the q6_K fold entry points for MMQ_KERNEL_AUTO: the
// vector-ALU dot4 kernel for n <= 8, the binary16-MFMA kernel above.
int q6k_auto_kernel(int64_t n) { return n <= mmq::kQ6kGemvMaxN ? MMQ_KERNEL_DOT4 : MMQ_KERNEL_F16; }

int q6k_fold_launcher(int kernel, int64_t m, int64_t n, FoldLaunch* f) {
    if (kernel == MMQ_KERNEL_AUTO) kernel = q6k_auto_kernel(n);
    switch (kernel) {
        case MMQ_KERNEL_DOT4:
            if (n > mmq::kQ6kGemvMaxN) return MMQ_ERR_KERNEL;
            *f = mmq::launch_q6k_gemv;
            return threads_ok((m + 15) / 16, 256) ? MMQ_OK : MMQ_ERR_OVERFLOW;
        case MMQ_KERNEL_F16:
            *f = mmq::launch_q6k_f16;
            return threads_ok((m + 127) / 128 * ((n + 127) / 128), 1024) ? MMQ_OK : MMQ_ERR_OVERFLOW;
        case MMQ_KERNEL_I8:
            *f = mmq::launch_q6k_i8;
            return threads_ok((m + 127) / 128 * ((n + 127) / 128), 256) ? MMQ_OK : MMQ_ERR_OVERFLOW;
        default:
            return MMQ_ERR_KERNEL;
    }
}

int q6k_fold_entry(const void* w, int64_t m, int64_t k, const int8_t* q, const uint32_t* ds,
                   int64_t n, void* out, bool half_out, int kernel, hipStream_t stream) {
    bool empty = false;
    int rc = check_mmq(w, m, k, q, n, out, &empty, mmq::kQ6kBlockBytes);
    if (rc != MMQ_OK || empty) return rc;
    if (!ds) return MMQ_ERR_NULL;
    if (!aligned16(ds)) return MMQ_ERR_ALIGN;
    FoldLaunch launch = nullptr;
    rc = q6k_fold_launcher(kernel, m, n, &launch);
    if (rc != MMQ_OK) return rc;
    rc = check_device();
    if (rc != MMQ_OK) return rc;
    return hip_status(launch(static_cast<const uint8_t*>(w), (int)m, (int)k, q, ds, (int)n, out, half_out,
                             stream));
}

}  // namespace

extern "C" {

int q8_quantize_rows(const float* x, int64_t n, int64_t k, int8_t* q, uint32_t* ds,
                     hipStream_t stream) {
    if (n < 0 || k <= 0 || (k & 31) != 0) return MMQ_ERR_SHAPE;
    if (n > kMaxDim || k > kMaxK || n * k >= kMaxElems) return MMQ_ERR_OVERFLOW;
    if (!threads_ok(n * (k / 32) * 4, 1)) return MMQ_ERR_OVERFLOW;   // 4 lanes per 32-block
    if (n == 0) return MMQ_OK;
    if (!x || !q || !ds) return MMQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(ds)) return MMQ_ERR_ALIGN;
    const int dev = check_device();
    if (dev != MMQ_OK) return dev;
    return hip_status(mmq::launch_q8_quantize(x, n * (k / 32), q, ds, stream));
}

int q8_quantize_rows_tiled(const float* x, int64_t n, int64_t k, uint16_t* qt, uint32_t* ds,
                           hipStream_t stream) {
    if (n < 0 || k <= 0 || (k & 255) != 0) return MMQ_ERR_SHAPE;
    if (n > kMaxDim - 127 || k > kMaxK || (n + 127) / 128 * 128 * k >= kMaxElems) return MMQ_ERR_OVERFLOW;
    if (!threads_ok((n + 127) / 128 * 128 * (k / 32) * 4, 1)) return MMQ_ERR_OVERFLOW;   // 4 lanes per 32-block
    if (n == 0) return MMQ_OK;
    if (!x || !qt || !ds) return MMQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(qt) || !aligned16(ds)) return MMQ_ERR_ALIGN;
    const int dev = check_device();
    if (dev != MMQ_OK) return dev;
    return hip_status(mmq::launch_q8_quantize_tiled(x, (int)n, (int)k, qt, ds, stream));
}

int q8_quantize_silu_mul(const float* gate, const float* up, int64_t n, int64_t k, int8_t* q,
                         uint32_t* ds, hipStream_t stream) {
    if (n < 0 || k <= 0 || (k & 31) != 0) return MMQ_ERR_SHAPE;
    if (n > kMaxDim || k > kMaxK || n * k >= kMaxElems) return MMQ_ERR_OVERFLOW;
    if (!threads_ok(n * (k / 32) * 4, 1)) return MMQ_ERR_OVERFLOW;
    if (n == 0) return MMQ_OK;
    if (!gate || !up || !q || !ds) return MMQ_ERR_NULL;
    if (!aligned16(gate) || !aligned16(up) || !aligned16(q) || !aligned16(ds)) return MMQ_ERR_ALIGN;
    const int dev = check_device();
    if (dev != MMQ_OK) return dev;
    return hip_status(mmq::launch_q8_quantize_silu_mul(gate, up, n * (k / 32), q, ds, stream));
}

int q8_quantize_silu_mul_tiled(const float* gate, const float* up, int64_t n, int64_t k, uint16_t* qt,
                               uint32_t* ds, hipStream_t stream) {
    if (n < 0 || k <= 0 || (k & 255) != 0) return MMQ_ERR_SHAPE;
    if (n > kMaxDim - 127 || k > kMaxK || (n + 127) / 128 * 128 * k >= kMaxElems) return MMQ_ERR_OVERFLOW;
    if (!threads_ok((n + 127) / 128 * 128 * (k / 32) * 4, 1)) return MMQ_ERR_OVERFLOW;   // 4 lanes per 32-block
    if (n == 0) return MMQ_OK;
    if (!gate || !up || !qt || !ds) return MMQ_ERR_NULL;
    if (!aligned16(gate) || !aligned16(up) || !aligned16(qt) || !aligned16(ds)) return MMQ_ERR_ALIGN;
    const int dev = check_device();
    if (dev != MMQ_OK) return dev;
    return hip_status(mmq::launch_q8_quantize_silu_mul_tiled(gate, up, (int)n, (int)k, qt, ds, stream));
}

int mmq_q4k_q8(const void* w, int64_t m, int64_t k, const int8_t* q, const uint32_t* ds,
               int64_t n, int32_t* dots, hipStream_t stream) {
    (void)ds;  // not read: the block dots do not depend on the scales
    bool empty = false;
    int rc = check_mmq(w, m, k, q, n, dots, &empty);
    if (rc != MMQ_OK || empty) return rc;
    if (n * m >= kMaxElems / (k / 32)) return MMQ_ERR_OVERFLOW;
    if (!threads_ok((m + 127) / 128 * ((n + 127) / 128), 256)) return MMQ_ERR_OVERFLOW;
    if (ds && !aligned16(ds)) return MMQ_ERR_ALIGN;
    rc = check_device();
    if (rc != MMQ_OK) return rc;
    return hip_status(mmq::launch_mmq_dots(static_cast<const uint8_t*>(w), (int)m, (int)k, q,
                                           (int)n, dots, stream));
}

int mmq_q4k_q8_fp32out(const void* w, int64_t m, int64_t k, const int8_t* q,
                       const uint32_t* ds, int64_t n, float* out, hipStream_t stream) {
    return fold_entry(w, m, k, q, ds, n, out, false, MMQ_KERNEL_AUTO, stream);
}

int mmq_q4k_q8_f16out(const void* w, int64_t m, int64_t k, const int8_t* q,
                      const uint32_t* ds, int64_t n, uint16_t* out, hipStream_t stream) {
    return fold_entry(w, m, k, q, ds, n, out, true, MMQ_KERNEL_AUTO, stream);
}

int mmq_q4k_q8_fold(const void* w, int64_t m, int64_t k, const int8_t* q, const uint32_t* ds, int64_t n,
                    void* out, int out_f16, int kernel, hipStream_t stream) {
    return fold_entry(w, m, k, q, ds, n, out, out_f16 != 0, kernel, stream);
}

int mmq_q6k_q8(const void* w, int64_t m, int64_t k, const int8_t* q, const uint32_t* ds,
               int64_t n, int32_t* dots, hipStream_t stream) {
    (void)ds;  // not read: the group dots do not depend on the scales
    bool empty = false;
    int rc = check_mmq(w, m, k, q, n, dots, &empty, mmq::kQ6kBlockBytes);
    if (rc != MMQ_OK || empty) return rc;
    if (n * m >= kMaxElems / (k / 16)) return MMQ_ERR_OVERFLOW;
    if (!threads_ok((m + 127) / 128 * ((n + 127) / 128), 256)) return MMQ_ERR_OVERFLOW;
    if (ds && !aligned16(ds)) return MMQ_ERR_ALIGN;
    rc = check_device();
    if (rc != MMQ_OK) return rc;
    return hip_status(mmq::launch_q6k_dots(static_cast<const uint8_t*>(w), (int)m, (int)k, q,
                                           (int)n, dots, stream));
}

int mmq_q6k_q8_fp32out(const void* w, int64_t m, int64_t k, const int8_t* q,
                       const uint32_t* ds, int64_t n, float* out, hipStream_t stream) {
    return q6k_fold_entry(w, m, k, q, ds, n, out, false, MMQ_KERNEL_AUTO, stream);
}

int mmq_q6k_q8_f16out(const void* w, int64_t m, int64_t k, const int8_t* q,
                      const uint32_t* ds, int64_t n, uint16_t* out, hipStream_t stream) {
    return q6k_fold_entry(w, m, k, q, ds, n, out, true, MMQ_KERNEL_AUTO, stream);
}

int mmq_q6k_q8_fold(const void* w, int64_t m, int64_t k, const int8_t* q, const uint32_t* ds, int64_t n,
                    void* out, int out_f16, int kernel, hipStream_t stream) {
    return q6k_fold_entry(w, m, k, q, ds, n, out, out_f16 != 0, kernel, stream);
}

int mmq_kernel_choice(int format, int64_t m, int64_t k, int64_t n) {
    if (n < 0 || m < 0 || k <= 0 || (k & 255) != 0) return MMQ_ERR_SHAPE;
    switch (format) {
        case MMQ_FORMAT_Q4K: return q4k_auto_kernel(m, k, n);
        case MMQ_FORMAT_Q4K_REPACKED: return q4kr_auto_kernel(m, n);
        case MMQ_FORMAT_Q6K: return q6k_auto_kernel(n);
        case MMQ_FORMAT_Q4K_TILES:
        case MMQ_FORMAT_Q4K_REPACKED_TILES:
        case MMQ_FORMAT_Q6K_TILES: return MMQ_KERNEL_F16;
        default: return MMQ_ERR_KERNEL;
    }
}

int q4k_repack(const void* w, int64_t m, int64_t k, void* wr, hipStream_t stream) {
    if (m < 0 || k <= 0 || (k & 255) != 0) return MMQ_ERR_SHAPE;
    if (m > kMaxDim || k > kMaxK) return MMQ_ERR_OVERFLOW;
    if (m * (k / 256) * 144 >= kMaxElems || (m + 15) / 16 * (k / 256) * mmq::kRepackRecordBytes >= kMaxElems)
        return MMQ_ERR_OVERFLOW;
    if (!threads_ok((m + 15) / 16 * (k / 256), 64)) return MMQ_ERR_OVERFLOW;   // 64 lanes per record
    if (m == 0) return MMQ_OK;
    if (!w || !wr) return MMQ_ERR_NULL;
    if (!aligned16(w) || !aligned16(wr)) return MMQ_ERR_ALIGN;
    const int dev = check_device();
    if (dev != MMQ_OK) return dev;
    return hip_status(mmq::launch_q4k_repack(static_cast<const uint8_t*>(w), (int)m, (int)k,
                                             static_cast<uint8_t*>(wr), stream));
}

int mmq_q4kr_q8_fp32out(const void* wr, int64_t m, int64_t k, const int8_t* q,
                        const uint32_t* ds, int64_t n, float* out, hipStream_t stream) {
    bool empty = false;
    int rc = check_mmq(wr, m, k, q, n, out, &empty);
    if (rc != MMQ_OK || empty) return rc;
    if ((m + 15) / 16 * (k / 256) * mmq::kRepackRecordBytes >= kMaxElems) return MMQ_ERR_OVERFLOW;
    if (!ds) return MMQ_ERR_NULL;
    if (!aligned16(ds)) return MMQ_ERR_ALIGN;
    const bool f16 = q4kr_auto_kernel(m, n) == MMQ_KERNEL_F16;
    if (f16 ? !threads_ok((m + 127) / 128 * ((n + 63) / 64), 1024) : !threads_ok((m + 15) / 16, 256))
        return MMQ_ERR_OVERFLOW;
    rc = check_device();
    if (rc != MMQ_OK) return rc;
    if (f16)
        return hip_status(mmq::launch_mmq_fp32_f16_repacked(static_cast<const uint8_t*>(wr), (int)m, (int)k,
                                                            q, ds, (int)n, out, stream));
    // Up to 8 tokens per launch; more tokens run as slices of 8 (each reads
    // the weights again: this layout serves the few-token path).  Slice
    // starts stay 16-byte aligned: 8 rows of q, ds and out are 8k, k/4 and
    // 32m bytes.
    for (int64_t t0 = 0; t0 < n; t0 += mmq::kGemvMaxN) {
        const int nn = (int)(n - t0 < mmq::kGemvMaxN ? n - t0 : mmq::kGemvMaxN);
        rc = hip_status(mmq::launch_mmq_fp32_gemv_repacked(
            static_cast<const uint8_t*>(wr), (int)m, (int)k, q + t0 * k, ds + t0 * (k / 32), nn,
            out + t0 * m, false, stream));
        if (rc != MMQ_OK) return rc;
    }
    return MMQ_OK;
}

int mmq_q4k_q8t_fp32out(const void* w, int64_t m, int64_t k, const uint16_t* qt,
                        const uint32_t* ds, int64_t n, float* out, hipStream_t stream) {
    return tiles_fold_entry(w, false, m, k, qt, ds, n, out, stream);
}

int mmq_q4kr_q8t_fp32out(const void* wr, int64_t m, int64_t k, const uint16_t* qt,
                         const uint32_t* ds, int64_t n, float* out, hipStream_t stream) {
    return tiles_fold_entry(wr, true, m, k, qt, ds, n, out, stream);
}

int mmq_q6k_q8t_fp32out(const void* w, int64_t m, int64_t k, const uint16_t* qt,
                        const uint32_t* ds, int64_t n, float* out, hipStream_t stream) {
    bool empty = false;
    int rc = check_mmq(w, m, k, reinterpret_cast<const int8_t*>(qt), n, out, &empty, mmq::kQ6kBlockBytes);
    if (rc != MMQ_OK || empty) return rc;
    if (n > kMaxDim - 127 || (n + 127) / 128 * 128 * k >= kMaxElems) return MMQ_ERR_OVERFLOW;
    if (!threads_ok((m + 127) / 128 * ((n + 127) / 128), 1024)) return MMQ_ERR_OVERFLOW;
    if (!ds) return MMQ_ERR_NULL;
    if (!aligned16(ds)) return MMQ_ERR_ALIGN;
    rc = check_device();
    if (rc != MMQ_OK) return rc;
    return hip_status(mmq::launch_q6k_f16_tiles(static_cast<const uint8_t*>(w), (int)m, (int)k, qt, ds,
                                                (int)n, out, stream));
}

const char* mmq_status_string(int status) {
    switch (status) {
        case MMQ_OK: return "MMQ_OK";
        case MMQ_ERR_NULL: return "MMQ_ERR_NULL: a required pointer is NULL";
        case MMQ_ERR_SHAPE: return "MMQ_ERR_SHAPE: invalid size (negative, k == 0, or k not a multiple of 32/256)";
        case MMQ_ERR_ALIGN: return "MMQ_ERR_ALIGN: a pointer is not 16-byte aligned";
        case MMQ_ERR_OVERFLOW: return "MMQ_ERR_OVERFLOW: size beyond the kernels' index range";
        case MMQ_ERR_DEVICE: return "MMQ_ERR_DEVICE: no HIP device, or the current device is not gfx950";
        case MMQ_ERR_HIP: return "MMQ_ERR_HIP: the HIP runtime reported a launch error";
        case MMQ_ERR_KERNEL: return "MMQ_ERR_KERNEL: unknown kernel or format, or a kernel outside its token range";
        default: return "unknown mmq status";
    }
}

}  // extern "C"
