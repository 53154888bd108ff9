/*
 * mmq.h - C ABI of the q4_K x q8 quantized matrix multiply (MMQ) for MI355X.
 *
 * The operation (the yusiwen.cn "minfer" pages: r31 "q-major sda scale-read
 * repack", sections 1 and 2, and r22 "qa8 XOR swizzle"): LLM prefill
 * multiplies a weight matrix W[m x k], stored as 4-bit k-quant (q4_K)
 * super-blocks, by activations X[n x k] that are quantized per token and per
 * 32-element block to int8 with a per-block scale word.  Each 32-element
 * chunk is an exact integer dot product, rescaled by the two-term rank-1 fold
 *
 *   out[t][o] = sum_c (d*sc)[o,c]*da[t,c]*D[t][o][c] - (dmin*m)[o,c]*da[t,c]*ssum[t,c]
 *   D[t][o][c] = sum_{i<32} q4[o][32c+i] * q8[t][32c+i]
 *
 * Data formats
 *   q4_K weights: m rows, each row k/256 super-blocks of 144 bytes, rows
 *     contiguous (row o's super-block b at byte (o*(k/256) + b)*144).  Block:
 *     d (binary16) at 0, dmin (binary16) at 2, twelve bytes of 6-bit (sc, m)
 *     pairs at 4 (GGUF k-quant packing), 128 bytes of nibbles at 16: weight
 *     64p+i is the low nibble of byte 32p+i, weight 64p+32+i its high nibble.
 *   q8 activations: q int8 [n][k] row-major and one 32-bit scale word per
 *     (token, 32-element block), ds uint32 [n][k/32]: binary16 da in the low
 *     16 bits, ssum = sum of the block's 32 q values as a two's-complement
 *     16-bit integer in the high 16 bits (r31 page, section 3.2).
 *
 * Conventions for every call
 *   - All array pointers are DEVICE pointers, allocated and owned by the
 *     caller; the library allocates nothing, keeps no pointer after
 *     returning, and keeps no global state other than a per-device
 *     "is this a gfx950" check.  Calls are reentrant.
 *   - Work is enqueued asynchronously on `stream` (NULL = the default
 *     stream); the caller keeps every buffer alive until the stream has
 *     finished.  Output buffers must not overlap inputs.
 *   - Every pointer must be 16-byte aligned.
 *   - n or m equal to 0 is an empty call: it returns MMQ_OK and touches
 *     nothing (pointers may then be NULL).  Negative sizes are MMQ_ERR_SHAPE.
 *   - Argument errors are detected on the host before any HIP call and
 *     before anything is enqueued.  No call throws or aborts.
 *   - Inputs must be finite.
 */
#ifndef Q4Q8_MMQ_H
#define Q4Q8_MMQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

enum mmq_status {
    MMQ_OK = 0,
    MMQ_ERR_NULL = -1,      /* a required pointer is NULL */
    MMQ_ERR_SHAPE = -2,     /* negative size, k not a multiple of 32 (quantize) or 256 (MMQ), k == 0 */
    MMQ_ERR_ALIGN = -3,     /* a pointer is not 16-byte aligned */
    MMQ_ERR_OVERFLOW = -4,  /* a size beyond the kernels' index range (see limits below) */
    MMQ_ERR_DEVICE = -5,    /* no HIP device, or the current device is not gfx950 */
    MMQ_ERR_HIP = -6,       /* the HIP runtime reported an error at launch */
    MMQ_ERR_KERNEL = -7     /* unknown kernel or format id, or a kernel outside its token range */
};

/* Size limits (MMQ_ERR_OVERFLOW beyond them): n, m <= 2^31 - 1; k <= 2^24;
 * n*k and m*k/256*144 below 2^40; for mmq_q4k_q8 also n*m*(k/32) < 2^40;
 * and every launch the call makes below 2^32 work-items (HIP's grid limit):
 * for the quantizers n*k/8 (tiled: ceil(n/128)*128*k/8), for the matmuls
 * 1024 per tile of 128 rows x 64 tokens, 512 per 16 rows (few tokens). */

/*
 * q8_quantize_rows - per-token, per-32-element q8 quantization of activations.
 * (Workload definition of the q8 activations: da = max|x|/127, q = round(x/da),
 * ssum = sum q; packed scale word as in the r31 page, section 3.2.)
 *
 *   x   : float [n][k], row-major, k % 32 == 0.
 *   q   : int8 [n][k] (out).   q = round(x / da), fp32 division, ties away from
 *         zero, in [-127, 127]; da = fp32(max|x| / 127) of the block.
 *   ds  : uint32 [n][k/32] (out).  binary16(da) (round to nearest even,
 *         subnormals kept) | (uint16)ssum << 16.  An all-zero block gives
 *         q = 0 and ds = 0.
 */
int q8_quantize_rows(const float *x, int64_t n, int64_t k, int8_t *q, uint32_t *ds,
                     hipStream_t stream);

/*
 * q8_quantize_silu_mul - the q8 quantization of an FFN down projection's
 * input h = SiLU(gate) * up, without writing h.  (The pages' later
 * "quantize-transpose prepass", named on the r22 page, moved activation
 * quantization into a pass of its own; fusing the gate product into that
 * pass is this library's reading.)
 *
 *   gate, up : float [n][k] each, row-major, k % 32 == 0 (the gate and up
 *              projections' outputs).
 *   q, ds    : as for q8_quantize_rows, of
 *              h = float32( g*u / (1 + exp(-g)) ) evaluated in float64
 *              (g*u exact, IEEE add and divide, one rounding to float32).
 * The result equals q8_quantize_rows applied to that h.  Errors and empty
 * calls as for q8_quantize_rows.
 */
int q8_quantize_silu_mul(const float *gate, const float *up, int64_t n, int64_t k, int8_t *q,
                         uint32_t *ds, hipStream_t stream);

/*
 * mmq_q4k_q8 - exact per-block integer dot products (the int32 result of the
 * 32-deep integer contraction, before the two-term rescale; r31 page, section 1).
 *
 *   w    : q4_K super-blocks of W [m][k] (m*(k/256)*144 bytes), k % 256 == 0.
 *   q    : int8 [n][k] q8 activations.
 *   ds   : the activations' scale words; accepted for a signature uniform with
 *          mmq_q4k_q8_fp32out and not read (may be NULL).
 *   dots : int32 [n][m][k/32] (out), dots[t][o][c] = D[t][o][c], exact.
 * A parity/inspection entry: its output is 4*n*m*k/32 bytes.
 */
int mmq_q4k_q8(const void *w, int64_t m, int64_t k, const int8_t *q, const uint32_t *ds,
               int64_t n, int32_t *dots, hipStream_t stream);

/*
 * mmq_q4k_q8_fp32out - the quantized matmul with the two-term rank-1 fold
 * applied per 32-element chunk (r31 page, sections 1-2), float32 result.
 *
 *   w   : q4_K super-blocks of W [m][k], k % 256 == 0.
 *   q   : int8 [n][k];  ds : uint32 [n][k/32] (as written by q8_quantize_rows).
 *   out : float [n][m] (out), token-major: out[t][o].  The summation order is
 *         the kernel's; results agree with the exact value to float32
 *         rounding of the accumulation: relative L2 error <= 1e-5, and every
 *         element within 1e-3 of its token row's largest |value|, for every
 *         k accepted (no float32 sum runs over more than 256 super-blocks).
 */
int mmq_q4k_q8_fp32out(const void *w, int64_t m, int64_t k, const int8_t *q,
                       const uint32_t *ds, int64_t n, float *out, hipStream_t stream);

/*
 * mmq_q4k_q8_f16out - the same quantized matmul and fold as
 * mmq_q4k_q8_fp32out, stored as IEEE binary16: out[t][o] is the float32
 * result rounded to nearest-even (overflow to +-inf), halving the output
 * bytes.  The pages only name a binary16 step after the output store (the
 * r22 page's round index, "r23 - f16 wall decomposition"); a binary16 output
 * is this library's reading of it.
 *
 *   w, q, ds : as for mmq_q4k_q8_fp32out.
 *   out      : binary16 bit patterns [n][m] (out), token-major, 16-byte
 *              aligned.  For the same inputs and binary, out[t][o] equals the
 *              binary16 rounding of mmq_q4k_q8_fp32out's out[t][o] bit for bit.
 * Errors and empty calls as for mmq_q4k_q8_fp32out.
 */
int mmq_q4k_q8_f16out(const void *w, int64_t m, int64_t k, const int8_t *q,
                      const uint32_t *ds, int64_t n, uint16_t *out, hipStream_t stream);

/*
 * Kernels behind the fold entry points.  Every one computes the same exact
 * integer dots and the same fold; they differ in how the work maps onto the
 * chip, and each meets the same accuracy bar on every shape it accepts.
 */
enum mmq_kernel {
    MMQ_KERNEL_AUTO = 0,  /* the entry point's own choice, by m, k and n (mmq_kernel_choice) */
    MMQ_KERNEL_DOT4 = 1,  /* vector-ALU 4-way int8 dots, weights streamed once; n <= 8 */
    MMQ_KERNEL_FEW = 2,   /* int8 MFMA on 16-token tiles, weights streamed once; n <= 64 (q4_K) */
    MMQ_KERNEL_F16 = 3,   /* binary16 MFMA on exact sc*q4 and q8 operands, 128-row tiles; any n */
    MMQ_KERNEL_I8 = 4,    /* int8 MFMA on 128 x 128 tiles with a three-operation fold; any n */
    MMQ_KERNEL_NARROW = 5, /* int8 4x4x4 MFMA, weights staged through LDS, streamed once; n <= 16 */
    MMQ_KERNEL_STREAM = 6  /* the narrow kernel's arithmetic, tokens held in LDS per workgroup of many
                              row tiles, weights streamed in 576-byte runs; n <= 16 */
};

/*
 * mmq_q4k_q8_fold - mmq_q4k_q8_fp32out (out_f16 == 0) or mmq_q4k_q8_f16out
 * (out_f16 != 0) on a kernel the caller names, for comparisons, benchmarks
 * and validation of every kernel on any shape.  With MMQ_KERNEL_AUTO it is
 * exactly that entry point.  A kernel outside its token range (DOT4 above 8
 * tokens, NARROW and STREAM above 16, FEW above 64) or an unknown id returns MMQ_ERR_KERNEL before any
 * HIP call; other arguments, errors and empty calls as for
 * mmq_q4k_q8_fp32out.
 */
int mmq_q4k_q8_fold(const void *w, int64_t m, int64_t k, const int8_t *q, const uint32_t *ds,
                    int64_t n, void *out, int out_f16, int kernel, hipStream_t stream);

/*
 * q6_K weights: the second k-quant format, named in the r31 page's closing
 * notes (its "q6_K line" of rounds); the pages print no layout, and the
 * GGUF k-quant super-block is taken: 256 weights in 210 bytes, rows
 * contiguous (row o's super-block b at byte (o*(k/256) + b)*210, so blocks
 * are only 2-byte aligned).  Block: ql[128] at 0 (low nibbles), qh[64] at 128
 * (2-bit high parts), sixteen int8 scales at 192 (one per 16 weights),
 * binary16 d at 208.  Weight 128h + 32g + l (h < 2, g < 4, l < 32) has the
 * code q = (nibble g/2 of ql[64h + 32(g%2) + l]) | (bits 2g..2g+1 of
 * qh[32h + l]) << 4 and the value d*sc[(128h + 32g + l)/16]*(q - 32).  The
 * same q8 activations as above.  There is no min term: with G = k/16 groups,
 *
 *   out[t][o] = sum_g d[o]*sc[o,g]*da[t,g/2]*D[t][o][g]
 *   D[t][o][g] = sum_{i<16} (q[o][16g+i] - 32) * q8[t][16g+i]
 *
 * Limits, errors, alignment (of w itself) and empty calls as above, with
 * m*(k/256)*210 below 2^40 and, for mmq_q6k_q8, n*m*(k/16) below 2^40.
 */

/*
 * mmq_q6k_q8 - exact per-group integer dot products of q6_K weights.
 *
 *   w    : q6_K super-blocks of W [m][k] (m*(k/256)*210 bytes), k % 256 == 0.
 *   q    : int8 [n][k] q8 activations.
 *   ds   : accepted for a uniform signature, not read (may be NULL).
 *   dots : int32 [n][m][k/16] (out), dots[t][o][g] = D[t][o][g], exact.
 */
int mmq_q6k_q8(const void *w, int64_t m, int64_t k, const int8_t *q, const uint32_t *ds,
               int64_t n, int32_t *dots, hipStream_t stream);

/*
 * mmq_q6k_q8_fp32out - the q6_K quantized matmul, float32 result.
 *
 *   w   : q6_K super-blocks of W [m][k], k % 256 == 0.
 *   q   : int8 [n][k];  ds : uint32 [n][k/32] (as written by q8_quantize_rows;
 *         only the binary16 da is read).
 *   out : float [n][m] (out), token-major.  The summation order is the
 *         kernel's; the same accuracy bar as mmq_q4k_q8_fp32out.
 */
int mmq_q6k_q8_fp32out(const void *w, int64_t m, int64_t k, const int8_t *q,
                       const uint32_t *ds, int64_t n, float *out, hipStream_t stream);

/*
 * mmq_q6k_q8_f16out - mmq_q6k_q8_fp32out's float32 result stored as binary16
 * (nearest-even, bit for bit the rounding of the float32 result of the same
 * inputs and binary), as mmq_q4k_q8_f16out is for q4_K.
 */
int mmq_q6k_q8_f16out(const void *w, int64_t m, int64_t k, const int8_t *q,
                      const uint32_t *ds, int64_t n, uint16_t *out, hipStream_t stream);

/*
 * mmq_q6k_q8_fold - mmq_q4k_q8_fold for q6_K weights: MMQ_KERNEL_AUTO,
 * MMQ_KERNEL_DOT4 (n <= 8), MMQ_KERNEL_F16 or MMQ_KERNEL_I8 (MMQ_KERNEL_FEW,
 * MMQ_KERNEL_NARROW and MMQ_KERNEL_STREAM return MMQ_ERR_KERNEL).
 */
int mmq_q6k_q8_fold(const void *w, int64_t m, int64_t k, const int8_t *q, const uint32_t *ds,
                    int64_t n, void *out, int out_f16, int kernel, hipStream_t stream);

/*
 * q4k_repack - load-time re-layout of q4_K weights (read by the few-token
 * dot4 kernel and the binary16-MFMA prefill kernel).
 * (The pages name a "load-time B pre-expansion" round and a scale
 * "predecode" round, r18 and r35 in the r17 and r31 pages' notes; the
 * layout is this library's.)
 *
 *   w  : q4_K super-blocks of W [m][k] (as for mmq_q4k_q8), k % 256 == 0.
 *   wr : ceil(m/16) * (k/256) * 2368 bytes (out), 16-byte aligned.  Rows in
 *        tiles of 16, one 2368-byte record per (tile, super-block), records
 *        tile-major.  Record: [0, 64) dword r = d | dmin << 16 of row r;
 *        [64, 320) dword 16p + r = sc[2p] | sc[2p+1] << 8 | m[2p] << 16 |
 *        m[2p+1] << 24 (the 6-bit fields as bytes); [320, 2368) the 16 bytes
 *        at 320 + 512p + 256h + 16r are qs bytes 32p + 16h .. +15 of row r
 *        (p < 4, h < 2, r < 16).  Rows past m are zero.
 * Pure byte work: the same values, 148 bytes per row and super-block
 * against 144.  Errors as for mmq_q4k_q8 (m == 0 is an empty call).
 */
int q4k_repack(const void *w, int64_t m, int64_t k, void *wr, hipStream_t stream);

/*
 * mmq_q4kr_q8_fp32out - mmq_q4k_q8_fp32out on repacked weights (wr from
 * q4k_repack of the same m, k).  For n <= 8 it runs the vector-ALU dot4
 * kernel with the same arithmetic, in the same order, as
 * mmq_q4k_q8_fp32out's kernel for that n, so the two results are equal bit
 * for bit.  Above 16 tokens, where the tiles fill the CUs (at least 160
 * tiles of 128 rows x 128 tokens) or n > 40, it runs the binary16-MFMA
 * kernel on the records, again with mmq_q4k_q8_fp32out's arithmetic and
 * order for that kernel (equal bit for bit where mmq_q4k_q8_fp32out takes it,
 * n > 64).  Other token counts run as slices of 8 tokens, each reading the
 * weights again.  Other arguments, errors and empty calls as for
 * mmq_q4k_q8_fp32out.
 */
int mmq_q4kr_q8_fp32out(const void *wr, int64_t m, int64_t k, const int8_t *q,
                        const uint32_t *ds, int64_t n, float *out, hipStream_t stream);

/*
 * q8_quantize_rows_tiled - q8_quantize_rows with the codes written as the
 * binary16 matrix-core operands of the prefill matmul, in its tile order (a
 * quantize-transpose pass ahead of the matmul: the r22 page, section 5,
 * names a later "quantize-transpose prepass" that changed the activation
 * side's layout at its root; this layout is the library's).  The codes and
 * scale words are q8_quantize_rows' bit for bit.
 *
 *   x  : float32 [n][k], k % 256 == 0.
 *   qt : ceil(n/128) * 128 * k binary16 values (out, 2 bytes each): tokens in
 *        tiles of 128, k in stages of 128, one block of 16 x 128 slots of 8
 *        values (32768 bytes) per (tile T, stage s), blocks tile-major.  Slot
 *        ((c*2 + h)*2 + g)*128 + tt of block (T, s) holds the codes of token
 *        128T + tt at k = 128s + 32c + 16g + 8h + e for e = 0,2,1,3,4,6,5,7
 *        (c < 4, h < 2, g < 2, tt < 128).  Tokens past n hold zeros.
 *   ds : uint32 [n][k/32] (out), as for q8_quantize_rows.
 * Errors as for q8_quantize_rows, except that k must be a multiple of 256
 * (MMQ_ERR_SHAPE) and n at most 2^31 - 128.
 */
int q8_quantize_rows_tiled(const float *x, int64_t n, int64_t k, uint16_t *qt, uint32_t *ds,
                           hipStream_t stream);

/*
 * q8_quantize_silu_mul_tiled - q8_quantize_silu_mul (h = SiLU(gate) * up,
 * never written) with the codes written as operand tiles, as
 * q8_quantize_rows_tiled does; codes and words bit for bit those of
 * q8_quantize_silu_mul.  Errors as for q8_quantize_rows_tiled, with `up`
 * checked beside `gate`.
 */
int q8_quantize_silu_mul_tiled(const float *gate, const float *up, int64_t n, int64_t k,
                               uint16_t *qt, uint32_t *ds, hipStream_t stream);

/*
 * mmq_q4k_q8t_fp32out / mmq_q4kr_q8t_fp32out - mmq_q4k_q8_fp32out (q4_K
 * rows) and mmq_q4kr_q8_fp32out (q4k_repack records) with the activations
 * as operand tiles (qt and ds from q8_quantize_rows_tiled of the same n and
 * k).  Every n runs the binary16-MFMA kernel, whose producers copy the tiles
 * straight into LDS instead of converting q8; the arithmetic and its order
 * are that kernel's, so the result equals mmq_q4k_q8_fp32out's bit for bit
 * wherever that takes the binary16 kernel (n > 64, and n > 32 where m
 * gives at least 160 tiles of 128 x 128).  Meant for prefill.
 * With few tokens it is faster than mmq_q4k_q8_fp32out only where m gives
 * many 128-row tiles (m = 28672 at n = 33); with few row tiles (m = 8192)
 * or n <= 8 the int8-code entry point is faster.  Other arguments, errors and
 * empty calls as for mmq_q4k_q8_fp32out / mmq_q4kr_q8_fp32out, and n at most
 * 2^31 - 128.
 */
int mmq_q4k_q8t_fp32out(const void *w, int64_t m, int64_t k, const uint16_t *qt,
                        const uint32_t *ds, int64_t n, float *out, hipStream_t stream);
int mmq_q4kr_q8t_fp32out(const void *wr, int64_t m, int64_t k, const uint16_t *qt,
                         const uint32_t *ds, int64_t n, float *out, hipStream_t stream);

/*
 * mmq_q6k_q8t_fp32out - mmq_q6k_q8_fp32out with the activations as operand
 * tiles (from q8_quantize_rows_tiled; one tiled quantization serves q4_K and
 * q6_K layers alike).  Every n runs the q6_K binary16-MFMA kernel, whose
 * producers copy the tiles straight into LDS; same arithmetic in the same
 * order, so the result equals mmq_q6k_q8_fp32out's bit for bit wherever that
 * takes the binary16 kernel (n > 8).  Other arguments, errors and empty
 * calls as for mmq_q6k_q8_fp32out, and n at most 2^31 - 128.
 */
int mmq_q6k_q8t_fp32out(const void *w, int64_t m, int64_t k, const uint16_t *qt,
                        const uint32_t *ds, int64_t n, float *out, hipStream_t stream);

/* Weight and activation formats of the fold entry points. */
enum mmq_format {
    MMQ_FORMAT_Q4K = 0,                /* mmq_q4k_q8_fp32out / _f16out */
    MMQ_FORMAT_Q4K_REPACKED = 1,       /* mmq_q4kr_q8_fp32out */
    MMQ_FORMAT_Q6K = 2,                /* mmq_q6k_q8_fp32out / _f16out */
    MMQ_FORMAT_Q4K_TILES = 3,          /* mmq_q4k_q8t_fp32out */
    MMQ_FORMAT_Q4K_REPACKED_TILES = 4, /* mmq_q4kr_q8t_fp32out */
    MMQ_FORMAT_Q6K_TILES = 5           /* mmq_q6k_q8t_fp32out */
};

/*
 * mmq_kernel_choice - the kernel (enum mmq_kernel, never MMQ_KERNEL_AUTO)
 * that the fold entry point of `format` runs for an m x k weight and n
 * tokens; host logic only, no HIP call.  MMQ_ERR_SHAPE for negative sizes or
 * k not a positive multiple of 256, MMQ_ERR_KERNEL for an unknown format.
 */
int mmq_kernel_choice(int format, int64_t m, int64_t k, int64_t n);

/* A static, human-readable name for a status code (never NULL). */
const char *mmq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* Q4Q8_MMQ_H */
