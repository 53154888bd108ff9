/*
 * oracle.c - plain, slow CPU reference for the q4_K (and q6_K) x q8 quantized
 * matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * What it computes (sources: the yusiwen.cn "minfer" pages, r31 "q-major sda
 * scale-read repack", sections 1-2, and r22 "qa8 XOR swizzle"; the workload
 * definition of the q8 activation quantizer):
 *
 *   q8 activations, per token t and 32-element block c:
 *       amax = max |x|;  da = amax / 127 (fp32);  q = round(x / da) (fp32
 *       divide, ties away from zero);  ssum = sum q;  the block's scale word is
 *       binary16(da) in the low 16 bits and ssum (two's complement i16) in the
 *       high 16 bits (r31 page, section 3.2: the read side takes the f16 from
 *       the low half and the signed short from the high half).
 *   block dots:  D[t][o][c] = sum_{i<32} q4[o][32c+i] * q8[t][32c+i]  (exact).
 *   output (the two-term rank-1 fold, r31 page sections 1-2):
 *       out[t][o] = sum_c (d*sc)[o,c]*da[t,c]*D[t][o][c]
 *                       - (dmin*m)[o,c]*da[t,c]*ssum[t,c]
 *     with da the binary16-decoded block scale, accumulated in float64 in
 *     chunk order.  Each product is exact in float64 (at most 45 significant
 *     bits), so only the additions round.
 *
 * The q4_K byte layout (144 bytes per 256 weights) is the GGUF k-quant
 * super-block: d, dmin binary16; twelve bytes of packed 6-bit (sc, m); 128
 * bytes of nibbles, low nibbles of bytes 32p..32p+31 = weights 64p..64p+31,
 * high nibbles = weights 64p+32..64p+63.
 *
 * q6_K weights (the second k-quant format; named in the r31 page's closing
 * notes, no layout printed): GGUF super-block of 210 bytes, signed 8-bit
 * scale per 16 weights, 6-bit codes q with weight d*sc*(q - 32).  Group dots
 * D[t][o][g] = sum_{i<16} (q - 32)*q8 (exact), output
 * sum_g d*sc[g]*da[t][g/2]*D in float64 in group order (no min term).
 *
 * Fused SiLU-gate quantize (oracle_q8_quantize_silu_mul): the quantizer applied
 * to h = float32(g*u / (1 + exp(-g))) evaluated in float64.
 *
 * Readings taken where the pages are silent: rounding ties go away from zero
 * (C roundf); q is computed from the fp32 da, the rescale uses the binary16
 * da; an all-zero block has da = 0, q = 0, ssum = 0; q is clamped to
 * [-127, 127] (a no-op for finite input).  Inputs are assumed finite.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 * (no fast-math, no hand SIMD).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ binary16
 * Conversions written from the IEEE 754 binary16 definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent field 0 = subnormal
 * (value = fraction * 2^-24), 31 = inf/NaN.
 */
double oracle_f16_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Round an fp32 value to the nearest binary16, ties to even, keeping
 * subnormals and overflowing to infinity. */
uint16_t oracle_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs((double)x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00u);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);                 /* a = f * 2^e2 with f in [0.5, 1) */
    int E = e2 - 1;                /* a in [2^E, 2^(E+1)) */
    if (E < -14)
        E = -14;                   /* subnormal range shares the quantum 2^-24 */
    const double quantum = ldexp(1.0, E - 10);
    const double n = rint(a / quantum);   /* exact scaling; rint = ties to even */
    uint32_t bits;
    if (n >= 1024.0)
        bits = ((uint32_t)(E + 15) << 10) + (uint32_t)(n - 1024.0);
    else
        bits = (uint32_t)n;        /* subnormal (E == -14) */
    if (bits >= 0x7c00u)
        bits = 0x7c00u;            /* overflow -> infinity */
    return (uint16_t)(sign | bits);
}

/* ------------------------------------------------------------ q8 quantizer */
int oracle_q8_quantize(const float *x, int64_t n, int64_t k, int8_t *q, uint32_t *ds)
{
    if (n < 0 || k < 0 || k % 32)
        return -1;
    const int64_t nb = k / 32;
    for (int64_t t = 0; t < n; t++) {
        for (int64_t c = 0; c < nb; c++) {
            const float *xb = x + t * k + c * 32;
            int8_t *qb = q + t * k + c * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; i++) {
                const float a = fabsf(xb[i]);
                if (a > amax)
                    amax = a;
            }
            int ssum = 0;
            uint16_t d16 = 0;
            if (amax == 0.0f) {
                for (int i = 0; i < 32; i++)
                    qb[i] = 0;
            } else {
                const float da = amax / 127.0f;
                for (int i = 0; i < 32; i++) {
                    float r = roundf(xb[i] / da);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    qb[i] = (int8_t)r;
                    ssum += qb[i];
                }
                d16 = oracle_f32_to_f16(da);
            }
            ds[t * nb + c] = (uint32_t)d16 | ((uint32_t)(uint16_t)(int16_t)ssum << 16);
        }
    }
    return 0;
}

/* ------------------------------------------------- fused SiLU-gate quantize */
/* The FFN down-projection input h = SiLU(gate) * up, quantized to q8 without
 * writing h (the pages' later "quantize-transpose prepass" moved activation
 * quantization into a prepass of its own; fusing the gate into it is this
 * library's reading).  h is defined as the float32 rounding of the float64
 * value  g*u / (1 + exp(-g)):  g*u is exact in float64 (two 24-bit
 * significands), then one IEEE add, one IEEE divide and the round to float32;
 * only exp() is a library function.  The quantization of h is exactly
 * oracle_q8_quantize. */
void oracle_silu_mul(const float *g, const float *u, int64_t count, float *h)
{
    for (int64_t i = 0; i < count; i++) {
        const double gd = (double)g[i];
        const double s = 1.0 + exp(-gd);
        h[i] = (float)(gd * (double)u[i] / s);
    }
}

int oracle_q8_quantize_silu_mul(const float *g, const float *u, int64_t n, int64_t k,
                                int8_t *q, uint32_t *ds)
{
    if (n < 0 || k < 0 || k % 32)
        return -1;
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
    for (int64_t t = 0; t < n; t++) {
        float row[k > 0 ? k : 1];
        oracle_silu_mul(g + t * k, u + t * k, k, row);
        rc |= oracle_q8_quantize(row, 1, k, q + t * k, ds + t * (k / 32));
    }
    return rc;
}

/* ------------------------------------------------------------ q4_K decoding */
/* Decode one 144-byte super-block into its fields. */
static void decode_block(const uint8_t *b, double *d, double *dmin,
                         int sc[8], int mn[8], int q[256])
{
    const uint16_t hd = (uint16_t)(b[0] | (b[1] << 8));
    const uint16_t hm = (uint16_t)(b[2] | (b[3] << 8));
    *d = oracle_f16_to_double(hd);
    *dmin = oracle_f16_to_double(hm);
    const uint8_t *s = b + 4;
    for (int j = 0; j < 8; j++) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            mn[j] = s[j + 4] & 63;
        } else {
            sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
    }
    const uint8_t *qs = b + 16;
    for (int p = 0; p < 4; p++) {
        for (int i = 0; i < 32; i++) {
            q[64 * p + i] = qs[32 * p + i] & 15;
            q[64 * p + 32 + i] = qs[32 * p + i] >> 4;
        }
    }
}

/* Unpack an m x k q4_K matrix into plain fields (for round-trip checks).
 * q: [m][k]; sc, mn: [m][k/32]; d, dmin: binary16 bits [m][k/256]. */
int oracle_q4k_unpack(const uint8_t *w, int64_t m, int64_t k, uint8_t *q,
                      uint8_t *sc, uint8_t *mn, uint16_t *d, uint16_t *dmin)
{
    if (m < 0 || k < 0 || k % 256)
        return -1;
    const int64_t S = k / 256;
    for (int64_t o = 0; o < m; o++) {
        for (int64_t b = 0; b < S; b++) {
            const uint8_t *blk = w + (o * S + b) * 144;
            double dd, dm;
            int s8[8], m8[8], q256[256];
            decode_block(blk, &dd, &dm, s8, m8, q256);
            d[o * S + b] = (uint16_t)(blk[0] | (blk[1] << 8));
            dmin[o * S + b] = (uint16_t)(blk[2] | (blk[3] << 8));
            for (int j = 0; j < 8; j++) {
                sc[o * (k / 32) + b * 8 + j] = (uint8_t)s8[j];
                mn[o * (k / 32) + b * 8 + j] = (uint8_t)m8[j];
            }
            for (int i = 0; i < 256; i++)
                q[o * k + b * 256 + i] = (uint8_t)q256[i];
        }
    }
    return 0;
}

/* ------------------------------------------------------------- block dots */
/* dots[t][o][c] = sum_{i<32} q4[o][32c+i] * q8[t][32c+i]  (int32, exact). */
int oracle_blockdots(const uint8_t *w, int64_t m, int64_t k, const int8_t *q8,
                     int64_t n, int32_t *dots)
{
    if (m < 0 || n < 0 || k < 0 || k % 256)
        return -1;
    const int64_t S = k / 256, C = k / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t o = 0; o < m; o++) {
        for (int64_t b = 0; b < S; b++) {
            double dd, dm;
            int sc[8], mn[8], q4[256];
            decode_block(w + (o * S + b) * 144, &dd, &dm, sc, mn, q4);
            for (int64_t t = 0; t < n; t++) {
                for (int j = 0; j < 8; j++) {
                    const int8_t *a = q8 + t * k + b * 256 + j * 32;
                    int32_t acc = 0;
                    for (int i = 0; i < 32; i++)
                        acc += q4[j * 32 + i] * a[i];
                    dots[(t * m + o) * C + b * 8 + j] = acc;
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------- load-time repack */
/* q4_K weights re-laid out for the few-token path (the pages' "load-time B
 * pre-expansion" and scale "predecode" rounds name the step, not a format;
 * this layout is the library's): rows in tiles of 16, one 2368-byte record
 * per (tile, super-block), records in tile-major order.  Record:
 *   [0, 64)      dword r:          d | dmin << 16 (binary16 bits) of row r
 *   [64, 320)    dword 16p + r:    sc[2p] | sc[2p+1] << 8 | m[2p] << 16 | m[2p+1] << 24
 *   [320, 2368)  bytes 320 + 512p + 256h + 16r + i:  qs byte 32p + 16h + i of row r
 * for pair p < 4, half h < 2, row r < 16, i < 16.  Rows past m are zero
 * (d = dmin = 0: they contribute nothing).  wr holds ceil(m/16)*(k/256)*2368
 * bytes. */
int oracle_q4k_repack(const uint8_t *w, int64_t m, int64_t k, uint8_t *wr)
{
    if (m < 0 || k < 0 || k % 256)
        return -1;
    const int64_t S = k / 256, tiles = (m + 15) / 16;
    memset(wr, 0, (size_t)(tiles * S * 2368));
    for (int64_t o = 0; o < m; o++) {
        const int64_t t = o / 16, r = o % 16;
        for (int64_t b = 0; b < S; b++) {
            const uint8_t *blk = w + (o * S + b) * 144;
            uint8_t *rec = wr + (t * S + b) * 2368;
            double dd, dm;
            int sc[8], mn[8], q4[256];
            decode_block(blk, &dd, &dm, sc, mn, q4);
            memcpy(rec + 4 * r, blk, 4);   /* d, dmin as stored */
            for (int p = 0; p < 4; p++) {
                uint8_t *sw = rec + 64 + 4 * (16 * p + r);
                sw[0] = (uint8_t)sc[2 * p];
                sw[1] = (uint8_t)sc[2 * p + 1];
                sw[2] = (uint8_t)mn[2 * p];
                sw[3] = (uint8_t)mn[2 * p + 1];
                for (int h = 0; h < 2; h++)
                    memcpy(rec + 320 + 512 * p + 256 * h + 16 * r, blk + 16 + 32 * p + 16 * h, 16);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------ q8 operand tiles */
/* The q8 codes laid out as binary16 matrix-core operands (the pages name a
 * later "quantize-transpose prepass" that changed the activation side's
 * layout at its root, r22 page, section 5; no layout is printed, this one is
 * the library's: the binary16 matmul kernel's LDS operand order).  Tokens in tiles of 128 and k in stages of 128: one block of
 * 16 x 128 slots of 8 binary16 values (32768 bytes) per (tile T, stage s),
 * blocks tile-major.  Slot ((c * 2 + h) * 2 + g) * 128 + tt of block (T, s)
 * holds the codes of token 128 T + tt at k = 128 s + 32 c + 16 g + 8 h + e for
 * e = 0, 2, 1, 3, 4, 6, 5, 7 (in that order); each code is exact in binary16.
 * Tokens past n hold zeros. */
int oracle_q8_tiles(const int8_t *q8, int64_t n, int64_t k, uint16_t *qt)
{
    static const int order[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    if (n < 0 || k < 0 || k % 128)
        return -1;
    const int64_t tiles = (n + 127) / 128, stages = k / 128;
    for (int64_t T = 0; T < tiles; T++)
        for (int64_t s = 0; s < stages; s++)
            for (int c = 0; c < 4; c++)
                for (int h = 0; h < 2; h++)
                    for (int g = 0; g < 2; g++)
                        for (int tt = 0; tt < 128; tt++) {
                            const int64_t row = (c * 2 + h) * 2 + g;
                            uint16_t *slot = qt + (((T * stages + s) * 16 + row) * 128 + tt) * 8;
                            const int64_t t = 128 * T + tt;
                            for (int e = 0; e < 8; e++) {
                                const int64_t kk = 128 * s + 32 * c + 16 * g + 8 * h + order[e];
                                slot[e] = t < n ? oracle_f32_to_f16((float)q8[t * k + kk]) : 0;
                            }
                        }
    return 0;
}

/* ----------------------------------------------------------------- output */
/* out[t][o] in float64, chunk order, from the two-term fold. */
int oracle_out_f64(const uint8_t *w, int64_t m, int64_t k, const int8_t *q8,
                   const uint32_t *ds, int64_t n, double *out)
{
    if (m < 0 || n < 0 || k < 0 || k % 256)
        return -1;
    const int64_t S = k / 256, C = k / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t o = 0; o < m; o++) {
        for (int64_t t = 0; t < n; t++)
            out[t * m + o] = 0.0;
        for (int64_t b = 0; b < S; b++) {
            double d, dmin;
            int sc[8], mn[8], q4[256];
            decode_block(w + (o * S + b) * 144, &d, &dmin, sc, mn, q4);
            for (int64_t t = 0; t < n; t++) {
                double acc = out[t * m + o];
                for (int j = 0; j < 8; j++) {
                    const int8_t *a = q8 + t * k + b * 256 + j * 32;
                    int32_t D = 0;
                    for (int i = 0; i < 32; i++)
                        D += q4[j * 32 + i] * a[i];
                    const uint32_t word = ds[t * C + b * 8 + j];
                    const double da = oracle_f16_to_double((uint16_t)(word & 0xffffu));
                    const int ssum = (int16_t)(uint16_t)(word >> 16);
                    const double main_term = (d * sc[j]) * da * (double)D;
                    const double corr_term = (dmin * mn[j]) * da * (double)ssum;
                    acc += main_term - corr_term;
                }
                out[t * m + o] = acc;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------ q6_K decoding */
/* q6_K (the second k-quant weight format; the pages name it, in the r31
 * page's closing notes, but print no layout).  The GGUF k-quant super-block
 * of 256 weights in 210 bytes: ql[128] low nibbles, qh[64] high bit pairs,
 * sixteen signed 8-bit scales (one per 16 weights), binary16 d.  Weight
 * e = 128h + 32g + l has the code
 *     q = (nibble g/2 of ql[64h + 32(g%2) + l]) | (bits 2g..2g+1 of qh[32h + l]) << 4
 * and the value d * sc[e/16] * (q - 32). */
static void decode_q6k_block(const uint8_t *b, double *d, int sc[16], int q[256])
{
    const uint8_t *ql = b, *qh = b + 128;
    *d = oracle_f16_to_double((uint16_t)(b[208] | (b[209] << 8)));
    for (int j = 0; j < 16; j++)
        sc[j] = (int8_t)b[192 + j];
    for (int h = 0; h < 2; h++)
        for (int g = 0; g < 4; g++)
            for (int l = 0; l < 32; l++) {
                const int lo = (ql[64 * h + 32 * (g & 1) + l] >> (4 * (g >> 1))) & 15;
                const int hi = (qh[32 * h + l] >> (2 * g)) & 3;
                q[128 * h + 32 * g + l] = lo | (hi << 4);
            }
}

/* Unpack an m x k q6_K matrix into plain fields (for round-trip checks).
 * q: [m][k] codes 0..63; sc: [m][k/16]; d: binary16 bits [m][k/256]. */
int oracle_q6k_unpack(const uint8_t *w, int64_t m, int64_t k, uint8_t *q,
                      int8_t *sc, uint16_t *d)
{
    if (m < 0 || k < 0 || k % 256)
        return -1;
    const int64_t S = k / 256;
    for (int64_t o = 0; o < m; o++) {
        for (int64_t b = 0; b < S; b++) {
            const uint8_t *blk = w + (o * S + b) * 210;
            double dd;
            int s16[16], q256[256];
            decode_q6k_block(blk, &dd, s16, q256);
            d[o * S + b] = (uint16_t)(blk[208] | (blk[209] << 8));
            for (int j = 0; j < 16; j++)
                sc[o * (k / 16) + b * 16 + j] = (int8_t)s16[j];
            for (int i = 0; i < 256; i++)
                q[o * k + b * 256 + i] = (uint8_t)q256[i];
        }
    }
    return 0;
}

/* Group dots: dots[t][o][g] = sum_{i<16} (q6[o][16g+i] - 32) * q8[t][16g+i]
 * (int32, exact; one value per 16-weight scale group). */
int oracle_q6k_dots(const uint8_t *w, int64_t m, int64_t k, const int8_t *q8,
                    int64_t n, int32_t *dots)
{
    if (m < 0 || n < 0 || k < 0 || k % 256)
        return -1;
    const int64_t S = k / 256, G = k / 16;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t o = 0; o < m; o++) {
        for (int64_t b = 0; b < S; b++) {
            double dd;
            int sc[16], q6[256];
            decode_q6k_block(w + (o * S + b) * 210, &dd, sc, q6);
            for (int64_t t = 0; t < n; t++) {
                for (int j = 0; j < 16; j++) {
                    const int8_t *a = q8 + t * k + b * 256 + j * 16;
                    int32_t acc = 0;
                    for (int i = 0; i < 16; i++)
                        acc += (q6[j * 16 + i] - 32) * a[i];
                    dots[(t * m + o) * G + b * 16 + j] = acc;
                }
            }
        }
    }
    return 0;
}

/* out[t][o] = sum_g d * sc[g] * da16[t][g/2] * D[t][o][g] in float64, in
 * group order.  Each product is exact in float64 (at most 11 + 8 + 11 + 17
 * significant bits), so only the additions round. */
int oracle_q6k_out_f64(const uint8_t *w, int64_t m, int64_t k, const int8_t *q8,
                       const uint32_t *ds, int64_t n, double *out)
{
    if (m < 0 || n < 0 || k < 0 || k % 256)
        return -1;
    const int64_t S = k / 256, C = k / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t o = 0; o < m; o++) {
        for (int64_t t = 0; t < n; t++)
            out[t * m + o] = 0.0;
        for (int64_t b = 0; b < S; b++) {
            double d;
            int sc[16], q6[256];
            decode_q6k_block(w + (o * S + b) * 210, &d, sc, q6);
            for (int64_t t = 0; t < n; t++) {
                double acc = out[t * m + o];
                for (int j = 0; j < 16; j++) {
                    const int8_t *a = q8 + t * k + b * 256 + j * 16;
                    int32_t D = 0;
                    for (int i = 0; i < 16; i++)
                        D += (q6[j * 16 + i] - 32) * a[i];
                    const uint32_t word = ds[t * C + b * 8 + j / 2];
                    const double da = oracle_f16_to_double((uint16_t)(word & 0xffffu));
                    acc += (d * sc[j]) * da * (double)D;
                }
                out[t * m + o] = acc;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------- threading */
void oracle_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
