/*
 * q4k_oracle.c -- plain, slow, obviously correct CPU oracle for the Q4_K
 * fused dequantize-and-multiply GEMV  y[b][r] = sum_c W[r][c] * x[b][c].
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path loads, links or
 * calls this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library; it has its own binary16 decode, its own 6-bit scale unpack and
 * its own nibble walk.  Build with -ffp-contract=off so that every float
 * operation below rounds exactly where it is written.
 *
 * What it follows (the pages are docs.rs source listings; cited by page title
 * and the function or doc comment the fact sits in):
 *  - memra-engine 0.83.1, src/f16_ffi.rs, extern block, doc comment of
 *    `memra_q4_K_dequant_f16`: a Q4_K tensor is a sequence of 144-byte
 *    superblocks; `ensure_f16_mirror`: a row of `in_f` weights holds
 *    in_f/256 superblocks of 144 bytes, so k must be a multiple of 256.
 *  - realizar 0.8.5, src/cuda/executor/uses.rs, doc of
 *    `batched_q4k_gemv_into`: weights are N x K/256 superblocks shared by the
 *    batch; the input is M x K row-major and the output M x N row-major.
 *  - The superblock field layout inside the 144 bytes is not printed on the
 *    pages.  It is the GGUF Q4_K layout (the format the pages' listings
 *    decode, by name):
 *    fp16 d at byte 0, fp16 dmin at byte 2, twelve bytes of packed 6-bit
 *    (scale, min) pairs for the eight 32-element sub-blocks at byte 4, and 128
 *    bytes of 4-bit quants at byte 16 where, in each 64-element chunk c, byte i
 *    holds element 64c+i in its low nibble and element 64c+32+i in its high
 *    nibble; each weight is w = d*sc_j*q - dmin*m_j.
 *  - The bit packing of the twelve scale bytes is not on the pages either;
 *    the reading taken is the GGUF K-quant packing (see oq_unpack_scales).
 *  - memra-engine 0.83.1, src/f16_ffi.rs, `f16_bits_to_f32` inside
 *    `ensure_f16_mirror`: binary16 decode keeping subnormals, infinities and
 *    NaN.  The decode below is written from the IEEE-754 binary16 definition.
 *
 * Pins (tests/, CPU only): exhaustive binary16 decode against numpy's
 * float16 conversion; exhaustive scale pack/unpack; one-hot layout brute
 * force; hand-computed golden superblocks; closed forms; exact dyadic dots;
 * quantizer round-trip; for the Q8 activations: exact round trips of
 * dyadic blocks, constant, zero, one-hot and mirrored blocks, the rounding
 * bound, non-finite blocks, and the Q8 GEMV against the f32 GEMV where the
 * quantized x is x itself; for Q6_K: a hand-computed golden superblock,
 * one-hot brute force over every element and code bit against an
 * independently written packer, every weight equal to the exact product of
 * its fields, closed forms, exact dyadic dots, special d, row strides; for
 * the fp16 mirror and GEMM: numpy's binary16 cast of the pinned weights,
 * integer-valued operands against exact integer products.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OQ_QK 256     /* elements per superblock */
#define OQ_SB 144     /* bytes per superblock    */

/* ---------------------------------------------------------------------------
 * binary16 -> binary32, from the definition:
 *   e == 0          : (-1)^s * 2^-14 * f/1024            (zero, subnormal)
 *   0 < e < 31      : (-1)^s * 2^(e-15) * (1 + f/1024)   (normal)
 *   e == 31, f == 0 : (-1)^s * inf
 *   e == 31, f != 0 : NaN
 * Every finite binary16 value is exactly representable in binary32, so the
 * double computation below followed by the cast is exact.
 * ------------------------------------------------------------------------- */
float oq_f16_to_f32(uint16_t h)
{
    const int s = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* 2^-14 * f / 2^10 */
    } else if (e == 31) {
        if (f == 0) {
            v = INFINITY;
        } else {
            v = NAN;
        }
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* 2^(e-15) * (1024+f) / 2^10 */
    }
    return (float)(s ? -v : v);
}

/* ---------------------------------------------------------------------------
 * binary32 -> binary16 with round-to-nearest-even, from the definition.  Used
 * only by the reference quantizer (the pages' own encoder rounds half up on
 * the normal path, so it is deliberately not the model here).
 * ------------------------------------------------------------------------- */
uint16_t oq_f32_to_f16_rne(float vf)
{
    double v = (double)vf;
    uint16_t sign = 0;
    if (signbit(v)) {
        sign = 0x8000;
        v = -v;
    }
    if (isnan(v)) {
        return (uint16_t)(sign | 0x7e00);
    }
    if (isinf(v)) {
        return (uint16_t)(sign | 0x7c00);
    }
    if (v == 0.0) {
        return sign;
    }
    /* subnormal range: multiples of 2^-24 below 2^-14 */
    if (v < ldexp(1.0, -14)) {
        double units = nearbyint(ldexp(v, 24));    /* RNE in the default mode */
        /* rounding up to 1024 units is exactly the smallest normal, 0x0400 */
        return (uint16_t)(sign | (uint16_t)units);
    }
    int ex;
    double fr = frexp(v, &ex);            /* v = fr * 2^ex, fr in [0.5, 1) */
    /* significand with 11 bits: 1024 <= sig < 2048, value = sig * 2^(ex-11) */
    double sig = nearbyint(ldexp(fr, 11));
    int e2 = ex - 11;
    if (sig == 2048.0) {                  /* carry out of the significand */
        sig = 1024.0;
        e2 += 1;
    }
    int biased = e2 + 10 + 15;            /* value = (sig/1024) * 2^(biased-15) */
    if (biased >= 31) {
        return (uint16_t)(sign | 0x7c00); /* overflow -> inf */
    }
    return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)((int)sig - 1024));
}

/* ---------------------------------------------------------------------------
 * The twelve scale bytes s[0..11] hold eight 6-bit scales sc_0..sc_7 and
 * eight 6-bit mins m_0..m_7 (GGUF K-quant packing):
 *   j < 4 : sc_j = low 6 bits of s[j],   m_j = low 6 bits of s[j+4]
 *   j >= 4: sc_j = low nibble of s[j+4]  plus (top two bits of s[j-4]) << 4
 *           m_j  = high nibble of s[j+4] plus (top two bits of s[j])   << 4
 * ------------------------------------------------------------------------- */
void oq_unpack_scales(const uint8_t s[12], uint8_t sc[8], uint8_t m[8])
{
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = (uint8_t)(s[j] % 64);
            m[j] = (uint8_t)(s[j + 4] % 64);
        } else {
            sc[j] = (uint8_t)((s[j + 4] % 16) + (s[j - 4] / 64) * 16);
            m[j] = (uint8_t)((s[j + 4] / 16) + (s[j] / 64) * 16);
        }
    }
}

/* The inverse, written from the same table one byte at a time (used by the
 * reference quantizer).  Inputs must be < 64. */
void oq_pack_scales(const uint8_t sc[8], const uint8_t m[8], uint8_t s[12])
{
    for (int j = 0; j < 4; ++j) {
        s[j] = (uint8_t)(sc[j] + (sc[j + 4] / 16) * 64);
        s[j + 4] = (uint8_t)(m[j] + (m[j + 4] / 16) * 64);
        s[j + 8] = (uint8_t)((sc[j + 4] % 16) + (m[j + 4] % 16) * 16);
    }
}

/* Sub-block index and 4-bit code of element e (0..255) of one superblock. */
static void oq_element_code(const uint8_t* qs, int e, int* j, int* q)
{
    const int c = e / 64;            /* 64-element chunk            */
    const int within = e % 64;
    const int hi = within / 32;      /* 0: low nibble, 1: high      */
    const int i = within % 32;       /* byte inside the chunk       */
    const uint8_t byte = qs[32 * c + i];
    *q = hi ? (byte / 16) : (byte % 16);
    *j = 2 * c + hi;                 /* sub-blocks in element order */
}

/* Dequantize one 144-byte superblock to 256 floats:
 *   w = fl32( fl32(d*sc_j) * q  -  fl32(dmin*m_j) )
 * d*sc_j, (d*sc_j)*q and dmin*m_j are exact in binary32 (at most 11+6+4
 * significant bits), so the only rounding is the subtraction. */
void oq_dequant_superblock(const uint8_t* blk, float* out)
{
    const float d = oq_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    const float dmin = oq_f16_to_f32((uint16_t)(blk[2] | (blk[3] << 8)));
    uint8_t sc[8], m[8];
    oq_unpack_scales(blk + 4, sc, m);
    const uint8_t* qs = blk + 16;
    for (int e = 0; e < OQ_QK; ++e) {
        int j, q;
        oq_element_code(qs, e, &j, &q);
        const float dsc = d * (float)sc[j];
        const float dm = dmin * (float)m[j];
        const float prod = dsc * (float)q;
        out[e] = prod - dm;
    }
}

static int oq_shape_ok(int64_t n, int64_t k)
{
    return n >= 0 && k > 0 && k % OQ_QK == 0;
}

/* out[r][c] for r < n, c < k. Returns 0, or -1 on a bad shape. */
int oq_dequant(const uint8_t* w, int64_t n, int64_t k, float* out)
{
    if (!oq_shape_ok(n, k)) {
        return -1;
    }
    const int64_t S = k / OQ_QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t s = 0; s < S; ++s) {
            oq_dequant_superblock(w + (r * S + s) * OQ_SB, out + r * k + s * OQ_QK);
        }
    }
    return 0;
}

/* One row: dequantize to f32, then for every vector b accumulate the dot in
 * f64 together with sum |w|*|x| (the tolerance scale). */
static void oq_row(const uint8_t* w, const float* x, int64_t k, int64_t m, int64_t r,
                   float* wrow, double* y_out, double* bound_out, int64_t ystride)
{
    const int64_t S = k / OQ_QK;
    for (int64_t s = 0; s < S; ++s) {
        oq_dequant_superblock(w + (r * S + s) * OQ_SB, wrow + s * OQ_QK);
    }
    for (int64_t b = 0; b < m; ++b) {
        const float* xb = x + b * k;
        double acc = 0.0, mag = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            const double wv = (double)wrow[c];
            const double xv = (double)xb[c];
            acc += wv * xv;
            mag += fabs(wv) * fabs(xv);
        }
        y_out[b * ystride] = acc;
        if (bound_out) {
            bound_out[b * ystride] = mag;
        }
    }
}

/* y[b][r], bound[b][r] for b < m, r < n (both m x n, row-major). */
int oq_gemv(const uint8_t* w, const float* x, int64_t n, int64_t k, int64_t m,
            double* y, double* bound)
{
    if (!oq_shape_ok(n, k) || m < 1) {
        return -1;
    }
    int bad = 0;
#pragma omp parallel
    {
        float* wrow = (float*)malloc((size_t)k * sizeof(float));
        if (!wrow) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < n; ++r) {
                oq_row(w, x, k, m, r, wrow, y + r, bound ? bound + r : NULL, n);
            }
            free(wrow);
        }
    }
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------------------
 * Simple reference quantizer (tests only): one row of k floats -> k/256
 * superblocks.  Per 32-element sub-block j: lo_j = min(0, min x), hi_j =
 * max x, step_j = (hi_j - lo_j)/15.  d = max_j step_j / 63 and
 * dmin = max_j(-lo_j) / 63, both rounded to binary16 (RNE).  sc_j and m_j are
 * nearbyint(step_j/d) and nearbyint(-lo_j/dmin), clamped to 0..63, and
 * q = clamp(nearbyint((x + dmin*m_j) / (d*sc_j)), 0, 15).
 * ------------------------------------------------------------------------- */
static int oq_clampi(double v, int lo, int hi)
{
    if (!(v >= lo)) {         /* also catches NaN */
        return lo;
    }
    if (v > hi) {
        return hi;
    }
    return (int)v;
}

int oq_quantize_row(const float* x, int64_t k, uint8_t* out)
{
    if (k <= 0 || k % OQ_QK != 0) {
        return -1;
    }
    const int64_t S = k / OQ_QK;
    for (int64_t s = 0; s < S; ++s) {
        const float* xs = x + s * OQ_QK;
        uint8_t* blk = out + s * OQ_SB;
        double step[8], neglo[8];
        double dmax = 0.0, mmax = 0.0;
        for (int j = 0; j < 8; ++j) {
            double lo = 0.0, hi = -INFINITY;
            for (int t = 0; t < 32; ++t) {
                /* sub-block j holds elements 64*(j/2) + 32*(j%2) + t */
                const double v = xs[64 * (j / 2) + 32 * (j % 2) + t];
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            if (hi < lo) hi = lo;
            step[j] = (hi - lo) / 15.0;
            neglo[j] = -lo;
            if (step[j] > dmax) dmax = step[j];
            if (neglo[j] > mmax) mmax = neglo[j];
        }
        const uint16_t dbits = oq_f32_to_f16_rne((float)(dmax / 63.0));
        const uint16_t mbits = oq_f32_to_f16_rne((float)(mmax / 63.0));
        const float d = oq_f16_to_f32(dbits);
        const float dmin = oq_f16_to_f32(mbits);
        uint8_t sc[8], mn[8];
        for (int j = 0; j < 8; ++j) {
            sc[j] = (uint8_t)(d > 0.0f ? oq_clampi(nearbyint(step[j] / d), 0, 63) : 0);
            mn[j] = (uint8_t)(dmin > 0.0f ? oq_clampi(nearbyint(neglo[j] / dmin), 0, 63) : 0);
        }
        blk[0] = (uint8_t)(dbits & 0xff);
        blk[1] = (uint8_t)(dbits >> 8);
        blk[2] = (uint8_t)(mbits & 0xff);
        blk[3] = (uint8_t)(mbits >> 8);
        oq_pack_scales(sc, mn, blk + 4);
        uint8_t* qs = blk + 16;
        memset(qs, 0, 128);
        for (int e = 0; e < OQ_QK; ++e) {
            const int c = e / 64, within = e % 64, hi = within / 32, i = within % 32;
            const int j = 2 * c + hi;
            const double dsc = (double)d * sc[j];
            const double dm = (double)dmin * mn[j];
            int q = 0;
            if (dsc > 0.0) {
                q = oq_clampi(nearbyint(((double)xs[e] + dm) / dsc), 0, 15);
            }
            qs[32 * c + i] = (uint8_t)(qs[32 * c + i] | (hi ? q * 16 : q));
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Q8 activations, for the pages' integer-dot variant (realizar 0.8.5,
 * src/cuda/executor/layers/modules_utilities.rs, `preload_hw_dp4a_modules`:
 * a Q8 quantize kernel for every GEMV input length, feeding the DP4A Q4_K
 * GEMV).  The pages name the kernels only; the block format is the reading
 * taken: blocks of 32 consecutive elements (one Q4_K sub-block), one f32
 * scale d = amax / 127 with amax the largest |x| of the block (NaN when the
 * block holds a NaN), and codes q = the nearest-even integer of x * (127 /
 * amax), that product and quotient rounded to f32; q = 0 where amax is 0 or
 * not a number, or where the product is not finite.
 * ------------------------------------------------------------------------- */
int oq_quantize_q8(const float* x, int64_t k, int8_t* q, float* d)
{
    if (k <= 0 || k % 32 != 0) {
        return -1;
    }
    for (int64_t b = 0; b < k / 32; ++b) {
        const float* xb = x + 32 * b;
        float amax = 0.0f;
        int has_nan = 0;
        for (int t = 0; t < 32; ++t) {
            const float a = fabsf(xb[t]);
            if (a != a) {
                has_nan = 1;
            } else if (a > amax) {
                amax = a;
            }
        }
        if (has_nan) {
            amax = NAN;
        }
        const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        d[b] = amax / 127.0f;
        for (int t = 0; t < 32; ++t) {
            const float v = xb[t] * inv;
            q[32 * b + t] = (int8_t)(isfinite(v) ? (int)rintf(v) : 0);
        }
    }
    return 0;
}

/* The GEMV against Q8 activations: y[b][r] = sum_c w[r][c] * xq[b][c] and
 * bound[b][r] = sum_c |w[r][c]| |xq[b][c]| in f64, where xq = d * q (exact
 * in f64) for the block of c.  q: m x k codes, d: m x k/32 scales. */
int oq_gemv_q8(const uint8_t* w, const int8_t* q, const float* d, int64_t n, int64_t k,
               int64_t m, double* y, double* bound)
{
    if (!oq_shape_ok(n, k) || m < 1) {
        return -1;
    }
    int bad = 0;
#pragma omp parallel
    {
        float* wrow = (float*)malloc((size_t)k * sizeof(float));
        if (!wrow) {
#pragma omp atomic write
            bad = 1;
        } else {
            const int64_t S = k / OQ_QK;
#pragma omp for schedule(static)
            for (int64_t r = 0; r < n; ++r) {
                for (int64_t s = 0; s < S; ++s) {
                    oq_dequant_superblock(w + (r * S + s) * OQ_SB, wrow + s * OQ_QK);
                }
                for (int64_t b = 0; b < m; ++b) {
                    double acc = 0.0, mag = 0.0;
                    for (int64_t c = 0; c < k; ++c) {
                        const double wv = (double)wrow[c];
                        const double xv = (double)d[b * (k / 32) + c / 32] * (double)q[b * k + c];
                        acc += wv * xv;
                        mag += fabs(wv) * fabs(xv);
                    }
                    y[b * n + r] = acc;
                    if (bound) {
                        bound[b * n + r] = mag;
                    }
                }
            }
            free(wrow);
        }
    }
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------------------
 * Q6_K, the other block format of the decode loop (realizar 0.8.5,
 * q4k_gemv_cached.rs, doc of `q6k_gemv_cached_async`: the same GEMV over
 * Q6_K weights, used for an LM head stored as Q6_K; memra-engine 0.83.1,
 * src/f16_ffi.rs, doc of `memra_q6_K_dequant_f16` and `ensure_f16_mirror`:
 * 210-byte superblocks of 256 weights, in_f / 256 of them per row).
 * The field layout inside the 210 bytes is not printed on the pages; the
 * reading taken is the GGUF Q6_K layout:
 *   bytes   0..127  ql: the low four bits of the codes,
 *   bytes 128..191  qh: the high two bits,
 *   bytes 192..207  sixteen signed 8-bit scales, scale s for elements
 *                   16 s .. 16 s + 15,
 *   bytes 208..209  fp16 d (little-endian).
 * Element e = 128 h + 32 t + l (h = 0, 1; t = 0..3; l = 0..31) takes its low
 * bits from ql byte 64 h + 32 (t % 2) + l (the low nibble for t < 2, the high
 * one for t >= 2) and its high bits from bits 2 t, 2 t + 1 of qh byte
 * 32 h + l; its code q is 0..63 and its weight w = d * sc * (q - 32).
 * ------------------------------------------------------------------------- */
#define OQ6_SB 210

/* code (0..63) and scale index of element e (0..255) of a Q6_K superblock */
static void oq6_element_code(const uint8_t* blk, int e, int* s, int* q)
{
    const int h = e / 128;
    const int t = (e % 128) / 32;
    const int l = e % 32;
    const uint8_t lo_byte = blk[64 * h + 32 * (t % 2) + l];
    const uint8_t hi_byte = blk[128 + 32 * h + l];
    const int lo = (t < 2) ? (lo_byte % 16) : (lo_byte / 16);
    const int hi = (hi_byte >> (2 * t)) % 4;
    *q = lo + 16 * hi;
    *s = e / 16;
}

/* Dequantize one 210-byte superblock to 256 floats: w = (d * sc) * (q - 32).
 * d has at most 11 significant bits, |sc| <= 128 and |q - 32| <= 32, so both
 * products are exact in binary32 (at most 11 + 7 + 5 significant bits, far
 * from overflow and underflow): every weight is the exact value of its
 * fields, with no rounding at all. */
void oq6_dequant_superblock(const uint8_t* blk, float* out)
{
    const float d = oq_f16_to_f32((uint16_t)(blk[208] | (blk[209] << 8)));
    for (int e = 0; e < OQ_QK; ++e) {
        int s, q;
        oq6_element_code(blk, e, &s, &q);
        const float sc = (float)(int8_t)blk[192 + s];
        const float dsc = d * sc;
        out[e] = dsc * (float)(q - 32);
    }
}

/* Rows of k / 256 superblocks, row r starting at byte r * row_stride
 * (row_stride >= 210 k / 256).  Returns 0, or -1 on a bad shape. */
static int oq6_shape_ok(int64_t n, int64_t k, int64_t row_stride)
{
    return oq_shape_ok(n, k) && row_stride >= (k / OQ_QK) * OQ6_SB;
}

/* out[r][c] for r < n, c < k. */
int oq6_dequant(const uint8_t* w, int64_t n, int64_t k, int64_t row_stride, float* out)
{
    if (!oq6_shape_ok(n, k, row_stride)) {
        return -1;
    }
    const int64_t S = k / OQ_QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t s = 0; s < S; ++s) {
            oq6_dequant_superblock(w + r * row_stride + s * OQ6_SB, out + r * k + s * OQ_QK);
        }
    }
    return 0;
}

/* y[b][r] = sum_c W[r][c] x[b][c] and bound[b][r] = sum_c |W[r][c]| |x[b][c]|,
 * in f64 over the f32 weights, for b < m (both m x n, row-major). */
int oq6_gemv(const uint8_t* w, const float* x, int64_t n, int64_t k, int64_t row_stride,
             int64_t m, double* y, double* bound)
{
    if (!oq6_shape_ok(n, k, row_stride) || m < 1) {
        return -1;
    }
    int bad = 0;
#pragma omp parallel
    {
        float* wrow = (float*)malloc((size_t)k * sizeof(float));
        if (!wrow) {
#pragma omp atomic write
            bad = 1;
        } else {
            const int64_t S = k / OQ_QK;
#pragma omp for schedule(static)
            for (int64_t r = 0; r < n; ++r) {
                for (int64_t s = 0; s < S; ++s) {
                    oq6_dequant_superblock(w + r * row_stride + s * OQ6_SB, wrow + s * OQ_QK);
                }
                for (int64_t b = 0; b < m; ++b) {
                    const float* xb = x + b * k;
                    double acc = 0.0, mag = 0.0;
                    for (int64_t c = 0; c < k; ++c) {
                        const double wv = (double)wrow[c];
                        const double xv = (double)xb[c];
                        acc += wv * xv;
                        mag += fabs(wv) * fabs(xv);
                    }
                    y[b * n + r] = acc;
                    if (bound) {
                        bound[b * n + r] = mag;
                    }
                }
            }
            free(wrow);
        }
    }
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------------------
 * The fp16 mirror and the prefill GEMM beside the decode path (memra-engine
 * 0.83.1, src/f16_ffi.rs: docs of `memra_q4_K_dequant_f16` and
 * `memra_q6_K_dequant_f16` -- GGUF superblocks to a row-major fp16 mirror
 * built at load time; `memra_f16_cvt` -- the f32 activations to fp16;
 * `memra_f16_pp_gemm` / `try_f16_gemm` -- y[m, out] = x[m, in] @ (fp16 W)^T
 * with f32 accumulation).  The reading taken: a mirror element is the f32
 * weight (as oq_dequant / oq6_dequant give it) rounded to binary16 to
 * nearest-even (oq_f32_to_f16_rne), an activation likewise; the reference
 * GEMM is the exact dot product of the two binary16 operands, in f64.
 * ------------------------------------------------------------------------- */

/* out[i] = binary16 bits of x[i], round to nearest even. */
void oq_f16_cvt(const float* x, int64_t count, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        out[i] = oq_f32_to_f16_rne(x[i]);
    }
}

/* The fp16 mirror of n rows of Q4_K (fmt 4, dense rows) or Q6_K (fmt 6,
 * rows at row_stride bytes): out[r*k + c] = binary16 of W[r][c]. */
int oq_mirror_f16(const uint8_t* w, int fmt, int64_t n, int64_t k, int64_t row_stride,
                  uint16_t* out)
{
    if (!oq_shape_ok(n, k) || (fmt != 4 && fmt != 6)) {
        return -1;
    }
    if (fmt == 6 && row_stride < (k / OQ_QK) * OQ6_SB) {
        return -1;
    }
    const int64_t S = k / OQ_QK;
    int bad = 0;
#pragma omp parallel
    {
        float* wrow = (float*)malloc((size_t)k * sizeof(float));
        if (!wrow) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < n; ++r) {
                for (int64_t s = 0; s < S; ++s) {
                    if (fmt == 4) {
                        oq_dequant_superblock(w + (r * S + s) * OQ_SB, wrow + s * OQ_QK);
                    } else {
                        oq6_dequant_superblock(w + r * row_stride + s * OQ6_SB, wrow + s * OQ_QK);
                    }
                }
                for (int64_t c = 0; c < k; ++c) {
                    out[r * k + c] = oq_f32_to_f16_rne(wrow[c]);
                }
            }
            free(wrow);
        }
    }
    return bad ? -2 : 0;
}

/* y[b][r] = sum_c W16[r][c] * X16[b][c] and bound[b][r] = sum_c |W16||X16|,
 * exactly in f64 (each product of two binary16 values is exact), for the
 * fp16 mirror w16 (n x k) and fp16 activations x16 (m x k). */
int oq_f16_gemm(const uint16_t* w16, const uint16_t* x16, int64_t m, int64_t n, int64_t k,
                double* y, double* bound)
{
    if (m < 1 || n < 1 || k < 1) {
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t b = 0; b < m; ++b) {
            double acc = 0.0, mag = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                const double wv = (double)oq_f16_to_f32(w16[r * k + c]);
                const double xv = (double)oq_f16_to_f32(x16[b * k + c]);
                acc += wv * xv;
                mag += fabs(wv) * fabs(xv);
            }
            y[b * n + r] = acc;
            if (bound) {
                bound[b * n + r] = mag;
            }
        }
    }
    return 0;
}

int oq_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oq_set_num_threads(int t)
{
#ifdef _OPENMP
    if (t > 0) {
        omp_set_num_threads(t);
    }
#else
    (void)t;
#endif
}
