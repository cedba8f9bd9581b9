/*
 * qmm_oracle.c -- the reference CPU implementation of y = x . W^T for GGUF
 * block-quantized weights W.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load it.  It shares no source, header, table or helper
 * with the HIP library, and the library never calls it.
 *
 * What it computes (plain definition, no blocking, fusion or reordering):
 *   1. Wd[n][k]: the exact real value of every weight element, decoded
 *      element by element from the block bytes by the per-kind rule below,
 *      held in IEEE binary64.  Every product below is exact in binary64
 *      (an f16 scale has an 11-bit significand and the integer factors have
 *      at most 8 bits each), and the one subtraction of the kinds that carry
 *      a minimum is exact as long as the two terms' exponents are within
 *      ~29 binades of each other, which every generated input satisfies.
 *   2. y[m][n] = sum_k Wd[n][k] * x[m][k], accumulated in binary64 with k
 *      ascending.
 *   3. bound[m][n] = sum_k |Wd[n][k]| * |x[m][k]|, the scale of the
 *      tolerance |y_gpu - y| <= 1e-3 * bound + 1e-6.
 *
 * Each element is evaluated with IEEE semantics in the order the format
 * names its factors, scale first: (d * sc) * q - dmin * m.  The sign of an
 * exact zero therefore follows binary arithmetic (for instance MXFP4 code 8
 * is -0.0 and a negative Q6_K scale times a zero code is -0.0).
 *
 * Sources (page titles as printed):
 *   [ferrox-mm]  docs.rs ferrox-cuda 0.21.0, src/mul_mm.rs
 *   [ferrox-cb]  docs.rs ferrox-cuda 0.20.0, src/mul_mm_kinds/codebook.rs
 *   [vulkore]    redgpu/Vulkore, examples/llm/quant_test.cpp
 * The block layouts of Q2_K, Q3_K and Q5_K are not printed on those pages;
 * they follow the public GGUF block definitions (parity unpinned by the
 * pages for Q2_K and Q3_K; Q5_K is tied to Q4_K by a cross-format test).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* GGUF type ids of the eleven kinds. */
enum {
    OK_Q4_0 = 2,
    OK_Q5_0 = 6,
    OK_Q8_0 = 8,
    OK_Q2_K = 10,
    OK_Q3_K = 11,
    OK_Q4_K = 12,
    OK_Q5_K = 13,
    OK_Q6_K = 14,
    OK_IQ4_NL = 20,
    OK_IQ4_XS = 23,
    OK_MXFP4 = 39
};

/* Bytes and elements of one block, per kind.  Returns 0 on success, -1 for a
 * kind this oracle does not know. */
int oracle_block_geometry(int kind, int *block_bytes, int *block_elems)
{
    int b, e;
    switch (kind) {
    case OK_Q8_0:   b = 34;  e = 32;  break; /* f16 d + 32 int8            */
    case OK_Q4_0:   b = 18;  e = 32;  break; /* f16 d + 16 B of nibbles     */
    case OK_Q5_0:   b = 22;  e = 32;  break; /* f16 d + u32 qh + 16 B       */
    case OK_Q2_K:   b = 84;  e = 256; break; /* 16 scales + 64 qs + d, dmin */
    case OK_Q3_K:   b = 110; e = 256; break; /* 32 hmask + 64 qs + 12 + d   */
    case OK_Q4_K:   b = 144; e = 256; break; /* d, dmin, 12 scales, 128 qs  */
    case OK_Q5_K:   b = 176; e = 256; break; /* d, dmin, 12, 32 qh, 128 qs  */
    case OK_Q6_K:   b = 210; e = 256; break; /* 128 ql, 64 qh, 16 sc, d     */
    case OK_IQ4_NL: b = 18;  e = 32;  break; /* f16 d + 16 B of codes       */
    case OK_IQ4_XS: b = 136; e = 256; break; /* d, scales_h, scales_l, 128  */
    case OK_MXFP4:  b = 17;  e = 32;  break; /* E8M0 byte + 16 B of codes   */
    default: return -1;
    }
    if (block_bytes) *block_bytes = b;
    if (block_elems) *block_elems = e;
    return 0;
}

/* IEEE 754 binary16 -> real: sign, 5 exponent bits (bias 15), 10 fraction
 * bits; exponent 0 is zero/subnormal (f * 2^-24), exponent 31 is Inf/NaN. */
static double binary16_value(unsigned h)
{
    const unsigned s = (h >> 15) & 1u;
    const unsigned e = (h >> 10) & 31u;
    const unsigned f = h & 1023u;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024u + f), (int)e - 25);
    return s ? -v : v;
}

/* OCP MX v1.0 E8M0 scale: 2^(e - 127).  e = 255 is NaN in that spec. */
static double e8m0_value(unsigned e)
{
    if (e == 255u) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* The 16-entry non-linear codebook shared by IQ4_NL and IQ4_XS
 * ([ferrox-cb], KVALUES_IQ4NL). */
static const double IQ4_VALUES[16] = {
    -127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113
};

/* E2M1 (sign, 2 exponent bits, 1 mantissa bit) values, code 0 first
 * ([ferrox-cb], KVALUES_MXFP4).  Code 8 is negative zero. */
static const double E2M1_VALUES[16] = {
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0
};

static unsigned u16_le(const uint8_t *p) { return (unsigned)p[0] | ((unsigned)p[1] << 8); }

static uint32_t u32_le(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* Two's-complement byte. */
static int int8_of(uint8_t b) { return b < 128 ? (int)b : (int)b - 256; }

/* Element t (0..31) of a 16-byte run of 4-bit codes: the low nibble of byte
 * t for t < 16, the high nibble of byte t - 16 otherwise ([ferrox-cb], the
 * IQ4_NL row; the same packing serves Q4_0, Q5_0, MXFP4 and each IQ4_XS
 * group). */
static unsigned split_nibble(const uint8_t *q, int t)
{
    return t < 16 ? (q[t] & 15u) : (unsigned)(q[t - 16] >> 4);
}

/* The 6-bit scale and minimum of 32-element group j (0..7) of a Q4_K/Q5_K
 * super-block, packed in 12 bytes ([vulkore], ref::q4k_scale_min). */
static void k4_scale_min(const uint8_t *s, int j, int *sc, int *mn)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *mn = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* The exact value of element r of the block at b. */
static double element_value(int kind, const uint8_t *b, int r)
{
    switch (kind) {
    case OK_Q8_0: {
        /* [vulkore] ref::q8_0: w = d * int8. */
        const double d = binary16_value(u16_le(b));
        return d * (double)int8_of(b[2 + r]);
    }
    case OK_Q4_0: {
        /* 18 B: f16 d then 32 nibbles in split order; w = d * (q - 8). */
        const double d = binary16_value(u16_le(b));
        return d * (double)((int)split_nibble(b + 2, r) - 8);
    }
    case OK_Q5_0: {
        /* [vulkore] ref::q5_0: bit r of the u32 qh is the fifth bit of
         * element r; w = d * (q - 16). */
        const double d = binary16_value(u16_le(b));
        const uint32_t qh = u32_le(b + 2);
        const unsigned q = split_nibble(b + 6, r) | (((qh >> r) & 1u) << 4);
        return d * (double)((int)q - 16);
    }
    case OK_Q4_K: {
        /* [vulkore] ref::q4_k: 64-element chunks; within a chunk the first
         * 32 elements are the low nibbles of its 32 bytes, the next 32 the
         * high nibbles; w = d*sc*q - dmin*m per 32-element group. */
        const double d = binary16_value(u16_le(b));
        const double dmin = binary16_value(u16_le(b + 2));
        int sc, mn;
        k4_scale_min(b + 4, r / 32, &sc, &mn);
        const uint8_t byte = b[16 + (r / 64) * 32 + r % 32];
        const unsigned q = (r % 64) < 32 ? (byte & 15u) : (unsigned)(byte >> 4);
        return d * (double)sc * (double)q - dmin * (double)mn;
    }
    case OK_Q5_K: {
        /* Public GGUF layout: d, dmin, the Q4_K 12-byte scale/min pack,
         * qh[32], qs[128].  Low four bits as Q4_K; the fifth bit of element
         * r is bit r/32 of qh[r % 32]. */
        const double d = binary16_value(u16_le(b));
        const double dmin = binary16_value(u16_le(b + 2));
        int sc, mn;
        k4_scale_min(b + 4, r / 32, &sc, &mn);
        const uint8_t byte = b[48 + (r / 64) * 32 + r % 32];
        const unsigned lo = (r % 64) < 32 ? (byte & 15u) : (unsigned)(byte >> 4);
        const unsigned q = lo | (((unsigned)(b[16 + r % 32] >> (r / 32)) & 1u) << 4);
        return d * (double)sc * (double)q - dmin * (double)mn;
    }
    case OK_Q6_K: {
        /* [vulkore] ref::q6_k: two 128-element halves, each four
         * interleaved 32-element quarters; w = d * sc * (q - 32). */
        const int h = r / 128, u = r % 128, l = u % 32, g = u / 32;
        const uint8_t byte = b[64 * h + l + 32 * (g & 1)];
        const unsigned lo = g < 2 ? (byte & 15u) : (unsigned)(byte >> 4);
        const unsigned hi = ((unsigned)b[128 + 32 * h + l] >> (2 * g)) & 3u;
        const int q = (int)(lo | (hi << 4)) - 32;
        const int sc = int8_of(b[192 + 8 * h + l / 16 + 2 * g]);
        const double d = binary16_value(u16_le(b + 208));
        return d * (double)sc * (double)q;
    }
    case OK_Q2_K: {
        /* Public GGUF layout: scales[16] (low nibble scale, high nibble
         * min, one byte per 16 elements), qs[64] (2-bit codes), d, dmin.
         * Element r: half n = r/128, shift 2*((r%128)/32), byte 32n + r%32. */
        const int n = r / 128, j = (r % 128) / 32, l = r % 32;
        const unsigned q = ((unsigned)b[16 + 32 * n + l] >> (2 * j)) & 3u;
        const unsigned s = b[r / 16];
        const double d = binary16_value(u16_le(b + 80));
        const double dmin = binary16_value(u16_le(b + 82));
        return d * (double)(s & 15u) * (double)q - dmin * (double)(s >> 4);
    }
    case OK_Q3_K: {
        /* Public GGUF layout: hmask[32], qs[64], 12 bytes of 6-bit scales,
         * d.  The 2-bit code is placed as in Q2_K; the high-mask bit
         * 4n + j of hmask[r % 32] clear means "subtract 4".  Scale i = r/16
         * has its low four bits in byte i (i < 8, low nibble) or byte i - 8
         * (high nibble), its top two bits at bits 2*(i/4) of byte 8 + i%4,
         * and is used as (scale - 32). */
        const int n = r / 128, j = (r % 128) / 32, l = r % 32;
        const int q2 = (int)(((unsigned)b[32 + 32 * n + l] >> (2 * j)) & 3u);
        const int hbit = ((unsigned)b[l] >> (4 * n + j)) & 1u;
        const int q = q2 - (hbit ? 0 : 4);
        const int i = r / 16;
        const uint8_t *sc = b + 96;
        const int low4 = i < 8 ? (sc[i] & 15) : (sc[i - 8] >> 4);
        const int high2 = (sc[8 + i % 4] >> (2 * (i / 4))) & 3;
        const double d = binary16_value(u16_le(b + 108));
        return d * (double)((low4 | (high2 << 4)) - 32) * (double)q;
    }
    case OK_IQ4_NL: {
        /* [ferrox-cb] IQ4_NL row: w = d * table[code]. */
        const double d = binary16_value(u16_le(b));
        return d * IQ4_VALUES[split_nibble(b + 2, r)];
    }
    case OK_IQ4_XS: {
        /* [ferrox-cb] IQ4_XS row: eight 32-element groups; group ib's 6-bit
         * scale is nibble (ib & 1) of scales_l[ib / 2] plus bits 2*ib of
         * scales_h as its top two bits; w = d * (ls - 32) * table[code]. */
        const double d = binary16_value(u16_le(b));
        const unsigned scales_h = u16_le(b + 2);
        const int ib = r / 32, t = r % 32;
        const unsigned ls = (((unsigned)b[4 + ib / 2] >> (4 * (ib & 1))) & 15u) |
                            (((scales_h >> (2 * ib)) & 3u) << 4);
        const unsigned code = split_nibble(b + 8 + 16 * ib, t);
        return d * (double)((int)ls - 32) * IQ4_VALUES[code];
    }
    case OK_MXFP4: {
        /* [ferrox-cb] MXFP4 row: E8M0 byte, then 32 E2M1 codes packed as
         * IQ4_NL packs its block; w = 2^(e-127) * e2m1[code]. */
        return e8m0_value(b[0]) * E2M1_VALUES[split_nibble(b + 1, r)];
    }
    default:
        return NAN;
    }
}

/* Decodes n_elems consecutive elements (a whole number of blocks) of W. */
int oracle_dequant(int kind, const uint8_t *W, int64_t n_elems, double *out)
{
    int bb, be;
    if (oracle_block_geometry(kind, &bb, &be) != 0) return -1;
    if (n_elems < 0 || n_elems % be != 0) return -2;
    for (int64_t i = 0; i < n_elems; ++i)
        out[i] = element_value(kind, W + (i / be) * bb, (int)(i % be));
    return 0;
}

static void decode_row(int kind, const uint8_t *row, int64_t K, int bb, int be, double *w)
{
    for (int64_t k = 0; k < K; ++k)
        w[k] = element_value(kind, row + (k / be) * bb, (int)(k % be));
}

/*
 * y = x . W^T for the selected rows of W.
 *   W        row n starts at W + n * row_bytes; row_bytes = (K / be) * bb.
 *   rows     NULL: rows 0 .. n_sel-1; else n_sel row indices.
 *   X        [M][K] binary64 activations (exact copies of the f32/f16 inputs).
 *   Y, B     [M][n_sel]: y and the bound sum |w||x| (B may be NULL).
 *   threads  OpenMP threads (<= 0: the runtime default).
 */
int oracle_matmul(int kind, const uint8_t *W, int64_t K, const int64_t *rows, int64_t n_sel,
                  const double *X, int64_t M, double *Y, double *B, int threads)
{
    int bb, be;
    if (oracle_block_geometry(kind, &bb, &be) != 0) return -1;
    if (K <= 0 || K % be != 0 || n_sel < 0 || M < 0) return -2;
    const int64_t row_bytes = (K / be) * bb;
#ifdef _OPENMP
    /* The count applies to this region only (omp_set_num_threads would
     * change every later call's default). */
    const int nt = threads > 0 ? threads : omp_get_max_threads();
#else
    (void)threads;
#endif
    int failed = 0;
#pragma omp parallel num_threads(nt)
    {
        double *w = (double *)malloc((size_t)K * sizeof(double));
        if (!w) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < n_sel; ++i) {
            if (!w) continue;
            const int64_t n = rows ? rows[i] : i;
            decode_row(kind, W + n * row_bytes, K, bb, be, w);
            for (int64_t m = 0; m < M; ++m) {
                const double *x = X + m * K;
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    acc += w[k] * x[k];
                    mag += fabs(w[k]) * fabs(x[k]);
                }
                Y[m * n_sel + i] = acc;
                if (B) B[m * n_sel + i] = mag;
            }
        }
        free(w);
    }
    return failed ? -3 : 0;
}

/*
 * Routed expert products: for every token t < M and slot s < topk, with
 * e = ids[t * topk + s], y[t][s][n] = sum_k W_e[n][k] * x[k] where x is
 * X[t] (x_per_slot == 0, X is [M][K]) or X[t][s] (x_per_slot != 0, X is
 * [M][topk][K]).  W holds E experts of N rows each, back to back.
 * Only the output rows listed in `rows` (n_sel of them; NULL: all N) are
 * computed; Y and B are [M][topk][n_sel].
 */
int oracle_moe(int kind, const uint8_t *W, int64_t E, int64_t N, int64_t K, const int32_t *ids,
               int64_t M, int64_t topk, const double *X, int x_per_slot, const int64_t *rows,
               int64_t n_sel, double *Y, double *B, int threads)
{
    int bb, be;
    if (oracle_block_geometry(kind, &bb, &be) != 0) return -1;
    if (K <= 0 || K % be != 0 || E <= 0 || N <= 0 || topk <= 0 || M < 0) return -2;
    const int64_t row_bytes = (K / be) * bb;
    const int64_t pairs = M * topk;
    for (int64_t p = 0; p < pairs; ++p)
        if (ids[p] < 0 || ids[p] >= E) return -4;
#ifdef _OPENMP
    /* The count applies to this region only (omp_set_num_threads would
     * change every later call's default). */
    const int nt = threads > 0 ? threads : omp_get_max_threads();
#else
    (void)threads;
#endif
    int failed = 0;
#pragma omp parallel num_threads(nt)
    {
        double *w = (double *)malloc((size_t)K * sizeof(double));
        if (!w) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t p = 0; p < pairs; ++p) {
            for (int64_t i = 0; i < n_sel; ++i) {
                if (!w) continue;
                const int64_t t = p / topk;
                const int64_t e = ids[p];
                const int64_t n = rows ? rows[i] : i;
                const double *x = x_per_slot ? X + p * K : X + t * K;
                decode_row(kind, W + (e * N + n) * row_bytes, K, bb, be, w);
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    acc += w[k] * x[k];
                    mag += fabs(w[k]) * fabs(x[k]);
                }
                Y[p * n_sel + i] = acc;
                if (B) B[p * n_sel + i] = mag;
            }
        }
        free(w);
    }
    return failed ? -3 : 0;
}

/* Number of OpenMP threads a parallel region would use. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
