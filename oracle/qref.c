/*
 * qref.c -- CPU oracle for the quantized-weight GEMV path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  The GPU library
 * shares no code, header, table or helper with it, and the product path
 * never calls it.
 *
 * Every function is the plain definition of what the method computes:
 * decode each weight from its bytes exactly as the pages define the format,
 * then y = W.x with every product formed exactly in double precision and the
 * sum accumulated in double; one final round-to-nearest-even to float.
 * No blocking, no fusion, no reordering.  Per-row work may run on several
 * OpenMP threads; each row's arithmetic is the same whatever the thread
 * count, so results do not depend on it.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fopenmp -shared -fPIC
 * (no fast-math: NaN, -0 and subnormals must behave as IEEE says).
 *
 * Planted mistakes: compiling with -DQREF_MUTATE=n swaps in one deliberate
 * error (listed at each site) so the tests can show that their pins catch it.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef QREF_MUTATE
#define QREF_MUTATE 0
#endif

static int g_threads = 1;

/* Number of OpenMP threads the GEMV functions use (1 = single thread). */
void qref_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int qref_get_threads(void) { return g_threads; }
int qref_mutation(void) { return QREF_MUTATE; }

/* ------------------------------------------------------------------------ */
/* Scalar decoders                                                           */
/* ------------------------------------------------------------------------ */

/*
 * OCP E4M3-FN byte -> value ("fmt=7: fp8-e4m3-b128 passthrough weight
 * format", section "Design"): sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent 0 holds the subnormals m * 2^-9; the only NaN
 * codes are exponent 15 with mantissa 7 (0x7F, 0xFF); there is no infinity,
 * and 0x80 is -0.
 */
double qref_e4m3(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 0xF, m = b & 7;
    double v;
#if QREF_MUTATE == 5 /* planted: NaN code decoded as an ordinary number */
    if (0) {
#else
    if (e == 15 && m == 7) {
#endif
        return NAN;
    } else if (e == 0) {
#if QREF_MUTATE == 6 /* planted: subnormals treated as normals */
        v = ldexp(8.0 + m, -10);
#else
        v = ldexp((double)m, -9);
#endif
    } else {
        v = ldexp(8.0 + m, e - 10); /* (1 + m/8) * 2^(e-7) */
    }
    return s ? -v : v;
}

/* IEEE binary16 bits -> value (subnormals, +-0, inf and NaN included). */
double qref_f16(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + m, e - 25);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Grouped int4 ("fmt=4")                                                    */
/* ------------------------------------------------------------------------ */

/*
 * Exact value of weight (o, i) of a grouped-int4 matrix, colibri PR #457
 * "metal: grouped-int4 (fmt=4) GEMV support", sections 1 and 3: rows of
 * (I+1)/2 bytes, column 2k in the low nibble of byte k and column 2k+1 in
 * its high nibble; the nibble q is unsigned and the weight is (q - 8) times
 * the f32 scale of group i/gs of that row (ceil(I/gs) scales per row).
 * The product is exact in double (a 4-bit integer times a 24-bit float).
 */
static double i4g_weight(const uint8_t *w, const float *s, int I, int gs,
                         int o, int i)
{
    size_t rb = (size_t)(I + 1) / 2;
    int ng = (I + gs - 1) / gs;
    uint8_t b = w[(size_t)o * rb + (size_t)i / 2];
#if QREF_MUTATE == 2 /* planted: nibbles swapped */
    int q = (i & 1) ? (b & 0xF) : (b >> 4);
#else
    int q = (i & 1) ? (b >> 4) : (b & 0xF);
#endif
#if QREF_MUTATE == 1 /* planted: group index off by one */
    int g = (i + 1) / gs;
    if (g >= ng) g = ng - 1;
#else
    int g = i / gs;
#endif
    double sc = (double)s[(size_t)o * ng + g];
#if QREF_MUTATE == 3 /* planted: 1% scale error */
    sc *= 1.01;
#endif
    return (double)(q - 8) * sc;
}

/* Decoded weights W[O][I] as f32: one rounding of the exact product. */
void qref_i4g_dequant(const uint8_t *w, const float *s, int O, int I, int gs,
                      float *W)
{
    for (int o = 0; o < O; o++)
        for (int i = 0; i < I; i++)
            W[(size_t)o * I + i] = (float)i4g_weight(w, s, I, gs, o, i);
}

/*
 * y[t][r] = sum_i W[rows[r]][i] * x[t][i] for t < S, r < nrows
 * (rows == NULL: all O rows, r = o).  x is f32[S][I], y is f32[S][nrows].
 */
void qref_i4g_gemv(const uint8_t *w, const float *s, const float *x, float *y,
                   int S, int I, int O, int gs, const int *rows, int nrows)
{
    int n = rows ? nrows : O;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int r = 0; r < n; r++) {
        int o = rows ? rows[r] : r;
        for (int t = 0; t < S; t++) {
            double acc = 0.0;
            for (int i = 0; i < I; i++)
                acc += i4g_weight(w, s, I, gs, o, i) * (double)x[(size_t)t * I + i];
            y[(size_t)t * n + r] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* fp8-e4m3 with 128x128 f32 block scales ("fmt=7")                          */
/* ------------------------------------------------------------------------ */

/*
 * Exact value of weight (o, i), "fmt=7: fp8-e4m3-b128 passthrough weight
 * format", section "Design": O*I raw E4M3-FN bytes row-major; one f32 per
 * 128x128 block, ceil(O/128)*ceil(I/128) of them in row-major block order;
 * the weight is decode(byte) MULTIPLIED by its block's scale (the sidecar
 * is named scale_inv, but it is applied as a multiplier).
 */
static double fp8_weight(const uint8_t *w, const float *sc, int O, int I,
                         int o, int i)
{
    int nbo = (O + 127) / 128, nbi = (I + 127) / 128;
#if QREF_MUTATE == 4 /* planted: block index transposed */
    (void)nbi;
    double s = (double)sc[(size_t)(i / 128) * nbo + o / 128];
#else
    (void)nbo;
    double s = (double)sc[(size_t)(o / 128) * nbi + i / 128];
#endif
    return qref_e4m3(w[(size_t)o * I + i]) * s;
}

void qref_fp8b128_dequant(const uint8_t *w, const float *sc, int O, int I,
                          float *W)
{
    for (int o = 0; o < O; o++)
        for (int i = 0; i < I; i++)
            W[(size_t)o * I + i] = (float)fp8_weight(w, sc, O, I, o, i);
}

void qref_fp8b128_gemv(const uint8_t *w, const float *sc, const float *x,
                       float *y, int S, int I, int O, const int *rows,
                       int nrows)
{
    int n = rows ? nrows : O;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int r = 0; r < n; r++) {
        int o = rows ? rows[r] : r;
        for (int t = 0; t < S; t++) {
            double acc = 0.0;
            for (int i = 0; i < I; i++)
                acc += fp8_weight(w, sc, O, I, o, i) * (double)x[(size_t)t * I + i];
            y[(size_t)t * n + r] = (float)acc;
        }
    }
}

/*
 * UE8M0 block scale byte -> value.  "fmt=7: fp8-e4m3-b128 passthrough weight
 * format", section "Design": the same weight geometry also ships with one
 * byte per 128x128 block holding a power-of-two exponent (dtype F8_E8M0).
 * The page names the dtype without its decode; the reading taken is that
 * dtype's usual definition: unsigned, no sign or mantissa bits, value
 * 2^(e - 127), and e = 255 is NaN (no zero, no infinity).
 */
double qref_e8m0(uint8_t e)
{
    if (e == 255)
        return NAN;
#if QREF_MUTATE == 11 /* planted: exponent bias 128 */
    return ldexp(1.0, (int)e - 128);
#else
    return ldexp(1.0, (int)e - 127);
#endif
}

/* Exact value of weight (o, i) with UE8M0 block scales (layout as fmt=7). */
static double fp8e8_weight(const uint8_t *w, const uint8_t *se, int O, int I,
                           int o, int i)
{
    int nbi = (I + 127) / 128;
    (void)O;
    return qref_e4m3(w[(size_t)o * I + i]) * qref_e8m0(se[(size_t)(o / 128) * nbi + i / 128]);
}

void qref_fp8ue8m0_dequant(const uint8_t *w, const uint8_t *se, int O, int I,
                           float *W)
{
    for (int o = 0; o < O; o++)
        for (int i = 0; i < I; i++)
            W[(size_t)o * I + i] = (float)fp8e8_weight(w, se, O, I, o, i);
}

void qref_fp8ue8m0_gemv(const uint8_t *w, const uint8_t *se, const float *x,
                        float *y, int S, int I, int O, const int *rows,
                        int nrows)
{
    int n = rows ? nrows : O;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int r = 0; r < n; r++) {
        int o = rows ? rows[r] : r;
        for (int t = 0; t < S; t++) {
            double acc = 0.0;
            for (int i = 0; i < I; i++)
                acc += fp8e8_weight(w, se, O, I, o, i) * (double)x[(size_t)t * I + i];
            y[(size_t)t * n + r] = (float)acc;
        }
    }
}


/* ------------------------------------------------------------------------ */
/* MQ4-v2: 136 bytes per 256 weights                                         */
/* ------------------------------------------------------------------------ */

/*
 * Exact value of weight (o, i), hipfire "MQ4 V2", sections 2 and 4: each row
 * is I/256 groups of 136 bytes, little-endian.  The dword at byte 0 holds the
 * fp16 scale (low half) and fp16 zero (high half) for weights 0..127 of the
 * group, the dword at byte 4 the pair for weights 128..255; the half is
 * chosen by the weight's own index j (j >= 128), never by a lane id.  The
 * 128 payload bytes start at byte 8; weight j is nibble j of the payload,
 * low nibble first (byte j/2, low nibble for even j).  w = q*scale + zero.
 */
static double mq4v2_weight(const uint8_t *w, int I, int o, int i)
{
    size_t G = (size_t)I / 256;
    const uint8_t *p = w + ((size_t)o * G + (size_t)i / 256) * 136;
    int j = i % 256;
#if QREF_MUTATE == 7 /* planted: half chosen at the wrong boundary */
    int h = j >= 64;
#else
    int h = j >= 128;
#endif
    uint32_t hd = (uint32_t)p[4 * h] | ((uint32_t)p[4 * h + 1] << 8) |
                  ((uint32_t)p[4 * h + 2] << 16) | ((uint32_t)p[4 * h + 3] << 24);
#if QREF_MUTATE == 8 /* planted: scale and zero fields swapped */
    double sc = qref_f16((uint16_t)(hd >> 16));
    double zp = qref_f16((uint16_t)(hd & 0xFFFF));
#else
    double sc = qref_f16((uint16_t)(hd & 0xFFFF));
    double zp = qref_f16((uint16_t)(hd >> 16));
#endif
    uint8_t b = p[8 + j / 2];
    int q = (j & 1) ? (b >> 4) : (b & 0xF);
    return (double)q * sc + zp;
}

void qref_mq4v2_dequant(const uint8_t *w, int O, int I, float *W)
{
    for (int o = 0; o < O; o++)
        for (int i = 0; i < I; i++)
            W[(size_t)o * I + i] = (float)mq4v2_weight(w, I, o, i);
}

void qref_mq4v2_gemv(const uint8_t *w, const float *x, float *y, int S, int I,
                     int O, const int *rows, int nrows)
{
    int n = rows ? nrows : O;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int r = 0; r < n; r++) {
        int o = rows ? rows[r] : r;
        for (int t = 0; t < S; t++) {
            double acc = 0.0;
            for (int i = 0; i < I; i++)
                acc += mq4v2_weight(w, I, o, i) * (double)x[(size_t)t * I + i];
            y[(size_t)t * n + r] = (float)acc;
        }
    }
}

/*
 * MQ4 v1 (qt=13) and the padded-compat form MQ4C (qt=45), hipfire "MQ4 V2",
 * sections 1b and 1e: the same 136-byte groups with the same 128 payload
 * bytes at [8..136) (weight j = nibble j, low nibble first), one header for
 * all 256 weights.  v1: f32 scale at byte 0, f32 zero at byte 4 ("v1 reads
 * two f32 fields").  MQ4C: one packed pair at byte 0, fp16 scale in the low
 * half and fp16 zero in the high half, as v2 packs its pairs; bytes 4..7 are
 * the required zero pad and are not read.  w = q*scale + zero.
 */
static uint32_t le32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
           ((uint32_t)p[3] << 24);
}

static double f32_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double mq4_group_weight(const uint8_t *w, int I, int o, int i, int fmt)
{
    size_t G = (size_t)I / 256;
    const uint8_t *p = w + ((size_t)o * G + (size_t)i / 256) * 136;
    int j = i % 256;
    double sc, zp;
    if (fmt == 1) {           /* v1 */
#if QREF_MUTATE == 13 /* planted: v1 fields swapped */
        sc = f32_bits(le32(p + 4));
        zp = f32_bits(le32(p));
#else
        sc = f32_bits(le32(p));
        zp = f32_bits(le32(p + 4));
#endif
    } else {                  /* MQ4C */
        uint32_t hd = le32(p);
        sc = qref_f16((uint16_t)(hd & 0xFFFF));
        zp = qref_f16((uint16_t)(hd >> 16));
    }
    uint8_t b = p[8 + j / 2];
    int q = (j & 1) ? (b >> 4) : (b & 0xF);
    return (double)q * sc + zp;
}

static void mq4_group_dequant(const uint8_t *w, int O, int I, float *W, int fmt)
{
    for (int o = 0; o < O; o++)
        for (int i = 0; i < I; i++)
            W[(size_t)o * I + i] = (float)mq4_group_weight(w, I, o, i, fmt);
}

static void mq4_group_gemv(const uint8_t *w, const float *x, float *y, int S, int I, int O,
                           const int *rows, int nrows, int fmt)
{
    int n = rows ? nrows : O;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int r = 0; r < n; r++) {
        int o = rows ? rows[r] : r;
        for (int t = 0; t < S; t++) {
            double acc = 0.0;
            for (int i = 0; i < I; i++)
                acc += mq4_group_weight(w, I, o, i, fmt) * (double)x[(size_t)t * I + i];
            y[(size_t)t * n + r] = (float)acc;
        }
    }
}

void qref_mq4v1_dequant(const uint8_t *w, int O, int I, float *W)
{
    mq4_group_dequant(w, O, I, W, 1);
}
void qref_mq4c_dequant(const uint8_t *w, int O, int I, float *W)
{
    mq4_group_dequant(w, O, I, W, 2);
}
void qref_mq4v1_gemv(const uint8_t *w, const float *x, float *y, int S, int I, int O,
                     const int *rows, int nrows)
{
    mq4_group_gemv(w, x, y, S, I, O, rows, nrows, 1);
}
void qref_mq4c_gemv(const uint8_t *w, const float *x, float *y, int S, int I, int O,
                    const int *rows, int nrows)
{
    mq4_group_gemv(w, x, y, S, I, O, rows, nrows, 2);
}

/*
 * f32 -> IEEE binary16 bits, round to nearest even (overflow to infinity,
 * subnormals kept, NaN stays NaN).  Every f32 is exact in double, so the
 * scaled value below is exact and one nearbyint() is the whole rounding.
 */
uint16_t qref_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    double v = fabs((double)f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00);
    if (isinf(f))
        return (uint16_t)(sign | 0x7C00);
    if (v == 0.0)
        return sign;
    int k;
    (void)frexp(v, &k);               /* v = m * 2^k, m in [0.5, 1) */
    int E = k - 1;                     /* v in [2^E, 2^(E+1)) */
    if (E < -14) {                     /* subnormal range: units of 2^-24 */
        double q = nearbyint(ldexp(v, 24));
        return (uint16_t)(sign | (uint16_t)q);   /* q = 1024 is the least normal */
    }
    double q = nearbyint(ldexp(v, 10 - E));       /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | ((E + 15) << 10) | ((int)q - 1024));
}

/*
 * MQ4-v2 encoder, hipfire "MQ4 V2", section 3, for weights already in the
 * rotated space (W f32 [O][I], I % 256 == 0) -> 136-byte groups.  Per group
 * and half h (weights 128h .. 128h+127): lo and hi are the half's min and
 * max; step = (hi - lo) / 15 in f32; the stored scale and zero are the fp16
 * roundings of step and lo; each code is chosen against the stored (f16
 * round-tripped) values, q = clamp(rint((w - z) / s), 0, 15) in f32, so the
 * decoder reproduces the encoder's reconstruction.  A half whose stored
 * scale is 0 -- the constant half of the page, and (our reading) a step too
 * small for fp16 -- gets q = 0: it decodes to the stored zero.  An extreme
 * of -0 counts as +0 (the two compare equal; this fixes the bits of the
 * stored values whichever zero comes first).  Weights must be finite.
 */
void qref_mq4v2_encode(const float *W, int O, int I, uint8_t *out)
{
    int G = I / 256;
    for (int o = 0; o < O; o++)
        for (int g = 0; g < G; g++) {
            const float *wg = W + (size_t)o * I + (size_t)g * 256;
            uint8_t *p = out + ((size_t)o * G + g) * 136;
            memset(p, 0, 136);
            for (int h = 0; h < 2; h++) {
                const float *wh = wg + 128 * h;
                float lo = wh[0], hi = wh[0];
                for (int i = 1; i < 128; i++) {
                    if (wh[i] < lo) lo = wh[i];
                    if (wh[i] > hi) hi = wh[i];
                }
                lo = lo + 0.0f;      /* a -0 extreme counts as +0 */
                hi = hi + 0.0f;
                volatile float step = (hi - lo) / 15.0f;
                uint16_t sc16 = qref_f32_to_f16(step);
                uint16_t zp16 = qref_f32_to_f16(lo);
#if QREF_MUTATE == 12 /* planted: codes chosen against the unrounded step */
                float st = step, z = (float)qref_f16(zp16);
#else
                float st = (float)qref_f16(sc16), z = (float)qref_f16(zp16);
#endif
                uint32_t hd = (uint32_t)sc16 | ((uint32_t)zp16 << 16);
                for (int b = 0; b < 4; b++)
                    p[4 * h + b] = (uint8_t)(hd >> (8 * b));
                for (int i = 0; i < 128; i++) {
                    int q = 0;
                    if (st != 0.0f) {
                        volatile float d = wh[i] - z;
                        volatile float r = d / st;
                        float qf = rintf(r);
                        q = qf < 0.0f ? 0 : (qf > 15.0f ? 15 : (int)qf);
                    }
                    int j = 128 * h + i;
                    p[8 + j / 2] |= (uint8_t)(q << (4 * (j & 1)));
                }
            }
        }
}

/* ------------------------------------------------------------------------ */
/* FWHT-256 pre-rotation                                                     */
/* ------------------------------------------------------------------------ */

static int popcount8(unsigned v)
{
    int c = 0;
    while (v) { c += v & 1; v >>= 1; }
    return c;
}

/*
 * Rotation of the activations into the space the MQ4 weights were quantised
 * in (hipfire "MQ4 V2", section 1: the weights are FWHT-256 rotated with
 * per-element signs).  Reading taken where the page is silent: per
 * 256-element block, x_rot = (1/16) * H * (signs . x) with H the Sylvester
 * Hadamard matrix H[i][j] = (-1)^popcount(i & j); the 1/16 makes it
 * orthonormal.  Written out densely in double, rounded once to f32.
 */
void qref_fwht256(const float *x, const int8_t *signs, float *xr, int S, int I)
{
    int nb = I / 256;
    for (int t = 0; t < S; t++)
        for (int b = 0; b < nb; b++) {
            const float *xb = x + (size_t)t * I + (size_t)b * 256;
            const int8_t *sb = signs + (size_t)b * 256;
            float *ob = xr + (size_t)t * I + (size_t)b * 256;
            for (int i = 0; i < 256; i++) {
                double acc = 0.0;
                for (int j = 0; j < 256; j++) {
                    double hij = (popcount8((unsigned)(i & j)) & 1) ? -1.0 : 1.0;
#if QREF_MUTATE == 9 /* planted: sign taken from the output index */
                    acc += hij * (double)sb[i] * (double)xb[j];
#else
                    acc += hij * (double)sb[j] * (double)xb[j];
#endif
                }
                ob[i] = (float)(acc / 16.0);
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Routed experts: gate-weighted sum of grouped-int4 GEMVs                   */
/* ------------------------------------------------------------------------ */

/*
 * y[t][r] = sum_k gates[t][k] * (W_{ids[t][k]} . x[t])[rows[r]]
 * (regolith audit "phase 0 + phase 2 m5 air validation", section 2.2: the
 * combine weights are the routing probabilities renormalised over the
 * selected experts; colibri PR #457, section 4: routed experts are
 * grouped-int4 matrices).  Expert e's packed weights start at byte
 * e*w_stride of w and its scales at float e*s_stride of s.  A duplicated id
 * contributes once per occurrence.  Out-of-range ids give NaN rows.
 */
void qref_moe_i4g(const uint8_t *w, const float *s, long long w_stride,
                  long long s_stride, int E, const int32_t *ids,
                  const float *gates, int T, int K, const float *x, float *y,
                  int I, int O, int gs, const int *rows, int nrows)
{
    int n = rows ? nrows : O;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int r = 0; r < n; r++) {
        int o = rows ? rows[r] : r;
        for (int t = 0; t < T; t++) {
            double acc = 0.0;
            for (int k = 0; k < K; k++) {
                int e = ids[(size_t)t * K + k];
                if (e < 0 || e >= E) { acc = NAN; break; }
                const uint8_t *we = w + (size_t)e * (size_t)w_stride;
                const float *se = s + (size_t)e * (size_t)s_stride;
                double dot = 0.0;
                for (int i = 0; i < I; i++)
                    dot += i4g_weight(we, se, I, gs, o, i) * (double)x[(size_t)t * I + i];
#if QREF_MUTATE == 10 /* planted: every expert weighted by the first gate */
                acc += (double)gates[(size_t)t * K] * dot;
#else
                acc += (double)gates[(size_t)t * K + k] * dot;
#endif
            }
            y[(size_t)t * n + r] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Router top-k                                                              */
/* ------------------------------------------------------------------------ */

/*
 * Top-K routing of T tokens over E experts, regolith audit "phase 0 + phase
 * 2 m5 air validation", sections 2.1 and 2.2: the logits of the valid
 * experts (columns 0..E-1 of rows of stride ld; columns >= E are masked out)
 * go through a softmax; the K most probable experts are picked in rank
 * order; each picked expert's gate is its probability renormalised over the
 * K picked ones.  Equal probabilities rank by the lower expert index (our
 * reading: the pages do not break ties).  The probability order is the
 * logit order, so picks compare logits; gates are formed in double,
 *     g_k = exp(l_k - m) / sum over picked j of exp(l_j - m),
 * with m the largest logit (the softmax's full normaliser cancels).  Logits
 * must be finite.
 */
void qref_router_topk(const float *logits, int T, int E, int ld, int K,
                      int32_t *ids, float *gates)
{
    for (int t = 0; t < T; t++) {
        const float *l = logits + (size_t)t * ld;
        int32_t *id = ids + (size_t)t * K;
        for (int k = 0; k < K; k++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                int taken = 0;
                for (int j = 0; j < k; j++)
                    taken |= id[j] == e;
                if (taken)
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;   /* strict: the lower index wins a tie */
            }
            id[k] = best;
        }
        double m = (double)l[id[0]], sum = 0.0;
#if QREF_MUTATE == 14 /* planted: gates normalised over all experts, not the picked */
        for (int e = 0; e < E; e++)
            sum += exp((double)l[e] - m);
#else
        for (int k = 0; k < K; k++)
            sum += exp((double)l[id[k]] - m);
#endif
        for (int k = 0; k < K; k++)
            gates[(size_t)t * K + k] = (float)(exp((double)l[id[k]] - m) / sum);
    }
}
