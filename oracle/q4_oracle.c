/*
 * q4_oracle.c -- plain, slow CPU oracle for 4-bit group-wise weight
 * quantization.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and
 * the benchmark's CPU-baseline leg load it.  It shares no code with the GPU
 * library.  The declarations and the page citations are in q4_oracle.h.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared q4_oracle.c -lm
 * (no -ffast-math: every division below must be the IEEE binary32 one).
 */
#include "q4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* The NF4 codebook exactly as printed in [n4n] "How 4-bit quantization
 * works" (three decimals).  Each literal becomes the nearest binary32.      */
const float orc_nf4_table[16] = {
    -1.0f,  -0.696f, -0.525f, -0.395f, -0.284f, -0.185f, -0.091f, 0.0f,
    0.079f, 0.161f,  0.246f,  0.338f,  0.441f,  0.562f,  0.720f,  1.0f};

/* The FP4 codebook (a reading: [hf4] "Developer" names the fp4 quant type
 * beside nf4 but prints no table).  Code bits: bit 3 the sign, bits 2..1 an
 * exponent e, bit 0 a mantissa bit m, as in the E2M1 element format: the
 * magnitude is m / 2 for e = 0 and 2^(e-1) (1 + m / 2) otherwise, i.e. 0,
 * 0.5, 1, 1.5, 2, 3, 4, 6.  Divided by 6 so that the largest magnitude is 1
 * and the block absmax scales it, as NF4's table; each value the nearest
 * binary32 of the exact fraction (code 8 is -0).  PARITY UNPINNED against
 * the pages; the tests pin it to the E2M1 definition. */
const float orc_fp4_table[16] = {
    0.0f,  (float)(1.0 / 12.0),  (float)(1.0 / 6.0),  0.25f,
    (float)(1.0 / 3.0),  0.5f,  (float)(2.0 / 3.0),  1.0f,
    -0.0f, -(float)(1.0 / 12.0), -(float)(1.0 / 6.0), -0.25f,
    -(float)(1.0 / 3.0), -0.5f, -(float)(2.0 / 3.0), -1.0f};

/* ------------------------------------------------------------------------ */
/* IEEE binary16 / bfloat16 conversions from the format definitions.        */

/* Round a finite, non-negative double v to a binary format with p significand
 * bits (hidden bit included) and smallest normal exponent emin, ties to even,
 * with gradual underflow.  v / quantum is exact (a power-of-two scaling), and
 * rint() rounds half to even in the default rounding mode. */
static double round_to_format(double v, int p, int emin)
{
    if (v == 0.0)
        return 0.0;
    int e;
    frexp(v, &e);          /* v = m * 2^e, m in [0.5, 1) */
    int E = e - 1;         /* exponent of the leading bit */
    if (E < emin)
        E = emin;          /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, E - (p - 1));
    return rint(v / quantum) * quantum;
}

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                 /* zero / subnormal */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25);     /* (1 + man/1024) * 2^(ex-15) */
    return (float)(sign ? -v : v);
}

uint16_t orc_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f))
        return 0x7e00;
    double v = fabs((double)f);
    if (isinf(f))
        return sign | 0x7c00;
    double r = round_to_format(v, 11, -14);
    if (r > 65504.0)
        return sign | 0x7c00;                         /* overflow to infinity */
    if (r == 0.0)
        return sign;
    int e;
    frexp(r, &e);
    int E = e - 1;
    if (E < -14)                                      /* subnormal: r = man * 2^-24 */
        return sign | (uint16_t)ldexp(r, 24);
    uint16_t man = (uint16_t)(ldexp(r, 10 - E) - 1024.0);
    return sign | (uint16_t)((E + 15) << 10) | man;
}

float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t orc_f32_to_bf16(float f)
{
    if (isnan(f))
        return 0x7fc0;
    double v = fabs((double)f);
    double bf16_max = ldexp(255.0, 120);              /* (2 - 2^-7) * 2^127 */
    double r = isinf(f) ? INFINITY : round_to_format(v, 8, -126);
    float rf = (float)(r > bf16_max ? INFINITY : r);  /* exact: r has <= 8 bits */
    if (signbit(f))
        rf = -rf;
    uint32_t u;
    memcpy(&u, &rf, 4);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* Coding rules.                                                            */

/* [hf4] "Block-wise quantisation, stated exactly": map to the nearest of the
 * 16 codebook entries.  Distances are taken in binary64, where x - Q[i] is
 * exact whenever x is near a decision point; a tie keeps the lower index
 * because only a strictly smaller distance replaces the current best. */
int orc_nf4_nearest(float x)
{
    int best = 0;
    double bestd = fabs((double)x - (double)orc_nf4_table[0]);
    for (int i = 1; i < 16; ++i) {
        double d = fabs((double)x - (double)orc_nf4_table[i]);
        if (d < bestd) {
            bestd = d;
            best = i;
        }
    }
    return best;
}

/* The same rule over the FP4 table: x = 0 (and anything nearer to 0 than to
 * +-1/12) takes code 0, the lower index of the tie between +0 and -0. */
int orc_fp4_nearest(float x)
{
    int best = 0;
    double bestd = fabs((double)x - (double)orc_fp4_table[0]);
    for (int i = 1; i < 16; ++i) {
        double d = fabs((double)x - (double)orc_fp4_table[i]);
        if (d < bestd) {
            bestd = d;
            best = i;
        }
    }
    return best;
}

static int clampi(int v, int lo, int hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

static int valid_shape(int fmt, int g, int64_t N, int64_t K)
{
    if (fmt < ORC_NF4 || fmt > ORC_FP4)
        return 0;
    if (g != 32 && g != 64 && g != 128)
        return 0;
    if (N <= 0 || K <= 0 || K % g != 0)
        return 0;
    return 1;
}

static void put_nibble(uint8_t *buf, int64_t idx, int v)
{
    if (idx % 2 == 0)
        buf[idx / 2] = (uint8_t)((buf[idx / 2] & 0xf0) | (v & 0xf));
    else
        buf[idx / 2] = (uint8_t)((buf[idx / 2] & 0x0f) | ((v & 0xf) << 4));
}

static int get_nibble(const uint8_t *buf, int64_t idx)
{
    uint8_t b = buf[idx / 2];
    return idx % 2 == 0 ? (b & 0xf) : (b >> 4);
}

/* One group of g weights of one row.  gi is the flat group index
 * row * (K / g) + group; e0 the flat index of the group's first element. */
static void quantize_group(int fmt, int g, const uint16_t *wg, int64_t gi,
                           int64_t e0, uint8_t *codes, void *scales,
                           uint8_t *zeros)
{
    if (fmt == ORC_NF4 || fmt == ORC_NF4_DQ || fmt == ORC_FP4) {
        /* [hf4]: c = max|w| over the block, stored as binary32 (an fp16 value
         * widened, so exact); code = nearest Q[i] to w / c (FP4: the same
         * with its own table; a zero block codes to its zero entry). */
        float c = 0.0f;
        for (int k = 0; k < g; ++k) {
            float a = fabsf(orc_f16_to_f32(wg[k]));
            if (a > c)
                c = a;
        }
        ((float *)scales)[gi] = c;
        for (int k = 0; k < g; ++k) {
            int code = fmt == ORC_FP4 ? 0 : 7;       /* the 0 entry for c == 0 */
            if (c != 0.0f) {
                float x = orc_f16_to_f32(wg[k]) / c;  /* binary32 division */
                code = fmt == ORC_FP4 ? orc_fp4_nearest(x) : orc_nf4_nearest(x);
            }
            put_nibble(codes, e0 + k, code);
        }
    } else if (fmt == ORC_INT4_SYM) {
        /* [n4n]: levels -8..7, implicit zero point, scale = max|w| / 7;
         * [atlas]: the scale is stored in FP16.  Codes use the stored scale,
         * q = clamp(round_half_even(w / s), -8, 7), nibble = q + 8. */
        float a = 0.0f;
        for (int k = 0; k < g; ++k) {
            float v = fabsf(orc_f16_to_f32(wg[k]));
            if (v > a)
                a = v;
        }
        uint16_t s16 = orc_f32_to_f16(a / 7.0f);
        ((uint16_t *)scales)[gi] = s16;
        float s = orc_f16_to_f32(s16);
        for (int k = 0; k < g; ++k) {
            int q = 0;
            if (s != 0.0f)
                q = clampi((int)rintf(orc_f16_to_f32(wg[k]) / s), -8, 7);
            put_nibble(codes, e0 + k, q + 8);
        }
    } else {
        /* [atlas]: levels 0..15 and an integer zero-point so that the group's
         * range fits [0, 15]; [n4n]: q = round((w - zp) / s), w = q*s + zp with
         * zp = -z*s.  Range taken as [min(0, min w), max(0, max w)] so that
         * zero is a level; s = fp16((hi - lo) / 15); z = round(-lo / s);
         * q = clamp(round(w / s) + z, 0, 15). */
        float lo = 0.0f, hi = 0.0f;
        for (int k = 0; k < g; ++k) {
            float v = orc_f16_to_f32(wg[k]);
            if (v < lo)
                lo = v;
            if (v > hi)
                hi = v;
        }
        uint16_t s16 = orc_f32_to_f16((hi - lo) / 15.0f);
        ((uint16_t *)scales)[gi] = s16;
        float s = orc_f16_to_f32(s16);
        int z = 0;
        if (s != 0.0f)
            z = clampi((int)rintf(-lo / s), 0, 15);
        put_nibble(zeros, gi, z);
        for (int k = 0; k < g; ++k) {
            int q = 0;
            if (s != 0.0f)
                q = clampi((int)rintf(orc_f16_to_f32(wg[k]) / s) + z, 0, 15);
            put_nibble(codes, e0 + k, q);
        }
    }
}

/* [dq] The block constants quantized again: consecutive runs of
 * ORC_DQ_BLOCK absmax values (flat group order; the last run may be short)
 * share one binary32 constant s2 = c2 / 127 with c2 the run's largest
 * absmax, and each absmax becomes the 8-bit code q = rint(c / s2) clamped to
 * 0..127 (symmetric absmax 8-bit coding; the absmax values are >= 0, so only
 * the non-negative half of the levels occurs).  s2 == 0 (an all-zero run)
 * gives q = 0. */
void orc_double_quant(const float *c, int64_t n, uint8_t *qc, float *s2)
{
    for (int64_t b = 0; b * ORC_DQ_BLOCK < n; ++b) {
        int64_t i0 = b * ORC_DQ_BLOCK;
        int64_t i1 = i0 + ORC_DQ_BLOCK < n ? i0 + ORC_DQ_BLOCK : n;
        float c2 = 0.0f;
        for (int64_t i = i0; i < i1; ++i)
            if (c[i] > c2)
                c2 = c[i];
        float s = c2 / 127.0f;                      /* binary32 division */
        s2[b] = s;
        for (int64_t i = i0; i < i1; ++i) {
            int q = 0;
            if (s != 0.0f)
                q = clampi((int)rintf(c[i] / s), 0, 127);
            qc[i] = (uint8_t)q;
        }
    }
}

int64_t orc_dq_s2_offset(int64_t n_groups) { return (n_groups + 15) / 16 * 16; }

int orc_quantize(int fmt, int g, const uint16_t *w, int64_t N, int64_t K,
                 uint8_t *codes, void *scales, uint8_t *zeros)
{
    if (!valid_shape(fmt, g, N, K) || !w || !codes || !scales)
        return -1;
    if ((fmt == ORC_INT4_ASYM) != (zeros != NULL))
        return -1;
    int64_t G = K / g;
    if (zeros) /* a half-filled last byte keeps a zero high nibble */
        memset(zeros, 0, (size_t)((N * G + 1) / 2));
    /* NF4_DQ: the codes are those of NF4 (made with the exact absmax); the
     * absmax array is kept aside and then quantized as a whole */
    void *first = scales;
    float *c = NULL;
    if (fmt == ORC_NF4_DQ) {
        c = (float *)malloc((size_t)(N * G) * sizeof(float));
        if (!c)
            return -1;
        first = c;
    }
    for (int64_t r = 0; r < N; ++r)
        for (int64_t j = 0; j < G; ++j)
            quantize_group(fmt, g, w + r * K + j * g, r * G + j, r * K + j * g,
                           codes, first, zeros);
    if (c) {
        int64_t nb = (N * G + ORC_DQ_BLOCK - 1) / ORC_DQ_BLOCK;
        float *s2 = (float *)malloc((size_t)nb * sizeof(float));
        if (!s2) {
            free(c);
            return -1;
        }
        uint8_t *out = (uint8_t *)scales;
        int64_t off = orc_dq_s2_offset(N * G);
        memset(out, 0, (size_t)off);
        orc_double_quant(c, N * G, out, s2);
        memcpy(out + off, s2, (size_t)nb * sizeof(float));
        free(s2);
        free(c);
    }
    return 0;
}

/* [n4n] dequantize: value = table entry (or integer level) times the block
 * scale, one binary32 product, then one round-to-nearest-even to the output
 * dtype.  Sym: (nib - 8) * s; asym: (q - z) * s ([n4n] affine form with
 * zp = -z*s); NF4: Q[i] * c ([hf4]); NF4_DQ: Q[i] * c' with the absmax
 * recovered as c' = q * s2 ([dq], one binary32 product). */
static float dequant_value(int fmt, int nib, int64_t gi, int64_t n_groups,
                           const void *scales, const uint8_t *zeros)
{
    if (fmt == ORC_NF4)
        return orc_nf4_table[nib] * ((const float *)scales)[gi];
    if (fmt == ORC_FP4)
        return orc_fp4_table[nib] * ((const float *)scales)[gi];
    if (fmt == ORC_NF4_DQ) {
        const uint8_t *qc = (const uint8_t *)scales;
        float s2;
        memcpy(&s2, qc + orc_dq_s2_offset(n_groups) + 4 * (gi / ORC_DQ_BLOCK), 4);
        float c = (float)qc[gi] * s2;
        return orc_nf4_table[nib] * c;
    }
    float s = orc_f16_to_f32(((const uint16_t *)scales)[gi]);
    if (fmt == ORC_INT4_SYM)
        return (float)(nib - 8) * s;
    return (float)(nib - get_nibble(zeros, gi)) * s;
}

int orc_dequantize(int fmt, int g, const uint8_t *codes, const void *scales,
                   const uint8_t *zeros, int64_t N, int64_t K, int out_t,
                   uint16_t *out)
{
    if (!valid_shape(fmt, g, N, K) || !codes || !scales || !out)
        return -1;
    if ((fmt == ORC_INT4_ASYM) != (zeros != NULL))
        return -1;
    if (out_t != ORC_F16 && out_t != ORC_BF16)
        return -1;
    for (int64_t e = 0; e < N * K; ++e) {
        int64_t gi = e / g; /* K % g == 0: flat groups never straddle rows */
        float v = dequant_value(fmt, get_nibble(codes, e), gi, N * K / g, scales,
                                zeros);
        out[e] = out_t == ORC_F16 ? orc_f32_to_f16(v) : orc_f32_to_bf16(v);
    }
    return 0;
}

/* [hf4] "Where the accuracy goes" / [bnb]: the layer dequantizes the weights
 * to the compute dtype and runs an ordinary 16-bit matmul.  The reference
 * takes what = dequantized weight rounded to the activation dtype, and sums the
 * exact products x * what in binary64, in k order. */
int orc_matmul(int fmt, int g, int act_t, const uint16_t *x, int64_t M,
               const uint8_t *codes, const void *scales, const uint8_t *zeros,
               int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
               double *y, double *absdot)
{
    if (!valid_shape(fmt, g, N, K) || !x || M <= 0 || !codes || !scales || !y)
        return -1;
    if ((fmt == ORC_INT4_ASYM) != (zeros != NULL))
        return -1;
    if (act_t != ORC_F16 && act_t != ORC_BF16)
        return -1;
    if (rows == NULL && nrows != N)
        return -1;
    double *wrow = (double *)malloc((size_t)K * sizeof(double));
    if (!wrow)
        return -1;
    int64_t G = K / g;
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t n = rows ? rows[j] : j;
        if (n < 0 || n >= N) {
            free(wrow);
            return -1;
        }
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = n * K + k;
            float v = dequant_value(fmt, get_nibble(codes, e), n * G + k / g,
                                    N * G, scales, zeros);
            wrow[k] = act_t == ORC_F16 ? orc_f16_to_f32(orc_f32_to_f16(v))
                                       : orc_bf16_to_f32(orc_f32_to_bf16(v));
        }
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                uint16_t xb = x[m * K + k];
                double xv = act_t == ORC_F16 ? orc_f16_to_f32(xb)
                                             : orc_bf16_to_f32(xb);
                double p = xv * wrow[k]; /* exact: two 16-bit significands */
                acc += p;
                aacc += fabs(p);
            }
            y[m * nrows + j] = acc;
            if (absdot)
                absdot[m * nrows + j] = aacc;
        }
    }
    free(wrow);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Element-wise loops over the scalar routines above, so that tests can sweep
 * many values per call. */
void orc_f32_to_f16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_f16(in[i]);
}

void orc_f16_to_f32_array(const uint16_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f16_to_f32(in[i]);
}

void orc_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_bf16(in[i]);
}

void orc_nf4_nearest_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)orc_nf4_nearest(in[i]);
}

/* [n4n] "QLoRA fine-tunes in 4-bit": the gradient reaches the layer input
 * through the dequantized weights, which stay fixed.  Reference
 * dx[m][j] = sum_n dy[m][n] * what[n][cols[j]] in binary64, summed in n
 * order, with what rounded to the activation dtype as in orc_matmul;
 * absdot[m][j] = sum_n |dy[m][n] * what[n][cols[j]]|.  cols == NULL means
 * columns 0..K-1 (ncols must then equal K). */
int orc_matmul_dx(int fmt, int g, int act_t, const uint16_t *dy, int64_t M,
                  const uint8_t *codes, const void *scales, const uint8_t *zeros,
                  int64_t N, int64_t K, const int64_t *cols, int64_t ncols,
                  double *dx, double *absdot)
{
    if (!valid_shape(fmt, g, N, K) || !dy || M <= 0 || !codes || !scales || !dx)
        return -1;
    if ((fmt == ORC_INT4_ASYM) != (zeros != NULL))
        return -1;
    if (act_t != ORC_F16 && act_t != ORC_BF16)
        return -1;
    if (cols == NULL && ncols != K)
        return -1;
    double *wcol = (double *)malloc((size_t)N * sizeof(double));
    if (!wcol)
        return -1;
    int64_t G = K / g;
    for (int64_t j = 0; j < ncols; ++j) {
        int64_t k = cols ? cols[j] : j;
        if (k < 0 || k >= K) {
            free(wcol);
            return -1;
        }
        for (int64_t n = 0; n < N; ++n) {
            int64_t e = n * K + k;
            float v = dequant_value(fmt, get_nibble(codes, e), n * G + k / g,
                                    N * G, scales, zeros);
            wcol[n] = act_t == ORC_F16 ? orc_f16_to_f32(orc_f32_to_f16(v))
                                       : orc_bf16_to_f32(orc_f32_to_bf16(v));
        }
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                uint16_t b = dy[m * N + n];
                double yv = act_t == ORC_F16 ? orc_f16_to_f32(b) : orc_bf16_to_f32(b);
                double p = yv * wcol[n]; /* exact: two 16-bit significands */
                acc += p;
                aacc += fabs(p);
            }
            dx[m * ncols + j] = acc;
            if (absdot)
                absdot[m * ncols + j] = aacc;
        }
    }
    free(wcol);
    return 0;
}
