/*
 * oracle.c -- plain, slow, single-threaded CPU definition of the fused
 * rank-sum + residual-add + RMSNorm (+ per-token FP8 e4m3) epilogue.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this file's library. The HIP library never links,
 * includes or calls it, and it shares no code, header, table or constant
 * with the HIP sources: every rounding rule below is written from the
 * format definitions (IEEE-754 binary16, bfloat16 = the top half of
 * binary32, OCP FP8 E4M3 "fn": bias 7, max 448, no infinities).
 *
 * What is computed (sources: ROCm/aiter PR #6699 "gfx1250 fused
 * all-reduce + RMSNorm", section Changes and the commit notes; PR #3462
 * "optimize fused AllReduce + RMSNorm", section Technical Details):
 *
 *   O1  a   = RNE_T( x_0 + x_1 + ... + x_{R-1} )   fp32 adds, rank 0 first,
 *             the accumulator starts at x_0 (fixed rank order, same
 *             rounding to bf16/fp16 as an unfused all-reduce).
 *   O2  h   = RNE_T( fl32(a + res) ),  residual_out = h   (the residual add
 *             of the unfused add+RMSNorm op, PR #6699 bench script).
 *   O3  ss  = sum_j h_j^2 in fp64, left to right;
 *       rstd = 1 / sqrt(ss / H + eps)  (fp64; eps is the fp32 argument).
 *   O4  w_eff = w (or 1 + w under gemma_norm, PR #6699 Changes);
 *       y_j = RNE_T( fl64( fl64(h_j * w_eff_j) * rstd ) ), one rounding
 *       from fp64 to T.
 *   O5  per-token FP8 (PR #6699 Changes: quantise the bf16/fp16-rounded
 *       output with the dynamic per-token steps):
 *       amax = max_j |y_j| ; scale = fl32(amax / 448) ;
 *       q_j = E4M3_RNE_sat( fl32(y_j / scale) ) ; amax == 0 gives
 *       scale = 0 and q_j = signed zero.
 *
 * The pages also name per-group and MXFP4 quant forms of the fused op
 * (PR #6699 Motivation and Changes) without defining them; this oracle
 * reads them as:
 *   O6  per-group FP8: O5's steps on each group of 128 consecutive
 *       columns (scales [M][H/128] fp32). No page gives a group size:
 *       128 (the usual 1 x 128 activation grouping) is a choice, and the
 *       pins hold O6 to this reading only;
 *   O7  MXFP4 (OCP Microscaling Formats v1.0, MXFP4): blocks of 32
 *       columns, E8M0 scale X = 2^(floor(log2(amax)) - 2), elements
 *       E2M1_RNE_sat(y / X), two per byte with the even column in the low
 *       nibble (codes [M][H/2], scales [M][H/32] bytes).
 *
 * For T = fp32 the RNE_T steps of O1/O2 are the fp32 operations
 * themselves and O4 rounds fp64 -> fp32 once.
 *
 * Non-finite values (the pages define none; read here as IEEE arithmetic
 * plus three rules): a maximum over |y| is NaN when any y it covers is NaN
 * (max_abs_nan below); the E4M3 code of any NaN is 0x7F, with no sign (a
 * NaN's sign is not fixed by the arithmetic that made it); in an MXFP4
 * block whose scale is the NaN code a NaN element is 0x7, other elements
 * +-6's code with the sign of y.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * -ffp-contract=off keeps every fp32/fp64 operation a separate IEEE
 * operation, as written.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* dtype codes and flag bits, as this oracle reads them (the same meaning
 * as the library's flags argument, restated here on purpose). */
#define ORC_DT_BF16 0
#define ORC_DT_FP16 1
#define ORC_DT_FP32 2
#define ORC_DT_MASK 3
#define ORC_GEMMA 4
#define ORC_FP8 8
#define ORC_FP8G 16        /* per-group FP8: scale per group of ORC_FP8_GROUP columns */
#define ORC_MXFP4 32       /* MXFP4: E8M0 scale per block of ORC_MX_BLOCK columns, E2M1 elements */
#define ORC_FP8_GROUP 128
#define ORC_MX_BLOCK 32

/* ------------------------------------------------------------------ */
/* Rounding to p significant bits (round to nearest, ties to even).    */
/* ------------------------------------------------------------------ */

/* Round finite v to the nearest number of the form k * 2^q with
 * |k| < 2^p, where q = max(floor(log2|v|), emin) - (p - 1): p significant
 * bits for normal numbers, a fixed quantum 2^(emin-p+1) below 2^emin
 * (gradual underflow). Ties go to the even k (nearbyint in the default
 * rounding mode). The exponent range above is unbounded; callers apply
 * their own overflow rule. */
static double round_p(double v, int p, int emin)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    (void)frexp(v, &e);          /* v = f * 2^e with 0.5 <= |f| < 1 */
    int lead = e - 1;            /* exponent of the leading bit */
    if (lead < emin)
        lead = emin;
    int q = lead - (p - 1);
    double k = nearbyint(ldexp(v, -q)); /* exact scaling, then RNE */
    return ldexp(k, q);
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float bits_f32(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* bfloat16: 8 significant bits, the exponent range of binary32. */
static uint16_t orc_bf16_from_double(double v)
{
    if (isnan(v))
        return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    double r = round_p(v, 8, -126);
    const double maxf = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > maxf)
        r = copysign(INFINITY, r);
    /* r has at most 8 significant bits and lies in the binary32 range, so
     * the conversion to float is exact and bf16 is its top half. */
    return (uint16_t)(f32_bits((float)r) >> 16);
}

static double orc_bf16_to_double(uint16_t b)
{
    return (double)bits_f32((uint32_t)b << 16);
}

/* binary16: 11 significant bits, emin = -14, max 65504. */
static uint16_t orc_fp16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0;
    if (isnan(v))
        return (uint16_t)(sign | 0x7E00u);
    double r = fabs(round_p(v, 11, -14));
    if (r > 65504.0)
        return (uint16_t)(sign | 0x7C00u);
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -14)) /* subnormal: multiple of 2^-24 */
        return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    int e;
    double f = frexp(r, &e); /* r = f * 2^e, f in [0.5, 1) */
    int lead = e - 1;
    uint16_t mant = (uint16_t)(ldexp(f, 11) - 1024.0); /* 10 fraction bits */
    return (uint16_t)(sign | (uint16_t)((lead + 15) << 10) | mant);
}

static double orc_fp16_to_double(uint16_t h)
{
    double s = (h & 0x8000u) ? -1.0 : 1.0;
    int ex = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    if (ex == 0x1F)
        return m ? NAN : s * INFINITY;
    if (ex == 0)
        return s * ldexp((double)m, -24);
    return s * ldexp((double)(1024 + m), ex - 15 - 10);
}

/* OCP FP8 E4M3 ("fn"): 4 significant bits, emin = -6, max 448, no
 * infinities, S.1111.111 is NaN. Out-of-range finite values saturate to
 * +-448. */
static uint8_t orc_e4m3_from_float(float x)
{
    if (isnan(x))
        return 0x7Fu; /* one NaN code, no sign */
    uint8_t sign = signbit(x) ? 0x80u : 0;
    double r = fabs(round_p((double)x, 4, -6));
    if (isinf(x) || r > 448.0)
        r = 448.0;
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -6)) /* subnormal: multiple of 2^-9 */
        return (uint8_t)(sign | (uint8_t)ldexp(r, 9));
    int e;
    double f = frexp(r, &e);
    int lead = e - 1;
    uint8_t mant = (uint8_t)(ldexp(f, 4) - 8.0); /* 3 fraction bits */
    return (uint8_t)(sign | (uint8_t)((lead + 7) << 3) | mant);
}

/* Running max of |y| that a NaN takes over and keeps. */
static float max_abs_nan(float amax, float y)
{
    if (isnan(amax) || isnan(y))
        return NAN;
    return fabsf(y) > amax ? fabsf(y) : amax;
}

/* OCP FP4 E2M1 (the MX element format): 2 significant bits, emin = 0
 * (normals 1, 1.5, 2, 3, 4, 6; the subnormal 0.5), no infinities or NaN.
 * Finite values round to nearest, ties to even, and saturate to +-6. The
 * code is S.EE.M in the low nibble. NaN and infinities are not defined by
 * the format; here NaN maps to +-6's code like the infinities. */
static uint8_t orc_e2m1_from_float(float x)
{
    uint8_t sign = signbit(x) ? 0x8u : 0;
    if (isnan(x) || isinf(x))
        return (uint8_t)(sign | 0x7u);
    double r = fabs(round_p((double)x, 2, 0));
    if (r > 6.0)
        r = 6.0;
    if (r == 0.0)
        return sign;
    if (r < 1.0) /* the subnormal 0.5 */
        return (uint8_t)(sign | 1u);
    int e;
    double f = frexp(r, &e); /* r = f * 2^e, f in [0.5, 1) */
    uint8_t mant = (uint8_t)(ldexp(f, 2) - 2.0);
    return (uint8_t)(sign | (uint8_t)(e << 1) | mant);
}

/* MX shared scale of a block (OCP Microscaling Formats v1.0, section 6.3):
 * X = 2^(floor(log2(amax)) - emax_elem) with emax_elem = 2 for E2M1,
 * returned as its E8M0 code (biased exponent, bias 127), the exponent
 * clamped to [-127, 127]. An all-zero block takes 2^-127 (code 0); a block
 * with a NaN or an infinity takes the E8M0 NaN code 0xFF. */
static uint8_t orc_mx_scale_code(float amax)
{
    if (isnan(amax) || isinf(amax))
        return 0xFFu;
    if (amax == 0.0f)
        return 0;
    int e;
    frexp((double)amax, &e); /* floor(log2(amax)) = e - 1 */
    int se = (e - 1) - 2;
    if (se < -127)
        se = -127;
    if (se > 127)
        se = 127;
    return (uint8_t)(se + 127);
}

/* ------------------------------------------------------------------ */
/* Element access in the storage type T.                                */
/* ------------------------------------------------------------------ */

static float load_t(const void *base, size_t idx, int dt)
{
    if (dt == ORC_DT_FP32)
        return ((const float *)base)[idx];
    uint16_t b = ((const uint16_t *)base)[idx];
    /* every bf16/fp16 value is exactly representable in binary32 */
    return (float)(dt == ORC_DT_BF16 ? orc_bf16_to_double(b) : orc_fp16_to_double(b));
}

/* RNE of a double to T, returned as the exact float value of the result. */
static float round_t(double v, int dt)
{
    if (dt == ORC_DT_FP32)
        return (float)v; /* one IEEE rounding (default mode: RNE) */
    if (dt == ORC_DT_BF16)
        return (float)orc_bf16_to_double(orc_bf16_from_double(v));
    return (float)orc_fp16_to_double(orc_fp16_from_double(v));
}

static void store_t(void *base, size_t idx, float v, int dt)
{
    /* v is already a value of T (an output of round_t) */
    if (dt == ORC_DT_FP32)
        ((float *)base)[idx] = v;
    else if (dt == ORC_DT_BF16)
        ((uint16_t *)base)[idx] = orc_bf16_from_double((double)v);
    else
        ((uint16_t *)base)[idx] = orc_fp16_from_double((double)v);
}

/* ------------------------------------------------------------------ */
/* The fused epilogue, rows [row_begin, row_end).                       */
/* ------------------------------------------------------------------ */

/*
 * rank_in[r]  : R host arrays [M][H] of T.
 * residual    : [M][H] T.        weight : [H] T.
 * out         : [M][H] T or NULL (with FP8 this is the optional T mirror).
 * residual_out: [M][H] T (may equal residual).
 * fp8_out     : [M][H] bytes, fp8_scale : [M] float; required with FP8.
 * h_scratch   : [H] float scratch supplied by the caller.
 * Returns 0, or -1 for an argument this oracle does not define.
 */
int oracle_fused_rows(const void *const *rank_in, int R, const void *residual,
                      const void *weight, void *out, void *residual_out,
                      void *fp8_out, float *fp8_scale, int M, int H, float eps,
                      int flags, int row_begin, int row_end, float *h_scratch)
{
    int dt = flags & ORC_DT_MASK;
    int gemma = (flags & ORC_GEMMA) != 0;
    int fp8 = (flags & ORC_FP8) != 0;
    int fp8g = (flags & ORC_FP8G) != 0;
    int mx = (flags & ORC_MXFP4) != 0;
    if (R < 1 || H < 1 || M < 0 || dt > ORC_DT_FP32)
        return -1;
    if (fp8 + fp8g + mx > 1)
        return -1;
    if ((fp8 || fp8g || mx) && (dt == ORC_DT_FP32 || !fp8_out || !fp8_scale))
        return -1;
    if ((fp8g && H % ORC_FP8_GROUP) || (mx && H % ORC_MX_BLOCK))
        return -1;
    if (row_begin < 0 || row_end > M || row_begin > row_end)
        return -1;

    for (int m = row_begin; m < row_end; ++m) {
        size_t row = (size_t)m * (size_t)H;

        /* O1 + O2: rank-ordered fp32 sum, RNE to T, residual add, RNE to T */
        for (int j = 0; j < H; ++j) {
            float acc = load_t(rank_in[0], row + j, dt);
            for (int r = 1; r < R; ++r)
                acc = acc + load_t(rank_in[r], row + j, dt);
            float a = round_t((double)acc, dt);
            float s = a + load_t(residual, row + j, dt); /* fp32 add */
            float h = round_t((double)s, dt);
            h_scratch[j] = h;
        }
        for (int j = 0; j < H; ++j)
            store_t(residual_out, row + j, h_scratch[j], dt);

        /* O3: fp64 sum of squares, left to right */
        double ss = 0.0;
        for (int j = 0; j < H; ++j)
            ss = ss + (double)h_scratch[j] * (double)h_scratch[j];
        double rstd = 1.0 / sqrt(ss / (double)H + (double)eps);

        /* O4: y = RNE_T((h * w_eff) * rstd) from fp64; O5 needs max|y| */
        float amax = 0.0f;
        for (int j = 0; j < H; ++j) {
            double weff = (double)load_t(weight, (size_t)j, dt);
            if (gemma)
                weff = weff + 1.0;
            double y64 = ((double)h_scratch[j] * weff) * rstd;
            float y = round_t(y64, dt);
            h_scratch[j] = y; /* h is no longer needed */
            if (out)
                store_t(out, row + j, y, dt);
            amax = max_abs_nan(amax, y);
        }

        /* O5: dynamic per-token FP8 of the T-rounded output */
        if (fp8) {
            float scale = amax / 448.0f;
            fp8_scale[m] = scale;
            uint8_t *q = (uint8_t *)fp8_out + row;
            for (int j = 0; j < H; ++j) {
                float y = h_scratch[j];
                if (amax == 0.0f)
                    q[j] = signbit(y) ? 0x80u : 0x00u;
                else
                    q[j] = orc_e4m3_from_float(y / scale); /* fp32 division */
            }
        }

        /* per-group FP8: the per-token steps on each group of columns */
        if (fp8g) {
            int ng = H / ORC_FP8_GROUP;
            uint8_t *q = (uint8_t *)fp8_out + row;
            for (int g = 0; g < ng; ++g) {
                const float *yg = h_scratch + (size_t)g * ORC_FP8_GROUP;
                float gmax = 0.0f;
                for (int j = 0; j < ORC_FP8_GROUP; ++j)
                    gmax = max_abs_nan(gmax, yg[j]);
                float scale = gmax / 448.0f;
                ((float *)fp8_scale)[(size_t)m * ng + g] = scale;
                for (int j = 0; j < ORC_FP8_GROUP; ++j) {
                    float y = yg[j];
                    q[(size_t)g * ORC_FP8_GROUP + j] = gmax == 0.0f ? (signbit(y) ? 0x80u : 0x00u)
                                                                     : orc_e4m3_from_float(y / scale);
                }
            }
        }

        /* MXFP4: E8M0 block scale, E2M1 elements of y / X (exact: X is a power
         * of two), two per byte, the even column in the low nibble */
        if (mx) {
            int nb = H / ORC_MX_BLOCK;
            uint8_t *q = (uint8_t *)fp8_out + (size_t)m * (size_t)(H / 2);
            for (int b = 0; b < nb; ++b) {
                const float *yb = h_scratch + (size_t)b * ORC_MX_BLOCK;
                float bmax = 0.0f;
                int bad = 0;
                for (int j = 0; j < ORC_MX_BLOCK; ++j) {
                    if (isnan(yb[j]))
                        bad = 1;
                    else if (fabsf(yb[j]) > bmax)
                        bmax = fabsf(yb[j]);
                }
                uint8_t code = orc_mx_scale_code(bad ? NAN : bmax);
                ((uint8_t *)fp8_scale)[(size_t)m * nb + b] = code;
                for (int j = 0; j < ORC_MX_BLOCK; j += 2) {
                    uint8_t c[2];
                    for (int t = 0; t < 2; ++t) {
                        float y = yb[j + t];
                        if (code == 0xFFu && isnan(y))
                            c[t] = 0x7u;
                        else if (code == 0xFFu)
                            c[t] = (uint8_t)((signbit(y) ? 0x8u : 0) | 0x7u);
                        else
                            c[t] = orc_e2m1_from_float((float)ldexp((double)y, 127 - (int)code));
                    }
                    q[(size_t)(b * ORC_MX_BLOCK + j) / 2] = (uint8_t)(c[0] | (c[1] << 4));
                }
            }
        }
    }
    return 0;
}

/* Step O1 alone over n elements: the plain rank all-reduce (the flattened
 * message sweep of PR #5807 "Specialize partial tiles in two-stage custom
 * all-reduce", section Proposed modifications; the rank order of PR #3462
 * Technical Details). out may be one of the inputs. Returns 0, or -1 for an
 * argument this oracle does not define. */
int oracle_rank_sum(const void *const *rank_in, int R, void *out, size_t n, int dt)
{
    if (R < 1 || dt < 0 || dt > ORC_DT_FP32)
        return -1;
    for (size_t i = 0; i < n; ++i) {
        float acc = load_t(rank_in[0], i, dt);
        for (int r = 1; r < R; ++r)
            acc = acc + load_t(rank_in[r], i, dt);
        store_t(out, i, round_t((double)acc, dt), dt);
    }
    return 0;
}

/* Quantisation step O5 alone, applied to given T rows (used to check the
 * FP8 bytes of a result against its own T mirror and scale). */
int oracle_quant_rows(const void *y_in, int dt, int M, int H, uint8_t *q_out,
                      float *scale_out)
{
    if (dt != ORC_DT_BF16 && dt != ORC_DT_FP16)
        return -1;
    for (int m = 0; m < M; ++m) {
        size_t row = (size_t)m * (size_t)H;
        float amax = 0.0f;
        for (int j = 0; j < H; ++j) {
            float y = load_t(y_in, row + j, dt);
            amax = max_abs_nan(amax, y);
        }
        float scale = amax / 448.0f;
        scale_out[m] = scale;
        for (int j = 0; j < H; ++j) {
            float y = load_t(y_in, row + j, dt);
            if (amax == 0.0f)
                q_out[row + j] = signbit(y) ? 0x80u : 0x00u;
            else
                q_out[row + j] = orc_e4m3_from_float(y / scale);
        }
    }
    return 0;
}

/* Vector forms of the encoders, for the pin tests. */
void orc_bf16_from_double_n(const double *v, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_bf16_from_double(v[i]);
}

void orc_fp16_from_double_n(const double *v, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_fp16_from_double(v[i]);
}

void orc_e2m1_from_float_n(const float *v, uint8_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_e2m1_from_float(v[i]);
}

void orc_e4m3_from_float_n(const float *v, uint8_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_from_float(v[i]);
}
