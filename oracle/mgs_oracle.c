/*
 * mgs_oracle.c — plain, slow, single-threaded CPU reference implementation.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg. The HIP library never includes, links or
 * calls anything here, and this file uses nothing of the library's.
 *
 * Every function writes out the definition it follows, with no blocking,
 * fusion or reordering beyond that definition. Citations are listed in
 * mgs_oracle.h ([ROWWISE], [BLOCKSIZE], [MXA2A], OFP8, MX).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * Floating point is IEEE binary32 / binary64 with round-to-nearest-even; the
 * entry points clear the x86 flush-to-zero and denormals-are-zero bits for
 * their duration so subnormals are honoured whatever the caller set.
 */
#include "mgs_oracle.h"

#include <float.h>
#include <math.h>
#include <string.h>
#include <xmmintrin.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs binary32 arithmetic evaluated in binary32"
#endif

/* ---- floating-point environment -------------------------------------- */

/* MXCSR: FTZ is bit 15, DAZ bit 6, rounding control bits 13-14 (00 = RNE). */
static unsigned fpenv_enter(void)
{
    unsigned saved = _mm_getcsr();
    _mm_setcsr(saved & ~(0x8000u | 0x0040u | 0x6000u));
    return saved;
}

static void fpenv_leave(unsigned saved) { _mm_setcsr(saved); }

/* ---- formats ---------------------------------------------------------- */

float oracle_bf16_to_f32(uint16_t bits)
{
    /* bf16 is the most significant half of an IEEE binary32 word. */
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return f;
}

double oracle_e4m3_decode(uint8_t code)
{
    /* OFP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits.
     * Exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN. */
    int s = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 15 && m == 7)
        return s ? -NAN : NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp((double)(8 + m), e - 7 - 3);
    return s ? -mag : mag;
}

uint8_t oracle_e4m3_encode(double v)
{
    /* Saturating round-to-nearest-even onto the E4M3 grid (OFP8 E4M3;
     * saturation bounds from fp8_dtype_min / fp8_dtype_max in the
     * [BLOCKSIZE] kernel-argument dict). */
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a, quantum, n, fl, frac, r, value;

    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    a = fabs(v);
    if (a > 448.0)
        a = 448.0;                          /* clamp to the finite range */

    /* Spacing of the grid around a: 2^-9 in the subnormal range below
     * 2^-6, else 2^(E-3) for a in [2^E, 2^(E+1)) (3 mantissa bits). */
    if (a < 0x1p-6) {
        quantum = 0x1p-9;
    } else {
        int ex;
        (void)frexp(a, &ex);                /* a = f * 2^ex, f in [0.5, 1) */
        quantum = ldexp(1.0, (ex - 1) - 3);
    }
    n = a / quantum;                        /* exact: power-of-two divisor */
    fl = floor(n);
    frac = n - fl;
    if (frac > 0.5)
        r = fl + 1.0;
    else if (frac < 0.5)
        r = fl;
    else                                    /* tie: pick the even multiple */
        r = (((int64_t)fl & 1) == 0) ? fl : fl + 1.0;
    value = r * quantum;                    /* exact, and <= 448 */

    if (value == 0.0)
        return sign;
    if (value < 0x1p-6)                     /* subnormal: m * 2^-9, m = 1..7 */
        return (uint8_t)(sign | (uint8_t)(value / 0x1p-9));
    {
        int ex, E, m;
        (void)frexp(value, &ex);
        E = ex - 1;                         /* value in [2^E, 2^(E+1)) */
        m = (int)((value / ldexp(1.0, E) - 1.0) * 8.0);
        return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)m);
    }
}

void oracle_e4m3_encode_array(const double *v, int64_t n, uint8_t *out)
{
    unsigned env = fpenv_enter();
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(v[i]);
    fpenv_leave(env);
}

void oracle_e4m3_encode_f32_bits(uint32_t first, int64_t n, uint8_t *out)
{
    unsigned env = fpenv_enter();
    int64_t i;
    for (i = 0; i < n; ++i) {
        uint32_t w = first + (uint32_t)i;
        float f;
        memcpy(&f, &w, sizeof f);
        out[i] = oracle_e4m3_encode((double)f);
    }
    fpenv_leave(env);
}

/* ---- per-group scaling --------------------------------------------------- */

float oracle_group_scale(float amax, int pow2)
{
    /* [BLOCKSIZE] kernel-argument dict: fp8_dtype_max = 448, EPS = 1e-12,
     * round_scales_to_power_of_2. The stored scale is the multiplier that
     * maps amax onto 448; rounding to a power of two goes downwards so
     * amax * scale never exceeds 448. */
    const float fp8_max = 448.0f;
    const float eps = 1e-12f;
    float denom = amax > eps ? amax : eps;
    float s = fp8_max / denom;              /* one binary32 division */
    if (pow2) {
        int ex;
        (void)frexpf(s, &ex);               /* s = f * 2^ex, f in [0.5, 1) */
        s = ldexpf(1.0f, ex - 1);           /* 2^floor(log2 s) */
    }
    return s;
}

static int offsets_ok(const int32_t *off, int32_t G, int64_t extent)
{
    int32_t g;
    int64_t prev = 0;
    if (G < 1 || !off)
        return 0;
    for (g = 0; g < G; ++g) {
        if ((int64_t)off[g] < prev)
            return 0;
        prev = off[g];
    }
    return prev == extent;
}

int oracle_quant_groups_dim0(const uint16_t *x, int64_t M, int64_t K,
                             const int32_t *offsets, int32_t G, int pow2,
                             uint8_t *q, float *scales)
{
    /* [BLOCKSIZE] description: per-token-group scaling along dim0. Group g
     * owns rows [off[g-1], off[g]); for every column k of that group the
     * scale comes from max |x| over the group's rows in column k. */
    unsigned env;
    int32_t g;
    if (M < 0 || K < 0 || !offsets_ok(offsets, G, M))
        return -1;
    env = fpenv_enter();
    for (g = 0; g < G; ++g) {
        int64_t r0 = g ? offsets[g - 1] : 0, r1 = offsets[g], r, k;
        float *srow = scales + (int64_t)g * K;
        /* amax per column over the group's rows (0 for an empty group) */
        for (k = 0; k < K; ++k)
            srow[k] = 0.0f;
        for (r = r0; r < r1; ++r)
            for (k = 0; k < K; ++k) {
                float a = fabsf(oracle_bf16_to_f32(x[r * K + k]));
                if (a > srow[k])
                    srow[k] = a;
            }
        /* amax -> scale, in place */
        for (k = 0; k < K; ++k)
            srow[k] = oracle_group_scale(srow[k], pow2);
        /* q = e4m3(fl32(x * s)): the product is rounded to binary32 first */
        for (r = r0; r < r1; ++r)
            for (k = 0; k < K; ++k) {
                float v = oracle_bf16_to_f32(x[r * K + k]) * srow[k];
                q[r * K + k] = oracle_e4m3_encode((double)v);
            }
    }
    fpenv_leave(env);
    return 0;
}

int oracle_quant_groups_dim1(const uint16_t *x, int64_t M, int64_t K,
                             const int32_t *offsets, int32_t G, int pow2,
                             uint8_t *q, float *scales)
{
    /* [ROWWISE] Summary: per-group rowwise scaling. Group g owns columns
     * [off[g-1], off[g]); row r of that group gets one scale from max |x|
     * over those columns of row r. */
    unsigned env;
    int64_t r;
    if (M < 0 || K < 0 || !offsets_ok(offsets, G, K))
        return -1;
    env = fpenv_enter();
    for (r = 0; r < M; ++r) {
        int32_t g;
        for (g = 0; g < G; ++g) {
            int64_t c0 = g ? offsets[g - 1] : 0, c1 = offsets[g], c;
            float amax = 0.0f, s;
            for (c = c0; c < c1; ++c) {
                float a = fabsf(oracle_bf16_to_f32(x[r * K + c]));
                if (a > amax)
                    amax = a;
            }
            s = oracle_group_scale(amax, pow2);
            scales[r * G + g] = s;
            for (c = c0; c < c1; ++c) {
                float v = oracle_bf16_to_f32(x[r * K + c]) * s;
                q[r * K + c] = oracle_e4m3_encode((double)v);
            }
        }
    }
    fpenv_leave(env);
    return 0;
}

/* ---- MX block-32 cast ------------------------------------------------------ */

int oracle_mx_exponent(float amax, int mode)
{
    /* [MXA2A] Summary / investigation comment: FLOOR and RCEIL scaling
     * types. The block is divided by 2^e. FLOOR takes e from the exponent
     * of amax less the exponent of the largest power of two within the
     * E4M3 range (256 = 2^8); RCEIL takes the smallest e that brings amax
     * into [-448, 448]. E8M0 (MX spec) stores e + 127; its range is
     * [-127, 127] (255 is NaN). */
    int e;
    if (amax == 0.0f) {
        e = -127;
    } else {
        int ex, E;
        (void)frexp((double)amax, &ex);     /* exact, also for subnormals */
        E = ex - 1;                         /* floor(log2 amax) */
        if (mode == 0) {
            e = E - 8;
        } else {
            e = E - 9;                      /* 448 * 2^(E-9) < 2^E <= amax */
            while ((double)amax > ldexp(448.0, e))
                ++e;
        }
    }
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

int oracle_mx_quant_dim0(const uint16_t *x, int64_t M, int64_t K, int mode,
                         uint8_t *q, uint8_t *scales)
{
    /* One E8M0 scale per 32 consecutive elements of a row; elements are
     * multiplied by 2^-e exactly and cast to E4M3 with saturation. */
    unsigned env;
    int64_t r, b, nb;
    if (M < 0 || K < 0 || K % 32 != 0 || (mode != 0 && mode != 1))
        return -1;
    nb = K / 32;
    env = fpenv_enter();
    for (r = 0; r < M; ++r)
        for (b = 0; b < nb; ++b) {
            const uint16_t *blk = x + r * K + b * 32;
            float amax = 0.0f;
            int i, e;
            for (i = 0; i < 32; ++i) {
                float a = fabsf(oracle_bf16_to_f32(blk[i]));
                if (a > amax)
                    amax = a;
            }
            e = oracle_mx_exponent(amax, mode);
            scales[r * nb + b] = (uint8_t)(e + 127);
            for (i = 0; i < 32; ++i) {
                double v = (double)oracle_bf16_to_f32(blk[i]) * ldexp(1.0, -e);
                q[r * K + b * 32 + i] = oracle_e4m3_encode(v);
            }
        }
    fpenv_leave(env);
    return 0;
}

/* ---- MX dequantisation -------------------------------------------------- */

uint16_t oracle_f64_to_bf16(double v)
{
    /* Round an exact value once, to nearest even, onto the bf16 grid
     * (8 significant bits, exponents -126..127, subnormal step 2^-133);
     * magnitudes from (2 - 2^-8) * 2^127 up round to infinity. NaN gives
     * the quiet NaN 0x7FC0. */
    uint16_t sign;
    double a, quantum, r;
    int e;
    float f;
    uint32_t w;
    if (v != v)
        return 0x7FC0;
    sign = signbit(v) ? 0x8000 : 0;
    a = fabs(v);
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127))
        return sign | 0x7F80;
    if (a < ldexp(1.0, -126)) {
        quantum = ldexp(1.0, -133);
    } else {
        frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
        quantum = ldexp(1.0, e - 1 - 7);
    }
    r = rint(a / quantum) * quantum;  /* rint: nearest, ties to even */
    f = (float)r;                     /* exact: r is on the bf16 grid */
    memcpy(&w, &f, sizeof w);
    return sign | (uint16_t)(w >> 16);
}

int oracle_mx_dequant_dim0(const uint8_t *q, const uint8_t *scales, int64_t M, int64_t K,
                           uint16_t *y)
{
    /* y = bf16(E4M3(q) * 2^(byte - 127)) per block of 32 along a row (the
     * receiving side of the quantise -> all-to-all -> dequantise pipeline).
     * E8M0 byte 0xFF is NaN (OCP MX), and so is an E4M3 NaN code: both give
     * 0x7FC0. The product of a 4-bit significand and a power of two is exact
     * in binary64, so the one rounding is the cast to bf16. */
    unsigned env;
    int64_t r, k, nb;
    if (M < 0 || K < 0 || K % 32 != 0)
        return -1;
    nb = K / 32;
    env = fpenv_enter();
    for (r = 0; r < M; ++r)
        for (k = 0; k < K; ++k) {
            const uint8_t s = scales[r * nb + k / 32];
            const double d = oracle_e4m3_decode(q[r * K + k]);
            if (s == 0xFF || d != d)
                y[r * K + k] = 0x7FC0;
            else
                y[r * K + k] = oracle_f64_to_bf16(d * ldexp(1.0, (int)s - 127));
        }
    fpenv_leave(env);
    return 0;
}
