/*
 * CPU oracle for the delayed-scaling FP8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this code.  It shares no source, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * Everything here is a plain, slow restatement of what the pages define,
 * written so that it can be checked against them by eye.  The only
 * concession to speed is OpenMP over independent outputs (rows of a cast or a
 * product, columns of a column sum, listed samples): each output is computed
 * exactly as in a single-threaded loop, every sum in the same order, so the
 * results do not depend on the thread count.  It follows:
 *
 *   - the OCP FP8 formats float8_e4m3fn and float8_e5m2 (the finfo table and
 *     the worked cast table in "Accelerating PyTorch Training Workloads with
 *     FP8 -- Part 2", section on PyTorch-native FP8 data types);
 *   - the per-tensor amax and the amax-history "max" recipe with history
 *     length 16 ("CPU Overhead of te.Linear FP8 Layers", the DelayedScaling
 *     recipe in the reproduction script; "support delayed scaling of weight in
 *     float8 all-gather", the amax / amax-history / scale buffers);
 *   - the scale-inverse snapshot held by each FP8 tensor ("[PyTorch] Refactor
 *     FP8 workspaces in linear modules", first motivation);
 *   - the per-tensor-scaled FP8 matrix product with bias (the torch._scaled_mm
 *     example of the Part 2 blog).
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   - the cast computes v = fp32(x) * scale as one IEEE fp32 multiply and
 *     rounds v to FP8 with round-to-nearest-even and SATURATION: every finite
 *     overflow and +-inf goes to +-max, NaN goes to sign|0x7F, where the sign
 *     of a NaN product is sign(x) XOR sign(scale) (IEEE leaves it open);
 *   - amax is the maximum of |x| over the UNSCALED source, ordered by the
 *     sign-cleared fp32 bit pattern (so a NaN dominates everything);
 *   - the scale formula is the conventional one, not printed on the pages:
 *     scale = fp8_max / (max(history) * 2^margin) in fp32, kept unchanged when
 *     the history maximum is zero or not finite or the quotient is not a
 *     finite positive number;
 *   - the product is the exact sum of decoded FP8 products (accumulated here
 *     in fp64), times both scale-inverses, plus bias, rounded once to the
 *     output type.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -fopenmp -ffp-contract=off -fno-fast-math
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* Threads the parallel loops below use (OMP_NUM_THREADS, else all cores). */
int orc_num_threads(void) { return omp_get_max_threads(); }

#define ORC_E4M3 0
#define ORC_E5M2 1

/* Field widths of the two OCP 8-bit formats (Part 2 blog: float8_e4m3fn has
 * 3 mantissa bits, float8_e5m2 has 2). */
typedef struct {
    int ebits;
    int mbits;
    int bias;
} orc_fmt;

static int orc_get_fmt(int fmt, orc_fmt *f) {
    if (fmt == ORC_E4M3) { f->ebits = 4; f->mbits = 3; f->bias = 7;  return 0; }
    if (fmt == ORC_E5M2) { f->ebits = 5; f->mbits = 2; f->bias = 15; return 0; }
    return -1;
}

/* Largest finite magnitude: E4M3 has no infinities and only S.1111.111 is NaN,
 * so its largest finite code is 0x7E = 1.75 * 2^8 = 448; E5M2 keeps IEEE-style
 * infinities, so its largest finite code is 0x7B = 1.75 * 2^15 = 57344. */
double orc_fp8_max(int fmt) {
    orc_fmt f;
    if (orc_get_fmt(fmt, &f)) return NAN;
    if (fmt == ORC_E4M3) return ldexp(1.75, 15 - f.bias);   /* exponent field 15 */
    return ldexp(1.75, 30 - f.bias);                        /* exponent field 30 */
}

static uint8_t orc_max_code(int fmt) { return fmt == ORC_E4M3 ? 0x7E : 0x7B; }

/* Value of an FP8 code, straight from the field definition. */
double orc_fp8_decode(uint8_t code, int fmt) {
    orc_fmt f;
    if (orc_get_fmt(fmt, &f)) return NAN;
    int s = code >> 7;
    int e = (code >> f.mbits) & ((1 << f.ebits) - 1);
    int m = code & ((1 << f.mbits) - 1);
    int emax_field = (1 << f.ebits) - 1;
    double v;
    if (fmt == ORC_E4M3 && e == emax_field && m == (1 << f.mbits) - 1) return NAN;
    if (fmt == ORC_E5M2 && e == emax_field) {
        if (m != 0) return NAN;
        return s ? -INFINITY : INFINITY;
    }
    if (e == 0)
        v = ldexp((double)m, 1 - f.bias - f.mbits);              /* subnormal */
    else
        v = ldexp(1.0 + ldexp((double)m, -f.mbits), e - f.bias); /* normal */
    return s ? -v : v;
}

/* Saturating round-to-nearest-even of an fp32 value to an FP8 code. */
uint8_t orc_fp8_encode(float v, int fmt) {
    orc_fmt f;
    if (orc_get_fmt(fmt, &f)) return 0;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return sign | 0x7F;
    double a = fabs((double)v);
    double maxval = orc_fp8_max(fmt);
    if (a >= maxval) return sign | orc_max_code(fmt);            /* saturate */
    if (a == 0.0) return sign;                                   /* signed zero */

    int emin = 1 - f.bias;                  /* exponent of the smallest normal */
    int ex;
    frexp(a, &ex);                          /* a = g * 2^ex, g in [0.5, 1) */
    int e = ex - 1;                         /* floor(log2(a)) */
    if (e < emin) e = emin;                 /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, e - f.mbits);
    double n = nearbyint(a / quantum);      /* exact division; ties to even */
    double r = n * quantum;                 /* rounded magnitude */
    if (r == 0.0) return sign;
    if (r > maxval) return sign | orc_max_code(fmt);   /* cannot happen, kept for safety */

    /* Re-encode the rounded magnitude. */
    int rex;
    frexp(r, &rex);
    int re = rex - 1;
    int efield, mfield;
    if (re < emin) {                        /* subnormal: r = m * 2^(emin - mbits) */
        efield = 0;
        mfield = (int)ldexp(r, f.mbits - emin);
    } else {
        efield = re + f.bias;
        mfield = (int)(ldexp(r, f.mbits - re) - ldexp(1.0, f.mbits));
    }
    return sign | (uint8_t)((efield << f.mbits) | mfield);
}

/* ---- bfloat16 <-> fp32 ------------------------------------------------ */

static uint32_t orc_f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float orc_bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* bf16 is the top half of an fp32 pattern, so widening is exact. */
float orc_bf16_to_f32(uint16_t b) { return orc_bits_f32((uint32_t)b << 16); }

/* Round a double to the nearest bf16 (8 significant bits, fp32 exponent
 * range with subnormals), ties to even; overflow to infinity. */
uint16_t orc_f64_to_bf16(double x) {
    if (isnan(x)) return signbit(x) ? 0xFFC0 : 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    if (e < -126) e = -126;
    double quantum = ldexp(1.0, e - 7);
    double r = nearbyint(a / quantum) * quantum;
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    /* r is representable in bf16, hence exactly in fp32. */
    return sign | (uint16_t)(orc_f32_bits((float)r) >> 16);
}

/* ---- amax, cast, transpose ------------------------------------------- */

/* Order of magnitudes used for amax: the fp32 pattern with the sign cleared,
 * compared as an unsigned integer.  For non-NaN values this is the order of
 * |x|; every NaN compares above +inf. */
static uint32_t orc_abs_key(float x) { return orc_f32_bits(x) & 0x7FFFFFFFu; }

static float orc_load_src(const void *x, int src, int64_t idx) {
    if (src == 0) return orc_bf16_to_f32(((const uint16_t *)x)[idx]);
    return ((const float *)x)[idx];
}

/*
 * One cast of a row-major [rows, cols] source with leading dimension ld
 * (elements) to FP8 with the given scale.  Writes q [rows, cols] and / or its
 * transpose qt [cols, rows] (either may be NULL), folds |x| into *amax_inout
 * and writes 1/scale to *scale_inv_out (either may be NULL).
 * src: 0 = bf16, 1 = fp32.  Returns 0, or -1 for a bad argument.
 */
int orc_cast_transpose_amax(const void *x, int src, int64_t rows, int64_t cols,
                            int64_t ld, float scale, int fmt, uint8_t *q,
                            uint8_t *qt, float *amax_inout, float *scale_inv_out) {
    orc_fmt f;
    if (orc_get_fmt(fmt, &f) || (src != 0 && src != 1) || rows < 0 || cols < 0 || ld < cols)
        return -1;
    uint32_t amax_key = amax_inout ? orc_abs_key(*amax_inout) : 0u;
#pragma omp parallel for reduction(max : amax_key) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            float xv = orc_load_src(x, src, r * ld + c);
            uint32_t k = orc_abs_key(xv);
            if (k > amax_key) amax_key = k;
            float v = xv * scale;                  /* one fp32 multiply */
            uint8_t code;
            if (isnan(v))   /* sign of a NaN product: the multiply's sign rule */
                code = 0x7F | ((signbit(xv) ? 0x80 : 0) ^ (signbit(scale) ? 0x80 : 0));
            else
                code = orc_fp8_encode(v, fmt);
            if (q) q[r * cols + c] = code;
            if (qt) qt[c * rows + r] = code;
        }
    }
    if (amax_inout) *amax_inout = orc_bits_f32(amax_key);
    if (scale_inv_out) *scale_inv_out = 1.0f / scale;
    return 0;
}

/*
 * Bias gradient of y = x W^T + b over a row-major [rows, cols] output
 * gradient dY with leading dimension ld (elements): dbias[c] = sum over r of
 * dY[r, c], of the unscaled source.  The training loop of "CPU Overhead of
 * te.Linear FP8 Layers" (reproduction script: biased linears, fp32
 * parameters in the FP8 run, loss.backward()) needs it for every biased
 * linear.  The sum is accumulated in fp64 (exact whenever the inputs'
 * exponent span and count fit in fp64's 53-bit significand, as for every
 * test input; otherwise the fp64 sum is the reference) and rounded once to
 * fp32.  src: 0 = bf16, 1 = fp32.
 * Returns 0, or -1 for a bad argument.
 */
int orc_dbias(const void *x, int src, int64_t rows, int64_t cols, int64_t ld, float *dbias) {
    if ((src != 0 && src != 1) || rows < 0 || cols < 0 || ld < cols || !dbias) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        double acc = 0.0;
        for (int64_t r = 0; r < rows; ++r) acc += (double)orc_load_src(x, src, r * ld + c);
        dbias[c] = (float)acc;
    }
    return 0;
}

/*
 * Producer-fused cast: the elementwise operation that produces a linear's
 * input in the toy block of "CPU Overhead of te.Linear FP8 Layers"
 * (reproduction script, TEBlock.forward: the modulation multiplies the block
 * input by one column slice of the modulation linear's output and divides it
 * by another; the residual adds put linear outputs back onto the stream),
 * rounded to bf16, followed by the cast of its result.  All arithmetic in
 * fp32, as torch does for bf16 tensors:
 *   op 1 (modulate): y = bf16(a * x / b), one multiply then one correctly
 *        rounded division, round to nearest even.  Nothing is sanitised: a
 *        zero divisor gives +-inf, 0/0 gives NaN, a quotient beyond the bf16
 *        range rounds to +-inf; a NaN result is written as 0x7FC0;
 *   op 2 (residual add): y = bf16(x + a); a NaN result is 0x7FC0;
 *   op 3 (residual add of two terms, as the block adds the cross-attention
 *        outputs): y = bf16(bf16(x + a) + b), the two bf16 adds torch performs
 *        one after the other, each rounded; a NaN at either step is 0x7FC0;
 *   op 4 (the library's finite modulation, on no page): op 1, then a y that
 *        is infinite or NaN becomes +0.
 * x, a, b are bf16 [rows, cols] with leading dimensions ldx, lda, ldb (b is
 * read by ops 1 and 3); y is bf16 [rows, cols], row-major.  The cast is then
 * exactly orc_cast_transpose_amax of y (so +-inf saturates to +-max and NaN
 * becomes 0x7F with its sign).  Returns 0, or -1 for a bad argument.
 */
static uint16_t orc_f32_to_bf16_canon(float f) {
    if (isnan(f)) return 0x7FC0;
    return orc_f64_to_bf16((double)f);   /* f is exact in fp64: one rounding */
}

int orc_produce_cast(int op, const uint16_t *x, int64_t ldx, const uint16_t *a, int64_t lda,
                     const uint16_t *b, int64_t ldb, int64_t rows, int64_t cols, float scale,
                     int fmt, uint16_t *y, uint8_t *q, uint8_t *qt, float *amax_inout,
                     float *scale_inv_out) {
    if ((op < 1 || op > 4) || rows < 0 || cols < 0 || ldx < cols || lda < cols ||
        !y || (op != 2 && (!b || ldb < cols)))
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            float xv = orc_bf16_to_f32(x[r * ldx + c]);
            float av = orc_bf16_to_f32(a[r * lda + c]);
            uint16_t out;
            if (op == 1 || op == 4) {
                float bv = orc_bf16_to_f32(b[r * ldb + c]);
                float prod = av * xv;
                out = orc_f32_to_bf16_canon(prod / bv);
                if (op == 4 && !isfinite(orc_bf16_to_f32(out))) out = 0x0000;
            } else if (op == 2) {
                out = orc_f32_to_bf16_canon(xv + av);
            } else {
                float t = orc_bf16_to_f32(orc_f32_to_bf16_canon(xv + av));
                float bv = orc_bf16_to_f32(b[r * ldb + c]);
                out = orc_f32_to_bf16_canon(t + bv);
            }
            y[r * cols + c] = out;
        }
    }
    return orc_cast_transpose_amax(y, 0, rows, cols, cols, scale, fmt, q, qt, amax_inout,
                                   scale_inv_out);
}

/*
 * Gradient of the modulation producer (ops 1 and 4 above) with respect to
 * its three inputs.  The forward is y = a * x / b; with the gradient dy of y,
 * its derivatives are dx = dy * a / b, da = dy * x / b and
 * db = -dy * (a * x / b) / b.  Steps, each an fp32 operation rounded to
 * nearest even on the exactly widened bf16 inputs:
 *   u  = (a * x) / b     the forward's quotient before its bf16 rounding
 *   t  = dy / b
 *   dx = bf16(t * a),  da = bf16(t * x),  db = bf16(-(t * u))
 * A NaN result is written as 0x7FC0.  Op 4 (the finite modulation): where the
 * forward's y = bf16(u) is infinite or NaN, the forward wrote the constant +0,
 * so dx, da and db are +0 there.  All tensors bf16 [rows, cols] with their
 * own leading dimensions.  Returns 0, or -1 for a bad argument.
 */
int orc_modulate_backward(int op, const uint16_t *dy, int64_t lddy, const uint16_t *x,
                          int64_t ldx, const uint16_t *a, int64_t lda, const uint16_t *b,
                          int64_t ldb, int64_t rows, int64_t cols, uint16_t *dx, int64_t lddx,
                          uint16_t *da, int64_t ldda, uint16_t *db, int64_t lddb) {
    if ((op != 1 && op != 4) || rows < 0 || cols < 0 || !dy || !x || !a || !b || !dx || !da ||
        !db || lddy < cols || ldx < cols || lda < cols || ldb < cols || lddx < cols ||
        ldda < cols || lddb < cols)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            float gv = orc_bf16_to_f32(dy[r * lddy + c]);
            float xv = orc_bf16_to_f32(x[r * ldx + c]);
            float av = orc_bf16_to_f32(a[r * lda + c]);
            float bv = orc_bf16_to_f32(b[r * ldb + c]);
            float prod = av * xv;
            float u = prod / bv;
            float t = gv / bv;
            float ta = t * av, tx = t * xv, tu = t * u;
            uint16_t ox = orc_f32_to_bf16_canon(ta);
            uint16_t oa = orc_f32_to_bf16_canon(tx);
            uint16_t ob = orc_f32_to_bf16_canon(-tu);
            if (op == 4 && !isfinite(orc_bf16_to_f32(orc_f32_to_bf16_canon(u))))
                ox = oa = ob = 0x0000;
            dx[r * lddx + c] = ox;
            da[r * ldda + c] = oa;
            db[r * lddb + c] = ob;
        }
    }
    return 0;
}

/*
 * Dynamic scaling, the comparator of delayed scaling: "support delayed
 * scaling of weight in float8 all-gather" contrasts the two recipes
 * (dynamic scaling reads a tensor twice -- once for its amax, once for the
 * cast -- where delayed scaling takes the amax in the cast's own read).  Here:
 *   amax  = max |x| of this very tensor (sign-cleared fp32 bit order);
 *   scale = fp8_max / (amax * 2^margin) in fp32, with the scale update's
 *           guard: *scale_inout is kept when amax is zero or not finite or
 *           the quotient is not a finite positive number;
 * then the cast of x with that scale, as orc_cast_transpose_amax (no amax
 * accumulation).  Writes *amax_out, *scale_inout and *scale_inv_out.
 * Returns 0, or -1 for a bad argument.
 */
int orc_dynamic_cast(const void *x, int src, int64_t rows, int64_t cols, int64_t ld, int margin,
                     int fmt, float *scale_inout, uint8_t *q, uint8_t *qt, float *amax_out,
                     float *scale_inv_out) {
    orc_fmt f;
    if (orc_get_fmt(fmt, &f) || (src != 0 && src != 1) || rows < 0 || cols < 0 || ld < cols ||
        !scale_inout || !amax_out)
        return -1;
    uint32_t best = 0;
#pragma omp parallel for reduction(max : best) schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint32_t k = orc_abs_key(orc_load_src(x, src, r * ld + c));
            if (k > best) best = k;
        }
    float amax = orc_bits_f32(best);
    *amax_out = amax;
    if (isfinite(amax) && amax > 0.0f) {
        float fp8_max = (float)orc_fp8_max(fmt);
        float s = fp8_max / ldexpf(amax, margin);   /* fp32, correctly rounded */
        if (isfinite(s) && s > 0.0f) *scale_inout = s;
    }
    return orc_cast_transpose_amax(x, src, rows, cols, ld, *scale_inout, fmt, q, qt, NULL,
                                   scale_inv_out);
}

/* ---- amax history and scale update ----------------------------------- */

/*
 * Delayed-scaling update of T per-tensor records at once.
 *   hist      [T, H]  amax history, newest first (hist[t*H + 0])
 *   amax_cur  [T]     amax recorded since the last update; reset to 0 here
 *   scale     [T]     quantisation scale used by the next casts
 *   scale_inv [T]     1 / scale
 *   fmt       [T]     0 = E4M3, 1 = E5M2 (selects fp8_max)
 * algo 0 = "max" over the history window (the only algorithm the pages use).
 * Returns 0, or -1 for a bad argument.
 */
int orc_scale_update(float *hist, float *amax_cur, float *scale, float *scale_inv,
                     const uint8_t *fmt, int T, int H, int margin, int algo) {
    if (T < 0 || H < 1 || algo != 0) return -1;
    for (int t = 0; t < T; ++t) {
        if (fmt[t] != ORC_E4M3 && fmt[t] != ORC_E5M2) return -1;
    }
    for (int t = 0; t < T; ++t) {
        float *h = hist + (int64_t)t * H;
        /* Roll the window by one and record the newest amax in front. */
        for (int i = H - 1; i > 0; --i) h[i] = h[i - 1];
        h[0] = amax_cur[t];
        /* "max" over the window, in the same order as amax itself. */
        uint32_t best = orc_abs_key(h[0]);
        float m = h[0];
        for (int i = 1; i < H; ++i) {
            uint32_t k = orc_abs_key(h[i]);
            if (k > best) { best = k; m = h[i]; }
        }
        m = fabsf(m);
        if (isfinite(m) && m > 0.0f) {
            float fp8_max = (float)orc_fp8_max(fmt[t]);
            float denom = ldexpf(m, margin);
            float s = fp8_max / denom;             /* fp32, correctly rounded */
            if (isfinite(s) && s > 0.0f) scale[t] = s;
        }
        scale_inv[t] = 1.0f / scale[t];
        amax_cur[t] = 0.0f;
    }
    return 0;
}

/* ---- scaled FP8 matrix product --------------------------------------- */

static double orc_bias_at(const uint16_t *bias, int64_t j) {
    return bias ? (double)orc_bf16_to_f32(bias[j]) : 0.0;
}

static void orc_store_out(void *out, int out_kind, int64_t idx, double y) {
    if (out_kind == 0)
        ((uint16_t *)out)[idx] = orc_f64_to_bf16(y);
    else
        ((float *)out)[idx] = (float)y;
}

/* Decoded copy of rows [0, n) of an FP8 matrix with K columns (stride ld). */
static double *orc_decode_rows(const uint8_t *X, int fmt, int64_t ld, int64_t n, int64_t K) {
    double *d = (double *)malloc((size_t)(n * K > 0 ? n * K : 1) * sizeof(double));
    if (!d) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = 0; k < K; ++k) d[i * K + k] = orc_fp8_decode(X[i * ld + k], fmt);
    return d;
}

/* sum_k a[k] * b[k], k ascending, in fp64 (FP8 x FP8 products are exact). */
static double orc_dot(const double *a, const double *b, int64_t K) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += a[k] * b[k];
    return acc;
}

/*
 * out[i, j] = round_out( (sum_k dec(A[i,k]) * dec(B[j,k])) * sinv_a * sinv_b
 *                        + bias[j] )
 * A is [M, K] row-major (lda), B is [N, K] row-major (ldb): the "NT" product
 * torch._scaled_mm computes for a row-major first operand and a transposed
 * second one.  out is [M, N] row-major (ldo); out_kind 0 = bf16 (RNE),
 * 1 = fp32 (RNE).  bias is bf16 [N] or NULL.  Returns 0 or -1.
 */
int orc_gemm_nt(const uint8_t *A, int fa, int64_t lda, const uint8_t *B, int fb,
                int64_t ldb, int64_t M, int64_t N, int64_t K, float sinv_a,
                float sinv_b, const uint16_t *bias, int out_kind, void *out,
                int64_t ldo) {
    orc_fmt f;
    if (orc_get_fmt(fa, &f) || orc_get_fmt(fb, &f) || M < 0 || N < 0 || K < 0 ||
        (out_kind != 0 && out_kind != 1))
        return -1;
    double *da = orc_decode_rows(A, fa, lda, M, K);
    double *db = orc_decode_rows(B, fb, ldb, N, K);
    if (!da || !db) { free(da); free(db); return -1; }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double acc = orc_dot(da + i * K, db + j * K, K);
            double y = acc * (double)sinv_a * (double)sinv_b + orc_bias_at(bias, j);
            orc_store_out(out, out_kind, i * ldo + j, y);
        }
    free(da);
    free(db);
    return 0;
}

/*
 * FP8-output form of the product: torch._scaled_mm called with an FP8
 * out_dtype returns the FP8 output together with its amax (the example in
 * the Part 2 blog, section on torch._scaled_mm).  The pages print the call,
 * not its arithmetic; the reading taken here is "the fp32 product, then the
 * ordinary cast of it":
 *   v[i, j]   = fp32( acc * sinv_a * sinv_b + bias[j] ), rounded once, as the
 *               fp32 output of orc_gemm_nt;
 *   codes     = the cast of v with the output's own scale (one fp32 multiply,
 *               saturating round-to-nearest-even, NaN -> sign|0x7F);
 *   *amax_inout folds in max |v| over the UNSCALED v -- the amax that a
 *               delayed-scaling history of the output records, as the cast
 *               records the amax of its unscaled source;
 *   *scale_inv_out = 1 / scale_out, the output's scale-inverse snapshot.
 * codes is [M, N] row-major (ldo).  v_out (fp32 [M, N], row-major, may be
 * NULL) receives v.  Returns 0 or -1.
 */
int orc_gemm_nt_fp8out(const uint8_t *A, int fa, int64_t lda, const uint8_t *B, int fb,
                       int64_t ldb, int64_t M, int64_t N, int64_t K, float sinv_a,
                       float sinv_b, const uint16_t *bias, float scale_out, int fo,
                       uint8_t *codes, int64_t ldo, float *v_out, float *amax_inout,
                       float *scale_inv_out) {
    orc_fmt f;
    if (orc_get_fmt(fo, &f) || M < 0 || N < 0 || ldo < N || !codes) return -1;
    float *v = (float *)malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(float));
    if (!v) return -1;
    int rc = orc_gemm_nt(A, fa, lda, B, fb, ldb, M, N, K, sinv_a, sinv_b, bias, 1, v, N);
    if (rc == 0) {
        uint8_t *q = (uint8_t *)malloc((size_t)(M * N > 0 ? M * N : 1));
        if (!q) rc = -1;
        else {
            rc = orc_cast_transpose_amax(v, 1, M, N, N, scale_out, fo, q, NULL, amax_inout,
                                         scale_inv_out);
            for (int64_t i = 0; rc == 0 && i < M; ++i)
                memcpy(codes + i * ldo, q + i * N, (size_t)N);
            free(q);
        }
        if (rc == 0 && v_out) memcpy(v_out, v, (size_t)(M * N) * sizeof(float));
    }
    free(v);
    return rc;
}

/* The same definition evaluated only at the listed (rows[s], cols[s]) pairs;
 * out receives `count` values of the output type, in list order. */
int orc_gemm_nt_sampled(const uint8_t *A, int fa, int64_t lda, const uint8_t *B,
                        int fb, int64_t ldb, int64_t K, float sinv_a, float sinv_b,
                        const uint16_t *bias, int out_kind, const int64_t *rows,
                        const int64_t *cols, int64_t count, void *out) {
    orc_fmt f;
    if (orc_get_fmt(fa, &f) || orc_get_fmt(fb, &f) || K < 0 || count < 0 ||
        (out_kind != 0 && out_kind != 1))
        return -1;
    double *da = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    double *db = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    if (!da || !db) { free(da); free(db); return -1; }
    for (int64_t s = 0; s < count; ++s) {
        for (int64_t k = 0; k < K; ++k) {
            da[k] = orc_fp8_decode(A[rows[s] * lda + k], fa);
            db[k] = orc_fp8_decode(B[cols[s] * ldb + k], fb);
        }
        double acc = orc_dot(da, db, K);
        double y = acc * (double)sinv_a * (double)sinv_b + orc_bias_at(bias, cols[s]);
        orc_store_out(out, out_kind, s, y);
    }
    free(da);
    free(db);
    return 0;
}
