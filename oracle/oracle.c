/*
 * oracle.c -- plain, slow, FP64 reference for the MTP draft sweep.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark load it (through oracle/__init__.py).  It shares no code,
 * header or table with the HIP path.
 *
 * Sources (web pages of the metrale API docs):
 *   [MTP]   metrale_model_arch/glm5next_mtp_head.rs  -- module doc (the draft
 *           formula), `forward_one`, the `head_fp8` field doc, `norm`.
 *   [LAYER] metrale_model_arch/glm5next_layer/mod.rs -- module invariants
 *           (every norm is `rms_norm_vanilla`, x*w/rms, never 1+w).
 *
 * Every reduction below is a sequential loop in index order, accumulated in
 * double.  Threads (pthreads), where offered, only split independent output
 * rows, so results do not depend on the thread count.
 *
 * Readings where the pages are silent:
 *   rms = sqrt(mean(x^2) + eps) with eps passed as f32; BF16 rounding (RNE) after
 *   each norm, after eh_proj and for the logits; FP8 is OCP E4M3FN with a per-row
 *   f32 scale amax/448, y = fl32(w/s), saturate to +-448, round to nearest even;
 *   argmax over the BF16 logits, lowest index on ties.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* BF16 is the top half of an IEEE binary32; widening is exact. */
double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One correctly rounded step double -> BF16, round to nearest, ties to even.
 * BF16 keeps 8 significant bits; its smallest quantum (subnormals) is 2^-133.
 * For |x| in [2^(e-1), 2^e) the quantum is 2^(e-8).  Scaling by a power of two
 * is exact, nearbyint() rounds half to even in the default rounding mode, and
 * the rounded value has at most 8 significant bits, so the final conversion to
 * float is exact.  Overflow, NaN and Inf are outside the contract. */
uint16_t orc_bf16_from_double(double x)
{
    if (x == 0.0)
        return signbit(x) ? 0x8000u : 0x0000u;
    int e;
    (void)frexp(x, &e);
    int qe = e - 8;
    if (qe < -133)
        qe = -133;
    double r = ldexp(nearbyint(ldexp(x, -qe)), qe);
    float f = (float)r;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t b = (uint16_t)(u >> 16);
    if (r == 0.0) /* rounded to zero: keep the sign of x */
        b = signbit(x) ? 0x8000u : 0x0000u;
    return b;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; largest finite magnitude 1.75 * 2^8 = 448.
 * Normal  (E >= 1): (1 + M/8) * 2^(E-7);  subnormal (E == 0): (M/8) * 2^-6. */
double orc_e4m3_decode(uint8_t c)
{
    int s = (c >> 7) & 1;
    int E = (c >> 3) & 15;
    int M = c & 7;
    if (E == 15 && M == 7)
        return NAN;
    double mag = (E == 0) ? ldexp((double)M / 8.0, -6) : ldexp(1.0 + (double)M / 8.0, E - 7);
    return s ? -mag : mag;
}

/* Nearest E4M3FN code of y, saturating to +-448, ties to the even code, sign of
 * zero kept.  E4M3 keeps 4 significant bits; for |y| in [2^(e-1), 2^e) the
 * quantum is 2^(e-4), never below the subnormal quantum 2^-9.  Because the
 * codes are ordered by magnitude and an even code has an even mantissa field,
 * rounding the scaled significand half-to-even picks the even code on a tie. */
uint8_t orc_e4m3_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80u : 0x00u;
    double a = fabs((double)y);
    if (a > 448.0)
        a = 448.0;
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);
    int qe = e - 4;
    if (qe < -9)
        qe = -9;
    double r = ldexp(nearbyint(ldexp(a, -qe)), qe);
    if (r > 448.0) /* cannot happen after the clamp; kept for clarity */
        r = 448.0;
    if (r == 0.0)
        return sign;
    /* Re-express the rounded magnitude as a code. */
    (void)frexp(r, &e); /* r in [2^(e-1), 2^e) */
    int E = (e - 1) + 7;
    uint8_t code;
    if (E >= 1) {
        double m = ldexp(r, -(e - 1)); /* in [1, 2) with 3 fraction bits */
        int M = (int)((m - 1.0) * 8.0);
        code = (uint8_t)((E << 3) | M);
    } else {
        int M = (int)ldexp(r, 9); /* r = M * 2^-9, M in 1..7 */
        code = (uint8_t)M;
    }
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------ */
/* Draft-sweep steps                                                         */
/* ------------------------------------------------------------------------ */

/* rms_norm_vanilla ([LAYER] invariants; launched by `norm` in [MTP]):
 * out_j = BF16(x_j * w_j / sqrt(sum_i x_i^2 / n + eps)). */
static double rms_of(const uint16_t *x, int64_t n, float eps)
{
    double ss = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double v = orc_bf16_to_double(x[j]);
        ss += v * v;
    }
    return sqrt(ss / (double)n + (double)eps);
}

void orc_rmsnorm(const uint16_t *x, const uint16_t *w, int64_t n, float eps, uint16_t *out)
{
    double r = rms_of(x, n, eps);
    for (int64_t j = 0; j < n; ++j)
        out[j] = orc_bf16_from_double(orc_bf16_to_double(x[j]) * orc_bf16_to_double(w[j]) / r);
}

/* The same norm with each output left in FP64, before the BF16 rounding that
 * orc_rmsnorm applies: the value every stored element is rounded from. */
void orc_rmsnorm_unrounded(const uint16_t *x, const uint16_t *w, int64_t n, float eps,
                           double *out)
{
    double r = rms_of(x, n, eps);
    for (int64_t j = 0; j < n; ++j)
        out[j] = orc_bf16_to_double(x[j]) * orc_bf16_to_double(w[j]) / r;
}

/* Gather + enorm + hnorm + concat ([MTP] module doc and `forward_one`):
 * concat[0:H] = enorm(embed[token]), concat[H:2H] = hnorm(hidden).
 * The embedding row is contiguous in the [V][H] table.  Returns -1 (and writes
 * nothing) when token >= V. */
int orc_front(const uint16_t *embed, int64_t V, int64_t H, uint32_t token,
              const uint16_t *hidden, const uint16_t *enorm_w, const uint16_t *hnorm_w,
              float eps, uint16_t *concat)
{
    if ((int64_t)token >= V)
        return -1;
    orc_rmsnorm(embed + (int64_t)token * H, enorm_w, H, eps, concat);
    orc_rmsnorm(hidden, hnorm_w, H, eps, concat + H);
    return 0;
}

/* y_i = sum_j W[i][j] * x_j over a row-major [n][k] BF16 matrix, unrounded. */
typedef struct {
    const uint16_t *W;
    const uint8_t *q;
    const float *s;
    const uint16_t *x;
    double *out;
    int64_t k, r0, r1;
} rows_job;

static void *gemv_bf16_rows(void *p)
{
    rows_job *jb = (rows_job *)p;
    for (int64_t i = jb->r0; i < jb->r1; ++i) {
        const uint16_t *row = jb->W + i * jb->k;
        double acc = 0.0;
        for (int64_t j = 0; j < jb->k; ++j)
            acc += orc_bf16_to_double(row[j]) * orc_bf16_to_double(jb->x[j]);
        jb->out[i] = acc;
    }
    return NULL;
}

/* FP8-weight row: s_i * sum_j dec(q[i][j]) * x_j, the scale applied once. */
static void *gemv_fp8_rows(void *p)
{
    rows_job *jb = (rows_job *)p;
    double dec[256];
    for (int c = 0; c < 256; ++c)
        dec[c] = orc_e4m3_decode((uint8_t)c);
    for (int64_t i = jb->r0; i < jb->r1; ++i) {
        const uint8_t *row = jb->q + i * jb->k;
        double acc = 0.0;
        for (int64_t j = 0; j < jb->k; ++j)
            acc += dec[row[j]] * orc_bf16_to_double(jb->x[j]);
        jb->out[i] = (double)jb->s[i] * acc;
    }
    return NULL;
}

static void run_rows(void *(*fn)(void *), rows_job base, int64_t n, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > n)
        nthreads = n > 0 ? (int)n : 1;
    pthread_t th[256];
    int started[256] = {0};
    rows_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].r0 = n * t / nthreads;
        jobs[t].r1 = n * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) {
        started[t] = pthread_create(&th[t], NULL, fn, &jobs[t]) == 0;
        if (!started[t])
            fn(&jobs[t]); /* no thread available: do the rows here */
    }
    fn(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (started[t])
            pthread_join(th[t], NULL);
}

/* dense_gemv ([MTP] `forward_one`: eh_proj with n=H, k=2H; lm_head with n=V,
 * k=H): W is row-major [n][k]. */
void orc_gemv_bf16(const uint16_t *W, int64_t n, int64_t k, const uint16_t *x, double *out,
                   int nthreads)
{
    rows_job b = {W, NULL, NULL, x, out, k, 0, 0};
    run_rows(gemv_bf16_rows, b, n, nthreads);
}

/* dense_gemv_fp8w ([MTP] `forward_one`, `head_fp8` doc): the FP8 E4M3 copy of
 * lm_head, per-row scale. */
void orc_gemv_fp8(const uint8_t *q, const float *s, int64_t n, int64_t k, const uint16_t *x,
                  double *out, int nthreads)
{
    rows_job b = {NULL, q, s, x, out, k, 0, 0};
    run_rows(gemv_fp8_rows, b, n, nthreads);
}

void orc_round_bf16(const double *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_from_double(in[i]);
}

/* argmax over BF16 logits ([MTP] `forward_one` argmax_bf16; lower index wins a
 * tie, as the cross-rank pick's `>=` makes the lower rank win).  Values compare
 * as numbers, so -0 == +0. */
int64_t orc_argmax_bf16(const uint16_t *logits, int64_t n)
{
    int64_t best = 0;
    double bv = orc_bf16_to_double(logits[0]);
    for (int64_t i = 1; i < n; ++i) {
        double v = orc_bf16_to_double(logits[i]);
        if (v > bv) {
            bv = v;
            best = i;
        }
    }
    return best;
}

/* FP8 quantisation of lm_head ([MTP] `head_fp8` doc: an E4M3 copy for drafting
 * only, which may fail).  Per row v:
 *   a   = max_j |L[v][j]|          (any NaN/Inf: failure)
 *   s_v = a > 0 ? fl32(a / 448) : 1
 *   q   = E4M3FN_RNE(clamp(fl32(L[v][j] / s_v), -448, 448))
 * Returns 0, or 1 when a weight is not finite (q and s are then unspecified). */
typedef struct {
    const uint16_t *L;
    uint8_t *q;
    float *s;
    int64_t H, r0, r1;
    int bad;
} quant_job;

static void *quant_rows(void *p)
{
    quant_job *jb = (quant_job *)p;
    for (int64_t v = jb->r0; v < jb->r1; ++v) {
        const uint16_t *row = jb->L + v * jb->H;
        float a = 0.0f;
        for (int64_t j = 0; j < jb->H; ++j) {
            float w = (float)orc_bf16_to_double(row[j]);
            if (!isfinite(w))
                jb->bad = 1;
            float m = fabsf(w);
            if (m > a)
                a = m;
        }
        float s = (a > 0.0f) ? a / 448.0f : 1.0f;
        jb->s[v] = s;
        for (int64_t j = 0; j < jb->H; ++j) {
            float y = (float)orc_bf16_to_double(row[j]) / s;
            if (y > 448.0f)
                y = 448.0f;
            if (y < -448.0f)
                y = -448.0f;
            jb->q[v * jb->H + j] = orc_e4m3_encode(y);
        }
    }
    return NULL;
}

int orc_quantize_fp8(const uint16_t *L, int64_t V, int64_t H, uint8_t *q, float *s, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > V)
        nthreads = V > 0 ? (int)V : 1;
    pthread_t th[256];
    int started[256] = {0};
    quant_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        quant_job j = {L, q, s, H, V * t / nthreads, V * (t + 1) / nthreads, 0};
        jobs[t] = j;
    }
    for (int t = 1; t < nthreads; ++t) {
        started[t] = pthread_create(&th[t], NULL, quant_rows, &jobs[t]) == 0;
        if (!started[t])
            quant_rows(&jobs[t]);
    }
    quant_rows(&jobs[0]);
    int bad = jobs[0].bad;
    for (int t = 1; t < nthreads; ++t) {
        if (started[t])
            pthread_join(th[t], NULL);
        bad |= jobs[t].bad;
    }
    return bad ? 1 : 0;
}
