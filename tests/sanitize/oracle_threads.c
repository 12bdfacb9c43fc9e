/* Drives the oracle's row-parallel loops (pthreads split independent rows)
 * from 1 to 24 threads and checks that every thread count gives the same bits.
 * Built with a thread sanitizer by tests/test_sanitizers_cpu.py, so a data
 * race between the row workers is reported as well. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_gemv_bf16(const uint16_t *W, int64_t n, int64_t k, const uint16_t *x, double *out,
                   int nthreads);
void orc_gemv_fp8(const uint8_t *q, const float *s, int64_t n, int64_t k, const uint16_t *x,
                  double *out, int nthreads);
int orc_quantize_fp8(const uint16_t *L, int64_t V, int64_t H, uint8_t *q, float *s, int nthreads);

static uint32_t lcg = 12345u;
static uint16_t rnd_bf16(void)
{
    lcg = lcg * 1664525u + 1013904223u;
    /* a finite BF16 pattern between about 2^-8 and 2^7, either sign */
    uint16_t exp = (uint16_t)(119 + (lcg >> 28));
    return (uint16_t)(((lcg >> 16) & 0x8000u) | (exp << 7) | ((lcg >> 9) & 0x7Fu));
}

int main(void)
{
    const int64_t n = 203, k = 96;
    uint16_t *W = malloc(sizeof(uint16_t) * n * k), *x = malloc(sizeof(uint16_t) * k);
    uint8_t *q = malloc(n * k), *q1 = malloc(n * k);
    float *s = malloc(sizeof(float) * n), *s1 = malloc(sizeof(float) * n);
    double *y = malloc(sizeof(double) * n), *y1 = malloc(sizeof(double) * n);
    for (int64_t i = 0; i < n * k; ++i)
        W[i] = rnd_bf16();
    for (int64_t i = 0; i < k; ++i)
        x[i] = rnd_bf16();
    int bad = 0;
    orc_gemv_bf16(W, n, k, x, y1, 1);
    if (orc_quantize_fp8(W, n, k, q1, s1, 1) != 0)
        bad = 1;
    for (int t = 2; t <= 24; t += 3) {
        orc_gemv_bf16(W, n, k, x, y, t);
        bad |= memcmp(y, y1, sizeof(double) * n) != 0;
        if (orc_quantize_fp8(W, n, k, q, s, t) != 0)
            bad = 1;
        bad |= memcmp(q, q1, n * k) != 0 || memcmp(s, s1, sizeof(float) * n) != 0;
        double *z = malloc(sizeof(double) * n), *z1 = malloc(sizeof(double) * n);
        orc_gemv_fp8(q, s, n, k, x, z, t);
        orc_gemv_fp8(q, s, n, k, x, z1, 1);
        bad |= memcmp(z, z1, sizeof(double) * n) != 0;
        free(z);
        free(z1);
    }
    /* more threads than rows */
    orc_gemv_bf16(W, 3, k, x, y, 16);
    bad |= memcmp(y, y1, sizeof(double) * 3) != 0;
    free(W); free(x); free(q); free(q1); free(s); free(s1); free(y); free(y1);
    printf(bad ? "MISMATCH\n" : "threads ok\n");
    return bad;
}
