/* The FP8 quantiser's fast quotient, checked over every input it can meet.
 *
 * For a row with amax a (a positive finite BF16 value) the scale is
 * s = fl32(a / 448), and the kernel forms, for each BF16 weight w with
 * |w| <= a,
 *     t = fl32(w * rs),  r = fma(-t, s, w),  y = -fma(-r, rs, -t),
 * with rs = fl32(1 / s), in place of the correctly rounded y0 = fl32(w / s).
 * This program checks, for every such (a, w) with s >= 2^-100 (the rows the
 * kernel sends this way), that the E4M3FN code of y equals that of y0, both
 * encoded by the oracle's encoder (orc_e4m3_encode, which saturates to 448).
 * Rows are split over threads.  Prints the counts; exit status 1 on any
 * difference.  Built and run by tests/test_quant_math_cpu.py. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint8_t orc_e4m3_encode(float y);

static float bf(uint32_t b)
{
    uint32_t u = b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

typedef struct {
    uint32_t a0, a1;
    long long pairs, same_quotient, code_diff;
} job;

static void *run(void *p)
{
    job *j = (job *)p;
    for (uint32_t a = j->a0; a < j->a1; ++a) {
        const float amax = bf(a);
        const float s = amax / 448.0f;
        if (!(s >= 0x1p-100f))
            continue;
        const float rs = 1.0f / s;
        for (uint32_t wb = 0; wb < 0x10000u; ++wb) {
            if ((wb & 0x7FFFu) > a)
                continue;
            const float w = bf(wb);
            const float t = w * rs;
            const float r = fmaf(-t, s, w);
            const float y = -fmaf(-r, rs, -t);
            const float y0 = w / s;
            j->pairs++;
            if (bits(y) == bits(y0)) {
                j->same_quotient++;
                continue;
            }
            if (orc_e4m3_encode(y) != orc_e4m3_encode(y0)) {
                if (j->code_diff < 5)
                    printf("amax %a w %a: %a vs %a\n", amax, w, y, y0);
                j->code_diff++;
            }
        }
    }
    return NULL;
}

int main(int argc, char **argv)
{
    int nt = argc > 1 ? atoi(argv[1]) : 8;
    if (nt < 1 || nt > 64)
        nt = 8;
    pthread_t th[64];
    job jobs[64];
    const uint32_t top = 0x7F80u; /* positive finite BF16 patterns 1 .. 0x7F7F */
    for (int i = 0; i < nt; ++i) {
        /* interleave-free contiguous ranges weighted toward large a (more w) */
        jobs[i].a0 = 1u + (uint32_t)((top - 1u) * sqrt((double)i / nt));
        jobs[i].a1 = 1u + (uint32_t)((top - 1u) * sqrt((double)(i + 1) / nt));
        jobs[i].pairs = jobs[i].same_quotient = jobs[i].code_diff = 0;
        pthread_create(&th[i], NULL, run, &jobs[i]);
    }
    long long pairs = 0, same = 0, diff = 0;
    for (int i = 0; i < nt; ++i) {
        pthread_join(th[i], NULL);
        pairs += jobs[i].pairs;
        same += jobs[i].same_quotient;
        diff += jobs[i].code_diff;
    }
    printf("pairs %lld same quotient %lld code differences %lld\n", pairs, same, diff);
    return diff != 0;
}
