/* Host check of the requantiser's quotient: with y = fl(1/b), the one-step
 * q = fma(fma(-b, a*y, a), y, a*y) and the IEEE quotient a/b give the same
 * code rint(.) for every divisor significand (b in [1, 2); the code of a
 * normal-range quotient depends only on the significands) and every
 * dividend a within +-24 ulps of k*b, k = +-0.5 .. +-7.5 (the only places
 * where two quotients a few ulps apart can round to different integers),
 * and also near the binade edges 1, 2, 4, 8.  Prints the counts; exit
 * status 1 on any code mismatch.  Threads: argv[1] (default 8). */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float flt(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

typedef struct { int id, nth; long n, code_bad, quot_bad; } job;

static void *run(void *p)
{
    job *j = p;
    static const float tg[] = {0.5f, 1.5f, 2.5f, 3.5f, 4.5f, 5.5f, 6.5f, 7.5f,
                               1.0f, 2.0f, 4.0f, 8.0f};
    for (uint32_t m = (uint32_t)j->id; m < (1u << 23); m += (uint32_t)j->nth) {
        const float b = flt((127u << 23) | m);
        const float y = 1.0f / b;
        for (int t = 0; t < (int)(sizeof tg / sizeof tg[0]); ++t)
            for (int sgn = 0; sgn < 2; ++sgn) {
                const uint32_t c = bits(tg[t] * b);
                for (int d = -24; d <= 24; ++d) {
                    float a = flt(c + (uint32_t)d);
                    if (sgn) a = -a;
                    const float ref = a / b;
                    const float q0 = a * y;
                    const float q = fmaf(fmaf(-b, q0, a), y, q0);
                    j->n++;
                    if (rintf(q) != rintf(ref)) j->code_bad++;
                    if (bits(q) != bits(ref)) j->quot_bad++;
                }
            }
    }
    return NULL;
}

int main(int argc, char **argv)
{
    int nth = argc > 1 ? atoi(argv[1]) : 8;
    if (nth < 1 || nth > 64) nth = 8;
    pthread_t th[64];
    job jb[64];
    for (int i = 0; i < nth; ++i) {
        jb[i] = (job){i, nth, 0, 0, 0};
        pthread_create(&th[i], NULL, run, &jb[i]);
    }
    long n = 0, cb = 0, qb = 0;
    for (int i = 0; i < nth; ++i) {
        pthread_join(th[i], NULL);
        n += jb[i].n;
        cb += jb[i].code_bad;
        qb += jb[i].quot_bad;
    }
    printf("cases %ld code_mismatches %ld quotient_mismatches %ld\n", n, cb, qb);
    return cb != 0;
}
