/* Exhaustive pin of the oracle's bf16 hop: every one of the 2^32 (a, b) pairs
 * of bf16 bit patterns.  Test code, not part of the oracle or the library.
 *
 * Reference route, sharing nothing with the oracle's own arithmetic:
 *   1. a + b in fp64.  Two bf16 values sum exactly in fp64 when their exponents
 *      differ by at most 45; beyond that the smaller one is below 2^-45 of the
 *      larger, so the fp64 sum cannot sit on an fp32 rounding tie.
 *   2. one cast to fp32 (IEEE nearest-even, done by the CPU), which is then the
 *      correctly rounded fp32 sum in every case;
 *   3. fp32 -> bf16 nearest-even by the integer carry rule
 *      (u + 0x7FFF + bit 16 of u) >> 16, with a NaN result mapped to the
 *      canonical quiet NaN 0x7FC0 (the hop's stated NaN rule).
 * The oracle computes the fp32 sum in fp32 arithmetic and rounds to bf16 by
 * comparing the distances to the two neighbours in fp64.
 *
 * Prints the number of mismatches (and the first few) and exits 0 only when
 * there are none.  Build: gcc -O2 -ffp-contract=off -fno-fast-math -pthread. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint16_t or_hop_bf16(uint16_t a, uint16_t b);

static float f32_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static uint16_t ref_hop(uint16_t a, uint16_t b) {
    const double s = (double)f32_of((uint32_t)a << 16) + (double)f32_of((uint32_t)b << 16);
    const float s32 = (float)s;
    if (isnan(s32)) return 0x7FC0u;
    const uint32_t u = bits_of(s32);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

#define THREADS 8
typedef struct { uint32_t a0, a1; uint64_t bad; uint32_t first[4][3]; } job_t;

static void* run(void* p) {
    job_t* j = (job_t*)p;
    for (uint32_t a = j->a0; a < j->a1; ++a)
        for (uint32_t b = 0; b < 65536u; ++b) {
            const uint16_t got = or_hop_bf16((uint16_t)a, (uint16_t)b), want = ref_hop((uint16_t)a, (uint16_t)b);
            if (got != want) {
                if (j->bad < 4) { j->first[j->bad][0] = a; j->first[j->bad][1] = b; j->first[j->bad][2] = (uint32_t)got << 16 | want; }
                ++j->bad;
            }
        }
    return NULL;
}

int main(void) {
    pthread_t th[THREADS];
    job_t jobs[THREADS];
    for (int i = 0; i < THREADS; ++i) {
        memset(&jobs[i], 0, sizeof jobs[i]);
        jobs[i].a0 = (uint32_t)(65536u / THREADS * i);
        jobs[i].a1 = (uint32_t)(65536u / THREADS * (i + 1));
        pthread_create(&th[i], NULL, run, &jobs[i]);
    }
    uint64_t bad = 0;
    for (int i = 0; i < THREADS; ++i) {
        pthread_join(th[i], NULL);
        for (uint64_t k = 0; k < jobs[i].bad && k < 4; ++k)
            printf("mismatch a=0x%04x b=0x%04x oracle=0x%04x reference=0x%04x\n", jobs[i].first[k][0],
                   jobs[i].first[k][1], jobs[i].first[k][2] >> 16, jobs[i].first[k][2] & 0xFFFFu);
        bad += jobs[i].bad;
    }
    printf("pairs=4294967296 mismatches=%llu\n", (unsigned long long)bad);
    return bad == 0 ? 0 : 1;
}
