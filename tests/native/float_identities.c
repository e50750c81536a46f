/* Exhaustive host check of the two FP32 identities the encoder uses in place
 * of IEEE divisions (the host follows IEEE 754 binary32 with FMA and gradual
 * underflow, as the GPU kernels do):
 *
 *   1. x / L for L = 3 and L = 15: with r = RN(1/L), q = RN(x * r),
 *      e = fma(-q, L, x), q' = fma(e, r, q) equals RN(x / L) for every float
 *      x in [0, 2^120], subnormals included.
 *   2. 1 / s for every positive finite binary16 value s (as FP32): from any
 *      r0 within 2 ulp of RN(1/s), e = fma(-r0, s, 1), r1 = fma(e, r0, r0)
 *      equals RN(1/s).
 *
 * Prints one line per identity with its mismatch count; exit status 0 iff all
 * counts are zero.  Built with -ffp-contract=off so that only the explicit
 * fmaf calls fuse. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t as_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

enum { THREADS = 8, BLOCK = 1 << 20 };
static const uint32_t TOP = 0x7B800000u; /* 2^120 */

typedef struct { int t; float L; unsigned long long bad; } job;

/* blocks of BLOCK consecutive bit patterns, dealt round-robin to the threads
 * (the subnormal and tiny binades, where the host is slow, are spread out) */
static void *div_job(void *arg) {
  job *j = arg;
  const float L = j->L, r = 1.0f / j->L;
  for (uint64_t b = (uint64_t)j->t * BLOCK; b <= TOP; b += (uint64_t)THREADS * BLOCK) {
    const uint64_t end = b + BLOCK <= (uint64_t)TOP + 1 ? b + BLOCK : (uint64_t)TOP + 1;
    for (uint64_t i = b; i < end; ++i) {
      const float x = as_float((uint32_t)i);
      const float q = x * r;
      const float e = fmaf(-q, L, x);
      const float q2 = fmaf(e, r, q);
      if (as_bits(q2) != as_bits(x / L)) j->bad++;
    }
  }
  return NULL;
}

int main(void) {
  int fail = 0;
  const float levels[2] = {3.0f, 15.0f};
  for (int k = 0; k < 2; ++k) {
    pthread_t th[THREADS];
    job jb[THREADS];
    for (int t = 0; t < THREADS; ++t) {
      jb[t].t = t; jb[t].L = levels[k]; jb[t].bad = 0;
      pthread_create(&th[t], NULL, div_job, &jb[t]);
    }
    unsigned long long bad = 0;
    for (int t = 0; t < THREADS; ++t) { pthread_join(th[t], NULL); bad += jb[t].bad; }
    printf("div_levels L=%g x in [0, 2^120]: %llu mismatches\n", levels[k], bad);
    fail |= bad != 0;
  }
  unsigned long long bad = 0, tried = 0;
  for (uint32_t h = 1; h < 0x7C00u; ++h) {
    const uint32_t e = h >> 10, m = h & 0x3ffu;
    const float s = e ? ldexpf((float)(1024 + m), (int)e - 25) : ldexpf((float)m, -24);
    const float want = 1.0f / s;
    float r0 = nextafterf(nextafterf(want, 0.0f), 0.0f);
    for (int c = 0; c < 5; ++c, r0 = nextafterf(r0, INFINITY)) {
      const float er = fmaf(-r0, s, 1.0f);
      const float r1 = fmaf(er, r0, r0);
      tried++;
      if (as_bits(r1) != as_bits(want)) bad++;
    }
  }
  printf("recip binary16 s > 0, 5 starting values each (%llu cases): %llu mismatches\n", tried, bad);
  fail |= bad != 0;
  return fail;
}
