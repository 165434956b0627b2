/*
 * Host-side emulation of two arithmetic shortcuts the HIP kernels take, checked
 * against the plain definitions (test infrastructure; compiled by the test suite
 * with gcc, no contraction):
 *   div14_mismatches: fp32(s / 14) as q = s * fl(1/14), r = fma(-q, 14, s),
 *     fma(r, fl(1/14), q), over every positive finite binary16 value s;
 *   rint_quot_mismatches: the quantizers' division-free code, t = v * fl(1/s),
 *     taken when |t - rint(t)| < 0.5 - 4e-6 and |t| <= 8, else rint(v / s),
 *     against rint(v / s) (ties to even) on random scales and values, half of
 *     them constructed on and next to the rounding boundaries.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float h2f(uint32_t h) {
    int e = (int)((h >> 10) & 31), m = (int)(h & 1023);
    return e ? ldexpf((float)(m | 1024), e - 25) : ldexpf((float)m, -24);
}

long div14_mismatches(void) {
    volatile float fourteen = 14.0f;
    const float c = 1.0f / fourteen;
    long bad = 0;
    for (uint32_t h = 1; h < 0x7c00; ++h) {
        const float s = h2f(h);
        const float q = s * c;
        const float r = fmaf(-q, fourteen, s);
        bad += fmaf(r, c, q) != s / fourteen;
    }
    return bad;
}

static uint64_t rng_state;
static uint64_t next64(void) {                 /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float nextf_toward(float x, int up) { return nextafterf(x, up ? INFINITY : -INFINITY); }

static float rint_quot(float v, float s, float rs) {
    const float t = v * rs;
    const float q = rintf(t);
    if (fabsf(t - q) < 0.5f - 4e-6f && fabsf(t) <= 8.0f) return q;
    return rintf(v / s);
}

long rint_quot_mismatches(uint64_t seed, long n) {
    rng_state = seed;
    long bad = 0;
    for (long i = 0; i < n; ++i) {
        const uint64_t u = next64();
        const float s = h2f(0x0400 + (uint32_t)(u % (0x7bff - 0x0400)));   /* normal fp16 scales */
        const float rs = 1.0f / s;
        float v;
        const int kind = (int)((u >> 32) & 3);
        const int k = (int)((u >> 40) % 17) - 8;
        if (kind == 0) {
            v = (float)(((int64_t)(u >> 20) % 2000001) - 1000000) * 1e-5f * s;   /* |v/s| <= 10 */
        } else {
            v = ((float)k + 0.5f) * s;                                        /* a tie (rounded) */
            if (kind == 2) v = nextf_toward(v, 1);
            if (kind == 3) v = nextf_toward(v, 0);
        }
        bad += rint_quot(v, s, rs) != rintf(v / s);
    }
    return bad;
}
