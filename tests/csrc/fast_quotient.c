/*
 * Host emulation of the GPU quantizers' quotient route, for a CPU test.
 *
 * The kernels compute a group's scale s = fl32(amax / 448) and r = fl32(1 / s)
 * once, both correctly rounded (formed on the device without a division and
 * checked equal to the correctly rounded quotients on every argument by a GPU
 * test; here by IEEE division), then for every element x of the group
 *     q0 = fl32(x * r);  res = fma(-q0, s, x);  q1 = fma(res, r, q0);
 *     t  = copysign(q1, x)
 * when s >= 2^-92, and t = fl32(x / s) otherwise.  The definition of the code
 * is E4M3(fl32(x / s)) (correctly rounded division, then the encoder).  The
 * route is Markstein's correction of a quotient by fused multiply-adds with a
 * correctly rounded reciprocal; this file checks, by brute force, that it
 * gives the same code as the definition:
 *   - if |fl32(x / s)| >= 2^-11, t must equal fl32(x / s) bit for bit (the
 *     encoder then sees the same input);
 *   - below 2^-11 the definition's code is a signed zero (E4M3 rounds
 *     magnitudes up to 2^-10 to zero), so t must have |t| <= 2^-10 and the
 *     sign of x.
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -fPIC
 *        -shared (no FMA contraction: the products and sums are exactly the
 *        ones written; fmaf is the C library's correctly rounded one).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float f_of(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t u_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static const float kFastScaleMin = 0x1p-92f;

/* 1 when the route's code matches the definition's for (x, amax). */
static int route_ok(float x, float amax)
{
    const float s = amax / 448.0f;
    const float r = 1.0f / s;
    const float q = x / s;                         /* the definition's quotient */
    float t;
    if (s >= kFastScaleMin) {
        const float q0 = x * r;
        const float res = fmaf(-q0, s, x);
        const float q1 = fmaf(res, r, q0);
        t = copysignf(q1, x);
    } else {
        t = q;
    }
    if (fabsf(q) >= 0x1p-11f)
        return u_of(t) == u_of(q);
    return fabsf(t) <= 0x1p-10f && signbit(t) == signbit(x);
}

/* The fast route's domain: whether s = fl32(amax / 448) takes it. */
int fq_is_fast(float amax) { return amax / 448.0f >= kFastScaleMin; }

/*
 * Every pair of positive finite bf16 values x <= amax (amax > 0), both signs
 * of x.  Returns the number of mismatches; the first is reported through
 * *bad_x / *bad_amax (bf16 bit patterns).  *pairs receives the pair count and
 * *fast_pairs how many of them took the fast route.
 */
int64_t fq_check_bf16(int64_t* pairs, int64_t* fast_pairs, uint32_t* bad_x, uint32_t* bad_amax)
{
    int64_t bad = 0, n = 0, nf = 0;
    uint32_t bx = 0, ba = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad, n, nf)
    for (int32_t a = 1; a <= 0x7F7F; ++a) {
        const float amax = f_of((uint32_t)a << 16);
        const int fast = fq_is_fast(amax);
        for (int32_t xb = 0; xb <= a; ++xb) {
            const float x = f_of((uint32_t)xb << 16);
            for (int sgn = 0; sgn < 2; ++sgn) {
                const float xs = sgn ? -x : x;
                ++n;
                nf += fast;
                if (!route_ok(xs, amax)) {
#pragma omp critical
                    {
                        if (bad == 0 || (uint32_t)a < ba) {
                            ba = (uint32_t)a;
                            bx = u_of(xs) >> 16;
                        }
                    }
                    ++bad;
                }
            }
        }
    }
    *pairs = n;
    *fast_pairs = nf;
    *bad_x = bx;
    *bad_amax = ba;
    return bad;
}

/* splitmix64: the published mixing function, a seeded counter-based stream. */
static uint64_t splitmix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/*
 * n random pairs with amax an arbitrary positive finite fp32 in the fast
 * route's domain ([448 * 2^-92, max float]), x uniform over the fp32 bit
 * patterns from 0 to amax (every magnitude up to amax), random sign; plus,
 * for each amax, x = amax.  These are the inputs the FP8-source requantizer
 * produces (values and their group maxima are arbitrary fp32 products).
 */
int64_t fq_check_random(uint64_t seed, int64_t n, uint32_t* bad_x, uint32_t* bad_amax)
{
    const uint32_t lo = u_of(448.0f * 0x1p-92f), hi = 0x7F7FFFFFu;
    int64_t bad = 0;
    uint32_t bx = 0, ba = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i < n; ++i) {
        const uint64_t z = splitmix64(seed * 0x100000001B3ull + (uint64_t)i);
        const uint32_t au = lo + (uint32_t)((z & 0xFFFFFFFFull) % (uint64_t)(hi - lo + 1));
        const uint32_t xu = (uint32_t)((z >> 32) % ((uint64_t)au + 1));
        const float amax = f_of(au);
        const float x = f_of(xu | ((uint32_t)(z >> 63) << 31));
        const int ok = fq_is_fast(amax) && route_ok(x, amax) && route_ok(amax, amax);
        if (!ok) {
#pragma omp critical
            {
                if (bad == 0) {
                    bx = u_of(x);
                    ba = au;
                }
            }
            ++bad;
        }
    }
    *bad_x = bx;
    *bad_amax = ba;
    return bad;
}

/* The route on one pair (for the fixtures in the test). */
float fq_route(float x, float amax)
{
    const float s = amax / 448.0f;
    const float r = 1.0f / s;
    if (s < kFastScaleMin)
        return x / s;
    const float q0 = x * r;
    const float res = fmaf(-q0, s, x);
    const float q1 = fmaf(res, r, q0);
    return copysignf(q1, x);
}

/* The uncorrected product fl32(x * r), to show the correction is needed. */
float fq_product_only(float x, float amax)
{
    const float s = amax / 448.0f;
    return x * (1.0f / s);
}
