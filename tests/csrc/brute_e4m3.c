/*
 * Brute-force E4M3 encoder used only to pin the oracle's encoder.
 *
 * It does not know the E4M3 bit layout: it receives the table of the 127
 * non-negative finite E4M3 magnitudes (index = code, taken by the test from an
 * independent library decoder), and for every fp32 input picks the table
 * entry nearest to |v| in exact fp64 distance, breaking ties towards the even
 * code.  Inputs above the largest entry therefore map to it (saturation).
 * The sign bit of the input is OR-ed in.
 *
 * count_mismatches() walks a range of fp32 bit patterns (NaN/Inf skipped) and
 * counts where the candidate encoder disagrees with this brute force.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*enc_fn)(float);

static double tab[127];

void set_table(const double* mags) { memcpy(tab, mags, sizeof tab); }

static uint8_t brute(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    /* binary search: largest index i with tab[i] <= a */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (tab[mid] <= a) lo = mid; else hi = mid - 1;
    }
    int best = lo;
    if (lo < 126) {
        double d0 = a - tab[lo], d1 = tab[lo + 1] - a;
        if (d1 < d0 || (d1 == d0 && ((lo + 1) % 2 == 0)))
            best = lo + 1;
    }
    return (uint8_t)(sign | best);
}

uint8_t brute_encode(float v) { return brute(v); }

/* Mismatches over fp32 bit patterns [lo, hi) ; first mismatch stored. */
int64_t count_mismatches(uint64_t lo, uint64_t hi, enc_fn enc, uint32_t* first_bad)
{
    int64_t bad = 0;
    uint32_t first = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static, 65536) reduction(+:bad)
    for (int64_t i = (int64_t)lo; i < (int64_t)hi; ++i) {
        uint32_t u = (uint32_t)i;
        if (((u >> 23) & 0xFF) == 0xFF) continue;       /* NaN / Inf */
        float v;
        memcpy(&v, &u, 4);
        if (enc(v) != brute(v)) {
            ++bad;
#pragma omp critical
            if (u < first) first = u;
        }
    }
    *first_bad = first;
    return bad;
}

/* Vectorised helper: encode n floats with the candidate encoder. */
void encode_many(const float* in, int64_t n, enc_fn enc, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = enc(in[i]);
}
