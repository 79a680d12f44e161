/*
 * fp8_oracle.c -- plain, slow, obviously-correct CPU oracle for the FP8
 * block-scaled quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the bench's
 * cpu_baseline leg do.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes (source: the Jet-RL technical summary on gist.science,
 * paper 2601.14243, section "Quantization scheme"; the numeric format and
 * rounding are the project's stated definitions, listed per function):
 *   - activations are quantized in 1x128 groups (one scale per row per 128
 *     consecutive columns),
 *   - weights are quantized in 128x128 blocks,
 *   - the backward GEMMs (DGrad, WGrad) also run in FP8; WGrad groups both
 *     operands 128-along-tokens (the page's "1x128 and 128x1" kernels),
 *   - gradients between operators stay BF16; activations saved for backward
 *     are FP8.
 * Scale of a group = fp32(amax / 448), codes = E4M3(fp32(x / scale)) with
 * round-to-nearest-even and saturation at +-448.  GEMMs are fp64 dot products
 * of decoded codes times their scales.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared
 * (no FMA contraction, no flush-to-zero, IEEE single division).  OpenMP is
 * used only across independent rows, so results do not depend on threads.
 *
 * It also holds the two producer operators that feed a linear layer (RMSNorm
 * and SwiGLU, section "Implementation": fused activation / RMSNorm kernels),
 * whose BF16 outputs are then quantized by the 1x128 activation quantizer.
 *
 * It also holds 4-bit MXFP4 weights for the rollout GEMM (QeRL, abstract:
 * NVFP4 weights, read here as the OCP MX format the MI355X takes), with the
 * GEMM on dequantized operands like the FP8 ones.
 *
 * Every function below is pinned by a CPU test against something other than
 * itself (exhaustive brute force, closed forms, exact rationals or an
 * independent library routine), except the FP8-source transpose-quant, whose
 * requantization reading has no independent pin: parity unpinned for
 * oracle_quant_transpose_fp8 beyond the invariants it shares with the rest.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GROUP 128

/* fp32 expressions must be evaluated in fp32 (no excess precision). */
#if !defined(__FLT_EVAL_METHOD__) || __FLT_EVAL_METHOD__ != 0
#error "the oracle needs FLT_EVAL_METHOD == 0 (x86-64 SSE or equivalent)"
#endif

/* ---------------------------------------------------------------- format */

/*
 * OCP E4M3FN decode: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, NaN only at 0x7F / 0xFF.  Exponent field 0 is subnormal:
 * F * 2^-9; otherwise (8 + F) * 2^(E - 10).
 */
double oracle_e4m3_decode(uint8_t c)
{
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int f = c & 0x7;
    double v;
    if (e == 0xF && f == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)f, -9);
    else
        v = ldexp((double)(8 + f), e - 10);
    return s ? -v : v;
}

/* Code of a non-negative magnitude that is exactly an E4M3 value <= 448. */
static uint8_t e4m3_code_of_exact(double r)
{
    if (r < ldexp(1.0, -6)) {                 /* subnormal: r = F * 2^-9 */
        return (uint8_t)(r * 512.0);
    }
    int e2;
    double m = frexp(r, &e2);                 /* r = m * 2^e2, m in [0.5,1) */
    int E = e2 - 1;                           /* r = (1 + F/8) * 2^E       */
    int F = (int)((m * 2.0 - 1.0) * 8.0);
    return (uint8_t)(((E + 7) << 3) | F);
}

/*
 * fp32 -> E4M3 code.  Round |v| to the nearest E4M3 value; on a tie choose
 * the value with the even code (equivalently, the even mantissa, which also
 * holds across the subnormal/normal seam); magnitudes that round above 448
 * saturate to 448 (0x7E).  The sign bit of v is kept, so -0 and negative
 * values that round to zero give 0x80.  NaN/Inf inputs are outside the
 * contract (the quantizer never produces them from finite inputs).
 *
 * Steps: the E4M3 quantum around |v| is 2^(E-3) with E = max(floor(log2|v|),
 * -6); |v| / quantum is exact in fp64, nearbyint() rounds it to the nearest
 * integer with ties to even; the product is the rounded magnitude.
 */
uint8_t oracle_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    if (E < -6)
        E = -6;
    double quantum = ldexp(1.0, E - 3);
    double k = nearbyint(a / quantum);
    double r = k * quantum;
    if (r > 448.0)
        return (uint8_t)(sign | 0x7E);
    return (uint8_t)(sign | e4m3_code_of_exact(r));
}

float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/*
 * fp64 -> bf16 with round-to-nearest-even (single rounding of the exact
 * fp64 value).  Used to compare exactly-representable GEMM results.
 */
uint16_t oracle_f64_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;                           /* a in [2^E, 2^(E+1)) */
    if (E < -126)
        E = -126;                             /* bf16 subnormal quantum 2^-133 */
    double quantum = ldexp(1.0, E - 7);
    double r = nearbyint(a / quantum) * quantum;
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80);     /* overflow -> inf */
    float f = (float)r;                       /* exact: r has <= 8 bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* ---------------------------------------------------------- quantization */

/* One group: amax over n values (stride apart), scale, codes.  Steps of the
 * definition: a = max|x| (exact in fp32); s = fp32(a / 448); q = E4M3(fp32(x
 * / s)); an all-zero group gets s = 0 and signed-zero codes. */
static float quant_group(const float* vals, int64_t n, uint8_t* codes)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float m = fabsf(vals[i]);
        if (m > a)
            a = m;
    }
    if (a == 0.0f) {
        for (int64_t i = 0; i < n; ++i)
            codes[i] = signbit(vals[i]) ? 0x80 : 0x00;
        return 0.0f;
    }
    float s = a / 448.0f;                     /* IEEE fp32 division, RNE */
    for (int64_t i = 0; i < n; ++i) {
        float t = vals[i] / s;                /* IEEE fp32 division, RNE */
        codes[i] = oracle_e4m3_encode(t);
    }
    return s;
}

/* Activation quant, 1x128 groups: x bf16 [M,K] -> q [M,K], s [M][K/128]. */
void oracle_quant_act(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s)
{
    int64_t G = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float vals[GROUP];
        uint8_t codes[GROUP];
        for (int64_t g = 0; g < G; ++g) {
            for (int i = 0; i < GROUP; ++i)
                vals[i] = oracle_bf16_to_f32(x[m * K + g * GROUP + i]);
            s[m * G + g] = quant_group(vals, GROUP, codes);
            memcpy(q + m * K + g * GROUP, codes, GROUP);
        }
    }
}

/* Weight quant, 128x128 blocks aligned at (0,0): w bf16 [N,K] -> q [N,K],
 * s [N/128][K/128] row-major. */
void oracle_quant_weight(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s)
{
    int64_t BN = N / GROUP, BK = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < BN * BK; ++b) {
        int64_t bi = b / BK, bj = b % BK;
        float vals[GROUP * GROUP];
        uint8_t codes[GROUP * GROUP];
        for (int r = 0; r < GROUP; ++r)
            for (int c = 0; c < GROUP; ++c)
                vals[r * GROUP + c] =
                    oracle_bf16_to_f32(w[(bi * GROUP + r) * K + bj * GROUP + c]);
        s[bi * BK + bj] = quant_group(vals, GROUP * GROUP, codes);
        for (int r = 0; r < GROUP; ++r)
            memcpy(q + (bi * GROUP + r) * K + bj * GROUP, codes + r * GROUP, GROUP);
    }
}

/* Transpose-quant from BF16, groups of 128 consecutive rows (tokens) per
 * column: x bf16 [T,C] -> qT [C,T], sT [C][T/128]. */
void oracle_quant_transpose_bf16(const uint16_t* x, int64_t T, int64_t C, uint8_t* qT, float* sT)
{
    int64_t G = T / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        float vals[GROUP];
        uint8_t codes[GROUP];
        for (int64_t g = 0; g < G; ++g) {
            for (int i = 0; i < GROUP; ++i)
                vals[i] = oracle_bf16_to_f32(x[(g * GROUP + i) * C + c]);
            sT[c * G + g] = quant_group(vals, GROUP, codes);
            memcpy(qT + c * T + g * GROUP, codes, GROUP);
        }
    }
}

/* Transpose-requant of a saved FP8 tensor (1x128 row-group scales along C):
 * v = fp32(dec(q) * s_row) with a plain fp32 multiply, then the same
 * 128-along-T quantization as above.  q [T,C], s_row [T][C/128] -> qT [C,T],
 * sT [C][T/128].  Parity unpinned beyond shared invariants (see header). */
void oracle_quant_transpose_fp8(const uint8_t* q, const float* s_row, int64_t T, int64_t C,
                                uint8_t* qT, float* sT)
{
    int64_t G = T / GROUP, GC = C / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        float vals[GROUP];
        uint8_t codes[GROUP];
        for (int64_t g = 0; g < G; ++g) {
            for (int i = 0; i < GROUP; ++i) {
                int64_t t = g * GROUP + i;
                float d = (float)oracle_e4m3_decode(q[t * C + c]);   /* exact */
                vals[i] = d * s_row[t * GC + c / GROUP];             /* fp32 multiply */
            }
            sT[c * G + g] = quant_group(vals, GROUP, codes);
            memcpy(qT + c * T + g * GROUP, codes, GROUP);
        }
    }
}

/* ------------------------------------------------------------ dequantize */

/* out[r,c] = dec(q[r,c]) * s[r][c/128], in fp64 (exact: <= 28 significant
 * bits). */
void oracle_dequant_rowgroup(const uint8_t* q, const float* s, int64_t R, int64_t C, double* out)
{
    int64_t G = C / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c)
            out[r * C + c] = oracle_e4m3_decode(q[r * C + c]) * (double)s[r * G + c / GROUP];
}

/* out[r,c] = dec(q[r,c]) * s[r/128][c/128], in fp64. */
void oracle_dequant_block(const uint8_t* q, const float* s, int64_t R, int64_t C, double* out)
{
    int64_t G = C / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c)
            out[r * C + c] =
                oracle_e4m3_decode(q[r * C + c]) * (double)s[(r / GROUP) * G + c / GROUP];
}

/* ------------------------------------------------------------------ GEMM */

/*
 * C[m*N + n] = sum_{k ascending} A(m,k) * B(n,k) in fp64, where
 * A(m,k) = A[m*sam + k*sak] and B(n,k) = B[n*sbn + k*sbk].  Strides let the
 * same routine express the forward (X W^T), DGrad (dY W) and WGrad
 * (dY^T X) contractions on dequantized operands.
 */
void oracle_gemm(int64_t M, int64_t N, int64_t K,
                 const double* A, int64_t sam, int64_t sak,
                 const double* B, int64_t sbn, int64_t sbk, double* C)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += A[m * sam + k * sak] * B[n * sbn + k * sbk];
            C[m * N + n] = acc;
        }
}

/* ------------------------------------------------ producer operators
 *
 * The summary's "Quantization scheme" section keeps the activations saved for
 * the backward pass in FP8, produced fused with the operator in front of the
 * linear layer, and "Implementation" names fused activation and RMSNorm
 * kernels.  The pages define neither operator.  The oracle takes their
 * textbook forms with every precision fixed, so that the fused result is the
 * producer's BF16 output (tensors between operators stay BF16) quantized by
 * oracle_quant_act:
 *   RMSNorm:  y = x * r * gamma,  r = 1 / sqrt(mean(x^2) + eps)
 *   SwiGLU:   h = silu(g) * u,    silu(g) = g / (1 + exp(-g))
 */

/* Sum of 2^j consecutive fp64 values as a balanced binary tree: the left half
 * and the right half are summed the same way, then added. */
static double tree_sum(const double* v, int n)
{
    if (n == 1)
        return v[0];
    return tree_sum(v, n / 2) + tree_sum(v + n / 2, n / 2);
}

/*
 * RMSNorm of BF16 rows, BF16 output.  Per row of K (K % 128 == 0):
 *   ss   = sum of x^2 in fp64 (each square is exact); each 128-element group
 *          is summed as a balanced binary tree, then the group sums are added
 *          in ascending group order starting from 0;
 *   r    = 1 / sqrt(ss / K + eps), three IEEE fp64 operations and sqrt;
 *   rstd = fp32(r) (round to nearest even);
 *   y[k] = bf16_rne(fp32(fp32(x[k] * rstd) * gamma[k])), two fp32 multiplies.
 * eps >= 0; a row with ss / K + eps == 0 is outside the contract.
 */
void oracle_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                         uint16_t* y, float* rstd)
{
    int64_t G = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * K;
        double sq[GROUP];
        double ss = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            for (int i = 0; i < GROUP; ++i) {
                double v = (double)oracle_bf16_to_f32(row[g * GROUP + i]);
                sq[i] = v * v;
            }
            ss += tree_sum(sq, GROUP);
        }
        double r = 1.0 / sqrt(ss / (double)K + (double)eps);
        float rs = (float)r;
        if (rstd)
            rstd[m] = rs;
        for (int64_t k = 0; k < K; ++k) {
            float t = oracle_bf16_to_f32(row[k]) * rs;            /* fp32 multiply */
            float u = t * oracle_bf16_to_f32(gamma[k]);           /* fp32 multiply */
            y[m * K + k] = oracle_f64_to_bf16((double)u);         /* exact widening, one RNE */
        }
    }
}

/*
 * Backward of the RMSNorm above, y = x * r * gamma, with r the rstd the
 * forward saved (the rounding of y is passed straight through).  From
 * dr/dx_i = -r^3 x_i / K, the textbook gradients are
 *   dx_j     = r g_j - x_j r^3 c / K,   g_j = gamma_j dy_j,   c = sum_i g_i x_i
 *   dgamma_k = sum_t dy[t,k] x[t,k] r_t
 * evaluated in fp64 in a fixed order:
 *   g_i = gamma_i * dy_i and p_i = g_i * x_i (both exact);
 *   c = sum of p over the row: each 128-group a balanced binary tree, the
 *       group sums added in ascending order (the forward's order for ss);
 *   k = ((r * r) * r) * (c / K);  dx_j = bf16(r * g_j - x_j * k), one rounding;
 *   dgamma_k = fp32 of the sum over t of (dy * x) * r_t, the rows of each block
 *       of 128 rows added in ascending order from 0, the block sums added in
 *       ascending order from 0 (a last block may be shorter).
 * x, dy: BF16 [M,K]; gamma: BF16 [K]; rstd: fp32 [M]; dx: BF16 [M,K];
 * dgamma: fp32 [K] (may be NULL).
 */
void oracle_rmsnorm_bwd(const uint16_t* x, const uint16_t* gamma, const float* rstd, const uint16_t* dy,
                        int64_t M, int64_t K, uint16_t* dx, float* dgamma)
{
    int64_t G = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* xr = x + m * K;
        const uint16_t* dr = dy + m * K;
        double p[GROUP];
        double c = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            for (int i = 0; i < GROUP; ++i) {
                int64_t k = g * GROUP + i;
                double gi = (double)oracle_bf16_to_f32(gamma[k]) * (double)oracle_bf16_to_f32(dr[k]);
                p[i] = gi * (double)oracle_bf16_to_f32(xr[k]);
            }
            c += tree_sum(p, GROUP);
        }
        double r = (double)rstd[m];
        double kk = ((r * r) * r) * (c / (double)K);
        for (int64_t k = 0; k < K; ++k) {
            double gi = (double)oracle_bf16_to_f32(gamma[k]) * (double)oracle_bf16_to_f32(dr[k]);
            double v = r * gi - (double)oracle_bf16_to_f32(xr[k]) * kk;
            dx[m * K + k] = oracle_f64_to_bf16(v);
        }
    }
    if (!dgamma)
        return;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        double total = 0.0;
        for (int64_t b0 = 0; b0 < M; b0 += GROUP) {
            double block = 0.0;
            for (int64_t t = b0; t < M && t < b0 + GROUP; ++t) {
                double prod = (double)oracle_bf16_to_f32(dy[t * K + k]) * (double)oracle_bf16_to_f32(x[t * K + k]);
                block += prod * (double)rstd[t];
            }
            total += block;
        }
        dgamma[k] = (float)total;
    }
}

/* Flag for a fp64 value whose BF16 rounding is within 2^-44 (relative) of a
 * midpoint between two BF16 neighbours (either neighbour is then correct). */
static uint8_t bf16_near_tie(double v)
{
    double a = fabs(v);
    if (a == 0.0 || !isfinite(a))
        return 0;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    if (E < -126)
        E = -126;
    double t = a / ldexp(1.0, E - 7);                     /* exact: a in BF16 quanta */
    double d = fabs((t - floor(t)) - 0.5);
    return d <= ldexp(t, -44);
}

/*
 * SwiGLU of BF16 gate / up rows, BF16 output: h = bf16_rne(v) with
 * v = (g / (1 + exp(-g))) * u evaluated in fp64 (C library exp, IEEE
 * division and multiply).  v differs from the exact value by a few fp64 ulps,
 * which can change the BF16 rounding only when the exact value lies next to
 * a midpoint between two BF16 neighbours; such elements are flagged in
 * `near_tie` (|v - midpoint| <= 2^-44 |v|), where either neighbour is a
 * correct result.  g and u have row stride ld (elements), h is dense [M,F].
 */
void oracle_swiglu_bf16(const uint16_t* g, const uint16_t* u, int64_t ld, int64_t M, int64_t F,
                        uint16_t* h, uint8_t* near_tie)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t f = 0; f < F; ++f) {
            double gv = (double)oracle_bf16_to_f32(g[m * ld + f]);
            double uv = (double)oracle_bf16_to_f32(u[m * ld + f]);
            double v = (gv / (1.0 + exp(-gv))) * uv;
            h[m * F + f] = oracle_f64_to_bf16(v);
            if (near_tie)
                near_tie[m * F + f] = bf16_near_tie(v);
        }
}

/*
 * Backward of SwiGLU h = silu(g) * u for BF16 gate g, up u and output
 * gradient dh (gradients between operators stay BF16).  With
 * s = 1 / (1 + exp(-g)) and silu(g) = g * s, the textbook derivatives
 *   d_up   = dh * silu(g)
 *   d_gate = dh * u * s * (1 + g * (1 - s))
 * are evaluated in fp64 (C library exp, IEEE operations in that order) and
 * rounded once to BF16.  Output dgu is [M, 2F]: d_gate in columns [0, F),
 * d_up in [F, 2F) (the layout of the fused gate/up projection).  near_tie
 * ([M, 2F], may be NULL) flags values within 2^-44 of a BF16 midpoint.
 * g, u and dh have row stride ld (elements).
 */
void oracle_swiglu_bwd_bf16(const uint16_t* g, const uint16_t* u, const uint16_t* dh, int64_t ld, int64_t M,
                            int64_t F, uint16_t* dgu, uint8_t* near_tie)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t f = 0; f < F; ++f) {
            double gv = (double)oracle_bf16_to_f32(g[m * ld + f]);
            double uv = (double)oracle_bf16_to_f32(u[m * ld + f]);
            double dv = (double)oracle_bf16_to_f32(dh[m * ld + f]);
            double s = 1.0 / (1.0 + exp(-gv));
            double d_up = dv * (gv * s);
            double d_gate = ((dv * uv) * s) * (1.0 + gv * (1.0 - s));
            dgu[m * 2 * F + f] = oracle_f64_to_bf16(d_gate);
            dgu[m * 2 * F + F + f] = oracle_f64_to_bf16(d_up);
            if (near_tie) {
                near_tie[m * 2 * F + f] = bf16_near_tie(d_gate);
                near_tie[m * 2 * F + F + f] = bf16_near_tie(d_up);
            }
        }
}

/* ------------------------------------------------ 4-bit weights (MXFP4)
 *
 * The QeRL page ("QeRL: Beyond Efficiency -- Quantization-enhanced
 * Reinforcement Learning for LLMs", abstract) speeds up the rollout with 4-bit
 * NVFP4 weights plus LoRA; the page gives no format details.  NVFP4 belongs to
 * NVIDIA's Blackwell; the MI355X converters and matrix cores take the OCP
 * Microscaling (MX) formats, so the 4-bit weights here are MXFP4 as the OCP
 * MX specification v1.0 defines it (the project's reading):
 *   - element E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit, no
 *     inf/NaN; exponent field 0 is subnormal (value 0.5 * mantissa);
 *   - 32 consecutive elements of a weight row (along K) share one E8M0 scale
 *     2^E, stored as the byte E + 127;
 *   - E = floor(log2(amax)) - 2 (2 is E2M1's largest exponent), clamped to
 *     [-127, 127]; an all-zero block takes E = -127;
 *   - an element is the E2M1 value nearest to v / 2^E, a tie going to the
 *     code with an even last bit; magnitudes past 6 saturate to 6; the sign
 *     of v is kept, zero results included;
 *   - two codes per byte, the even element of K in the low nibble.
 */

/* E2M1 value of a 4-bit code, from its fields. */
double oracle_e2m1_decode(uint8_t c)
{
    const int sgn = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    const double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return sgn ? -mag : mag;
}

/* Nearest E2M1 code to the exact value q (ties to the even code). */
static uint8_t e2m1_nearest(double q)
{
    const double a = fabs(q);
    int best = 0;
    double bd = a;                                   /* distance to code 0 (value 0) */
    for (int c = 1; c < 8; ++c) {
        const double d = fabs(a - oracle_e2m1_decode((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(q) ? 8 : 0));
}

/* Shared exponent of a block from its amax (fp64, exact). */
static int mx_shared_exp(double amax)
{
    if (amax == 0.0)
        return -127;
    int e;
    frexp(amax, &e);                                 /* amax = f * 2^e, f in [0.5, 1) */
    int E = (e - 1) - 2;
    if (E < -127)
        E = -127;
    if (E > 127)
        E = 127;
    return E;
}

/* w [N][K] bf16 (K % 32 == 0) -> codes [N][K/2], scales [N][K/32]. */
void oracle_mxfp4_quant(const uint16_t* w, int64_t N, int64_t K, uint8_t* codes, uint8_t* scales)
{
    const int64_t B = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < B; ++b) {
            const uint16_t* v = w + n * K + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                const double a = fabs((double)oracle_bf16_to_f32(v[i]));
                if (a > amax)
                    amax = a;
            }
            const int E = mx_shared_exp(amax);
            scales[n * B + b] = (uint8_t)(E + 127);
            for (int i = 0; i < 32; i += 2) {
                const uint8_t lo = e2m1_nearest(ldexp((double)oracle_bf16_to_f32(v[i]), -E));
                const uint8_t hi = e2m1_nearest(ldexp((double)oracle_bf16_to_f32(v[i + 1]), -E));
                codes[n * (K / 2) + b * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
}

/* out[n][k] = e2m1(code) * 2^(scale - 127), in fp64. */
void oracle_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, double* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t byte = codes[n * (K / 2) + k / 2];
            const uint8_t c = (k & 1) ? (byte >> 4) : (byte & 15);
            out[n * K + k] = ldexp(oracle_e2m1_decode(c), (int)scales[n * (K / 32) + k / 32] - 127);
        }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
