// producer_kernels.hip -- the operators in front of a linear layer, fused with
// its 1x128 FP8 activation quantization (gfx950).
//
// Jet-RL technical summary (gist.science 2601.14243): "Quantization scheme"
// keeps the activations saved for the backward pass in FP8, produced fused
// with the operator before the linear layer; "Implementation" names fused
// activation and RMSNorm kernels.  Each kernel here reads the producer's
// inputs once and writes FP8 codes and 1x128 scales, never the BF16
// intermediate.  The result is, bit for bit, the producer's BF16 output
// quantized by fp8_quant_act:
//   RMSNorm:  y = bf16(fp32(fp32(x * rstd) * gamma)),
//             rstd = fp32(1 / sqrt(ss / K + eps)) in fp64, where ss, the
//             fp64 sum of x^2, is summed as a balanced binary tree over each
//             128-group and the group sums are added in ascending order
//             (a fixed order, so the result does not depend on the launch);
//   SwiGLU:   h = bf16(silu(g) * u), silu(g) = g / (1 + exp(-g)), the
//             fp64 evaluation rounded once to BF16 (reached through an fp32
//             evaluation with a proven error bound, fp64 where that bound
//             cannot decide the rounding).
#include "fp8lin_device.hpp"
#include "fp8lin_launch.hpp"
#include "quant_tile.hpp"

namespace fp8lin {

// ------------------------------------------------------------ fp64 helpers

__device__ __forceinline__ double shfl_xor_f64(double v, int mask)
{
    const int lane = threadIdx.x & 63;
    const int src = (lane ^ mask) << 2;
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_ds_bpermute(src, (int)(b & 0xFFFFFFFFll));
    const int hi = __builtin_amdgcn_ds_bpermute(src, (int)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), lane);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Two fp32 -> two bf16 (low half = lo), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950 (denormals kept, as the kernels' fp32 mode).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// fp64 -> bf16 bits with one rounding to nearest even (finite inputs).
// At or above 2^-126 the 52-bit fraction is rounded to 7 bits on the integer
// pattern (a carry moves into the exponent, as rounding does); below, BF16's
// quantum is 2^-133 and the value is rounded as an integer multiple of it.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v)
{
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    const unsigned long long a = b & 0x7FFFFFFFFFFFFFFFull;
    float f;
    if (a >= 0x3810000000000000ull) {                      // |v| >= 2^-126
        unsigned long long r = a + ((1ull << 44) - 1) + ((a >> 45) & 1ull);
        r &= ~((1ull << 45) - 1);
        f = (float)__longlong_as_double((long long)r);     // exact (or +inf)
    } else {
        const double t = __builtin_rint(__longlong_as_double((long long)a) * 0x1p133);
        f = (float)(t * 0x1p-133);                         // exact
    }
    return (__float_as_uint(f) >> 16) | sign;
}

// Quantize the group held by 16 lanes (8 bf16 values per lane as 4 packed
// words): group amax, scale, codes.  Returns this lane's 8 codes and the
// group scale.
__device__ __forceinline__ uint2 quantize_group16(uint4 y, float& scale)
{
    const uint32_t am = max_over_16_lanes(absmax_bits_8xbf16(y));
    const GroupScale gs = group_scale(am);
    scale = gs.s;
    return quantize8(y, gs);
}

// ==================================================== RMSNorm -> FP8 1x128
//
// One wave per row: lane l holds elements [512 i + 8 l, +8) of pass i in
// registers (NV passes, 512 (NV - 1) < K <= 512 NV for K <= 8192), so the row
// is read from HBM once.  Lanes past the end of the row load a valid address
// (the row's first chunk) and zero it, so no load sits behind a branch and all
// of a row's loads, and gamma's, are in flight together.  The squares are
// summed in fp64 in the stated order: the lane's 8 values as a tree, then 16
// lanes by DPP exchanges (quad xor 1, quad xor 2, half-row mirror, row mirror:
// after each step every lane of a block holds the block's sum, so each step
// adds two sibling subtrees of the balanced tree over the 128-group), then the
// group sums in ascending order through lane reads.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const long long b = __double_as_longlong(v);
    const uint32_t lo = dpp<CTRL>((uint32_t)(b & 0xFFFFFFFFll));
    const uint32_t hi = dpp<CTRL>((uint32_t)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | lo);
}

__device__ __forceinline__ double sum_over_16_lanes(double t)
{
    t = t + dpp_f64<kDppQuadXor1>(t);
    t = t + dpp_f64<kDppQuadXor2>(t);
    t = t + dpp_f64<kDppRowHalfMirror>(t);
    t = t + dpp_f64<kDppRowMirror>(t);
    return t;
}

__device__ __forceinline__ double tree_sum_sq8(uint4 v)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    double sq[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double lo = (double)bf16_lo(w[j]);
        const double hi = (double)bf16_hi(w[j]);
        sq[2 * j] = lo * lo;
        sq[2 * j + 1] = hi * hi;
    }
    return ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
}

template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ gamma,
                                                            int64_t M, int K, float eps,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ s,
                                                            float* __restrict__ rstd_out)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M)
        return;                                             // wave-uniform
    const int G = K >> 7;
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * K);
    const uint4* gr = reinterpret_cast<const uint4*>(gamma);
    // Rows up to 8192 wide also hold gamma in registers from the start; wider
    // rows read it in the second pass (register budget).
    constexpr bool kGammaFirst = NV <= 16;
    uint4 v[NV], gw[kGammaFirst ? NV : 1];
    bool live[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        live[i] = 512 * i + 8 * lane < K;                   // uniform over each 16-lane group
        const int c = live[i] ? 64 * i + lane : lane & 15;
        v[i] = load_nt(xr + c);
        if (kGammaFirst)
            gw[i] = gr[c];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (!live[i])
            v[i] = make_uint4(0, 0, 0, 0);

    double t[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
        t[i] = sum_over_16_lanes(tree_sum_sq8(v[i]));
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double gsum = readlane_f64(t[i], 16 * j);
            ss = ss + (4 * i + j < G ? gsum : 0.0);          // adding +0 leaves ss unchanged
        }
    const double r = 1.0 / __builtin_sqrt(ss / (double)K + (double)eps);
    const float rs = (float)r;
    if (rstd_out != nullptr && lane == 0)
        rstd_out[row] = rs;

    uint2* qr = reinterpret_cast<uint2*>(q + row * K);
    float* sr = s + row * G;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const uint4 g4 = kGammaFirst ? gw[i] : gr[live[i] ? 64 * i + lane : lane & 15];
        const uint32_t xw[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        const uint32_t gg[4] = {g4.x, g4.y, g4.z, g4.w};
        uint32_t yw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = (bf16_lo(xw[j]) * rs) * bf16_lo(gg[j]);
            const float hi = (bf16_hi(xw[j]) * rs) * bf16_hi(gg[j]);
            yw[j] = pack_bf16x2(lo, hi);
        }
        float scale;
        const uint2 c = quantize_group16(make_uint4(yw[0], yw[1], yw[2], yw[3]), scale);
        if (live[i]) {
            qr[64 * i + lane] = c;
            if ((lane & 15) == 0)
                sr[4 * i + (lane >> 4)] = scale;
        }
    }
}

// ======================================================= RMSNorm backward
//
// y = x r gamma with r the forward's rstd (y's rounding passed straight
// through): dx_j = r g_j - x_j r^3 c / K with g_j = gamma_j dy_j and
// c = sum_i g_i x_i; dgamma_k = sum_t dy[t,k] x[t,k] r_t.  All in fp64 in a
// fixed order, so every bit is determined: g and g x are exact; c follows the
// forward's order for the sum of squares (a balanced tree over each 128-group
// by DPP exchanges, groups ascending through lane reads);
// dx_j = bf16(r g_j - x_j (((r r) r) (c / K))) with one rounding.  dgamma:
// each workgroup of the second kernel adds 128 tokens of 512 columns in
// ascending order, one fp64 accumulator per column, into the caller's
// workspace [ceil(M/128)][K]; the third adds those block sums in ascending
// order and rounds to fp32.
// One workgroup of 256 threads per row: thread t holds elements
// [2048 i + 8 t, +8) of pass i (NP passes, K <= 2048 NP) of x, dy and gamma;
// each 16-lane group reduces its 128-group by DPP and parks the sum in LDS,
// and every thread then adds the group sums in ascending order.
template <int NP>
__global__ __launch_bounds__(256) void rmsnorm_bwd_dx_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ gamma,
                                                             const float* __restrict__ rstd,
                                                             const uint16_t* __restrict__ dy, int K,
                                                             uint16_t* __restrict__ dx)
{
    __shared__ double gsum[128];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int G = K >> 7;
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * K);
    const uint4* dr = reinterpret_cast<const uint4*>(dy + row * K);
    const uint4* gr = reinterpret_cast<const uint4*>(gamma);
    uint4 xv[NP], dv[NP], gv[NP];
    bool live[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        live[i] = 2048 * i + 8 * tid < K;                   // uniform over each 16-lane group
        const int c = live[i] ? 256 * i + tid : tid & 15;   // past the end: a valid address, zeroed
        xv[i] = load_nt(xr + c);
        dv[i] = load_nt(dr + c);
        gv[i] = gr[c];
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        if (!live[i])
            dv[i] = make_uint4(0, 0, 0, 0);
        const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        const uint32_t dw[4] = {dv[i].x, dv[i].y, dv[i].z, dv[i].w};
        const uint32_t gw[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
        double p[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[2 * j] = ((double)bf16_lo(gw[j]) * (double)bf16_lo(dw[j])) * (double)bf16_lo(xw[j]);
            p[2 * j + 1] = ((double)bf16_hi(gw[j]) * (double)bf16_hi(dw[j])) * (double)bf16_hi(xw[j]);
        }
        const double t = sum_over_16_lanes(((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
        if (live[i] && (tid & 15) == 0)
            gsum[16 * i + (tid >> 4)] = t;
    }
    __syncthreads();
    double c = 0.0;
    for (int g = 0; g < G; ++g)
        c = c + gsum[g];
    const double r = (double)rstd[row];
    const double kk = ((r * r) * r) * (c / (double)K);
    uint4* out = reinterpret_cast<uint4*>(dx + row * K);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        const uint32_t dw[4] = {dv[i].x, dv[i].y, dv[i].z, dv[i].w};
        const uint32_t gw[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double glo = (double)bf16_lo(gw[j]) * (double)bf16_lo(dw[j]);
            const double ghi = (double)bf16_hi(gw[j]) * (double)bf16_hi(dw[j]);
            const uint32_t lo = f64_to_bf16_rne(r * glo - (double)bf16_lo(xw[j]) * kk);
            const uint32_t hi = f64_to_bf16_rne(r * ghi - (double)bf16_hi(xw[j]) * kk);
            o[j] = lo | (hi << 16);
        }
        if (live[i])
            out[256 * i + tid] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Block sums of dgamma: workgroup (bx, by) owns columns [512 bx, +512) (two
// per thread) and tokens [128 by, +128) (fewer in a last block), summed in
// ascending order.
__global__ __launch_bounds__(256) void rmsnorm_bwd_dgamma_partial_kernel(const uint16_t* __restrict__ x,
                                                                         const float* __restrict__ rstd,
                                                                         const uint16_t* __restrict__ dy,
                                                                         int64_t M, int64_t K,
                                                                         double* __restrict__ ws)
{
    const int64_t col = (int64_t)blockIdx.x * 512 + 2 * threadIdx.x;
    if (col >= K)
        return;
    const int64_t t0 = (int64_t)blockIdx.y * kGroup;
    const int64_t t1 = t0 + kGroup < M ? t0 + kGroup : M;
    double a0 = 0.0, a1 = 0.0;
    int64_t t = t0;
    for (; t + 8 <= t1; t += 8) {                            // 8 tokens' loads in flight
        uint32_t xw[8], dw[8];
        float rs[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            xw[u] = *reinterpret_cast<const uint32_t*>(x + (t + u) * K + col);
            dw[u] = *reinterpret_cast<const uint32_t*>(dy + (t + u) * K + col);
            rs[u] = rstd[t + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            a0 = a0 + ((double)bf16_lo(dw[u]) * (double)bf16_lo(xw[u])) * (double)rs[u];
            a1 = a1 + ((double)bf16_hi(dw[u]) * (double)bf16_hi(xw[u])) * (double)rs[u];
        }
    }
    for (; t < t1; ++t) {
        const uint32_t xw = *reinterpret_cast<const uint32_t*>(x + t * K + col);
        const uint32_t dw = *reinterpret_cast<const uint32_t*>(dy + t * K + col);
        const double rt = (double)rstd[t];
        a0 = a0 + ((double)bf16_lo(dw) * (double)bf16_lo(xw)) * rt;
        a1 = a1 + ((double)bf16_hi(dw) * (double)bf16_hi(xw)) * rt;
    }
    ws[(int64_t)blockIdx.y * K + col] = a0;
    ws[(int64_t)blockIdx.y * K + col + 1] = a1;
}

// dgamma[k] = fp32 of the block partials added in ascending block order; 32
// blocks' loads in flight per thread.
__global__ __launch_bounds__(64) void rmsnorm_bwd_dgamma_final_kernel(const double* __restrict__ ws,
                                                                      int64_t nblocks, int64_t K,
                                                                      float* __restrict__ dgamma)
{
    const int64_t k = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (k >= K)
        return;
    double total = 0.0;
    int64_t b = 0;
    for (; b + 32 <= nblocks; b += 32) {
        double v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u)
            v[u] = ws[(b + u) * K + k];
#pragma unroll
        for (int u = 0; u < 32; ++u)
            total = total + v[u];
    }
    for (; b < nblocks; ++b)
        total = total + ws[b * K + k];
    dgamma[k] = (float)total;
}

// ===================================================== SwiGLU -> FP8 1x128
//
// The reference evaluation is fp64: (g / (1 + exp(-g))) * u, rounded once to
// BF16; its error (a few fp64 ulps) cannot move the rounding except within
// 2^-44 of a BF16 midpoint.  The kernel first evaluates in fp32:
//   e = v_exp_f32(g * fl(-log2 e)),  v = (g * v_rcp_f32(1 + e)) * u.
// For |g| < 64 its relative error is at most (eps = 2^-24)
//   2|g| eps (the rounded exponent argument, times ln 2)
//   + 4 eps (exp, within 2 ulp) + 2 eps (rcp, within 1 ulp)
//   + 3 eps (the add and the two products)  <=  (2|g| + 9) eps,
// the two hardware bounds measured on every argument these kernels pass.
// Elements whose fp32 value may round differently from the exact one
// (needs_f64 with B = 2|g| + 10 ulps) and every |g| >= 64 are evaluated
// again in fp64, one flagged element at a time per lane; an exact zero
// (g = 0 or u = 0: a signed zero on both routes) never is.
__device__ __forceinline__ uint32_t swiglu_bf16_f64(float g, float u)
{
    const double gd = g, ud = u;
    return f64_to_bf16_rne((gd / (1.0 + exp(-gd))) * ud);
}

// The fp32 value (rounded to BF16 by the caller) and whether it must be
// evaluated again in fp64.
// True when the fp32 value v, within B ulps of the exact value, may round to
// a different BF16 than the exact value: a BF16 rounding midpoint lies within
// lim = B + 2 ulps of v (the 2 cover the second-order terms the bounds leave
// out and the rounding of lim's own evaluation, both far below one ulp), or v
// lies outside [2^-100, 2^101), where an intermediate could under- or
// overflow and the relative bounds do not hold.  A relative error of B eps
// (eps = 2^-24) is at most B ulps of the result.  The conditions are combined
// without short-circuits so that the test compiles to straight-line code.
__device__ __forceinline__ bool needs_f64(float v, float lim)
{
    // the distance in ulps from v to the midpoint of its BF16 interval,
    // |low 16 bits - 0x8000|: v_sad_u16 adds the absolute differences of both
    // 16-bit halves, so the high half is cleared first
    const uint32_t d = __builtin_amdgcn_sad_u16(__float_as_uint(v) & 0xFFFFu, 0x8000u, 0u);
    const float a = __builtin_fabsf(v);
    return ((float)d <= lim) | !((a >= 0x1p-100f) & (a < 0x1p101f));
}

__device__ __forceinline__ float swiglu_f32(float g, float u, bool& redo)
{
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
    const float v = (g * __builtin_amdgcn_rcpf(1.0f + e)) * u;
    const float ag = __builtin_fabsf(g);
    const bool exact_zero = (g == 0.0f) | (u == 0.0f);
    redo = !exact_zero & ((ag >= 64.0f) | needs_f64(v, fmaf(ag, 2.0f, 12.0f)));   // B = 2|g| + 10
    return v;
}

// The 8 BF16 results of one lane's 16-byte chunks of gate and up.
__device__ __forceinline__ uint4 swiglu8(uint4 gv, uint4 uv)
{
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t hw[4];
    uint32_t need = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        bool r0, r1;
        const float h0 = swiglu_f32(bf16_lo(gw[j]), bf16_lo(uw[j]), r0);
        const float h1 = swiglu_f32(bf16_hi(gw[j]), bf16_hi(uw[j]), r1);
        hw[j] = pack_bf16x2(h0, h1);
        need |= (r0 ? 1u << (2 * j) : 0u) | (r1 ? 2u << (2 * j) : 0u);
    }
    while (need != 0) {                                     // divergent: flagged elements only
        const int k = __builtin_ctz(need);
        need &= need - 1;
        uint32_t gsel = 0, usel = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((k >> 1) == j) {
                gsel = gw[j];
                usel = uw[j];
            }
        const bool hi = k & 1;
        const uint32_t hb = swiglu_bf16_f64(hi ? bf16_hi(gsel) : bf16_lo(gsel), hi ? bf16_hi(usel) : bf16_lo(usel));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((k >> 1) == j)
                hw[j] = hi ? ((hw[j] & 0xFFFFu) | (hb << 16)) : ((hw[j] & 0xFFFF0000u) | hb);
    }
    return make_uint4(hw[0], hw[1], hw[2], hw[3]);
}

// Elementwise with 1x128 groups: 16 lanes per group, 8 values per lane, a
// wave covers 4 groups per step and keeps UNROLL steps of loads in flight.
// Group gi is row gi / GF, columns [128 (gi % GF), +128) of gate and up (row
// stride ld); the output is dense [M, F].
template <int UNROLL>
__global__ __launch_bounds__(256) void swiglu_quant_kernel(const uint16_t* __restrict__ gate,
                                                           const uint16_t* __restrict__ up,
                                                           int64_t ld, uint32_t GF, uint32_t ngroups,
                                                           uint2* __restrict__ q,
                                                           float* __restrict__ s)
{
    const int lane = threadIdx.x & 63;
    const int sub = lane & 15;
    const int slot = lane >> 4;
    const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const uint32_t nwaves = (gridDim.x * blockDim.x) >> 6;
    for (uint32_t base = wave * (4 * UNROLL); base < ngroups; base += nwaves * (4 * UNROLL)) {
        uint4 gv[UNROLL], uv[UNROLL];
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
            const uint32_t gi = base + k * 4 + slot;
            // past the end: re-read group 0 (always valid) and discard the result
            const uint32_t gc = gi < ngroups ? gi : 0u;
            const uint32_t m = gc / GF, j = gc - m * GF;
            const int64_t off = (int64_t)m * ld + (int64_t)j * kGroup + sub * 8;
            gv[k] = load_nt(gate + off);
            uv[k] = load_nt(up + off);
        }
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
            const uint32_t gi = base + k * 4 + slot;
            float scale;
            const uint2 c = quantize_group16(swiglu8(gv[k], uv[k]), scale);
            if (gi < ngroups) {
                q[(int64_t)gi * 16 + sub] = c;
                if (sub == 0)
                    s[gi] = scale;
            }
        }
    }
}

// ======================================================== SwiGLU backward
//
// BF16 gradients of h = silu(g) u (gradients between operators stay BF16):
// s = 1 / (1 + exp(-g)), d_up = dh (g s), d_gate = ((dh u) s) (1 + g (1 - s)),
// each the fp64 evaluation in that order rounded once to BF16.  As in the
// forward, the kernel first evaluates in fp32 (eps = 2^-24; dh g and dh u are
// exact products of BF16 values), with d_gate written through the identity
// 1 + g (1 - s) = s z,  z = 1 + e (1 + g):
//   e = v_exp_f32(g fl(-log2 e))       rel. error <= 2|g| eps + 4 eps
//   s = v_rcp_f32(1 + e)               <= 2|g| eps + 7 eps
//   a = 1 + g                          <= eps (exact unless |g| < 2^-16)
//   z = fma(e, a, 1)                   <= R (2|g| + 5) eps + eps,  R = |e a| / |z|
//   d_up   = (dh g) s                   <= (2|g| + 8) eps
//   d_gate = (((dh u) s) z) s           <= (4|g| + 18 + R (2|g| + 5)) eps
// z vanishes with silu' (g ~ -1.28) like 1 + g (1 - s) does, but the error it
// amplifies there is e's alone and R ~ 1 / ((1 + e) |w|): about a tenth of the
// amplification of the direct form 1 + g t, t = e s, so far fewer results next
// to that zero need fp64.
// (exp within 2 ulp and rcp within 1 ulp, measured on every argument these
// kernels pass).  A relative error of B eps is at most B ulps of the fp32
// result, so an output whose fp32 bits lie more than B + 2 ulps from a BF16
// midpoint rounds as the exact value does (needs_f64).  The others, |g| >= 64
// (exponent argument error and exp range), results outside [2^-100, 2^101)
// (where an intermediate could under- or overflow) and z = 0 (R infinite) are evaluated
// again in fp64, one flagged element at a time per lane.
__device__ __forceinline__ void swiglu_bwd_f64(float gf, float uf, float df, uint32_t& bg, uint32_t& bu)
{
    const double g = gf, u = uf, d = df;
    const double sg = 1.0 / (1.0 + exp(-g));
    bg = f64_to_bf16_rne(((d * u) * sg) * (1.0 + g * (1.0 - sg)));
    bu = f64_to_bf16_rne(d * (g * sg));
}

__device__ __forceinline__ void swiglu_bwd_f32(float g, float u, float dh, float& vg, float& vu, bool& redo)
{
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
    const float s = __builtin_amdgcn_rcpf(1.0f + e);
    const float a = 1.0f + g;
    const float z = fmaf(e, a, 1.0f);                 // (1 + e) w, one rounding
    vu = (dh * g) * s;
    vg = (((dh * u) * s) * z) * s;                    // z before the second s: no intermediate underflow
    const float ag = __builtin_fabsf(g);
    const float limu = fmaf(ag, 2.0f, 10.0f);                                   // B_u = 2|g| + 8
    // d_gate's test without a reciprocal: with lim = B_g + 2 = Y + R X,
    // R = |e a| / |z|, a midpoint distance d satisfies d <= lim exactly when
    // (d - Y) |z| <= |e a| X (z = 0: always, as R is infinite).  The three
    // roundings of that comparison move it by far less than the 2-ulp margin.
    const float X = fmaf(ag, 2.0f, 5.0f), Y = fmaf(ag, 4.0f, 20.0f);
    const float dg = (float)__builtin_amdgcn_sad_u16(__float_as_uint(vg) & 0xFFFFu, 0x8000u, 0u);
    const float avg = __builtin_fabsf(vg);
    const bool near_g = (dg - Y) * __builtin_fabsf(z) <= __builtin_fabsf(e * a) * X;
    const bool out_g = !((avg >= 0x1p-100f) & (avg < 0x1p101f));
    redo = (ag >= 64.0f) | needs_f64(vu, limu) | near_g | out_g;
}

// The 8 (d_gate, d_up) pairs of 16-byte chunks of g, u and dh.
__device__ __forceinline__ void swiglu_bwd8(uint4 gv, uint4 uv, uint4 dv, uint4& og4, uint4& ou4)
{
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
    const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
    uint32_t og[4], ou[4];
    uint32_t need = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float vg0, vu0, vg1, vu1;
        bool r0, r1;
        swiglu_bwd_f32(bf16_lo(gw[j]), bf16_lo(uw[j]), bf16_lo(dw[j]), vg0, vu0, r0);
        swiglu_bwd_f32(bf16_hi(gw[j]), bf16_hi(uw[j]), bf16_hi(dw[j]), vg1, vu1, r1);
        og[j] = pack_bf16x2(vg0, vg1);
        ou[j] = pack_bf16x2(vu0, vu1);
        need |= (r0 ? 1u << (2 * j) : 0u) | (r1 ? 2u << (2 * j) : 0u);
    }
    while (need != 0) {                                     // divergent: flagged elements only
        const int k = __builtin_ctz(need);
        need &= need - 1;
        uint32_t gs = 0, us = 0, ds = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((k >> 1) == j) {
                gs = gw[j];
                us = uw[j];
                ds = dw[j];
            }
        const bool hi = k & 1;
        uint32_t bg, bu;
        swiglu_bwd_f64(hi ? bf16_hi(gs) : bf16_lo(gs), hi ? bf16_hi(us) : bf16_lo(us),
                       hi ? bf16_hi(ds) : bf16_lo(ds), bg, bu);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((k >> 1) == j) {
                og[j] = hi ? ((og[j] & 0xFFFFu) | (bg << 16)) : ((og[j] & 0xFFFF0000u) | bg);
                ou[j] = hi ? ((ou[j] & 0xFFFFu) | (bu << 16)) : ((ou[j] & 0xFFFF0000u) | bu);
            }
    }
    og4 = make_uint4(og[0], og[1], og[2], og[3]);
    ou4 = make_uint4(ou[0], ou[1], ou[2], ou[3]);
}

// A thread owns 8 consecutive columns of one row (16-byte loads of g, u, dh;
// 16-byte stores of d_gate into dgu[:, :F] and d_up into dgu[:, F:]).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* __restrict__ gate,
                                                         const uint16_t* __restrict__ up, int64_t ld,
                                                         const uint16_t* __restrict__ dh, int64_t F,
                                                         int64_t nchunks, uint16_t* __restrict__ dgu)
{
    const int64_t cpr = F >> 3;                             // 8-column chunks per row
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nchunks; i += (int64_t)gridDim.x * 256) {
        const int64_t m = i / cpr, c = (i - m * cpr) * 8;
        uint4 og, ou;
        swiglu_bwd8(load_nt(gate + m * ld + c), load_nt(up + m * ld + c), load_nt(dh + m * F + c), og, ou);
        uint16_t* row = dgu + m * 2 * F + c;
        *reinterpret_cast<uint4*>(row) = og;
        *reinterpret_cast<uint4*>(row + F) = ou;
    }
}

// =========================== SwiGLU backward fused with its FP8 quantization
//
// The gradient of the fused gate/up projection's output, dgu = [d_gate | d_up]
// [T, 2F], is consumed only as FP8: 1x128 row groups by the gate/up DGrad and
// 128-along-token groups (transposed) by its WGrad.  One workgroup per
// 128 (tokens) x 128 (columns of g, u, dh) tile computes both gradients of
// the tile in registers (swiglu_bwd8 on 8 rows x 8 columns per
// thread), writes their row quantization directly (gate columns f0.., up
// columns F + f0..), then parks each half in LDS in turn for the transposing
// quantizer's column phase.  dgu itself is never stored; the codes and scales
// are bit-identical to fp8_quant_transpose (dual) of fp8_swiglu_bwd's output.
__global__ __launch_bounds__(256) void swiglu_bwd_quant_kernel(const uint16_t* __restrict__ gate,
                                                               const uint16_t* __restrict__ up, int64_t ld,
                                                               const uint16_t* __restrict__ dh, int64_t T,
                                                               int64_t F, uint8_t* __restrict__ q,
                                                               float* __restrict__ s, uint8_t* __restrict__ qT,
                                                               float* __restrict__ sT)
{
    __shared__ uint4 tile[128 * 16];              // [row][16 chunks of 8 bf16] = 32 KB
    __shared__ uint32_t red[4 * 64];
    __shared__ __attribute__((aligned(16))) uint8_t ctile[128 * 128];
    const int tid = threadIdx.x;
    const int sub = tid & 15, r0 = tid >> 4;
    const int64_t t0 = (int64_t)blockIdx.y * kGroup, f0 = (int64_t)blockIdx.x * kGroup;
    const int64_t F2 = 2 * F, G2 = F2 / kGroup;
    uint4 vg[8], vu[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = t0 + r0 + 16 * i, col = f0 + sub * 8;
        swiglu_bwd8(load_nt(gate + row * ld + col), load_nt(up + row * ld + col), load_nt(dh + row * F + col),
                    vg[i], vu[i]);
    }
    // 1x128 row groups of both halves
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = t0 + r0 + 16 * i;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 v = h ? vu[i] : vg[i];
            const int64_t col = (h ? F : 0) + f0;
            const GroupScale gs = group_scale(max_over_16_lanes(absmax_bits_8xbf16(v)));
            *reinterpret_cast<uint2*>(q + row * F2 + col + sub * 8) = quantize8(v, gs);
            if (sub == 0)
                s[row * G2 + col / kGroup] = gs.s;
        }
    }
    // 128-along-token groups, transposed: the gate half, then the up half
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h)
            __syncthreads();                          // the gate half's tile and code tile are drained
#pragma unroll
        for (int i = 0; i < 8; ++i)
            tile[(r0 + 16 * i) * 16 + sub] = h ? vu[i] : vg[i];
        __syncthreads();
        transpose_quant_tile<false>(tile, red, ctile, qT, sT, (h ? F : 0) + f0, t0, T, F2);
    }
}

// ================================================================ launchers

template <int NV>
static void rmsnorm_launch(const uint16_t* xp, const uint16_t* gp, int64_t M, int K, float eps, uint8_t* q,
                           float* s, float* rstd, hipStream_t st)
{
    rmsnorm_quant_kernel<NV><<<(unsigned)((M + 3) / 4), 256, 0, st>>>(xp, gp, M, K, eps, q, s, rstd);
}

void launch_rmsnorm_quant(const void* x, const void* gamma, int64_t M, int64_t K, float eps, uint8_t* q,
                          float* s, float* rstd, hipStream_t st)
{
    // As many register passes as the row needs (K <= 8192); wider rows (to
    // 16384) take 32 passes, the surplus ones masked.
    using Fn = void (*)(const uint16_t*, const uint16_t*, int64_t, int, float, uint8_t*, float*, float*,
                        hipStream_t);
    static constexpr Fn by_passes[17] = {
        nullptr, rmsnorm_launch<1>, rmsnorm_launch<2>, rmsnorm_launch<3>, rmsnorm_launch<4>,
        rmsnorm_launch<5>, rmsnorm_launch<6>, rmsnorm_launch<7>, rmsnorm_launch<8>, rmsnorm_launch<9>,
        rmsnorm_launch<10>, rmsnorm_launch<11>, rmsnorm_launch<12>, rmsnorm_launch<13>, rmsnorm_launch<14>,
        rmsnorm_launch<15>, rmsnorm_launch<16>};
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* gp = static_cast<const uint16_t*>(gamma);
    const int64_t passes = (K + 511) / 512;
    if (passes <= 16)
        by_passes[passes](xp, gp, M, (int)K, eps, q, s, rstd, st);
    else
        rmsnorm_launch<32>(xp, gp, M, (int)K, eps, q, s, rstd, st);
}

void launch_swiglu_quant(const void* gate, const void* up, int64_t ld, int64_t M, int64_t F, uint8_t* q,
                         float* s, hipStream_t st)
{
    const uint32_t GF = (uint32_t)(F / kGroup);
    const uint32_t ngroups = (uint32_t)(M * (F / kGroup));
    constexpr int kUnroll = 2;
    int64_t blocks = ((int64_t)ngroups + 4 * 4 * kUnroll - 1) / (4 * 4 * kUnroll);
    if (blocks > 16384)
        blocks = 16384;
    swiglu_quant_kernel<kUnroll><<<(unsigned)(blocks < 1 ? 1 : blocks), 256, 0, st>>>(
        static_cast<const uint16_t*>(gate), static_cast<const uint16_t*>(up), ld, GF, ngroups,
        reinterpret_cast<uint2*>(q), s);
}

void launch_swiglu_bwd(const void* gate, const void* up, int64_t ld, const void* dh, int64_t M, int64_t F,
                       void* dgu, hipStream_t st)
{
    const int64_t nchunks = M * (F / 8);
    int64_t blocks = (nchunks + 255) / 256;
    if (blocks > 32768)
        blocks = 32768;
    swiglu_bwd_kernel<<<(unsigned)(blocks < 1 ? 1 : blocks), 256, 0, st>>>(
        static_cast<const uint16_t*>(gate), static_cast<const uint16_t*>(up), ld, static_cast<const uint16_t*>(dh),
        F, nchunks, static_cast<uint16_t*>(dgu));
}

void launch_swiglu_bwd_quant(const void* gate, const void* up, int64_t ld, const void* dh, int64_t T, int64_t F,
                             uint8_t* q, float* s, uint8_t* qT, float* sT, hipStream_t st)
{
    const dim3 grid((unsigned)(F / kGroup), (unsigned)(T / kGroup));
    swiglu_bwd_quant_kernel<<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(gate), static_cast<const uint16_t*>(up),
                                                  ld, static_cast<const uint16_t*>(dh), T, F, q, s, qT, sT);
}

// Diagnostic: the fp32 hardware functions the SwiGLU kernels evaluate with,
// and the division-free group-scale functions of the quantizers, one per
// element (fn 0: v_exp_f32 = 2^x; fn 1: v_rcp_f32 = 1/x; fn 2: div448_rn;
// fn 3: rcp_rn).
__global__ __launch_bounds__(256) void math_probe_kernel(const float* __restrict__ in, int64_t n,
                                                         float* __restrict__ out, int fn)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        const float x = in[i];
        out[i] = fn == 0 ? __builtin_amdgcn_exp2f(x)
                 : fn == 1 ? __builtin_amdgcn_rcpf(x)
                 : fn == 2 ? div448_rn(x)
                           : rcp_rn(x);
    }
}

void launch_math_probe(const float* in, int64_t n, float* out, int fn, hipStream_t st)
{
    int64_t b = (n + 255) / 256;
    if (b > 65536)
        b = 65536;
    math_probe_kernel<<<(unsigned)(b < 1 ? 1 : b), 256, 0, st>>>(in, n, out, fn);
}

// Diagnostic: the SwiGLU kernels' re-evaluation test (needs_f64) on given
// values with one bound, 1.0 where it flags the value, else 0.0.
__global__ __launch_bounds__(256) void flag_probe_kernel(const float* __restrict__ v, int64_t n, float lim,
                                                         float* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
        out[i] = needs_f64(v[i], lim) ? 1.0f : 0.0f;
}

void launch_flag_probe(const float* v, int64_t n, float lim, float* out, hipStream_t st)
{
    int64_t b = (n + 255) / 256;
    if (b > 65536)
        b = 65536;
    flag_probe_kernel<<<(unsigned)(b < 1 ? 1 : b), 256, 0, st>>>(v, n, lim, out);
}

template <int NP>
static void rmsnorm_bwd_dx_launch(const uint16_t* x, const uint16_t* g, const float* r, const uint16_t* dy, int64_t M,
                                  int K, uint16_t* dx, hipStream_t st)
{
    rmsnorm_bwd_dx_kernel<NP><<<(unsigned)M, 256, 0, st>>>(x, g, r, dy, K, dx);
}

void launch_rmsnorm_bwd(const void* x, const void* gamma, const float* rstd, const void* dy, int64_t M, int64_t K,
                        void* dx, float* dgamma, double* ws, hipStream_t st)
{
    using Fn = void (*)(const uint16_t*, const uint16_t*, const float*, const uint16_t*, int64_t, int, uint16_t*,
                        hipStream_t);
    static constexpr Fn by_passes[9] = {nullptr, rmsnorm_bwd_dx_launch<1>, rmsnorm_bwd_dx_launch<2>,
                                        rmsnorm_bwd_dx_launch<3>, rmsnorm_bwd_dx_launch<4>, rmsnorm_bwd_dx_launch<5>,
                                        rmsnorm_bwd_dx_launch<6>, rmsnorm_bwd_dx_launch<7>, rmsnorm_bwd_dx_launch<8>};
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* dp = static_cast<const uint16_t*>(dy);
    by_passes[(K + 2047) / 2048](xp, static_cast<const uint16_t*>(gamma), rstd, dp, M, (int)K,
                                 static_cast<uint16_t*>(dx), st);
    if (dgamma) {
        const int64_t nb = (M + kGroup - 1) / kGroup;
        const dim3 grid((unsigned)((K + 511) / 512), (unsigned)nb);
        rmsnorm_bwd_dgamma_partial_kernel<<<grid, 256, 0, st>>>(xp, rstd, dp, M, K, ws);
        rmsnorm_bwd_dgamma_final_kernel<<<(unsigned)((K + 63) / 64), 64, 0, st>>>(ws, nb, K, dgamma);
    }
}

}  // namespace fp8lin
