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
//   SwiGLU:   h = bf16(silu(g) * u), silu(g) = g / (1 + exp(-g)), evaluated
//             in fp64 and rounded once to BF16.
#include "fp8lin_device.hpp"
#include "fp8lin_launch.hpp"

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

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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
// registers (NV passes, K <= 512 NV), so the row is read from HBM once.  The
// squares are summed in fp64 in the stated order: 8 in-lane values as a
// tree, then 16 lanes by xor exchange (a balanced tree over the 128-group,
// identical in every lane because fp64 addition is commutative), then the
// group sums in ascending order through lane reads.  Gamma (shared by every
// row) is read in the second pass from the cache.
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
    uint4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
        v[i] = (512 * i + 8 * lane < K) ? load_nt(xr + 64 * i + lane) : make_uint4(0, 0, 0, 0);

    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (512 * i >= K)
            continue;                                       // wave-uniform
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        double sq[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double lo = (double)bf16_lo(w[j]);
            const double hi = (double)bf16_hi(w[j]);
            sq[2 * j] = lo * lo;
            sq[2 * j + 1] = hi * hi;
        }
        double t = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
        t = t + shfl_xor_f64(t, 1);
        t = t + shfl_xor_f64(t, 2);
        t = t + shfl_xor_f64(t, 4);
        t = t + shfl_xor_f64(t, 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (4 * i + j < G)                              // wave-uniform
                ss = ss + readlane_f64(t, 16 * j);
    }
    const double r = 1.0 / __builtin_sqrt(ss / (double)K + (double)eps);
    const float rs = (float)r;
    if (rstd_out != nullptr && lane == 0)
        rstd_out[row] = rs;

    const uint4* gr = reinterpret_cast<const uint4*>(gamma);
    uint2* qr = reinterpret_cast<uint2*>(q + row * K);
    float* sr = s + row * G;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (512 * i >= K)
            continue;                                       // wave-uniform
        const bool live = 512 * i + 8 * lane < K;           // uniform over each 16-lane group
        const uint4 gw = live ? gr[64 * i + lane] : make_uint4(0, 0, 0, 0);
        const uint32_t xw[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        const uint32_t gg[4] = {gw.x, gw.y, gw.z, gw.w};
        uint32_t yw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = (bf16_lo(xw[j]) * rs) * bf16_lo(gg[j]);
            const float hi = (bf16_hi(xw[j]) * rs) * bf16_hi(gg[j]);
            yw[j] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
        }
        float scale;
        const uint2 c = quantize_group16(make_uint4(yw[0], yw[1], yw[2], yw[3]), scale);
        if (live) {
            qr[64 * i + lane] = c;
            if ((lane & 15) == 0)
                sr[4 * i + (lane >> 4)] = scale;
        }
    }
}

// ===================================================== SwiGLU -> FP8 1x128
//
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
            if (gi < ngroups) {
                const uint32_t m = gi / GF, j = gi - m * GF;
                const int64_t off = (int64_t)m * ld + (int64_t)j * kGroup + sub * 8;
                gv[k] = load_nt(gate + off);
                uv[k] = load_nt(up + off);
            } else {
                gv[k] = make_uint4(0, 0, 0, 0);
                uv[k] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
            const uint32_t gi = base + k * 4 + slot;
            const uint32_t gw[4] = {gv[k].x, gv[k].y, gv[k].z, gv[k].w};
            const uint32_t uw[4] = {uv[k].x, uv[k].y, uv[k].z, uv[k].w};
            uint32_t hw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double g0 = (double)bf16_lo(gw[j]), g1 = (double)bf16_hi(gw[j]);
                const double u0 = (double)bf16_lo(uw[j]), u1 = (double)bf16_hi(uw[j]);
                const double h0 = (g0 / (1.0 + exp(-g0))) * u0;
                const double h1 = (g1 / (1.0 + exp(-g1))) * u1;
                hw[j] = f64_to_bf16_rne(h0) | (f64_to_bf16_rne(h1) << 16);
            }
            float scale;
            const uint2 c = quantize_group16(make_uint4(hw[0], hw[1], hw[2], hw[3]), scale);
            if (gi < ngroups) {
                q[(int64_t)gi * 16 + sub] = c;
                if (sub == 0)
                    s[gi] = scale;
            }
        }
    }
}

// ================================================================ launchers

void launch_rmsnorm_quant(const void* x, const void* gamma, int64_t M, int64_t K, float eps, uint8_t* q,
                          float* s, float* rstd, hipStream_t st)
{
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* gp = static_cast<const uint16_t*>(gamma);
    const unsigned blocks = (unsigned)((M + 3) / 4);
    const int k = (int)K;
    if (K <= 512)
        rmsnorm_quant_kernel<1><<<blocks, 256, 0, st>>>(xp, gp, M, k, eps, q, s, rstd);
    else if (K <= 1024)
        rmsnorm_quant_kernel<2><<<blocks, 256, 0, st>>>(xp, gp, M, k, eps, q, s, rstd);
    else if (K <= 2048)
        rmsnorm_quant_kernel<4><<<blocks, 256, 0, st>>>(xp, gp, M, k, eps, q, s, rstd);
    else if (K <= 4096)
        rmsnorm_quant_kernel<8><<<blocks, 256, 0, st>>>(xp, gp, M, k, eps, q, s, rstd);
    else if (K <= 8192)
        rmsnorm_quant_kernel<16><<<blocks, 256, 0, st>>>(xp, gp, M, k, eps, q, s, rstd);
    else
        rmsnorm_quant_kernel<32><<<blocks, 256, 0, st>>>(xp, gp, M, k, eps, q, s, rstd);
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

}  // namespace fp8lin
