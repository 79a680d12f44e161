// w4_kernels.hip -- 4-bit (MXFP4) weights for the rollout GEMM, gfx950.
//
// The QeRL page ("QeRL: Beyond Efficiency -- Quantization-enhanced
// Reinforcement Learning for LLMs", abstract) runs the rollout on 4-bit NVFP4
// weights and gives no format details.  NVFP4 belongs to NVIDIA's Blackwell;
// gfx950's converters and matrix cores take the OCP Microscaling formats, so
// the weights here are MXFP4 as OCP MX v1.0 defines it:
//   - E2M1 elements (sign, 2 exponent bits with bias 1, 1 mantissa bit;
//     magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6);
//   - 32 consecutive elements of a weight row share one E8M0 scale 2^E,
//     stored as E + 127, with E = floor(log2(amax)) - 2 clamped to
//     [-127, 127] (-127 for an all-zero block);
//   - an element is the E2M1 value nearest to v / 2^E, ties to the even
//     code, saturated at 6, sign kept; two per byte, even k in the low nibble.
//
// GEMM (activations keep the flow's FP8 1x128 groups):
//     Y[m,n] = sum_g sx[m,g] * sum_{k in g} dec(X[m,k]) * e2m1(W[n,k]) * 2^E[n,k/32]
// Both operands are converted exactly to fp16 and multiplied on the fp16
// matrix core (gfx950's FP8 matrix core truncates inside its sums).  An E2M1
// code is converted with its block's scale relative to the largest block
// scale Ec of the same column and 128-group, 2^(E - Ec) <= 1: exact in fp16
// unless the block lies more than 2^23 below that largest block (its terms
// are then below 2^-20 of the group's largest weight).  2^Ec and sx enter the
// fp32 promotion once per group.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_stream.hpp"
#include "fp8lin_launch.hpp"

namespace fp8lin {
namespace w4 {

// u32x4 (fp8lin_device.hpp), v8h and dec::cvt8 (decode_stream.hpp) are shared
// with the FP8 kernels.
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBlock = 32;

__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------- quantization

// E2M1 magnitude code of a = |v| / 2^E (a < 8): the nearest of
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even code, 6 for a > 5.
__device__ __forceinline__ uint32_t e2m1_mag(float a)
{
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
           (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

// 4-bit code of the bf16 `bits` scaled by 2^-E (exact: a power-of-two scaling).
__device__ __forceinline__ uint32_t e2m1_code(uint32_t bits, int negE)
{
    const float q = __builtin_amdgcn_ldexpf(__uint_as_float(bits << 16), negE);
    return e2m1_mag(fabsf(q)) | (((bits >> 15) & 1u) << 3);
}

// Four threads per 32-element block of W [N][K] bf16 (K % 32 == 0, so the
// blocks tile the flattened array): thread i converts elements [8i, 8i + 8),
// 16 contiguous bytes, so a wave's loads are one contiguous KB; the block's
// amax is combined over its four lanes.  Threads past the end read the last
// element group and store nothing (all lanes take part in the exchange).
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t* __restrict__ w, int64_t nthreads,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool valid = i < nthreads;
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w) + (valid ? i : nthreads - 1));
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t lo = v[c] & 0x7FFFu, hi = (v[c] >> 16) & 0x7FFFu;
        amax = amax > lo ? amax : lo;
        amax = amax > hi ? amax : hi;
    }
    amax = max_over_4_lanes(amax);
    // floor(log2(amax)) = exponent field - 127 for a normal amax; zero and
    // subnormal amax (floor(log2) <= -127) clamp to E = -127
    const int ef = (int)(amax >> 7);
    int E = ef == 0 ? -127 : ef - 127 - 2;
    E = E < -127 ? -127 : (E > 127 ? 127 : E);
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t lo = e2m1_code(v[c] & 0xFFFFu, -E), hi = e2m1_code(v[c] >> 16, -E);
        word |= (lo | (hi << 4)) << (8 * c);
    }
    if (valid) {
        reinterpret_cast<uint32_t*>(codes)[i] = word;
        if ((i & 3) == 0)
            scales[i >> 2] = (uint8_t)(E + 127);
    }
}

// ------------------------------------------------------------------ GEMM

// 8 E2M1 codes (one word, element 2i in the low nibble of byte i) -> 8 fp16
// times `scale` (a power of two, 2^-30 <= scale <= 1).
__device__ __forceinline__ v8h fp4x8_to_f16(uint32_t w, float scale)
{
    const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0);
    const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1);
    const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2);
    const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3);
    return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// A workgroup computes 64 rows x 64 columns of Y with four waves: wave
// (ct, kq) owns W columns [32ct, 32ct + 32) and the K half [64kq, 64kq + 64)
// of every 128-group, for both 32-row halves of X (two 32x32 tiles).  Lane
// (j = lane & 31, kh = lane >> 5) is A row j (an X row) and B column j (a W
// column); its K slots in MFMA step s (0..3) are
//     k = 128g + 64kq + 32kh + 8s + e,  e = 0..7,
// so its 32 W elements of a group are exactly the MX block 4g + 2kq + kh.
// The two K halves are added in a fixed order at the end.  Requires
// K % 128 == 0, K <= kMaxK, M, N >= 1; rows past M and columns past N read the
// last row / column and are not stored.
constexpr int kMaxK = 16384;

__global__ __launch_bounds__(256) void gemm_w4_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                                                      const uint8_t* __restrict__ w4,
                                                      const uint8_t* __restrict__ s4, int64_t M, int64_t N,
                                                      int64_t K, uint16_t* __restrict__ y)
{
    __shared__ __attribute__((aligned(16))) float lds_sx[kMaxK / kGroup][64];
    __shared__ __attribute__((aligned(16))) float lds_red[2][2][16][64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ct = wave & 1, kq = wave >> 1;
    const int j = lane & 31, kh = lane >> 5;
    const int64_t G = K / kGroup;
    const int64_t n0 = (int64_t)blockIdx.x * 64, m0 = (int64_t)blockIdx.y * 64;

    // lds_sx[g][r] = sx[m0 + r][g]
    for (int64_t idx = tid; idx < 64 * G; idx += 256) {
        const int64_t r = idx / G, g = idx - r * G;
        const int64_t row = m0 + r < M ? m0 + r : M - 1;
        lds_sx[g][r] = sx[row * G + g];
    }

    const int64_t col = n0 + 32 * ct + j;
    const int64_t ccol = col < N ? col : N - 1;
    // group g: W bytes [64g + 32kq + 16kh, +16) of the column (4 u32x4 per
    // group), its 4 scale bytes at word g, X bytes [128g + 64kq + 32kh, +32)
    // of the row (8 u32x4 per group)
    const u32x4* wp = reinterpret_cast<const u32x4*>(w4 + ccol * (K / 2) + 32 * kq + 16 * kh);
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(s4 + ccol * (K / kBlock));
    const u32x4* xp[2];
#pragma unroll
    for (int xt = 0; xt < 2; ++xt) {
        const int64_t row = m0 + 32 * xt + j;
        const int64_t crow = row < M ? row : M - 1;
        xp[xt] = reinterpret_cast<const u32x4*>(xq + crow * K + 64 * kq + 32 * kh);
    }

    v16f acc[2];
#pragma unroll
    for (int xt = 0; xt < 2; ++xt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[xt][r] = 0.f;

    u32x4 wv = __builtin_nontemporal_load(wp);
    uint32_t sv = sp[0];
    u32x4 xv[2][2];
#pragma unroll
    for (int xt = 0; xt < 2; ++xt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            xv[xt][h] = xp[xt][h];
    __syncthreads();                               // scale table built

    const int my_block = 2 * kq + kh;              // block 4g + my_block
    for (int64_t g = 0; g < G; ++g) {
        const u32x4 wc = wv;
        const uint32_t sc = sv;
        u32x4 xc[2][2];
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                xc[xt][h] = xv[xt][h];
        {
            const int64_t gn = g + 1 < G ? g + 1 : g;   // last group: a harmless re-read
            wv = __builtin_nontemporal_load(wp + 4 * gn);
            sv = sp[gn];
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    xv[xt][h] = xp[xt][8 * gn + h];
        }
        const int e0 = (int)(sc & 255u), e1 = (int)((sc >> 8) & 255u), e2 = (int)((sc >> 16) & 255u),
                  e3 = (int)(sc >> 24);
        const int ec = max(max(e0, e1), max(e2, e3));
        const int eb = (int)((sc >> (8 * my_block)) & 255u);
        const float cs = __builtin_amdgcn_ldexpf(1.0f, max(eb - ec, -30));
        v8h wf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            wf[s] = fp4x8_to_f16(wc[s], cs);
        v16f tmp[2];
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                tmp[xt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int xt = 0; xt < 2; ++xt) {
                const u32x4& xw = xc[xt][s >> 1];
                const v8h xf = dec::cvt8(xw[2 * (s & 1)], xw[2 * (s & 1) + 1]);
                tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf, wf[s], tmp[xt], 0, 0, 0);
            }
        // D[i][j]: register r holds X row i = 8(r/4) + 4kh + (r%4) of the tile
        const int esh = ec - 127;
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float4 s4v = *reinterpret_cast<const float4*>(&lds_sx[g][32 * xt + 8 * a + 4 * kh]);
                acc[xt][4 * a + 0] = fmaf(tmp[xt][4 * a + 0], __builtin_amdgcn_ldexpf(s4v.x, esh), acc[xt][4 * a + 0]);
                acc[xt][4 * a + 1] = fmaf(tmp[xt][4 * a + 1], __builtin_amdgcn_ldexpf(s4v.y, esh), acc[xt][4 * a + 1]);
                acc[xt][4 * a + 2] = fmaf(tmp[xt][4 * a + 2], __builtin_amdgcn_ldexpf(s4v.z, esh), acc[xt][4 * a + 2]);
                acc[xt][4 * a + 3] = fmaf(tmp[xt][4 * a + 3], __builtin_amdgcn_ldexpf(s4v.w, esh), acc[xt][4 * a + 3]);
            }
    }

    // K half 1 into LDS, then half 0 adds it and stores
    if (kq == 1) {
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                lds_red[ct][xt][r][lane] = acc[xt][r];
    }
    __syncthreads();
    if (kq == 0 && col < N) {
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + 32 * xt + 8 * (r >> 2) + 4 * kh + (r & 3);
                if (row < M)
                    y[row * N + col] = bf16_rne(acc[xt][r] + lds_red[ct][xt][r][lane]);
            }
    }
}


// Decode form (M <= 64, K % 256 == 0): X streams through the LDS ring of the
// FP8 decode GEMMs (wave 8, two groups per chunk, one barrier per chunk), so
// each workgroup reads X once; waves 0-7 load their W codes straight into
// registers one chunk ahead and read the scale words from an LDS table (one
// contiguous read of the workgroup's 64 scale rows at the start).  Wave
// (ct, kp, kq) owns W columns [32ct, +32) and, of each chunk, group kp and the
// K quarter pieces
// {4kh + 2kq + q} of it: lane (m, kh) holds X row m of each 32-row tile and W
// column m at k = 64kh + 32kq + 16q + e within the group -- its 32 W codes are
// the MX block 2kh + kq of the group.  Each chunk's partial products are
// promoted during the next chunk; the four (kp, kq) partials are added in a
// fixed order at the end.  Rows past M read row M - 1 and are not stored.
template <int NCH>
__global__ __launch_bounds__(576) void gemm_w4_decode_kernel(const uint8_t* __restrict__ xq,
                                                             const float* __restrict__ sx,
                                                             const uint8_t* __restrict__ w4,
                                                             const uint8_t* __restrict__ s4, int64_t M, int64_t N,
                                                             int64_t K, uint16_t* __restrict__ y)
{
    using namespace dec;
    constexpr int WDX = 4;
    static_assert(WDX * WCH >= 3 * 2 * 2 * 16 * 64 * 4, "partial sums fit in the X ring");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_x[WDX][WCH];
    __shared__ __attribute__((aligned(16))) float lds_sx[kMaxK / kGroup * 64];   // [g][row]
    __shared__ uint32_t lds_sw[64 * (kMaxK / kGroup + 1)];                       // [column][g], stride G + 1

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = K / kGroup, nch = NCH > 0 ? NCH : G / CH;
    const int64_t n0 = (int64_t)blockIdx.x * 64;

    if (wave < 8) {
        // the X scales [g][row] and the workgroup's W scale words (four E8M0
        // bytes per column and group) [column][g]; columns past N repeat N - 1
        // four entries of each table per thread and batch, the batch's loads
        // in flight together (a load-store loop would wait on each load)
        const int Gi = (int)G, GS = Gi + 1, nent = 64 * Gi;
        for (int base = 0; base < nent; base += 512 * 4) {
            float xs[4];
            uint32_t ws[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = min(base + tid + 512 * i, nent - 1);
                const int r = idx / Gi, g = idx - r * Gi;
                const int64_t row = r < M ? r : M - 1;
                const int64_t wc = n0 + r < N ? n0 + r : N - 1;
                xs[i] = sx[row * G + g];
                ws[i] = reinterpret_cast<const uint32_t*>(s4 + wc * (K / kBlock))[g];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = base + tid + 512 * i;
                if (idx < nent) {
                    const int r = idx / Gi, g = idx - r * Gi;
                    lds_sx[g * 64 + r] = xs[i];
                    lds_sw[r * GS + g] = ws[i];
                }
            }
        }
        const int ct = wave & 1, kp = (wave >> 1) & 1, kq = wave >> 2;
        const int m = lane & 31, kh = lane >> 5;
        const int64_t col = n0 + 32 * ct + m;
        const int64_t ccol = col < N ? col : N - 1;
        // chunk c: group 2c + kp, code bytes [64(2c + kp) + 32kh + 16kq, +16)
        // of the column (8 u32x4 per chunk), scale word 2c + kp
        const u32x4* wp = reinterpret_cast<const u32x4*>(w4 + ccol * (K / 2) + 64 * kp + 32 * kh + 16 * kq);
        const uint32_t* swl = lds_sw + (32 * ct + m) * GS + kp;   // + 2 words per chunk
        u32x4 wreg = __builtin_nontemporal_load(wp);
        const int my_block = 2 * kh + kq;

        v16f acc[2], prev[2];
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[xt][r] = prev[xt][r] = 0.f;
        int prev_g = 0, prev_esh = 0;
        // acc += t * sx[row][g] * 2^esh (rows of the lane's registers)
        auto promote = [&](const v16f (&t)[2], int g, int esh) {
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float4 sv = *reinterpret_cast<const float4*>(&lds_sx[g * 64 + 32 * xt + 8 * a + 4 * kh]);
                    acc[xt][4 * a + 0] = fmaf(t[xt][4 * a + 0], __builtin_amdgcn_ldexpf(sv.x, esh), acc[xt][4 * a + 0]);
                    acc[xt][4 * a + 1] = fmaf(t[xt][4 * a + 1], __builtin_amdgcn_ldexpf(sv.y, esh), acc[xt][4 * a + 1]);
                    acc[xt][4 * a + 2] = fmaf(t[xt][4 * a + 2], __builtin_amdgcn_ldexpf(sv.z, esh), acc[xt][4 * a + 2]);
                    acc[xt][4 * a + 3] = fmaf(t[xt][4 * a + 3], __builtin_amdgcn_ldexpf(sv.w, esh), acc[xt][4 * a + 3]);
                }
        };
        __syncthreads();                           // chunk 0 of X landed, table built
        constexpr int kUnroll = NCH > 0 ? NCH : 1;
#pragma unroll kUnroll
        for (int64_t c = 0; c < nch; ++c) {
            const uint8_t* xl = lds_x[c % WDX];
            u32x4 xv[2][2];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int xt = 0; xt < 2; ++xt)
                    xv[xt][q] = *reinterpret_cast<const u32x4*>(xl + w_off(32 * xt + m, 8 * kp + 4 * kh + 2 * kq + q));
            const u32x4 wc = wreg;
            const uint32_t sc = swl[2 * c];
            {
                const int64_t cn = c + 1 < nch ? c + 1 : c;   // last chunk: a harmless re-read
                wreg = __builtin_nontemporal_load(wp + 8 * cn);
            }
            if (c > 0)
                promote(prev, prev_g, prev_esh);
            const int e0 = (int)(sc & 255u), e1 = (int)((sc >> 8) & 255u), e2 = (int)((sc >> 16) & 255u),
                      e3 = (int)(sc >> 24);
            const int ec = max(max(e0, e1), max(e2, e3));
            const int eb = (int)((sc >> (8 * my_block)) & 255u);
            const float cs = __builtin_amdgcn_ldexpf(1.0f, max(eb - ec, -30));
            v16f tmp[2];
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    tmp[xt][r] = 0.f;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const v8h wlo = fp4x8_to_f16(wc[2 * q], cs), whi = fp4x8_to_f16(wc[2 * q + 1], cs);
#pragma unroll
                for (int xt = 0; xt < 2; ++xt) {
                    const v8h xlo = dec::cvt8(xv[xt][q].x, xv[xt][q].y);
                    const v8h xhi = dec::cvt8(xv[xt][q].z, xv[xt][q].w);
                    tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xlo, wlo, tmp[xt], 0, 0, 0);
                    tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xhi, whi, tmp[xt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
                prev[xt] = tmp[xt];
            prev_g = (int)(2 * c + kp);
            prev_esh = ec - 127;
            __syncthreads();                       // chunk c drained, chunk c + 1 landed
        }
        promote(prev, prev_g, prev_esh);           // the last chunk
        __syncthreads();                           // the loader drained: the X ring is idle
        // the (kp, kq) partials through the idle X ring as 16-byte vectors,
        // [part - 1][ct][xt][r / 4][lane][r % 4], added in a fixed order
        float* red = reinterpret_cast<float*>(&lds_x[0][0]);
        const int part = kp * 2 + kq;
        auto red_at = [&](int pp, int xt, int a4) { return red + ((((pp * 2 + ct) * 2 + xt) * 4 + a4) * 64 + lane) * 4; };
        if (part != 0) {
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4)
                    *reinterpret_cast<float4*>(red_at(part - 1, xt, a4)) =
                        make_float4(acc[xt][4 * a4], acc[xt][4 * a4 + 1], acc[xt][4 * a4 + 2], acc[xt][4 * a4 + 3]);
        }
        __syncthreads();
        if (part == 0) {
            // bf16 results staged row-major in the ring past the partials
            // ([64 rows][64 columns], this wave's 32 columns only, read back by
            // this wave), then stored 8 columns (16 bytes) per lane
            uint16_t* tile = reinterpret_cast<uint16_t*>(&lds_x[0][0] + 3 * 2 * 2 * 16 * 64 * 4);
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    float4 v = make_float4(acc[xt][4 * a4], acc[xt][4 * a4 + 1], acc[xt][4 * a4 + 2],
                                           acc[xt][4 * a4 + 3]);
#pragma unroll
                    for (int pp = 0; pp < 3; ++pp) {
                        const float4 o = *reinterpret_cast<const float4*>(red_at(pp, xt, a4));
                        v.x += o.x;
                        v.y += o.y;
                        v.z += o.z;
                        v.w += o.w;
                    }
                    const int row = 32 * xt + 8 * a4 + 4 * kh;
                    const int cl = 32 * ct + m;
                    tile[(row + 0) * 64 + cl] = bf16_rne(v.x);
                    tile[(row + 1) * 64 + cl] = bf16_rne(v.y);
                    tile[(row + 2) * 64 + cl] = bf16_rne(v.z);
                    tile[(row + 3) * 64 + cl] = bf16_rne(v.w);
                }
            // lane L: rows L / 4 + 16 i, columns 32 ct + 8 (L % 4) .. + 8
            const int c8 = 32 * ct + 8 * (lane & 3);
            const int64_t gc = n0 + c8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = (lane >> 2) + 16 * i;
                if (row >= M || gc >= N)
                    continue;
                const uint16_t* src = tile + row * 64 + c8;
                if (gc + 8 <= N && (N & 7) == 0) {
                    *reinterpret_cast<u32x4*>(y + row * N + gc) = *reinterpret_cast<const u32x4*>(src);
                } else {
                    for (int e = 0; e < 8 && gc + e < N; ++e)
                        y[row * N + gc + e] = src[e];
                }
            }
        }
    } else {
        stream_operand<WDX>(xq, M, 0, K, nch, (uint32_t)(uintptr_t)&lds_x[0][0], lane);
    }
}

}  // namespace w4

// ---------------------------------------------------------- launchers

void launch_mxfp4_quant(const void* w, int64_t N, int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t st)
{
    const int64_t nthreads = N * (K / 8);
    const unsigned grid = (unsigned)((nthreads + 255) / 256);
    w4::quant_mxfp4_kernel<<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(w), nthreads, codes, scales);
}

int64_t gemm_w4_max_k() { return w4::kMaxK; }

void launch_gemm_fwd_w4(const uint8_t* xq, const float* sx, const uint8_t* w4c, const uint8_t* s4, int64_t M,
                        int64_t N, int64_t K, void* y, hipStream_t st)
{
    uint16_t* out = static_cast<uint16_t*>(y);
    if (M <= 64 && K % (dec::CH * kGroup) == 0) {
        const unsigned grid = (unsigned)((N + 63) / 64);
        if (K == 4096)
            w4::gemm_w4_decode_kernel<16><<<grid, 576, 0, st>>>(xq, sx, w4c, s4, M, N, K, out);
        else
            w4::gemm_w4_decode_kernel<0><<<grid, 576, 0, st>>>(xq, sx, w4c, s4, M, N, K, out);
        return;
    }
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    w4::gemm_w4_kernel<<<grid, 256, 0, st>>>(xq, sx, w4c, s4, M, N, K, out);
}

}  // namespace fp8lin
