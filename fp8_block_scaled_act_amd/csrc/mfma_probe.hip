// mfma_probe.hip -- diagnostic: the block-scaled forward product on each of
// gfx950's FP8 matrix-core instructions, and on the fp16 one as a control.
//
// Jet-RL technical summary (gist.science 2601.14243), "Quantization scheme":
// the FP8 GEMMs of the layer multiply FP8 codes with one scale per 128-wide
// contraction group.  The library's GEMMs convert the codes exactly to fp16
// and use the fp16 matrix core, because the FP8 instructions do not sum their
// products exactly.  This file keeps that evidence reproducible: one plain
// kernel computes
//     Y[m][n] = sum_g sx[m][g] * sw[n/128][g] * P_g[m][n],
//     P_g[m][n] = sum_{k in g} dec(xq[m][k]) * dec(wq[n][k])
// with P_g from a chain of MFMA instructions of the chosen form (fp32 C
// operand, starting from zero at every group) and one fp32 FMA per group for
// the scale, writing the fp32 sums.  Only the instruction differs between the
// forms, so a difference in accuracy is the instruction's.
//
// Forms (lane l supplies row l % T of its operand and the T x T output tile
// of one wave is computed from both operands' k slices in the same lane
// order, so any k permutation the hardware applies cancels):
//   0  v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 both sides, unit E8M0
//      scales): one instruction per group, 32 codes per lane;
//   1  v_mfma_scale_f32_32x32x64_f8f6f4: two per group, 32 codes per lane;
//   2  v_mfma_f32_16x16x32_fp8_fp8: four per group, 8 codes per lane;
//   3  v_mfma_f32_32x32x16_fp8_fp8: eight per group, 8 codes per lane;
//   4  v_mfma_f32_32x32x16_f16 on the codes converted exactly to fp16 (the
//      instruction the library's GEMMs use): eight per group.
// Output layouts: 16 x 16 tiles, lane l register v holds row 4 (l / 16) + v,
// column l % 16; 32 x 32 tiles, row 8 (v / 4) + 4 (l / 32) + v % 4, column
// l % 32.  One wave per workgroup, no LDS: this kernel is for accuracy, not
// speed.
#include "decode_stream.hpp"
#include "fp8lin_device.hpp"
#include "fp8lin_launch.hpp"

namespace fp8lin {

namespace {

typedef float p4f __attribute__((ext_vector_type(4)));
typedef float p16f __attribute__((ext_vector_type(16)));
typedef int p8i __attribute__((ext_vector_type(8)));

constexpr int kUnitE8M0 = 127;                     // E8M0 code of 2^0

template <int FORM>
struct Form {
    static constexpr int T = (FORM == 0 || FORM == 2) ? 16 : 32;   // output tile edge
    static constexpr int NREG = T == 16 ? 4 : 16;                  // output registers per lane
};

// Row of the tile held by output register v of lane l.
template <int T>
__device__ __forceinline__ int out_row(int l, int v)
{
    return T == 16 ? 4 * (l >> 4) + v : 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
}

template <int FORM>
__device__ __forceinline__ void group_product(const uint8_t* a, const uint8_t* b, int lane,
                                              float (&out)[Form<FORM>::NREG])
{
    // a, b: the group's first code of the lane's operand row
    if constexpr (FORM == 0) {
        const int kg = lane >> 4;                  // 4 lane groups of 32 codes
        const p8i av = *reinterpret_cast<const p8i*>(a + 32 * kg);
        const p8i bv = *reinterpret_cast<const p8i*>(b + 32 * kg);
        p4f c = {0.f, 0.f, 0.f, 0.f};
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, kUnitE8M0, 0, kUnitE8M0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            out[v] = c[v];
    } else if constexpr (FORM == 1) {
        const int kg = lane >> 5;                  // 2 lane groups of 32 codes per step
        p16f c = {};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const p8i av = *reinterpret_cast<const p8i*>(a + 64 * s + 32 * kg);
            const p8i bv = *reinterpret_cast<const p8i*>(b + 64 * s + 32 * kg);
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, kUnitE8M0, 0, kUnitE8M0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v)
            out[v] = c[v];
    } else if constexpr (FORM == 2) {
        const int kg = lane >> 4;                  // 4 lane groups of 8 codes per step
        p4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const long av = *reinterpret_cast<const long*>(a + 32 * s + 8 * kg);
            const long bv = *reinterpret_cast<const long*>(b + 32 * s + 8 * kg);
            c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av, bv, c, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
            out[v] = c[v];
    } else {
        const int kg = lane >> 5;                  // 2 lane groups of 8 codes per step
        p16f c = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint2 av = *reinterpret_cast<const uint2*>(a + 16 * s + 8 * kg);
            const uint2 bv = *reinterpret_cast<const uint2*>(b + 16 * s + 8 * kg);
            if constexpr (FORM == 3)
                c = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(
                    (long)(((unsigned long)av.y << 32) | av.x), (long)(((unsigned long)bv.y << 32) | bv.x), c, 0,
                    0, 0);
            else
                c = __builtin_amdgcn_mfma_f32_32x32x16_f16(dec::cvt8(av.x, av.y), dec::cvt8(bv.x, bv.y), c, 0, 0,
                                                               0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v)
            out[v] = c[v];
    }
}

// grid: (N / T, ceil(M / T)), one wave.  Rows past M read row M - 1 and are
// not stored.  N % 128 == 0, so a tile's columns share one weight block.
template <int FORM>
__global__ __launch_bounds__(64) void gemm_fwd_mfma_probe_kernel(const uint8_t* __restrict__ xq,
                                                                 const float* __restrict__ sx,
                                                                 const uint8_t* __restrict__ wq,
                                                                 const float* __restrict__ sw, int64_t M,
                                                                 int64_t K, int64_t N, float* __restrict__ y)
{
    constexpr int T = Form<FORM>::T, NR = Form<FORM>::NREG;
    const int lane = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * T, m0 = (int64_t)blockIdx.y * T;
    const int64_t G = K / kGroup;
    const int64_t arow = m0 + (lane % T) < M ? m0 + (lane % T) : M - 1;
    const int64_t brow = n0 + (lane % T);
    float acc[NR];
#pragma unroll
    for (int v = 0; v < NR; ++v)
        acc[v] = 0.f;
    for (int64_t g = 0; g < G; ++g) {
        float p[NR];
        // MFMA side A = X rows (tile rows), side B = W rows (tile columns)
        group_product<FORM>(xq + arow * K + g * kGroup, wq + brow * K + g * kGroup, lane, p);
        const float s_w = sw[(n0 / kGroup) * G + g];
#pragma unroll
        for (int v = 0; v < NR; ++v) {
            int64_t r = m0 + out_row<T>(lane, v);
            r = r < M ? r : M - 1;
            acc[v] = fmaf(p[v], sx[r * G + g] * s_w, acc[v]);
        }
    }
#pragma unroll
    for (int v = 0; v < NR; ++v) {
        const int64_t r = m0 + out_row<T>(lane, v);
        if (r < M)
            y[r * N + n0 + (lane % T)] = acc[v];
    }
}

template <int FORM>
void launch_form(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M, int64_t N,
                 int64_t K, float* y, hipStream_t st)
{
    constexpr int T = Form<FORM>::T;
    const dim3 grid((unsigned)(N / T), (unsigned)((M + T - 1) / T));
    gemm_fwd_mfma_probe_kernel<FORM><<<grid, 64, 0, st>>>(xq, sx, wq, sw, M, K, N, y);
}

}  // namespace

int mfma_probe_tile(int form) { return (form == 0 || form == 2) ? 16 : 32; }

void launch_gemm_fwd_mfma_probe(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, float* y, int form, hipStream_t st)
{
    switch (form) {
    case 0: launch_form<0>(xq, sx, wq, sw, M, N, K, y, st); break;
    case 1: launch_form<1>(xq, sx, wq, sw, M, N, K, y, st); break;
    case 2: launch_form<2>(xq, sx, wq, sw, M, N, K, y, st); break;
    case 3: launch_form<3>(xq, sx, wq, sw, M, N, K, y, st); break;
    default: launch_form<4>(xq, sx, wq, sw, M, N, K, y, st); break;
    }
}

}  // namespace fp8lin
