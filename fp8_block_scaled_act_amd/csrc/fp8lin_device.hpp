// fp8lin_device.hpp -- device helpers shared by the gfx950 kernels of libfp8lin.
//
// Numeric contract (Jet-RL technical summary, "Quantization scheme": FP8 with
// 1x128 activation groups and 128x128 weight blocks; the format is fixed here
// as OCP E4M3FN): scale = fp32(amax / 448), code = E4M3(fp32(x / scale)) with
// round-to-nearest-even, saturation at +-448 and the sign of x kept; an
// all-zero group has scale 0 and signed-zero codes.
//
// The whole library is compiled with -ffp-contract=off: every fused
// multiply-add below is written out as fmaf on purpose.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

constexpr int kGroup = 128;

// -------------------------------------------------------- streaming loads

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (streamed once, not worth keeping in L2).
__device__ __forceinline__ uint4 load_nt(const void* p)
{
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest |value| of the 8 bf16 in a 16-byte chunk, as fp32 bits.  For finite
// non-negative floats the integer order of the bit patterns is the numeric
// order, so the maximum is taken on the 15-bit magnitudes with packed u16 max.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t absmax_bits_8xbf16(uint4 v)
{
    u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
    u16x2 b = __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu);
    u16x2 c = __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu);
    u16x2 d = __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu);
    u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                        __builtin_elementwise_max(c, d));
    uint32_t lo = m.x, hi = m.y;
    return (lo > hi ? lo : hi) << 16;
}

// ------------------------------------------------------- lane reductions

// DPP control codes (GCN/CDNA data-parallel primitives).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Maximum over each aligned group of 4 / 8 / 16 lanes; every lane of the
// group receives it.  All 64 lanes must be active.
__device__ __forceinline__ uint32_t max_over_4_lanes(uint32_t v)
{
    v = umax(v, dpp<kDppQuadXor1>(v));
    v = umax(v, dpp<kDppQuadXor2>(v));
    return v;
}
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t v)
{
    v = max_over_4_lanes(v);
    return umax(v, dpp<kDppRowHalfMirror>(v));
}
__device__ __forceinline__ uint32_t max_over_16_lanes(uint32_t v)
{
    v = max_over_8_lanes(v);
    return umax(v, dpp<kDppRowMirror>(v));
}
__device__ __forceinline__ uint32_t max_over_64_lanes(uint32_t v)
{
    v = max_over_16_lanes(v);
    uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return umax(umax(a, b), umax(c, d));
}

// --------------------------------------------------------- group scaling

// Per-group quantities.  s = fp32(amax / 448) and r = fp32(1 / s), both
// correctly rounded (the quotients IEEE division gives).  `fast` selects the
// quotient route below.
struct GroupScale {
    float s;
    float r;
    bool fast;
};

// Scales at or above 2^-92 keep the correction residual of the fast quotient
// exact whenever |x / s| >= 2^-11; below that magnitude every route yields a
// signed-zero code.  Smaller scales (amax < ~2^-83) take IEEE division.
constexpr float kFastScaleMin = 0x1p-92f;

// fp32(a / 448) without a division, for a in [2^-100, 2^128): 448 = 7 * 2^6,
// so a / 448 = fp32(a / 7) * 2^-6 exactly while that product is normal (it
// is at least 2^-109 here), and fp32(a / 7) is q = fp32(a * fp32(1/7))
// corrected once, fp32(q + (a - 7 q) * fp32(1/7)) with both steps fused (the
// residual is exact).  Checked against IEEE division on every such a.
__device__ __forceinline__ float div448_rn(float a)
{
    constexpr float c = 1.0f / 7.0f;
    const float q = a * c;
    return __builtin_amdgcn_ldexpf(fmaf(fmaf(-q, 7.0f, a), c, q), -6);
}

// fp32(1 / s) without a division, for s in [2^-92, 2^120): one Newton step
// y + y (1 - s y) on v_rcp_f32's estimate, both steps fused.  Checked against
// IEEE division on every such s.
__device__ __forceinline__ float rcp_rn(float s)
{
    const float y = __builtin_amdgcn_rcpf(s);
    return fmaf(fmaf(-s, y, 1.0f), y, y);
}

__device__ __forceinline__ GroupScale group_scale(uint32_t amax_bits)
{
    GroupScale g;
    const float a = __uint_as_float(amax_bits);
    const bool tiny = !(a >= 0x1p-100f);
    g.s = div448_rn(a);
    if (__builtin_amdgcn_ballot_w64(tiny) != 0)   // rare: the IEEE division only where needed
        if (tiny)
            g.s = a / 448.0f;
    g.fast = g.s >= kFastScaleMin;
    // r is read only by the fast quotient (s >= 2^-92; s < 2^120 for any finite amax)
    g.r = rcp_rn(g.s);
    if (amax_bits == 0) {                  // all-zero group: scale 0, codes = signs
        g.s = 0.0f;
        g.r = 0.0f;
        g.fast = true;
    }
    return g;
}

// fp32(x / s), correctly rounded, from the per-group reciprocal r = RN(1/s):
// q0 = RN(x r) is within one ulp of x/s, the residual x - q0 s is exact (FMA),
// and RN(q0 + residual * r) is the correctly rounded quotient (Markstein's
// theorem for division by FMA with a correctly rounded reciprocal).  The sign
// of x is re-applied so that zero quotients keep it, as IEEE division does.
// With r = 0 (all-zero group) the result is a signed zero.
__device__ __forceinline__ float quotient_fast(float x, float s, float r)
{
    float q0 = x * r;
    float res = fmaf(-q0, s, x);
    float q1 = fmaf(res, r, q0);
    return __builtin_copysignf(q1, x);
}

// IEEE division, then clamp to [-448, 448]: saturation is only reachable
// through tiny scales, and a value clamped to 448 encodes to 448 as any
// value above 448 does under round-then-saturate.
__device__ __forceinline__ float quotient_slow(float x, float s)
{
    float t = x / s;
    return __builtin_amdgcn_fmed3f(t, -448.0f, 448.0f);
}

// --------------------------------------------------------------- encode

// fp32 -> OCP E4M3FN, round-to-nearest-even, saturating, sign kept.
// Integer construction: below 2^-6 the code is RNE(|t| * 2^9) (subnormals,
// reaching 0x08 = 2^-6 exactly at the seam); otherwise the fp32 bits are
// rounded to 3 mantissa bits (ties to even) and re-biased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_encode(float t)
{
    uint32_t u = __float_as_uint(t);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    uint32_t nrm = (r >> 20) - (120u << 3);
    nrm = nrm < 0x7Eu ? nrm : 0x7Eu;
    uint32_t code = a < 0x3C800000u ? sub : nrm;
    return code | sign;
}

// Four codes packed little-endian into one dword.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d)
{
    return e4m3_encode(a) | (e4m3_encode(b) << 8) | (e4m3_encode(c) << 16) | (e4m3_encode(d) << 24);
}

// Hardware conversion: v_cvt_pk_fp8_f32 (two fp32 -> two FP8 codes per
// instruction, rounding per the MODE register, round-to-nearest-even by
// default).  Its FP8 flavour, tie handling, subnormals and out-of-range
// behaviour are checked against the definition on every fp32 input through
// the encoder diagnostic before any kernel relies on it.
__device__ __forceinline__ uint32_t e4m3_encode4_hw(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// ---------------------------------------------------------------- decode

// E4M3FN code -> fp32 (exact).  Finite codes only (0x7F/0xFF never occur in
// quantizer output).
__device__ __forceinline__ float e4m3_decode(uint32_t c)
{
    uint32_t e = (c >> 3) & 0xFu;
    uint32_t f = c & 7u;
    // normal: (8+f) * 2^(e-10) = bits with exponent e+120, mantissa f<<20
    float nrm = __uint_as_float(((e + 120u) << 23) | (f << 20));
    float sub = (float)f * 0x1p-9f;
    float v = e ? nrm : sub;
    return (c & 0x80u) ? -v : v;
}

// Hardware decode of four codes (v_cvt_pk_f32_fp8 on each 16-bit half).
__device__ __forceinline__ void e4m3_decode4_hw(uint32_t w, float* v)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    v[0] = lo.x;
    v[1] = lo.y;
    v[2] = hi.x;
    v[3] = hi.y;
}

// ------------------------------------------------------------ quantize 8

// Quantize the 8 bf16 values of a 16-byte chunk with a group's scale;
// returns 8 codes in a uint2.
__device__ __forceinline__ uint2 quantize8_bf16(uint4 v, const GroupScale& g)
{
    float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float t[8];
    if (g.fast) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            t[i] = quotient_fast(x[i], g.s, g.r);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            t[i] = quotient_slow(x[i], g.s);
    }
    return make_uint2(e4m3_encode4(t[0], t[1], t[2], t[3]), e4m3_encode4(t[4], t[5], t[6], t[7]));
}

// 4x4 byte transpose: rows r0..r3 (4 bytes each) -> columns c0..c3.
__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                             uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3)
{
    const uint32_t lo01 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
    const uint32_t lo23 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
    c0 = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    c1 = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    c2 = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    c3 = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// ---------------------------------------------- quantize with the hardware

// Encoder / decoder used by the kernels: the gfx950 conversion instructions.
// Checked on every fp32 input against the definition: v_cvt_pk_fp8_f32
// rounds to nearest even into OCP E4M3FN (subnormals and ties included) for
// |v| <= 464 and returns NaN above, so its inputs must stay within +-464; the
// fast quotient never exceeds 448 (1 + 2^-23) and the slow one is clamped to
// +-448.  v_cvt_pk_f32_fp8 decodes all 254 finite codes exactly.
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d)
{
    return e4m3_encode4_hw(a, b, c, d);
}

__device__ __forceinline__ void decode4(uint32_t w, float* v) { e4m3_decode4_hw(w, v); }

// Quotients of n values with one group's scale, encoded 4 at a time.
template <int N>
__device__ __forceinline__ void quantize_n(const float* x, const GroupScale& g, uint32_t* out)
{
    float t[N];
    if (g.fast) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            t[i] = quotient_fast(x[i], g.s, g.r);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            t[i] = quotient_slow(x[i], g.s);
    }
#pragma unroll
    for (int i = 0; i < N / 4; ++i)
        out[i] = encode4(t[4 * i], t[4 * i + 1], t[4 * i + 2], t[4 * i + 3]);
}

__device__ __forceinline__ uint2 quantize8(uint4 v, const GroupScale& g)
{
    float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    uint32_t c[2];
    quantize_n<8>(x, g, c);
    return make_uint2(c[0], c[1]);
}

}  // namespace fp8lin
