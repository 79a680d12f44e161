// decode_stream.hpp -- the X (or W) stream of the decode GEMMs: one loader
// wave moves 64 rows of an FP8 operand, two 128-groups (256 bytes of a row) at
// a time, from global memory into a D-deep LDS ring with
// global_load_lds_dwordx4, publishing each chunk at a workgroup barrier.
//
// LDS layout of a chunk (16-byte pieces; the rows of a 16-row stripe hit
// distinct banks): rows in 1 KB blocks of four, piece q of row r at
// (r / 4) * 1024 + 16 * (16 (r % 4) + (q ^ (r % 16))).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8lin_device.hpp"

namespace fp8lin {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

namespace dec {
constexpr int CH = 2;                              // groups per chunk
constexpr int WCH = 64 * CH * kGroup;              // bytes per chunk of one operand

__device__ __forceinline__ void dma16(uint32_t lds, const void* g)
{
    // the LDS address is wave-uniform; readfirstlane keeps it in an SGPR for M0
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(
                     __builtin_amdgcn_readfirstlane(lds)),
                 "v"(g)
                 : "memory");
}
// The 4-byte form: lane l's word lands at M0 + 4 * l.
__device__ __forceinline__ void dma4(uint32_t lds, const void* g)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(
                     __builtin_amdgcn_readfirstlane(lds)),
                 "v"(g)
                 : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ int w_off(int r, int q) { return (r >> 2) * 1024 + ((((r & 3) << 4) | (q ^ (r & 15))) << 4); }

// 8 codes (two words) -> 8 fp16, exact (scale 1.0)
__device__ __forceinline__ v8h cvt8(uint32_t a, uint32_t b)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)a, 1.0f, false);
    const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)a, 1.0f, true);
    const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b, 1.0f, false);
    const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b, 1.0f, true);
    return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// One loader wave: streams the 64 rows [row0, row0 + 64) of a [rows][K]
// FP8 operand (rows past `rows` read row rows - 1) chunk by chunk into a
// D-deep LDS ring at `base`, publishing chunk c + 1 at the barrier that
// ends chunk c.  Passes 3 + nch barriers, like the MMA waves.
template <int D>
__device__ __forceinline__ void stream_operand(const uint8_t* src, int64_t rows, int64_t row0, int64_t Kc,
                                               int64_t nch, uint32_t base, int lane)
{
    const int lr4 = lane >> 4, x = lane & 15;
    const uint8_t* rp[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t r = row0 + 4 * i + lr4;
        rp[i] = src + (r < rows ? r : rows - 1) * Kc + 16 * (x ^ ((4 * i + lr4) & 15));
    }
    auto chunk = [&](int64_t c, int slot) {
        const uint32_t dst = base + (uint32_t)(slot * WCH);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            dma16(dst + i * 1024, rp[i] + c * (CH * kGroup));
    };
    // waits until chunk c has landed when the chunks after it up to c + D - 2
    // (those that exist) were issued after it (vmcnt retires in order)
    auto wait_chunk = [&](int64_t c) {
        const int64_t after = nch - 1 - c < D - 2 ? nch - 1 - c : D - 2;
        if (after >= 2)
            wait_vm<32>();
        else if (after == 1)
            wait_vm<16>();
        else
            wait_vm<0>();
    };
    static_assert(D - 2 <= 2, "wait_chunk covers up to two chunks in flight behind the awaited one");
#pragma unroll
    for (int c = 0; c < D - 1; ++c)
        if (c < nch)
            chunk(c, c);
    wait_chunk(0);                                 // chunk 0 landed
    __syncthreads();
    for (int64_t c = 0; c < nch; ++c) {
        if (c + D - 1 < nch)
            chunk(c + D - 1, (int)((c + D - 1) % D));  // into the slot drained before the last barrier
        if (c + 1 < nch)
            wait_chunk(c + 1);                     // chunk c + 1 landed
        __syncthreads();
    }
    wait_vm<0>();                                  // nothing is in flight any more
    __syncthreads();
    __syncthreads();
}
}  // namespace dec

}  // namespace fp8lin
