// quant_tile.hpp -- the column phase of the transposing 1x128 quantizer,
// shared by the kernels that quantize a 128x128 BF16 tile 128-along-tokens
// (transposed output: each source column becomes an output row of codes).
#pragma once

#include "fp8lin_device.hpp"

namespace fp8lin {

// Transposed code tile in LDS: 128 output rows (columns of the source) x
// 128 tokens, 16-byte token chunks XOR-swizzled so both the quantizing
// waves' writes and the row-wise reads spread over the banks.
__device__ __forceinline__ int ct_off(int r, int tchunk) { return r * 128 + ((tchunk ^ ((r >> 2) & 7)) << 4); }

// Stores the 128x128 code tile to qT rows c0 + r (r < nrows), eight lanes per
// 128-byte row: every store instruction writes 8 full rows.
__device__ __forceinline__ void store_code_tile(const uint8_t* ctile, uint8_t* __restrict__ qT, int64_t c0,
                                                int64_t t0, int64_t T, int64_t nrows)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = (int)threadIdx.x + 256 * i;
        const int r = idx >> 3, pc = idx & 7;
        if (r < nrows)
            *reinterpret_cast<uint4*>(qT + (c0 + r) * T + t0 + 16 * pc) =
                *reinterpret_cast<const uint4*>(ctile + ct_off(r, pc));
    }
}

// Column phase for a 128 (tokens t0..) x 128 (columns c0..) BF16 tile parked
// in LDS as tile[row][16 chunks of 8 bf16]: per column, the amax over the
// tile's 128 tokens (each wave 32 tokens, each lane a pair of adjacent
// columns: a tile row is 64 consecutive dwords; the four waves combine
// through `red`), the scale, and 128 codes parked in the LDS code tile, then
// written out eight lanes per 128-byte output row of qT [C][T]; scales to
// sT [C][T/128].  RAGGED: columns at or past C are neither scaled nor
// written.  All 256 threads; two barriers.
template <bool RAGGED>
__device__ __forceinline__ void transpose_quant_tile(const uint4* tile, uint32_t* red, uint8_t* ctile,
                                                     uint8_t* __restrict__ qT, float* __restrict__ sT,
                                                     int64_t c0, int64_t t0, int64_t T, int64_t C)
{
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int cp = tid & 63;                  // columns 2cp, 2cp+1 of the tile
    const uint32_t* tile32 = reinterpret_cast<const uint32_t*>(tile);
    uint32_t d[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
        d[i] = tile32[(wave * 32 + i) * 64 + cp];
    u16x2 m = {0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[i] & 0x7FFF7FFFu));
    red[wave * 64 + cp] = __builtin_bit_cast(uint32_t, m);
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; ++w)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, red[w * 64 + cp]));
    const GroupScale g0 = group_scale((uint32_t)m.x << 16);
    const GroupScale g1 = group_scale((uint32_t)m.y << 16);

    const int64_t ca = c0 + 2 * cp;
    const int64_t GT = T / kGroup;
    float xv[32];
    uint32_t codes[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int64_t c = ca + half;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            xv[i] = half ? bf16_hi(d[i]) : bf16_lo(d[i]);
        quantize_n<32>(xv, half ? g1 : g0, codes);
        const int r = 2 * cp + half;
        *reinterpret_cast<uint4*>(&ctile[ct_off(r, 2 * wave)]) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
        *reinterpret_cast<uint4*>(&ctile[ct_off(r, 2 * wave + 1)]) = make_uint4(codes[4], codes[5], codes[6], codes[7]);
        if (wave == 0 && (!RAGGED || c < C))
            sT[c * GT + (t0 / kGroup)] = half ? g1.s : g0.s;
    }
    __syncthreads();
    store_code_tile(ctile, qT, c0, t0, T, RAGGED ? (C - c0 < 128 ? C - c0 : 128) : 128);
}

}  // namespace fp8lin
