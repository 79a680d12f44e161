// quant_kernels.hip -- FP8 E4M3 quantization kernels for gfx950.
//
// Jet-RL technical summary (gist.science 2601.14243), "Quantization scheme":
// activations in 1x128 groups, weights in 128x128 blocks, and the WGrad
// operands grouped 128-along-tokens (the "1x128 and 128x1" kernels), produced
// here by a transposing quantizer ("Implementation": dedicated quantization
// and transposition kernels).  All of these are HBM-streaming codecs: every
// kernel reads its input once and writes codes and scales once.
#include "fp8lin_device.hpp"
#include "fp8lin_launch.hpp"
#include "quant_tile.hpp"

namespace fp8lin {

// ============================================================ 1x128 groups
//
// A [M,K] tensor with K % 128 == 0 is a flat sequence of 128-element groups
// (group g covers elements [128g, 128g+128) and owns scale g), so the kernel
// is one-dimensional.  16 lanes hold one group (16 bytes of bf16 each), a
// wave holds 4 groups per step, and each wave keeps UNROLL steps of loads in
// flight before reducing.  The group amax is a 16-lane DPP reduction.
template <int UNROLL>
__global__ __launch_bounds__(256) void quant_rowgroup_kernel(const uint4* __restrict__ x,
                                                             uint2* __restrict__ q,
                                                             float* __restrict__ s,
                                                             int64_t ngroups)
{
    const int lane = threadIdx.x & 63;
    const int sub = lane & 15;
    const int slot = lane >> 4;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t base = wave * (4 * UNROLL); base < ngroups; base += nwaves * (4 * UNROLL)) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t g = base + u * 4 + slot;
            v[u] = g < ngroups ? load_nt(x + g * 16 + sub) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t g = base + u * 4 + slot;
            const uint32_t am = max_over_16_lanes(absmax_bits_8xbf16(v[u]));
            const GroupScale gs = group_scale(am);
            const uint2 c = quantize8(v[u], gs);
            if (g < ngroups) {
                q[g * 16 + sub] = c;
                if (sub == 0)
                    s[g] = gs.s;
            }
        }
    }
}

// ========================================================== 128x128 blocks
//
// One workgroup per block: 256 threads, 16 lanes per 256-byte row segment,
// 8 rows per thread held in registers, block amax by DPP + LDS, then the
// block is encoded from registers (one HBM read, one write).
__global__ __launch_bounds__(256) void quant_block_kernel(const uint16_t* __restrict__ w, int64_t K,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ s)
{
    __shared__ uint32_t red[4];
    const int tid = threadIdx.x;
    const int sub = tid & 15;
    const int r0 = tid >> 4;
    const int64_t row0 = (int64_t)blockIdx.y * kGroup;
    const int64_t col0 = (int64_t)blockIdx.x * kGroup;
    uint4 v[8];
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4* p = reinterpret_cast<const uint4*>(w + (row0 + r0 + 16 * i) * K + col0) + sub;
        v[i] = load_nt(p);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        am = umax(am, absmax_bits_8xbf16(v[i]));
    am = max_over_64_lanes(am);
    if ((tid & 63) == 0)
        red[tid >> 6] = am;
    __syncthreads();
    am = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    const GroupScale gs = group_scale(am);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint2* p = reinterpret_cast<uint2*>(q + (row0 + r0 + 16 * i) * K + col0) + sub;
        *p = quantize8(v[i], gs);
    }
    if (tid == 0)
        s[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = gs.s;
}

// ========================================================= weight transpose
//
// FP8 codes [R][C] -> [C][R] and 128x128 block scales [R/128][C/128] ->
// [C/128][R/128], bit for bit (a 128x128 block is the same block either way).
// One workgroup per 128x128 tile: rows are read 16 bytes per lane into an
// LDS tile; each thread then gathers a 16-row x 4-column block as 4x4 byte
// transposes and writes 4 output rows x 16 bytes (eight lanes cover one
// 128-byte output row).
__global__ __launch_bounds__(256) void transpose_codes_kernel(const uint8_t* __restrict__ src,
                                                              const float* __restrict__ s, int64_t R,
                                                              int64_t C, uint8_t* __restrict__ dst,
                                                              float* __restrict__ sT)
{
    constexpr int kPitch = 33;                // dwords per LDS row (32 + 1 pad)
    __shared__ uint32_t tile[128 * kPitch];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * kGroup;
    const int64_t c0 = (int64_t)blockIdx.x * kGroup;
    {
        const int sub = tid & 7, row = tid >> 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = load_nt(src + (r0 + row + 32 * i) * C + c0 + sub * 16);
            uint32_t* d = tile + (row + 32 * i) * kPitch + sub * 4;
            d[0] = v.x;
            d[1] = v.y;
            d[2] = v.z;
            d[3] = v.w;
        }
    }
    if (tid == 0)
        sT[(int64_t)blockIdx.x * gridDim.y + blockIdx.y] = s[(int64_t)blockIdx.y * gridDim.x + blockIdx.x];
    __syncthreads();
    const int rg = tid & 7;                   // source rows 16 rg .. 16 rg + 15
    const int cq = tid >> 3;                  // source columns 4 cq .. 4 cq + 3
    uint32_t out[4][4];                       // [column j][4-row block b]
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t* t = tile + (16 * rg + 4 * b) * kPitch + cq;
        transpose4x4(t[0], t[kPitch], t[2 * kPitch], t[3 * kPitch], out[0][b], out[1][b], out[2][b], out[3][b]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint4*>(dst + (c0 + 4 * cq + j) * R + r0 + 16 * rg) =
            make_uint4(out[j][0], out[j][1], out[j][2], out[j][3]);
}

// ==================================================== transpose, BF16 source
//
// Tile of 128 tokens (t) x 128 columns (c); one workgroup of 256 threads.
// Phase 1 reads the tile row-wise (16 lanes x 16 B per row, fully coalesced)
// into registers, optionally emits the 1x128 row quantization from there
// (dual output), and parks the bf16 tile in LDS.  Phase 2 gives each wave 32
// tokens and each lane a pair of adjacent columns: reading a tile row is 64
// consecutive dwords (no bank conflicts), the per-column amax over the
// wave's 32 tokens is a packed u16 max, the four waves combine through LDS,
// and each lane parks 32 codes per column in an LDS code tile that is then
// written out eight lanes per 128-byte output row.  RAGGED handles a last column tile with C % 128 != 0 (element-wise
// loads when rows are not 16-byte aligned); out-of-range columns read as 0 and
// are never written.
template <bool DUAL, bool RAGGED>
__global__ __launch_bounds__(256) void quant_transpose_bf16_kernel(const uint16_t* __restrict__ x,
                                                                   int64_t T, int64_t C,
                                                                   uint8_t* __restrict__ qT,
                                                                   float* __restrict__ sT,
                                                                   uint8_t* __restrict__ qrow,
                                                                   float* __restrict__ srow)
{
    __shared__ uint4 tile[128 * 16];          // [row][16 chunks of 8 bf16] = 32 KB
    __shared__ uint32_t red[4 * 64];
    __shared__ __attribute__((aligned(16))) uint8_t ctile[128 * 128];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * kGroup;
    const int64_t c0 = (int64_t)blockIdx.x * kGroup;

    // ---- phase 1: load rows
    {
        const int sub = tid & 15;
        const int r0 = tid >> 4;
        uint4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t row = t0 + r0 + 16 * i;
            const int64_t col = c0 + sub * 8;
            if (!RAGGED) {
                v[i] = load_nt(x + row * C + col);
            } else if ((C & 7) == 0) {
                v[i] = col < C ? *reinterpret_cast<const uint4*>(x + row * C + col) : make_uint4(0, 0, 0, 0);
            } else {
                uint32_t e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    e[j] = (col + j < C) ? x[row * C + col + j] : 0u;
                v[i] = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                  e[6] | (e[7] << 16));
            }
            tile[(r0 + 16 * i) * 16 + sub] = v[i];
        }
        if constexpr (DUAL) {
            const int64_t G = C / kGroup;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t row = t0 + r0 + 16 * i;
                const uint32_t am = max_over_16_lanes(absmax_bits_8xbf16(v[i]));
                const GroupScale gs = group_scale(am);
                *reinterpret_cast<uint2*>(qrow + row * C + c0 + sub * 8) = quantize8(v[i], gs);
                if (sub == 0)
                    srow[row * G + blockIdx.x] = gs.s;
            }
        }
    }
    __syncthreads();

    // ---- phase 2: columns
    transpose_quant_tile<RAGGED>(tile, red, ctile, qT, sT, c0, t0, T, C);
}

// ============================================ transpose, saved FP8 source
//
// Tile of 128 tokens x 128 columns of E4M3 codes with 1x128 row scales (one
// scale per token for the tile, because column tiles are 128-aligned).  The
// values are first dequantized exactly, v = fp32(dec(code) * row scale),
// then quantized 128-along-tokens as above.  Phase 2: wave = 32 tokens,
// lane = (column quad, half of the wave's tokens); quad reads are 32
// consecutive dwords per row.  Codes leave through the same LDS code tile.
__global__ __launch_bounds__(256) void quant_transpose_fp8_kernel(const uint8_t* __restrict__ src,
                                                                  const float* __restrict__ srow,
                                                                  int64_t T, int64_t C,
                                                                  uint8_t* __restrict__ qT,
                                                                  float* __restrict__ sT)
{
    constexpr int kPitch = 33;                // dwords per LDS row (32 + 1 pad)
    __shared__ uint32_t tile[128 * kPitch];
    __shared__ float rs[128];
    __shared__ uint32_t red[8 * 128];
    __shared__ __attribute__((aligned(16))) uint8_t ctile[128 * 128];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * kGroup;
    const int64_t c0 = (int64_t)blockIdx.x * kGroup;
    const int64_t GC = C / kGroup;
    {
        const int sub = tid & 7;
        const int r0 = tid >> 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = r0 + 32 * i;
            const uint4 v = load_nt(src + (t0 + row) * C + c0 + sub * 16);
            uint32_t* dst = tile + row * kPitch + sub * 4;
            dst[0] = v.x;
            dst[1] = v.y;
            dst[2] = v.z;
            dst[3] = v.w;
        }
        if (tid < 128)
            rs[tid] = srow[(t0 + tid) * GC + blockIdx.x];
    }
    __syncthreads();

    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int quad = lane & 31;               // columns 4quad .. 4quad+3
    const int half = lane >> 5;               // tokens wave*32 + half*16 + [0,16)
    const int rbase = wave * 32 + half * 16;
    float v[4][16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float dv[4];
        decode4(tile[(rbase + i) * kPitch + quad], dv);
        const float sc = rs[rbase + i];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j][i] = dv[j] * sc;
    }
    uint32_t am[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t a = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            a = umax(a, __float_as_uint(v[j][i]) & 0x7FFFFFFFu);
        am[j] = a;
        red[(wave * 2 + half) * 128 + quad * 4 + j] = a;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t a = 0;
#pragma unroll
        for (int p = 0; p < 8; ++p)
            a = umax(a, red[p * 128 + quad * 4 + j]);
        am[j] = a;
    }
    const int64_t GT = T / kGroup;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const GroupScale gs = group_scale(am[j]);
        uint32_t codes[4];
        quantize_n<16>(v[j], gs, codes);
        const int64_t c = c0 + quad * 4 + j;
        *reinterpret_cast<uint4*>(&ctile[ct_off(quad * 4 + j, rbase >> 4)]) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
        if (wave == 0 && half == 0)
            sT[c * GT + blockIdx.y] = gs.s;
    }
    __syncthreads();
    store_code_tile(ctile, qT, c0, t0, T, 128);
}

// ============================================================= diagnostics

// method 0: the kernels' encoder over all inputs (clamp to +-448, then the
// hardware conversion: the code any kernel produces for a quotient t);
// 1: hardware conversion on the raw input (out-of-range behaviour visible);
// 2: integer encoder.
__global__ __launch_bounds__(256) void encode_probe_kernel(const float* __restrict__ in, int64_t n,
                                                           uint8_t* __restrict__ out, int method)
{
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n)
        return;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        v[j] = (i + j < n) ? in[i + j] : 0.0f;
    uint32_t w;
    if (method == 1)
        w = e4m3_encode4_hw(v[0], v[1], v[2], v[3]);
    else if (method == 2)
        w = e4m3_encode4(v[0], v[1], v[2], v[3]);
    else
        w = encode4(__builtin_amdgcn_fmed3f(v[0], -448.0f, 448.0f), __builtin_amdgcn_fmed3f(v[1], -448.0f, 448.0f),
                    __builtin_amdgcn_fmed3f(v[2], -448.0f, 448.0f), __builtin_amdgcn_fmed3f(v[3], -448.0f, 448.0f));
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (i + j < n)
            out[i + j] = (uint8_t)(w >> (8 * j));
}

// method 0: the kernels' decoder; 1: hardware conversion; 2: integer decoder.
__global__ __launch_bounds__(256) void decode_probe_kernel(const uint8_t* __restrict__ in, int64_t n,
                                                           float* __restrict__ out, int method)
{
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n)
        return;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (i + j < n)
            w |= (uint32_t)in[i + j] << (8 * j);
    float v[4];
    if (method == 1) {
        e4m3_decode4_hw(w, v);
    } else if (method == 2) {
        for (int j = 0; j < 4; ++j)
            v[j] = e4m3_decode((w >> (8 * j)) & 0xFFu);
    } else {
        decode4(w, v);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (i + j < n)
            out[i + j] = v[j];
}

// ================================================================ launchers

static inline unsigned blocks_for(int64_t work, int64_t per_block, int64_t cap)
{
    int64_t b = (work + per_block - 1) / per_block;
    if (b > cap)
        b = cap;
    return (unsigned)(b < 1 ? 1 : b);
}

void launch_quant_rowgroup(const void* x, int64_t ngroups, uint8_t* q, float* s, hipStream_t st)
{
    // A few rows (decode) are latency-bound: one load per lane and more
    // workgroups; larger inputs keep two loads per lane in flight (measured:
    // 64x4096 2.2 us vs 2.9 us with four; 8192x3584 equal to four).
    const uint4* xv = static_cast<const uint4*>(x);
    uint2* qv = reinterpret_cast<uint2*>(q);
    if (ngroups < 8192)
        quant_rowgroup_kernel<1><<<blocks_for(ngroups, 4 * 4, 16384), 256, 0, st>>>(xv, qv, s, ngroups);
    else
        quant_rowgroup_kernel<2><<<blocks_for(ngroups, 4 * 4 * 2, 16384), 256, 0, st>>>(xv, qv, s, ngroups);
}

void launch_quant_block(const void* w, int64_t N, int64_t K, uint8_t* q, float* s, hipStream_t st)
{
    dim3 grid((unsigned)(K / kGroup), (unsigned)(N / kGroup));
    quant_block_kernel<<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(w), K, q, s);
}

void launch_transpose_codes(const uint8_t* src, const float* s, int64_t R, int64_t C, uint8_t* dst, float* sT,
                            hipStream_t st)
{
    dim3 grid((unsigned)(C / kGroup), (unsigned)(R / kGroup));
    transpose_codes_kernel<<<grid, 256, 0, st>>>(src, s, R, C, dst, sT);
}

void launch_quant_transpose_bf16(const void* x, int64_t T, int64_t C, uint8_t* qT, float* sT,
                                 uint8_t* qrow, float* srow, hipStream_t st)
{
    dim3 grid((unsigned)((C + kGroup - 1) / kGroup), (unsigned)(T / kGroup));
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const bool ragged = (C % kGroup) != 0;
    if (qrow)
        quant_transpose_bf16_kernel<true, false><<<grid, 256, 0, st>>>(xp, T, C, qT, sT, qrow, srow);
    else if (ragged)
        quant_transpose_bf16_kernel<false, true><<<grid, 256, 0, st>>>(xp, T, C, qT, sT, nullptr, nullptr);
    else
        quant_transpose_bf16_kernel<false, false><<<grid, 256, 0, st>>>(xp, T, C, qT, sT, nullptr, nullptr);
}

void launch_quant_transpose_fp8(const uint8_t* src, const float* srow, int64_t T, int64_t C,
                                uint8_t* qT, float* sT, hipStream_t st)
{
    dim3 grid((unsigned)(C / kGroup), (unsigned)(T / kGroup));
    quant_transpose_fp8_kernel<<<grid, 256, 0, st>>>(src, srow, T, C, qT, sT);
}

void launch_encode_probe(const float* in, int64_t n, uint8_t* out, int method, hipStream_t st)
{
    const unsigned grid = (unsigned)((n + 1023) / 1024);
    encode_probe_kernel<<<grid, 256, 0, st>>>(in, n, out, method);
}

void launch_decode_probe(const uint8_t* in, int64_t n, float* out, int method, hipStream_t st)
{
    const unsigned grid = (unsigned)((n + 1023) / 1024);
    decode_probe_kernel<<<grid, 256, 0, st>>>(in, n, out, method);
}

}  // namespace fp8lin
