// gemm_kernels.hip -- block-scaled FP8 GEMMs for gfx950.
//
// Jet-RL technical summary (gist.science 2601.14243), "Quantization scheme":
// the forward GEMM, the DGrad GEMM and the WGrad GEMM all run on FP8 codes,
// 1x128-grouped activations/gradients and 128x128-blocked weights (WGrad on
// operands grouped 128-along-tokens).  Every 128-wide contraction group g has
// one scale per row of the left operand and one per column (or per 128-column
// block) of the right operand:
//     C[m,n] = sum_g sa[m,g] * sb[n,g] * P_g[m,n],
//     P_g[m,n] = sum_{k in g} dec(A[m,k]) * dec(B[n,k]),
// with P_g promoted into fp32 accumulators once per group.
//
// Matrix-core choice.  gfx950's FP8 MFMA sums its products in a fixed-point
// window: products are aligned to the largest one of a chunk and truncated
// toward zero 13 bits below it (measured: 448 + 0.0586 in adjacent slots gives
// 448.03125; errors reach 2^-11.6 of the largest product on random codes).
// With the outlier channels of real activations that error exceeds the
// layer's accuracy bound.  Every E4M3 value is exactly an fp16 value, so the
// codes are converted exactly to fp16 (v_cvt_scalef32_pk_f16_fp8, scale 1)
// and multiplied on the fp16 matrix core (measured error <= 2^-20 of the
// largest product).  HBM traffic stays one byte per operand element.
//
// Kernels in this file:
//   gemm_kernel            generic tile; DGrad on the untransposed weight and
//                          a few small shapes (described below);
//   gemm_fwd_skinny_kernel forward for <= 64 rows and very long K;
//   gemm_fwd_decode_kernel forward for <= 64 rows: W streamed by LDS DMA;
//   gemm_nt_kernel         forward, WGrad and DGrad on the transposed
//                          weight: 128x128 tiles fed by LDS DMA.
//
// gemm_kernel: one workgroup of WM x WN waves, tile BM x BN of C, contraction
// stepped one group (128) at a time:
//   - FP8 operand tiles are read from global (16-byte loads), converted and
//     written to LDS as fp16, double-buffered: group g+1 is in flight while
//     group g is multiplied;
//   - an LDS row is one group of one row (column) of an operand: 16 chunks of
//     8 fp16.  Chunk p holds k in [16 (p mod 8) + 8 (p div 8), +8): a fixed
//     permutation of the group applied to both operands, which leaves the
//     contraction unchanged and lets 8 threads write a row without bank
//     conflicts.  Chunks are XOR-swizzled with swz(row) so fragment reads of 16
//     rows and staging writes hit distinct banks;
//   - one group = 4 chained 16x16x32 MFMAs (fp32 C operand, exact fp32 adds);
//     lane l supplies row (l % 16) and chunk 4 s + l / 16 for step s;
//     output lane l, register v: row 4 (l / 16) + v, column l % 16.
//   - promotion: acc += P_g * (sa * sb) with one fp32 FMA per element.
//
// DGrad contracts W [N,K] over its rows: the B tile (128 rows of W x BN
// columns) is read along W's rows (coalesced), transposed 4x4 bytes at a
// time in registers with v_perm and stored column-major, so the MFMA side is
// the same as for the NT products.  128x128 weight blocks make the transpose
// exact (the block-scale grid transposes).
#include "decode_stream.hpp"
#include "fp8lin_device.hpp"
#include "fp8lin_launch.hpp"

#include <atomic>
#include <mutex>

namespace fp8lin {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum class Mode { Fwd = 0, Dgrad = 1, Wgrad = 2 };

struct GemmArgs {
    const uint8_t* a;   // [M][Kc] codes
    const float* sa;    // [M][G]
    const uint8_t* b;   // Fwd/Wgrad: [N][Kc]; Dgrad: [Kc][N]
    const float* sb;    // Fwd: [N/128][G]; Dgrad: [G][N/128]; Wgrad: [N][G]
    uint16_t* c;        // bf16 [M][N]
    int64_t M, N, Kc;
    int tiles_m, tiles_n;
};

// LDS chunk swizzle of a 256-byte row (16 chunks of 16 bytes): a bijection
// on 16 consecutive rows (fragment reads take one chunk from each of 16 rows
// per 16-lane group), and rows 2j, 2j+1 map to opposite halves (a 16-lane
// group of a staging write covers 8 chunks of each of two rows).
__device__ __forceinline__ int swz(int row) { return ((row & 1) << 3) | ((row >> 1) & 7); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// 4 E4M3 codes -> 4 fp16 (exact: every E4M3 value is an fp16 value), two
// v_cvt_scalef32_pk_f16_fp8 with scale 1.0 (measured 1.5x the throughput of
// v_cvt_pk_f32_fp8 + v_cvt_pkrtz_f16_f32).
__device__ __forceinline__ u32x2 fp8x4_to_f16x4(uint32_t w)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false);
    const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// 16 codes (one 16-byte FP8 chunk) -> 32 bytes of fp16 as two 16-byte halves.
__device__ __forceinline__ void fp8x16_to_f16(u32x4 v, u32x4& lo, u32x4& hi)
{
    const u32x2 a = fp8x4_to_f16x4(v.x), b = fp8x4_to_f16x4(v.y);
    const u32x2 c = fp8x4_to_f16x4(v.z), d = fp8x4_to_f16x4(v.w);
    lo = u32x4{a.x, a.y, b.x, b.y};
    hi = u32x4{c.x, c.y, d.x, d.y};
}

// Byte offset in an LDS row (256 bytes = 16 fp16 chunks) of logical chunk p.
__device__ __forceinline__ int lds_chunk(int row, int p) { return row * 256 + ((p ^ swz(row)) << 4); }

// XCD-aware block order: hardware dispatches workgroup i to XCD i % 8.  The
// remap makes consecutive remapped ids live on one XCD (bijective for any
// count), then a grouped raster (GROUP_M row-tiles per band) keeps tiles that
// share A rows and B columns close in time on the same L2.
__device__ __forceinline__ void tile_coords(int bid, int nblocks, int tiles_m, int tiles_n, int& tm,
                                            int& tn)
{
    constexpr int kXcd = 8;
    constexpr int kGroupM = 8;
    const int q = nblocks / kXcd, r = nblocks % kXcd;
    const int xcd = bid % kXcd, idx = bid / kXcd;
    const int id = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    const int in_group = kGroupM * tiles_n;
    const int gid = id / in_group;
    const int first_m = gid * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int local = id % in_group;
    tm = first_m + local % gsize;
    tn = local / gsize;
}

template <int BM, int BN, int WM, int WN, Mode MODE>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const GemmArgs p)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    static_assert(TM >= 1 && TN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
    constexpr int A_CHUNKS = BM * 8 / NT;           // 16-byte FP8 chunks per thread
    constexpr int B_CHUNKS = BN * 8 / NT;
    static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1 && BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile too small");
    static_assert(BM <= NT && (MODE != Mode::Wgrad || 128 + BN <= NT), "scale staging threads");
    constexpr int DG_ROWS = 32 * BN / NT;           // Dgrad: W rows per thread (8 or 16)
    static_assert(MODE != Mode::Dgrad || DG_ROWS == 8 || DG_ROWS == 16, "Dgrad tile");

    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * 256];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * 256];
    __shared__ __attribute__((aligned(16))) float lds_sa[2][BM];
    __shared__ __attribute__((aligned(16))) float lds_sb[2][MODE == Mode::Wgrad ? BN : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 15, kg = lane >> 4;

    int tmi, tni;
    tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tmi, tni);
    const int64_t m0 = (int64_t)tmi * BM;
    const int64_t n0 = (int64_t)tni * BN;
    const int64_t G = p.Kc / kGroup;

    // ------------------------------------------------ stage registers
    u32x4 ra[A_CHUNKS];
    u32x4 rb[MODE == Mode::Dgrad ? 1 : B_CHUNKS];
    uint32_t rbd[MODE == Mode::Dgrad ? DG_ROWS : 1];
    float rsa = 0.f, rsb = 0.f;
    float rsbs = 1.f;                               // Fwd/Dgrad: the group's W-block scale

    auto load_global = [&](int64_t g) {
        const int64_t k0 = g * kGroup;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int idx = tid + NT * i;
            const int r = idx >> 3, c = idx & 7;
            int64_t row = m0 + r;
            row = row < p.M ? row : p.M - 1;
            ra[i] = *reinterpret_cast<const u32x4*>(p.a + row * p.Kc + k0 + c * 16);
        }
        if constexpr (MODE == Mode::Dgrad) {
            constexpr int KQ = BN / 4;              // 4-column groups across the tile
            const int kq = tid % KQ, rbk = tid / KQ;
            const uint8_t* base = p.b + (k0 + rbk * DG_ROWS) * p.N + n0 + kq * 4;
#pragma unroll
            for (int j = 0; j < DG_ROWS; ++j)
                rbd[j] = *reinterpret_cast<const uint32_t*>(base + j * p.N);
        } else {
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int idx = tid + NT * i;
                const int r = idx >> 3, c = idx & 7;
                int64_t row = n0 + r;
                row = row < p.N ? row : p.N - 1;
                rb[i] = *reinterpret_cast<const u32x4*>(p.b + row * p.Kc + k0 + c * 16);
            }
        }
        // Scale loads are unconditional (clamped indices): a load under a
        // branch makes the wait-count pass drain every outstanding load at
        // the join, which would serialize the prefetch.
        {
            int64_t row = m0 + (tid < BM ? tid : BM - 1);
            row = row < p.M ? row : p.M - 1;
            rsa = p.sa[row * G + g];
        }
        if constexpr (MODE == Mode::Wgrad) {
            const int t = tid - 128;
            int64_t col = n0 + (t < 0 ? 0 : (t < BN ? t : BN - 1));
            col = col < p.N ? col : p.N - 1;
            rsb = p.sb[col * G + g];
        } else if constexpr (MODE == Mode::Fwd) {
            rsbs = p.sb[(n0 / kGroup) * G + g];
        } else {
            rsbs = p.sb[g * (p.N / kGroup) + n0 / kGroup];
        }
    };

    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int idx = tid + NT * i;
            const int r = idx >> 3, c = idx & 7;
            u32x4 lo, hi;
            fp8x16_to_f16(ra[i], lo, hi);
            *reinterpret_cast<u32x4*>(&lds_a[buf][lds_chunk(r, c)]) = lo;
            *reinterpret_cast<u32x4*>(&lds_a[buf][lds_chunk(r, c + 8)]) = hi;
        }
        // Fwd/Dgrad: the row scale times the group's W-block scale, i.e. the
        // whole promotion factor of the row (one fp32 product, as before)
        if (tid < BM)
            lds_sa[buf][tid] = MODE == Mode::Wgrad ? rsa : rsa * rsbs;
    };
    auto store_b = [&](int buf) {
        if constexpr (MODE == Mode::Dgrad) {
            constexpr int KQ = BN / 4;
            const int kq = tid % KQ, rbk = tid / KQ;
            uint32_t cols[4][DG_ROWS / 4];
#pragma unroll
            for (int j = 0; j < DG_ROWS / 4; ++j)
                transpose4x4(rbd[4 * j], rbd[4 * j + 1], rbd[4 * j + 2], rbd[4 * j + 3], cols[0][j],
                             cols[1][j], cols[2][j], cols[3][j]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = kq * 4 + q;
                if constexpr (DG_ROWS == 16) {
                    // rows [16 rbk, 16 rbk + 16) of the group = FP8 chunk rbk
                    u32x4 lo, hi;
                    fp8x16_to_f16(u32x4{cols[q][0], cols[q][1], cols[q][2], cols[q][3]}, lo, hi);
                    *reinterpret_cast<u32x4*>(&lds_b[buf][lds_chunk(col, rbk)]) = lo;
                    *reinterpret_cast<u32x4*>(&lds_b[buf][lds_chunk(col, rbk + 8)]) = hi;
                } else {
                    // rows [8 rbk, 8 rbk + 8) = half (rbk & 1) of FP8 chunk rbk / 2
                    const u32x2 a = fp8x4_to_f16x4(cols[q][0]), b = fp8x4_to_f16x4(cols[q][1]);
                    *reinterpret_cast<u32x4*>(&lds_b[buf][lds_chunk(col, (rbk >> 1) + 8 * (rbk & 1))]) =
                        u32x4{a.x, a.y, b.x, b.y};
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int idx = tid + NT * i;
                const int r = idx >> 3, c = idx & 7;
                u32x4 lo, hi;
                fp8x16_to_f16(rb[i], lo, hi);
                *reinterpret_cast<u32x4*>(&lds_b[buf][lds_chunk(r, c)]) = lo;
                *reinterpret_cast<u32x4*>(&lds_b[buf][lds_chunk(r, c + 8)]) = hi;
            }
        }
        if constexpr (MODE == Mode::Wgrad) {
            if (tid >= 128 && tid < 128 + BN)
                lds_sb[buf][tid - 128] = rsb;
        }
    };

    // ------------------------------------------------ main loop
    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Group g + 1 is converted into the other LDS buffer between the MFMAs of
    // group g (its codes arrived in registers during the previous group), and
    // group g + 2 is requested right after: each wave interleaves conversion
    // with matrix work, and the loads have a full group of time to land.
    const int64_t nk = G;
    load_global(0);
    store_a(0);
    store_b(0);
    load_global(nk > 1 ? 1 : 0);
    __syncthreads();

    // fragment offsets inside a buffer (the buffer index is static after the
    // unroll by two, so it folds into the instructions' offset field)
    uint32_t offa[TM][4], offb[TN][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            offa[i][s] = (uint32_t)lds_chunk(wm * WTM + i * 16 + lr, 4 * s + kg);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            offb[j][s] = (uint32_t)lds_chunk(wn * WTN + j * 16 + lr, 4 * s + kg);
    }

    for (int64_t g0 = 0; g0 < nk; g0 += 2) {
#pragma unroll
        for (int buf = 0; buf < 2; ++buf) {
            const int64_t g = g0 + buf;
            if (g >= nk)
                break;                              // uniform: odd group count
            v4f tmp[TM][TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    tmp[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                v8h fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    fa[i] = *reinterpret_cast<const v8h*>(&lds_a[buf][offa[i][s]]);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    fb[j] = *reinterpret_cast<const v8h*>(&lds_b[buf][offb[j][s]]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        tmp[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], tmp[i][j], 0, 0, 0);
                // (the group after the last re-stages the last one into the idle buffer)
                if (s == 0)
                    store_a(buf ^ 1);
                if (s == 1) {
                    store_b(buf ^ 1);
                    load_global(g + 2 < nk ? g + 2 : nk - 1);
                }
            }

            // Promotion with this group's scale products.
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const v4f sav = *reinterpret_cast<const v4f*>(&lds_sa[buf][wm * WTM + i * 16 + 4 * kg]);
                if constexpr (MODE == Mode::Wgrad) {
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const float sbc = lds_sb[buf][wn * WTN + j * 16 + lr];
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[i][j][v] = fmaf(tmp[i][j][v], sav[v] * sbc, acc[i][j][v]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[i][j][v] = fmaf(tmp[i][j][v], sav[v], acc[i][j][v]);
                }
            }

            __syncthreads();
        }
    }

    // ------------------------------------------------ epilogue
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wn * WTN + j * 16 + lr;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = m0 + wm * WTM + i * 16 + 4 * kg + v;
                if (row < p.M && col < p.N)
                    p.c[row * p.N + col] = f32_to_bf16_rne(acc[i][j][v]);
            }
        }
}

// =================================================== skinny forward (decode)
//
// Rollout decode: at most 64 rows of X against a large W.  The weights are
// read once and dominate the traffic; the work per column is too small for
// one wave per SIMD to hide its latencies, so the contraction is also split
// inside the workgroup.  A workgroup covers 64 columns of Y with KSPLIT parts
// of K; each part has 4 / CT waves, each wave owns CT tiles of 16 columns
// (16 * CT rows of W) for its part.  A wave streams its W fragments straight
// from global memory into a register ring DEPTH groups deep and converts
// them to fp16 in registers; the waves of a part stage their X (64 rows,
// DEPTH groups at a time) as fp16 into their own LDS region, and each X
// fragment read from LDS feeds CT MFMAs.  At the end the partial sums of the
// parts are added in part order (deterministic) through LDS.
//
// The vector-memory counter retires loads in order, so waiting for any load
// also waits for every load issued before it: every load is consumed about
// DEPTH groups after it is issued and none sits under a branch.
// KSPLIT * DEPTH divides the number of groups.
//
// Lane (r, kg) of a wave holds, per column tile, W row n + r, bytes
// [16 kg, 16 kg + 16) and [64 + 16 kg, 64 + 16 kg + 16) of the group (two
// 64-byte runs per row per load instruction); each MFMA step uses 8 of those
// 32 codes, and X fragments are read from LDS at the same k positions.
template <int KSPLIT, int CT, int DEPTH>
__global__ __launch_bounds__(KSPLIT * 256 / CT) void gemm_fwd_skinny_kernel(const GemmArgs p)
{
    constexpr int WPP = 4 / CT;                    // waves per part
    constexpr int TPP = 64 * WPP;                  // threads per part
    constexpr int XCH = 512 / TPP;                 // X 16-byte chunks per thread per group
    __shared__ __attribute__((aligned(16))) uint8_t lds_x[KSPLIT][DEPTH][64 * 256];
    __shared__ __attribute__((aligned(16))) float lds_sx[KSPLIT][DEPTH][64];
    static_assert(4 * 64 * 16 * sizeof(float) <= (size_t)KSPLIT * DEPTH * 64 * 256 / (KSPLIT > 1 ? KSPLIT - 1 : 1),
                  "partial sums fit in the X regions");

    const int tid = threadIdx.x;
    const int ptid = tid % TPP;                    // thread index within its part
    const int lane = tid & 63;
    const int wip = ptid >> 6;                     // wave within the part
    const int kp = tid / TPP;                      // K part
    const int lr = lane & 15, kg = lane >> 4;
    const int64_t nw = (int64_t)blockIdx.x * 64 + wip * 16 * CT;   // first column of this wave
    const int64_t G = p.Kc / kGroup;
    const int64_t GP = G / KSPLIT;                 // groups per part
    const int64_t gbeg = kp * GP;
    const uint8_t* wrow[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t)
        wrow[t] = p.b + (nw + 16 * t + lr) * p.Kc + 16 * kg;
    const float* swp = p.sb + (nw / kGroup) * G;  // the wave's 16 CT columns lie in one 128-block

    // X staging for this part: chunks (rows clamped to M) and scale row
    const uint8_t* xsrc[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int idx = ptid + TPP * i;
        const int r = idx >> 3, c = idx & 7;
        const int64_t row = r < p.M ? r : p.M - 1;
        xsrc[i] = p.a + row * p.Kc + c * 16;
    }
    const int64_t sr = ptid < 64 ? ptid : 63;
    const float* sxsrc = p.sa + (sr < p.M ? sr : p.M - 1) * G;

    u32x4 wring[DEPTH][CT][2];
    u32x4 xr[DEPTH][XCH];
    float sxr[DEPTH];
    auto load_w = [&](int slot, int64_t g) {      // g relative to the part
        const int64_t gc = gbeg + (g < GP ? g : GP - 1);
#pragma unroll
        for (int t = 0; t < CT; ++t) {
            wring[slot][t][0] = *reinterpret_cast<const u32x4*>(wrow[t] + gc * kGroup);
            wring[slot][t][1] = *reinterpret_cast<const u32x4*>(wrow[t] + gc * kGroup + 64);
        }
    };
    auto load_xchunk = [&](int64_t g0) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int64_t g = gbeg + (g0 + d < GP ? g0 + d : GP - 1);
#pragma unroll
            for (int i = 0; i < XCH; ++i)
                xr[d][i] = *reinterpret_cast<const u32x4*>(xsrc[i] + g * kGroup);
            sxr[d] = sxsrc[g];
        }
    };
    auto store_xchunk = [&]() {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
#pragma unroll
            for (int i = 0; i < XCH; ++i) {
                const int idx = ptid + TPP * i;
                const int r = idx >> 3, c = idx & 7;
                u32x4 lo, hi;
                fp8x16_to_f16(xr[d][i], lo, hi);
                // the permuted group order of gemm_kernel: chunk c, c + 8
                *reinterpret_cast<u32x4*>(&lds_x[kp][d][lds_chunk(r, c)]) = lo;
                *reinterpret_cast<u32x4*>(&lds_x[kp][d][lds_chunk(r, c + 8)]) = hi;
            }
            if (ptid < 64)
                lds_sx[kp][d][ptid] = sxr[d];
        }
    };

    load_xchunk(0);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        load_w(d, d);

    v4f acc[CT][4];
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[t][i] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int64_t g0 = 0; g0 < GP; g0 += DEPTH) {
        __syncthreads();                           // previous chunk fully read
        store_xchunk();
        load_xchunk(g0 + DEPTH);
        __syncthreads();                           // chunk g0 visible
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int64_t g = g0 + d;
            u32x4 wf[CT][4];
#pragma unroll
            for (int t = 0; t < CT; ++t) {
                fp8x16_to_f16(wring[d][t][0], wf[t][0], wf[t][1]);
                fp8x16_to_f16(wring[d][t][1], wf[t][2], wf[t][3]);
            }
            load_w(d, g + DEPTH);

            v4f tmp[CT][4];
#pragma unroll
            for (int t = 0; t < CT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tmp[t][i] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                // step s of lane group kg takes logical chunk q = 4 s + kg, i.e.
                // k in [16 (q mod 8) + 8 (q div 8), +8): W fragment (0,2,1,3)[s]
                const int q = 4 * s + kg;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v8h fa = *reinterpret_cast<const v8h*>(&lds_x[kp][d][lds_chunk(16 * i + lr, q)]);
#pragma unroll
                    for (int t = 0; t < CT; ++t)
                        tmp[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            fa, __builtin_bit_cast(v8h, wf[t][(s & 1) * 2 + (s >> 1)]), tmp[t][i], 0, 0, 0);
                }
            }
            const float sw = swp[gbeg + g];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v4f sav = *reinterpret_cast<const v4f*>(&lds_sx[kp][d][16 * i + 4 * kg]);
                float ps[4];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    ps[v] = sav[v] * sw;
#pragma unroll
                for (int t = 0; t < CT; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[t][i][v] = fmaf(tmp[t][i][v], ps[v], acc[t][i][v]);
            }
        }
    }

    // partial sums of parts 1..KSPLIT-1 through LDS (all X reads are over
    // after the first barrier)
    if constexpr (KSPLIT > 1) {
        __syncthreads();
        float* part = reinterpret_cast<float*>(&lds_x[0][0][0]);
        const int slot = wip * CT;                 // 16-column tile index in the workgroup
        if (kp > 0) {
#pragma unroll
            for (int t = 0; t < CT; ++t) {
                float* dst = part + ((kp - 1) * 4 + slot + t) * (64 * 16) + lane * 16;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<v4f*>(dst + 4 * i) = acc[t][i];
            }
        }
        __syncthreads();
        if (kp == 0) {
#pragma unroll
            for (int k = 1; k < KSPLIT; ++k)
#pragma unroll
                for (int t = 0; t < CT; ++t) {
                    const float* src = part + ((k - 1) * 4 + slot + t) * (64 * 16) + lane * 16;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[t][i] += *reinterpret_cast<const v4f*>(src + 4 * i);
                }
        }
    }
    if (kp == 0) {
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t row = 16 * i + 4 * kg + v;
                    if (row < p.M)
                        p.c[row * p.N + nw + 16 * t + lr] = f32_to_bf16_rne(acc[t][i][v]);
                }
    }
}

// ===================================== decode forward, operands streamed by LDS DMA
//
// Rollout decode with K up to 16384: the same product for at most 64 rows of
// X, built so that the weight stream never waits for arithmetic.  A
// workgroup owns 64 columns of Y (64 rows of W); both operands travel from
// global memory into LDS rings by DMA and are converted to fp16 only as MFMA
// fragments.  One workgroup barrier per chunk of two groups publishes the
// next chunk and retires the oldest.
//  * wave 8 streams W, wave 9 streams X (rows past M read row M - 1; their
//    outputs are never stored) with global_load_lds_dwordx4: each lane's 16
//    bytes land at M0 + 16 * lane, one instruction moves four rows x 256
//    contiguous bytes (one chunk of a row).  The W ring is WDW chunks deep,
//    the X ring WDX (X is an L2 hit).  The instruction is issued from inline
//    assembly so that the compiler does not drain the vector-memory counter
//    at every barrier; each loader waits explicitly for the chunk it is about
//    to publish (vmcnt retires these loads in order).
//  * waves 0-7 (two per SIMD) first build every scale product sx[r,g]*sw[g]
//    (the 64 columns lie in one 128-column weight block, so sw is per group
//    only), then multiply on v_mfma_f32_32x32x16_f16: wave (ct, kp, kq) owns
//    W rows [32 ct, +32) on the MFMA M side and all 64 X rows (two 32-row
//    tiles on the N side) for k steps [4 kq, +4) of group kp of every chunk.
//    Codes are converted with v_cvt_scalef32_pk_f16_fp8 (scale 1: exact);
//    each W code is converted once, each X code twice (both column halves).
//    The four (kp, kq) partial sums are added in a fixed order at the end.
// Lane (m, kh) of a 32x32x16 step st holds k in [64 kh + 8 st, +8) of the
// group for both operands (a fixed permutation of the group, applied to both
// sides).  Output lane l holds X row l % 32 of its tile and W rows
// 8 (j / 4) + 4 (l / 32) + j % 4, j < 16, so each lane needs one scale
// product per tile and group.
//
// LDS layout of a chunk of either operand (16-byte pieces; the rows of a
// 16-row stripe hit distinct banks): rows in 1 KB blocks of four, piece q of
// row r at (r / 4) * 1024 + 16 * (16 (r % 4) + (q ^ (r % 16))).

typedef float v16f __attribute__((ext_vector_type(16)));

// Requires M <= 64, G = K / 128 even and G <= GM; every role passes
// 3 + G / 2 barriers.
// Scale products sx[r][g] * sw[g] of a 64-column block (the columns lie in
// one 128-column weight block), four per thread per batch with the batch's
// loads in flight together; rows past M repeat row M - 1.  Threads 0..511.
__device__ __forceinline__ void decode_scale_table(const GemmArgs& p, int64_t n0, int64_t G, int GP, int tid,
                                                   float* lds_ps)
{
    const float* swp = p.sb + (n0 / kGroup) * G;
    const int nps = 64 * (int)G;
    for (int base = 0; base < nps; base += 512 * 4) {
        float sv[4], wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = min(base + tid + 512 * i, nps - 1);
            const int row = idx / (int)G, g = idx - row * (int)G;
            const int64_t xrow = row < p.M ? row : p.M - 1;
            sv[i] = p.sa[xrow * G + g];
            wv[i] = swp[g];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = base + tid + 512 * i;
            if (idx < nps) {
                const int row = idx / (int)G, g = idx - row * (int)G;
                lds_ps[row * GP + g] = sv[i] * wv[i];
            }
        }
    }
}

// Adds the four (kp, kq) partial sums of the eight MMA waves in a fixed order
// through `red` (an idle LDS ring, >= 48 KB) and stores the 64 x 64 block of
// Y as bf16.  Passes one barrier.
__device__ __forceinline__ void decode_reduce_store(const GemmArgs& p, v16f (&acc)[2], float* red, int64_t n0,
                                                    int ct, int kp, int kq, int m, int kh, int lane)
{
    // partials as 16-byte vectors: [part - 1][ct][xt][r / 4][lane][r % 4]
    const int part = kp * 2 + kq;
    auto red_at = [&](int pp, int xt, int a4) { return red + ((((pp * 2 + ct) * 2 + xt) * 4 + a4) * 64 + lane) * 4; };
    if (part != 0) {
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4)
                *reinterpret_cast<v4f*>(red_at(part - 1, xt, a4)) =
                    v4f{acc[xt][4 * a4], acc[xt][4 * a4 + 1], acc[xt][4 * a4 + 2], acc[xt][4 * a4 + 3]};
    }
    __syncthreads();
    if (part == 0) {
#pragma unroll
        for (int xt = 0; xt < 2; ++xt) {
            const int64_t row = 32 * xt + m;
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
                for (int pp = 0; pp < 3; ++pp) {
                    const v4f o = *reinterpret_cast<const v4f*>(red_at(pp, xt, a4));
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[xt][4 * a4 + e] += o[e];
                }
            if (row < p.M) {
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    uint32_t v[2];
#pragma unroll
                    for (int b2 = 0; b2 < 2; ++b2) {
                        const int r0 = 4 * a4 + 2 * b2;
                        v[b2] = (uint32_t)f32_to_bf16_rne(acc[xt][r0]) |
                                ((uint32_t)f32_to_bf16_rne(acc[xt][r0 + 1]) << 16);
                    }
                    *reinterpret_cast<u32x2*>(p.c + row * p.N + n0 + 32 * ct + 8 * a4 + 4 * kh) = u32x2{v[0], v[1]};
                }
            }
        }
    }
}

template <int WDW, int WDX, int GM>
__global__ __launch_bounds__(640) void gemm_fwd_decode_kernel(const GemmArgs p)
{
    using namespace dec;
    static_assert(WDX * WCH >= 3 * 2 * 2 * 16 * 64 * 4, "partial sums fit in the X ring");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_w[WDW][WCH];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_x[WDX][WCH];
    __shared__ __attribute__((aligned(16))) float lds_ps[64 * (GM + 1)];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = p.Kc / kGroup, nch = G / CH;
    const int GP = (int)G | 1;                     // scale-table row stride (odd: no bank conflicts)
    const int64_t n0 = (int64_t)blockIdx.x * 64;

    if (wave < 8) {
        decode_scale_table(p, n0, G, GP, tid, lds_ps);
        const int ct = wave & 1, kp = (wave >> 1) & 1, kq = wave >> 2;
        const int m = lane & 31, kh = lane >> 5;
        const int wr = 32 * ct + m;
        v16f acc[2];
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[xt][r] = 0.f;
        __syncthreads();                           // chunk 0 of both operands landed, table built
        for (int64_t c = 0; c < nch; ++c) {
            const uint8_t* wl = lds_w[c % WDW];
            const uint8_t* xl = lds_x[c % WDX];
            u32x4 wv[2], xv[2][2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int pc = 8 * kp + 4 * kh + 2 * kq + q;
                wv[q] = *reinterpret_cast<const u32x4*>(wl + w_off(wr, pc));
#pragma unroll
                for (int xt = 0; xt < 2; ++xt)
                    xv[xt][q] = *reinterpret_cast<const u32x4*>(xl + w_off(32 * xt + m, pc));
            }
            v16f tmp[2];
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    tmp[xt][r] = 0.f;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const v8h wlo = cvt8(wv[q].x, wv[q].y), whi = cvt8(wv[q].z, wv[q].w);
#pragma unroll
                for (int xt = 0; xt < 2; ++xt) {
                    const v8h xlo = cvt8(xv[xt][q].x, xv[xt][q].y), xhi = cvt8(xv[xt][q].z, xv[xt][q].w);
                    tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wlo, xlo, tmp[xt], 0, 0, 0);
                    tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(whi, xhi, tmp[xt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int xt = 0; xt < 2; ++xt) {
                const float sc = lds_ps[(32 * xt + m) * GP + c * CH + kp];
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[xt][r] = fmaf(tmp[xt][r], sc, acc[xt][r]);
            }
            __syncthreads();                       // chunk c drained, chunk c + 1 landed
        }
        __syncthreads();                           // both loaders drained: the X ring is idle
        decode_reduce_store(p, acc, reinterpret_cast<float*>(&lds_x[0][0]), n0, ct, kp, kq, m, kh, lane);
    } else if (wave == 8) {
        stream_operand<WDW>(p.b, p.N, n0, p.Kc, nch, (uint32_t)(uintptr_t)&lds_w[0][0], lane);
    } else {
        stream_operand<WDX>(p.a, p.M, 0, p.Kc, nch, (uint32_t)(uintptr_t)&lds_x[0][0], lane);
    }
}

// ------------------------------------------- decode with a fragment-packed W
//
// The same product for <= 64 rows, with W in the decode layout written by
// fp8_weight_pack: for each 64-row block nb, chunk c (256 columns) and MMA
// wave w = ct + 2 kp + 4 kq, the 2 KB that wave multiplies are contiguous,
// ordered [q][lane][16 bytes], lane = m + 32 kh holding piece
// 8 kp + 4 kh + 2 kq + q of row 32 ct + m (the pieces the LDS version reads).
// So each MMA wave loads its W fragments with two fully coalesced 1 KB loads
// per chunk straight into registers, one chunk ahead, and W needs neither LDS
// nor a loader wave; X still streams through the LDS ring (wave 8).  The
// arithmetic, and so every result bit, is that of gemm_fwd_decode_kernel.
// NCH > 0 fixes K / 256 at compile time (fully unrolled loop); NCH == 0 reads
// it at run time.
__device__ __forceinline__ int64_t packed_piece(int64_t nb, int64_t nch, int64_t c, int w, int q, int lane)
{
    return (((nb * nch + c) * 8 + w) * 2 + q) * 64 + lane;   // in 16-byte pieces
}

template <int GM, int NCH>
__global__ __launch_bounds__(576) void gemm_fwd_decode_packed_kernel(const GemmArgs p)
{
    using namespace dec;
    constexpr int WDX = 4;
    static_assert(WDX * WCH >= 3 * 2 * 2 * 16 * 64 * 4, "partial sums fit in the X ring");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_x[WDX][WCH];
    __shared__ __attribute__((aligned(16))) float lds_ps[64 * (GM + 1)];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = p.Kc / kGroup, nch = NCH > 0 ? NCH : G / CH;
    const int GP = (int)G | 1;
    const int64_t n0 = (int64_t)blockIdx.x * 64;

    if (wave < 8) {
        decode_scale_table(p, n0, G, GP, tid, lds_ps);
        const u32x4* wsrc = reinterpret_cast<const u32x4*>(p.b) + packed_piece(blockIdx.x, nch, 0, wave, 0, lane);
        u32x4 wreg[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
            wreg[q] = __builtin_nontemporal_load(wsrc + q * 64);
        const int ct = wave & 1, kp = (wave >> 1) & 1, kq = wave >> 2;
        const int m = lane & 31, kh = lane >> 5;
        v16f acc[2];
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[xt][r] = 0.f;
        // acc += t * s, one scale per 32-row half
        auto promote = [&](const v16f (&t)[2], const float (&sc)[2]) {
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[xt][r] = fmaf(t[xt][r], sc[xt], acc[xt][r]);
        };
        // unrolled loop: chunk c's partial products are scaled into acc while
        // chunk c + 1 is multiplied (the same additions in the same order), so
        // the promotion overlaps the next chunk's LDS reads and MFMAs instead
        // of waiting on the last MFMA before each barrier
        v16f prev[2];
        float sprev[2] = {0.f, 0.f};
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
            float sc[2];
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
                sc[xt] = lds_ps[(32 * xt + m) * GP + c * CH + kp];
            v8h wlo[2], whi[2];
            if constexpr (NCH == 0) {
                // run-time loop: convert this chunk's W fragments before the
                // next chunk is loaded into their registers (otherwise the
                // loop's back edge copies them and waits for the loads)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    wlo[q] = cvt8(wreg[q].x, wreg[q].y);
                    whi[q] = cvt8(wreg[q].z, wreg[q].w);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            const u32x4 wv[2] = {wreg[0], wreg[1]};
            {
                const int64_t cn = c + 1 < nch ? c + 1 : c;  // last chunk: a harmless re-read
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    wreg[q] = __builtin_nontemporal_load(wsrc + cn * (8 * 2 * 64) + q * 64);
            }
            if constexpr (NCH == 0)
                __builtin_amdgcn_sched_barrier(0);
            if constexpr (NCH > 0) {
                if (c > 0)
                    promote(prev, sprev);
            }
            v16f tmp[2];
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    tmp[xt][r] = 0.f;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if constexpr (NCH > 0) {
                    wlo[q] = cvt8(wv[q].x, wv[q].y);
                    whi[q] = cvt8(wv[q].z, wv[q].w);
                }
#pragma unroll
                for (int xt = 0; xt < 2; ++xt) {
                    const v8h xlo = cvt8(xv[xt][q].x, xv[xt][q].y), xhi = cvt8(xv[xt][q].z, xv[xt][q].w);
                    tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wlo[q], xlo, tmp[xt], 0, 0, 0);
                    tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(whi[q], xhi, tmp[xt], 0, 0, 0);
                }
            }
            if constexpr (NCH > 0) {
#pragma unroll
                for (int xt = 0; xt < 2; ++xt) {
                    prev[xt] = tmp[xt];
                    sprev[xt] = sc[xt];
                }
            } else {
                promote(tmp, sc);
            }
            __syncthreads();                       // chunk c drained, chunk c + 1 landed
        }
        if constexpr (NCH > 0)
            promote(prev, sprev);                  // the last chunk
        __syncthreads();                           // the loader drained: the X ring is idle
        decode_reduce_store(p, acc, reinterpret_cast<float*>(&lds_x[0][0]), n0, ct, kp, kq, m, kh, lane);
    } else {
        stream_operand<WDX>(p.a, p.M, 0, p.Kc, nch, (uint32_t)(uintptr_t)&lds_x[0][0], lane);
    }
}

// ------------------------------------ decode on the packed W, split over K
//
// For weights with few output columns (N / 64 workgroups leave most CUs
// idle, e.g. the MLP down projection, N = 4096) the chunks of the contraction
// are divided over S workgroups per 64-column block (blockIdx.y = split).
// Each computes the packed kernel's product over its chunk range [c0, c1)
// (same roles, same per-chunk arithmetic, the four wave partials added in the
// same fixed order) and writes that fp32 64x64 partial tile to the caller's
// workspace, [S][M][N]; splitk_reduce_kernel then adds the S partials in
// ascending split order and rounds to BF16.  Deterministic, rows independent
// of the other rows of the call; not bit-identical to the unsplit kernels
// (the groups are added in another association).
template <int GM, int NL = 0>
__global__ __launch_bounds__(576) void gemm_fwd_decode_packed_splitk_kernel(const GemmArgs p, float* ws,
                                                                            int64_t per_split)
{
    using namespace dec;
    constexpr int WDX = 4;
    static_assert(WDX * WCH >= 3 * 2 * 2 * 16 * 64 * 4, "partial sums fit in the X ring");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_x[WDX][WCH];
    __shared__ __attribute__((aligned(16))) float lds_ps[64 * (GM + 1)];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = p.Kc / kGroup, nch = G / CH;
    const int GP = (int)G | 1;
    const int64_t n0 = (int64_t)blockIdx.x * 64;
    const int64_t c0 = (int64_t)blockIdx.y * per_split;
    const int64_t c1 = c0 + per_split < nch ? c0 + per_split : nch;
    const int64_t nloc = c1 - c0;                  // >= 1: the launcher sizes the splits

    if (wave < 8) {
        decode_scale_table(p, n0, G, GP, tid, lds_ps);
        const u32x4* wsrc = reinterpret_cast<const u32x4*>(p.b) + packed_piece(blockIdx.x, nch, 0, wave, 0, lane);
        u32x4 wreg[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
            wreg[q] = __builtin_nontemporal_load(wsrc + c0 * (8 * 2 * 64) + q * 64);
        const int ct = wave & 1, kp = (wave >> 1) & 1, kq = wave >> 2;
        const int m = lane & 31, kh = lane >> 5;
        v16f acc[2];
#pragma unroll
        for (int xt = 0; xt < 2; ++xt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[xt][r] = 0.f;
        __syncthreads();                           // local chunk 0 of X landed, table built
        if constexpr (NL > 0) {
            // every split has NL chunks: unrolled, and each chunk's partial
            // products are scaled into acc during the next chunk (the same
            // additions in the same order)
            v16f prev[2];
            float sprev[2] = {0.f, 0.f};
#pragma unroll
            for (int lc = 0; lc < NL; ++lc) {
                const int64_t c = c0 + lc;
                const uint8_t* xl = lds_x[lc % WDX];
                u32x4 xv[2][2];
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int xt = 0; xt < 2; ++xt)
                        xv[xt][q] = *reinterpret_cast<const u32x4*>(xl + w_off(32 * xt + m, 8 * kp + 4 * kh + 2 * kq + q));
                float sc[2];
#pragma unroll
                for (int xt = 0; xt < 2; ++xt)
                    sc[xt] = lds_ps[(32 * xt + m) * GP + c * CH + kp];
                const u32x4 wv[2] = {wreg[0], wreg[1]};
                {
                    const int64_t cn = lc + 1 < NL ? c + 1 : c;   // last chunk: a harmless re-read
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        wreg[q] = __builtin_nontemporal_load(wsrc + cn * (8 * 2 * 64) + q * 64);
                }
                if (lc > 0) {
#pragma unroll
                    for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[xt][r] = fmaf(prev[xt][r], sprev[xt], acc[xt][r]);
                }
                v16f tmp[2];
#pragma unroll
                for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        tmp[xt][r] = 0.f;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const v8h wlo = cvt8(wv[q].x, wv[q].y), whi = cvt8(wv[q].z, wv[q].w);
#pragma unroll
                    for (int xt = 0; xt < 2; ++xt) {
                        const v8h xlo = cvt8(xv[xt][q].x, xv[xt][q].y), xhi = cvt8(xv[xt][q].z, xv[xt][q].w);
                        tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wlo, xlo, tmp[xt], 0, 0, 0);
                        tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(whi, xhi, tmp[xt], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int xt = 0; xt < 2; ++xt) {
                    prev[xt] = tmp[xt];
                    sprev[xt] = sc[xt];
                }
                __syncthreads();                   // chunk drained, the next one landed
            }
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[xt][r] = fmaf(prev[xt][r], sprev[xt], acc[xt][r]);
        } else {
            for (int64_t lc = 0; lc < nloc; ++lc) {
                const int64_t c = c0 + lc;
                const uint8_t* xl = lds_x[lc % WDX];
                u32x4 xv[2][2];
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int xt = 0; xt < 2; ++xt)
                        xv[xt][q] = *reinterpret_cast<const u32x4*>(xl + w_off(32 * xt + m, 8 * kp + 4 * kh + 2 * kq + q));
                v8h wlo[2], whi[2];
                // convert this chunk's W fragments before the next chunk is
                // loaded into their registers
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    wlo[q] = cvt8(wreg[q].x, wreg[q].y);
                    whi[q] = cvt8(wreg[q].z, wreg[q].w);
                }
                __builtin_amdgcn_sched_barrier(0);
                {
                    const int64_t cn = c + 1 < c1 ? c + 1 : c;   // last chunk: a harmless re-read
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        wreg[q] = __builtin_nontemporal_load(wsrc + cn * (8 * 2 * 64) + q * 64);
                }
                __builtin_amdgcn_sched_barrier(0);
                v16f tmp[2];
#pragma unroll
                for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        tmp[xt][r] = 0.f;
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int xt = 0; xt < 2; ++xt) {
                        const v8h xlo = cvt8(xv[xt][q].x, xv[xt][q].y), xhi = cvt8(xv[xt][q].z, xv[xt][q].w);
                        tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wlo[q], xlo, tmp[xt], 0, 0, 0);
                        tmp[xt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(whi[q], xhi, tmp[xt], 0, 0, 0);
                    }
#pragma unroll
                for (int xt = 0; xt < 2; ++xt) {
                    const float sc = lds_ps[(32 * xt + m) * GP + c * CH + kp];
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[xt][r] = fmaf(tmp[xt][r], sc, acc[xt][r]);
                }
                __syncthreads();                       // chunk drained, the next one landed
            }
        }
        __syncthreads();                           // the loader drained: the X ring is idle
        // the four (kp, kq) partials in the fixed order of decode_reduce_store,
        // then the fp32 tile to ws[split]
        float* red = reinterpret_cast<float*>(&lds_x[0][0]);
        const int part = kp * 2 + kq;
        if (part != 0) {
#pragma unroll
            for (int xt = 0; xt < 2; ++xt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    red[(((part - 1) * 2 + ct) * 2 + xt) * 16 * 64 + r * 64 + lane] = acc[xt][r];
        }
        __syncthreads();
        if (part == 0) {
            float* dst = ws + (int64_t)blockIdx.y * p.M * p.N;
#pragma unroll
            for (int xt = 0; xt < 2; ++xt) {
                const int64_t row = 32 * xt + m;
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int pp = 0; pp < 3; ++pp)
                        acc[xt][r] += red[((pp * 2 + ct) * 2 + xt) * 16 * 64 + r * 64 + lane];
                if (row < p.M) {
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4)
                        *reinterpret_cast<float4*>(dst + row * p.N + n0 + 32 * ct + 8 * a4 + 4 * kh) =
                            make_float4(acc[xt][4 * a4], acc[xt][4 * a4 + 1], acc[xt][4 * a4 + 2],
                                        acc[xt][4 * a4 + 3]);
                }
            }
        }
    } else {
        stream_operand<WDX>(p.a + c0 * (CH * kGroup), p.M, 0, p.Kc, nloc, (uint32_t)(uintptr_t)&lds_x[0][0],
                            lane);
    }
}

// y[m][n] = bf16(sum over splits, ascending, of ws[split][m][n]); 4 columns
// per thread.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int S, int64_t mn,
                                                            uint16_t* __restrict__ y)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn)
        return;
    float4 a = *reinterpret_cast<const float4*>(ws + i);
    for (int k = 1; k < S; ++k) {
        const float4 b = *reinterpret_cast<const float4*>(ws + (int64_t)k * mn + i);
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    *reinterpret_cast<u32x2*>(y + i) =
        u32x2{(uint32_t)f32_to_bf16_rne(a.x) | ((uint32_t)f32_to_bf16_rne(a.y) << 16),
              (uint32_t)f32_to_bf16_rne(a.z) | ((uint32_t)f32_to_bf16_rne(a.w) << 16)};
}

// W codes [N][K] -> the decode layout above, one 16-byte piece per thread
// (stores coalesced, loads gathered; done once per weight update).
__global__ __launch_bounds__(256) void pack_decode_kernel(const uint8_t* __restrict__ wq, int64_t K,
                                                          int64_t npieces, u32x4* __restrict__ wqp)
{
    const int64_t nch = K / (dec::CH * kGroup);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < npieces; i += (int64_t)gridDim.x * 256) {
        const int lane = (int)(i & 63), q = (int)((i >> 6) & 1), w = (int)((i >> 7) & 7);
        const int64_t c = (i >> 10) % nch, nb = (i >> 10) / nch;
        const int ct = w & 1, kp = (w >> 1) & 1, kq = w >> 2, m = lane & 31, kh = lane >> 5;
        const int64_t row = nb * 64 + 32 * ct + m;
        const int pc = 8 * kp + 4 * kh + 2 * kq + q;
        wqp[i] = *reinterpret_cast<const u32x4*>(wq + row * K + c * (dec::CH * kGroup) + 16 * pc);
    }
}

// ------------------------------------------------------------ large NT GEMM
//
// C[m][n] = sum_g sa(m, g) sb(n, g) sum_{k in g} dec(a[m][k]) dec(b[n][k]) for
// the forward GEMM (sb(n, g) = sb[n / 128][g], a 128x128 weight block) and
// WGrad (sb(n, g) = sb[n][g]); both operands are row-major with the
// contraction contiguous.  A workgroup of four waves computes a 128 x 128
// tile of C, two workgroups per CU, one 128-wide group per step:
//  * every wave streams its share of the step's operands straight from
//    global memory into LDS with global_load_lds (9 instructions per wave and
//    step: 4 x 1 KB of A codes, 4 x 1 KB of B codes, one 256-byte run of row
//    scales), two steps deep; one barrier per step publishes step g and
//    retires step g - 1, whose slot then receives step g + 1;
//  * wave w multiplies A rows [64 (w % 2), +64) by B rows [64 (w / 2), +64)
//    as 2 x 2 tiles of v_mfma_f32_32x32x16_f16, converting codes exactly to
//    fp16 after the LDS read (v_cvt_scalef32_pk_f16_fp8, scale 1), and adds
//    each step's fp32 partial sums into the accumulators times sa * sb.
// MFMA side: B rows are the instruction's M side and A rows its N side, so a
// lane's 16 results share one A row (one sa per tile and step).  Lane (m, kh)
// of k-step st of a step holds k in [32 (st / 2) + 16 kh + 8 (st % 2), +8)
// for both operands, a fixed permutation of the group.
// LDS: a row of a step is 128 bytes, its 16-byte piece q at position
// q ^ ((row / 2) % 8), so the 16 rows a 16-lane fragment read touches cover
// all banks; the DMA writes eight whole rows per instruction.
namespace nt {
// Tile shapes: BA A rows x BB B rows per workgroup of NW waves, each wave a
// TA x TB block of 32 x 32 tiles (a WA x WB wave grid), D steps in flight.
// Every output element is computed by the same instruction sequence whatever
// the shape (one chain of MFMAs per group in a fixed k order, then one
// promotion), so all shapes give bit-identical results.
template <int BA_, int NW_, int D_, int BB_ = 128, int TA_ = 2, int TB_ = 2>
struct Cfg {
    static constexpr int BA = BA_, BB = BB_, NW = NW_, D = D_, TA = TA_, TB = TB_;
    static constexpr int WA = BA / (32 * TA);      // waves along A
    static constexpr int WB = BB / (32 * TB);      // waves along B (WA x WB = NW)
    static constexpr int RA = BA / 64, RB = BB / 64;   // 64-row scale runs of A and of B
    static constexpr int OFF_B = BA * kGroup;
    static constexpr int OFF_SA = OFF_B + BB * kGroup;
    static constexpr int OFF_SB = OFF_SA + BA * 4;
    static constexpr int STAGE = (OFF_SB + BB * 4 + 1023) / 1024 * 1024;
    static constexpr int NA = BA / 8 / NW;         // 1 KB A-code runs per wave and step
    static constexpr int NB = BB / 8 / NW;         // 1 KB B-code runs per wave and step
    static constexpr int NDMA = NA + NB + 1;       // + one 64-row run of scales
    static_assert(WA * WB == NW && NA * NW * 8 == BA && NB * NW * 8 == BB, "tile / wave split");
    static_assert(RA * 64 == BA && RB * 64 == BB && NW >= RA + RB, "every scale run has a wave");
};
// Two workgroups per CU (2 x 66 KB of LDS): while one waits at its step
// barrier the other computes.  Measured 5-8% ahead of one 256 x 128
// workgroup of 8 waves with three steps in flight (Cfg<256, 8, 3>), and
// level with or ahead of one with two steps in flight (Cfg<256, 8, 2>, 25%
// fewer operand bytes per flop: 16384 x 27648 x 5120 within 2%, 8192 x
// 18944 x 3584 6-8% slower), with bit-identical results.
using Pair = Cfg<128, 4, 2>;
// Rollout batches (M <= 64) on the batch-invariant forward: 64 x 64 tiles of
// four waves with one 32 x 32 tile each, so an 8B up-projection fills 224
// workgroups instead of 112 half-empty ones, four steps in flight (each wave
// has a quarter of Pair's arithmetic per step; measured 2 / 3 / 4 / 6 / 8
// steps: 28.5 / 23.1 / 20.8-21.9 / 24.1-24.6 / 23.6-23.8 us); bit-identical
// to Pair.
using Skinny = Cfg<64, 4, 4, 64, 1, 1>;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int piece(int row, int q) { return row * kGroup + ((q ^ ((row >> 1) & 7)) << 4); }

template <class C>
struct Sources {
    const uint8_t* a[C::NA];                       // 8-row runs of A codes
    const uint8_t* b[C::NB];                       // 8-row runs of B codes
    const float* s;                                // a 64-row run of A or B scales
    uint32_t dst_s;                                // its LDS offset within a step
};

// Waits until this wave's DMA of step g has landed, when `after` later steps
// (after <= AMAX) have been issued behind it: vmcnt retires in order, so at
// most after * NDMA of the wave's DMAs may still be outstanding.
template <int NDMA, int AMAX>
__device__ __forceinline__ void wait_step(int64_t after)
{
    if constexpr (AMAX == 0) {
        dec::wait_vm<0>();
    } else {
        if (after >= AMAX)
            dec::wait_vm<AMAX * NDMA>();
        else
            wait_step<NDMA, AMAX - 1>(after);
    }
}

// One wave's share of step g into LDS slot `st` (an LDS byte address).
template <class C>
__device__ __forceinline__ void issue_step(const Sources<C>& src, int wave, uint32_t st, int64_t g)
{
    using namespace dec;
#pragma unroll
    for (int i = 0; i < C::NA; ++i)
        dma16(st + (C::NA * wave + i) * 1024, src.a[i] + g * kGroup);
#pragma unroll
    for (int j = 0; j < C::NB; ++j)
        dma16(st + C::OFF_B + (C::NB * wave + j) * 1024, src.b[j] + g * kGroup);
    dma4(st + src.dst_s, src.s + g);
}
}  // namespace nt

template <Mode MODE, class C>
__global__ __launch_bounds__(C::NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void gemm_nt_kernel(
    const GemmArgs p)
{
    using namespace dec;
    using namespace nt;
    static_assert(MODE == Mode::Fwd || MODE == Mode::Wgrad, "NT operands only");
    static_assert(MODE != Mode::Fwd || 128 % C::BB == 0, "a forward tile's B rows lie in one weight block");
    constexpr int BA = C::BA, BB = C::BB, D = C::D, STAGE = C::STAGE;
    constexpr int OFF_B = C::OFF_B, OFF_SA = C::OFF_SA, OFF_SB = C::OFF_SB;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[D * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = p.Kc / kGroup;
    int tm, tn;
    tile_coords((int)blockIdx.x, (int)gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BA, n0 = (int64_t)tn * BB;

    // this wave's DMA sources (rows past the end read the last row; their
    // results are never stored)
    Sources<C> src;
    {
        const int r8 = lane >> 3, pos = lane & 7;
#pragma unroll
        for (int i = 0; i < C::NA; ++i) {
            const int row = 8 * (C::NA * wave + i) + r8;
            const int64_t gr = m0 + row < p.M ? m0 + row : p.M - 1;
            src.a[i] = p.a + gr * p.Kc + 16 * (pos ^ ((row >> 1) & 7));
        }
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
            const int row = 8 * (C::NB * wave + j) + r8;
            const int64_t gr = n0 + row < p.N ? n0 + row : p.N - 1;
            src.b[j] = p.b + gr * p.Kc + 16 * (pos ^ ((row >> 1) & 7));
        }
        if (wave < C::RA) {
            const int64_t gr = m0 + 64 * wave + lane < p.M ? m0 + 64 * wave + lane : p.M - 1;
            src.s = p.sa + gr * G;
            src.dst_s = OFF_SA + 256 * wave;
        } else {
            // the B-scale runs; with more waves than runs, the extra waves
            // repeat them (same values to the same words), so that every wave
            // issues NDMA
            const int run = (wave - C::RA) % C::RB;
            const int64_t r = n0 + 64 * run + lane;
            const int64_t gr = r < p.N ? r : p.N - 1;
            src.s = MODE == Mode::Fwd ? p.sb + (gr / kGroup) * G : p.sb + gr * G;
            src.dst_s = OFF_SB + 256 * run;
        }
    }
    const uint32_t base = (uint32_t)(uintptr_t)&lds[0];

    constexpr int TA = C::TA, TB = C::TB;
    const int wa = wave % C::WA, wb = wave / C::WA;
    const int a0 = 32 * TA * wa, b0 = 32 * TB * wb;    // the wave's first A row and B row in the tile
    const int m = lane & 31, kh = lane >> 5;
    v16f acc[TA][TB];
#pragma unroll
    for (int at = 0; at < TA; ++at)
#pragma unroll
        for (int bt = 0; bt < TB; ++bt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[at][bt][r] = 0.f;

#pragma unroll
    for (int s0 = 0; s0 < D - 1; ++s0)
        if (s0 < G)
            issue_step<C>(src, wave, base + s0 * STAGE, s0);
    for (int64_t g = 0; g < G; ++g) {
        // steps g + 1 .. min(g + D - 2, G - 1) were issued behind step g
        wait_step<C::NDMA, D - 2>(G - 1 - g);      // step g landed (this wave's part)
        __syncthreads();                           // all of step g landed; step g - 1 retired
        if (g + D - 1 < G)
            issue_step<C>(src, wave, base + (uint32_t)(((g + D - 1) % D) * STAGE), g + D - 1);
        const uint8_t* st = lds + (g % D) * STAGE;
        v16f tmp[TA][TB];
#pragma unroll
        for (int at = 0; at < TA; ++at)
#pragma unroll
            for (int bt = 0; bt < TB; ++bt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    tmp[at][bt][r] = 0.f;
        // pieces of k pair kp + 1 are read while pair kp is multiplied
        u32x4 avn[TA], bvn[TB];
#pragma unroll
        for (int t = 0; t < TA; ++t)
            avn[t] = *reinterpret_cast<const u32x4*>(st + piece(a0 + 32 * t + m, kh));
#pragma unroll
        for (int t = 0; t < TB; ++t)
            bvn[t] = *reinterpret_cast<const u32x4*>(st + OFF_B + piece(b0 + 32 * t + m, kh));
#pragma unroll
        for (int kp = 0; kp < 4; ++kp) {
            u32x4 av[TA], bv[TB];
#pragma unroll
            for (int t = 0; t < TA; ++t)
                av[t] = avn[t];
#pragma unroll
            for (int t = 0; t < TB; ++t)
                bv[t] = bvn[t];
            if (kp < 3) {
                const int q = 2 * (kp + 1) + kh;
#pragma unroll
                for (int t = 0; t < TA; ++t)
                    avn[t] = *reinterpret_cast<const u32x4*>(st + piece(a0 + 32 * t + m, q));
#pragma unroll
                for (int t = 0; t < TB; ++t)
                    bvn[t] = *reinterpret_cast<const u32x4*>(st + OFF_B + piece(b0 + 32 * t + m, q));
            }
            v8h alo[TA], ahi[TA], blo[TB], bhi[TB];
#pragma unroll
            for (int t = 0; t < TA; ++t) {
                alo[t] = cvt8(av[t].x, av[t].y);
                ahi[t] = cvt8(av[t].z, av[t].w);
            }
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                blo[t] = cvt8(bv[t].x, bv[t].y);
                bhi[t] = cvt8(bv[t].z, bv[t].w);
            }
            // the tiles' first k steps, then their second (with 2 x 2 tiles a
            // dependent pair is three instructions apart)
#pragma unroll
            for (int at = 0; at < TA; ++at)
#pragma unroll
                for (int bt = 0; bt < TB; ++bt)
                    tmp[at][bt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(blo[bt], alo[at], tmp[at][bt], 0, 0, 0);
#pragma unroll
            for (int at = 0; at < TA; ++at)
#pragma unroll
                for (int bt = 0; bt < TB; ++bt)
                    tmp[at][bt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bhi[bt], ahi[at], tmp[at][bt], 0, 0, 0);
        }
        const float* ssa = reinterpret_cast<const float*>(st + OFF_SA);
        const float* ssb = reinterpret_cast<const float*>(st + OFF_SB);
#pragma unroll
        for (int at = 0; at < TA; ++at) {
            const float sa = ssa[a0 + 32 * at + m];
#pragma unroll
            for (int bt = 0; bt < TB; ++bt) {
                if constexpr (MODE == Mode::Fwd) {
                    // the tile's B rows lie in one 128-row weight block
                    const float s = sa * ssb[0];
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[at][bt][r] = fmaf(tmp[at][bt][r], s, acc[at][bt][r]);
                } else {
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        const f32x4 sb4 =
                            *reinterpret_cast<const f32x4*>(ssb + b0 + 32 * bt + 8 * a4 + 4 * kh);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[at][bt][4 * a4 + e] = fmaf(tmp[at][bt][4 * a4 + e], sa * sb4[e],
                                                           acc[at][bt][4 * a4 + e]);
                    }
                }
            }
        }
    }

    // C rows are A rows (lane m of each tile), columns B rows: four
    // consecutive columns per lane and 8-byte stores (N % 4 == 0)
#pragma unroll
    for (int at = 0; at < TA; ++at) {
        const int64_t row = m0 + a0 + 32 * at + m;
        if (row >= p.M)
            continue;
#pragma unroll
        for (int bt = 0; bt < TB; ++bt)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int64_t col = n0 + b0 + 32 * bt + 8 * a4 + 4 * kh;
                if (col < p.N) {
                    const int r0 = 4 * a4;
                    const uint32_t v0 = (uint32_t)f32_to_bf16_rne(acc[at][bt][r0]) |
                                        ((uint32_t)f32_to_bf16_rne(acc[at][bt][r0 + 1]) << 16);
                    const uint32_t v1 = (uint32_t)f32_to_bf16_rne(acc[at][bt][r0 + 2]) |
                                        ((uint32_t)f32_to_bf16_rne(acc[at][bt][r0 + 3]) << 16);
                    *reinterpret_cast<u32x2*>(p.c + row * p.N + col) = u32x2{v0, v1};
                }
            }
    }
}

// Zeros for an empty contraction (C = 0).  A kernel rather than a memset so
// the call stays capturable without memset nodes.
__global__ __launch_bounds__(256) void fill_zero_kernel(uint16_t* __restrict__ c, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = i; k < n; k += stride)
        c[k] = 0;
}

// ================================================================ launchers

template <int BM, int BN, int WM, int WN, Mode MODE>
static void launch_gemm(GemmArgs p, hipStream_t st)
{
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.N + BN - 1) / BN);
    const unsigned nblocks = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
    gemm_kernel<BM, BN, WM, WN, MODE><<<nblocks, 64 * WM * WN, 0, st>>>(p);
}

void launch_fill_zero_bf16(void* c, int64_t n, hipStream_t st)
{
    int64_t b = (n + 255) / 256;
    if (b > 8192)
        b = 8192;
    fill_zero_kernel<<<(unsigned)(b < 1 ? 1 : b), 256, 0, st>>>(static_cast<uint16_t*>(c), n);
}

template <Mode MODE, class C = nt::Pair>
static void launch_gemm_nt(GemmArgs p, hipStream_t st)
{
    p.tiles_m = (int)((p.M + C::BA - 1) / C::BA);
    p.tiles_n = (int)((p.N + C::BB - 1) / C::BB);
    const unsigned nblocks = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
    gemm_nt_kernel<MODE, C><<<nblocks, C::NW * 64, 0, st>>>(p);
}

void launch_gemm_fwd(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                     int64_t N, int64_t K, void* y, hipStream_t st)
{
    GemmArgs p{xq, sx, wq, sw, static_cast<uint16_t*>(y), M, N, K, 0, 0};
    const int64_t G = K / kGroup;
    if (M <= 64 && G % 2 == 0 && G <= 64)
        gemm_fwd_decode_kernel<3, 4, 64><<<(unsigned)(N / 64), 640, 0, st>>>(p);
    else if (M <= 64 && G % 2 == 0 && G <= 128)
        gemm_fwd_decode_kernel<3, 4, 128><<<(unsigned)(N / 64), 640, 0, st>>>(p);
    else if (M <= 64 && G % 8 == 0)
        gemm_fwd_skinny_kernel<4, 1, 2><<<(unsigned)(N / 64), 1024, 0, st>>>(p);
    else if (M <= 64)
        launch_gemm<64, 64, 1, 4, Mode::Fwd>(p, st);
    else
        launch_gemm_nt<Mode::Fwd>(p, st);
}

void launch_gemm_fwd_unified(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                             int64_t N, int64_t K, void* y, hipStream_t st)
{
    // one kernel for every M: each output element is the same MFMA chain over
    // the same groups in ascending order, whichever tile its row falls in and
    // whichever tile shape (64 x 64 for rollout batches, 128 x 128 above)
    GemmArgs p{xq, sx, wq, sw, static_cast<uint16_t*>(y), M, N, K, 0, 0};
    if (M <= 64)
        launch_gemm_nt<Mode::Fwd, nt::Skinny>(p, st);
    else
        launch_gemm_nt<Mode::Fwd>(p, st);
}

// Splits per 64-column block for the split-K decode GEMM: none when the
// 64-column blocks already fill half the CUs, else enough workgroups to cover
// the 256 CUs with at least two chunks (512 columns of K) per split.
int64_t splitk_splits(int64_t N, int64_t K)
{
    const int64_t blocks = N / 64, nch = K / (dec::CH * kGroup);
    if (blocks >= 128)
        return 1;                                  // at least half the CUs busy: no split
    int64_t s = blocks > 0 ? (256 + blocks - 1) / blocks : 1;
    if (s > nch / 2)
        s = nch / 2;
    if (s < 1)
        s = 1;
    // equal chunk ranges, none empty
    const int64_t per = (nch + s - 1) / s;
    return (nch + per - 1) / per;
}

void launch_gemm_fwd_packed_splitk(const uint8_t* xq, const float* sx, const uint8_t* wqp, const float* sw,
                                   int64_t M, int64_t N, int64_t K, void* y, float* ws, hipStream_t st)
{
    const int64_t S = splitk_splits(N, K);
    if (S <= 1) {
        launch_gemm_fwd_packed(xq, sx, wqp, sw, M, N, K, y, st);
        return;
    }
    GemmArgs p{xq, sx, wqp, sw, static_cast<uint16_t*>(y), M, N, K, 0, 0};
    const int64_t nch = K / (dec::CH * kGroup);
    const int64_t per = (nch + S - 1) / S;
    const dim3 grid((unsigned)(N / 64), (unsigned)S);
    if (per == 14 && nch == S * per)               // the 8B down projection (K = 14336, 4 splits)
        gemm_fwd_decode_packed_splitk_kernel<128, 14><<<grid, 576, 0, st>>>(p, ws, per);
    else if (K / kGroup <= 64)
        gemm_fwd_decode_packed_splitk_kernel<64><<<grid, 576, 0, st>>>(p, ws, per);
    else
        gemm_fwd_decode_packed_splitk_kernel<128><<<grid, 576, 0, st>>>(p, ws, per);
    const int64_t mn = M * N;
    splitk_reduce_kernel<<<(unsigned)((mn / 4 + 255) / 256), 256, 0, st>>>(ws, (int)S, mn,
                                                                          static_cast<uint16_t*>(y));
}

// ------------------------------------------- allocation-free split-K scratch
//
// The fp32 partial sums [S][M][N] of the split-K decode GEMM for callers that
// cannot allocate: a file-scope device array, one copy per GPU, alive until
// the process ends and shared by every call on that GPU (calls that overlap
// on one GPU race on it).  Every element a call reads was written by the same
// call's split kernel, so nothing needs clearing.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// it looks up the device address once per device with hipGetSymbolAddress
// and uses that pointer.
static __device__ __align__(256) float scratch[kSplitkScratchBytes / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t splitk_scratch(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kScratchDevices)
        return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            // the current device is `dev`: the address is that GPU's copy
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            if (p == nullptr)
                return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

void launch_pack_decode(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wqp, hipStream_t st)
{
    const int64_t npieces = N * K / 16;
    int64_t b = (npieces + 255) / 256;
    if (b > 65536)
        b = 65536;
    pack_decode_kernel<<<(unsigned)b, 256, 0, st>>>(wq, K, npieces, reinterpret_cast<u32x4*>(wqp));
}

void launch_gemm_fwd_packed(const uint8_t* xq, const float* sx, const uint8_t* wqp, const float* sw, int64_t M,
                            int64_t N, int64_t K, void* y, hipStream_t st)
{
    GemmArgs p{xq, sx, wqp, sw, static_cast<uint16_t*>(y), M, N, K, 0, 0};
    const int64_t nch = K / (dec::CH * kGroup);
    const unsigned grid = (unsigned)(N / 64);
    // the model widths of the decode workloads get a fully unrolled loop
    if (nch == 14)
        gemm_fwd_decode_packed_kernel<64, 14><<<grid, 576, 0, st>>>(p);
    else if (nch == 16)
        gemm_fwd_decode_packed_kernel<64, 16><<<grid, 576, 0, st>>>(p);
    else if (nch == 20)
        gemm_fwd_decode_packed_kernel<64, 20><<<grid, 576, 0, st>>>(p);
    else if (nch <= 32)
        gemm_fwd_decode_packed_kernel<64, 0><<<grid, 576, 0, st>>>(p);
    else
        gemm_fwd_decode_packed_kernel<128, 0><<<grid, 576, 0, st>>>(p);
}

void launch_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw, int64_t T,
                       int64_t N, int64_t K, void* dx, hipStream_t st)
{
    // C = dX [T][K]; contraction over W's rows (N); B(n=k, kc=n) = wq[n][k].
    GemmArgs p{dyq, sdy, wq, sw, static_cast<uint16_t*>(dx), T, K, N, 0, 0};
    if (T <= 64)
        launch_gemm<64, 64, 1, 4, Mode::Dgrad>(p, st);
    else
        launch_gemm<128, 128, 4, 2, Mode::Dgrad>(p, st);
}

void launch_gemm_wgrad(const uint8_t* dyTq, const float* sdyT, const uint8_t* xTq, const float* sxT,
                       int64_t N, int64_t K, int64_t T, void* dw, hipStream_t st)
{
    // C = dW [N][K]; contraction over T.
    GemmArgs p{dyTq, sdyT, xTq, sxT, static_cast<uint16_t*>(dw), N, K, T, 0, 0};
    if (N <= 64)
        launch_gemm<64, 64, 1, 4, Mode::Wgrad>(p, st);
    else if (K % 4 != 0)
        launch_gemm<128, 128, 4, 2, Mode::Wgrad>(p, st);
    else
        launch_gemm_nt<Mode::Wgrad>(p, st);
}

}  // namespace fp8lin
