// fp8lin_api.cpp -- the C ABI of libfp8lin (declared in include/fp8lin.h).
//
// Each entry point validates its arguments on the host (pure checks, no HIP
// call), then checks once per device that it is a gfx950, then enqueues the
// kernels on the caller's stream and returns.  Nothing is allocated.
#include "fp8lin.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "fp8lin_launch.hpp"

static_assert(fp8lin::kSplitkScratchBytes == FP8LIN_SPLITK_SCRATCH_BYTES, "scratch size");

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kGroup = FP8LIN_GROUP;
constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kMaxBlocks = 0x7FFFFFFF;

// ---------------------------------------------------------------- checks

struct Buf {
    const void* p;
    int64_t bytes;
};

// a * b * c with overflow detection (all operands >= 0).
bool mul_ok(int64_t a, int64_t b, int64_t* out)
{
    if (a == 0 || b == 0) {
        *out = 0;
        return true;
    }
    if (a > INT64_MAX / b)
        return false;
    *out = a * b;
    return true;
}

bool bytes_of(int64_t rows, int64_t cols, int64_t elem, int64_t* out)
{
    int64_t n;
    return mul_ok(rows, cols, &n) && mul_ok(n, elem, out);
}

bool overlap(const Buf& x, const Buf& y)
{
    if (x.bytes <= 0 || y.bytes <= 0)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), a1 = a0 + (uintptr_t)x.bytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(y.p), b1 = b0 + (uintptr_t)y.bytes;
    return a0 < b1 && b0 < a1;
}

// NULL / alignment / aliasing of the buffers a call touches.  Buffers with 0
// bytes are not touched and may be anything.
fp8lin_status check_buffers(const Buf* in, int nin, const Buf* out, int nout)
{
    for (int i = 0; i < nin + nout; ++i) {
        const Buf& b = i < nin ? in[i] : out[i - nin];
        if (b.bytes > 0 && b.p == nullptr)
            return FP8LIN_ERR_NULL;
    }
    for (int i = 0; i < nin + nout; ++i) {
        const Buf& b = i < nin ? in[i] : out[i - nin];
        if (b.bytes > 0 && (reinterpret_cast<uintptr_t>(b.p) & 15u) != 0)
            return FP8LIN_ERR_ALIGN;
    }
    for (int o = 0; o < nout; ++o) {
        for (int i = 0; i < nin; ++i)
            if (overlap(out[o], in[i]))
                return FP8LIN_ERR_ALIAS;
        for (int o2 = o + 1; o2 < nout; ++o2)
            if (overlap(out[o], out[o2]))
                return FP8LIN_ERR_ALIAS;
    }
    return FP8LIN_OK;
}

// ----------------------------------------------------------- device check

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

fp8lin_status check_device()
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return FP8LIN_ERR_DEVICE;
    }
    if (dev < kMaxDevices) {
        const int st = g_arch_state[dev].load(std::memory_order_acquire);
        if (st == 1)
            return FP8LIN_OK;
        if (st == 2)
            return FP8LIN_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return FP8LIN_ERR_DEVICE;
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices)
        g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_release);
    return ok ? FP8LIN_OK : FP8LIN_ERR_DEVICE;
}

// Device check, then clear any stale error so the post-launch check sees
// only this call's launches.
fp8lin_status begin_launch()
{
    const fp8lin_status s = check_device();
    if (s != FP8LIN_OK)
        return s;
    (void)hipGetLastError();
    return FP8LIN_OK;
}

fp8lin_status end_launch()
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return FP8LIN_ERR_HIP;
    }
    return FP8LIN_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int fp8lin_version(void) { return FP8LIN_VERSION; }

const char* fp8lin_status_string(int status)
{
    switch (status) {
    case FP8LIN_OK: return "FP8LIN_OK: success";
    case FP8LIN_ERR_NULL: return "FP8LIN_ERR_NULL: a required pointer is NULL";
    case FP8LIN_ERR_SHAPE: return "FP8LIN_ERR_SHAPE: invalid size (negative, 128-group dimension not a multiple of 128, or too large)";
    case FP8LIN_ERR_ALIGN: return "FP8LIN_ERR_ALIGN: a base pointer is not 16-byte aligned";
    case FP8LIN_ERR_ALIAS: return "FP8LIN_ERR_ALIAS: an output overlaps an input or another output";
    case FP8LIN_ERR_DEVICE: return "FP8LIN_ERR_DEVICE: no HIP device, or the current device is not gfx950";
    case FP8LIN_ERR_HIP: return "FP8LIN_ERR_HIP: a HIP call or kernel launch failed";
    case FP8LIN_ERR_ARG: return "FP8LIN_ERR_ARG: invalid argument combination";
    case FP8LIN_ERR_SCRATCH:
        return "FP8LIN_ERR_SCRATCH: the shape needs more scratch than the library's static device buffer "
               "holds (FP8LIN_SPLITK_SCRATCH_BYTES); use the entry point that takes a workspace";
    default: return "FP8LIN: unknown status";
    }
}

int fp8lin_last_hip_error(void) { return g_last_hip_error; }

fp8lin_status fp8_quant_act(const void* x, int64_t M, int64_t K, uint8_t* xq, float* sx, void* stream)
{
    if (M < 0 || K < 0 || K % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    int64_t bx, bq, bs;
    if (!bytes_of(M, K, 2, &bx) || !bytes_of(M, K, 1, &bq) || !bytes_of(M, K / kGroup, 4, &bs))
        return FP8LIN_ERR_SHAPE;
    const Buf in[] = {{x, bx}};
    const Buf out[] = {{xq, bq}, {sx, bs}};
    fp8lin_status s = check_buffers(in, 1, out, 2);
    if (s != FP8LIN_OK)
        return s;
    if (bq == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_quant_rowgroup(x, M * (K / kGroup), xq, sx, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_quant_weight(const void* w, int64_t N, int64_t K, uint8_t* wq, float* sw, void* stream)
{
    if (N < 0 || K < 0 || N % kGroup != 0 || K % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    if (N / kGroup > kMaxGridY)
        return FP8LIN_ERR_SHAPE;
    int64_t bw, bq, bs;
    if (!bytes_of(N, K, 2, &bw) || !bytes_of(N, K, 1, &bq) || !bytes_of(N / kGroup, K / kGroup, 4, &bs))
        return FP8LIN_ERR_SHAPE;
    const Buf in[] = {{w, bw}};
    const Buf out[] = {{wq, bq}, {sw, bs}};
    fp8lin_status s = check_buffers(in, 1, out, 2);
    if (s != FP8LIN_OK)
        return s;
    if (bq == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_quant_block(w, N, K, wq, sw, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_weight_transpose(const uint8_t* wq, const float* sw, int64_t N, int64_t K, uint8_t* wqT,
                                  float* swT, void* stream)
{
    if (N < 0 || K < 0 || N % kGroup != 0 || K % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    if (N / kGroup > kMaxGridY)
        return FP8LIN_ERR_SHAPE;
    int64_t bq, bs;
    if (!bytes_of(N, K, 1, &bq) || !bytes_of(N / kGroup, K / kGroup, 4, &bs))
        return FP8LIN_ERR_SHAPE;
    const Buf in[] = {{wq, bq}, {sw, bs}};
    const Buf out[] = {{wqT, bq}, {swT, bs}};
    fp8lin_status s = check_buffers(in, 2, out, 2);
    if (s != FP8LIN_OK)
        return s;
    if (bq == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_transpose_codes(wq, sw, N, K, wqT, swT, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_quant_transpose(int kind, const void* src, const float* src_scales, int64_t T, int64_t C,
                                  uint8_t* dstT, float* sT, uint8_t* dst_rowq, float* s_rowq, void* stream)
{
    if (kind != FP8LIN_SRC_BF16 && kind != FP8LIN_SRC_FP8_ROWQ)
        return FP8LIN_ERR_ARG;
    const bool dual = dst_rowq != nullptr || s_rowq != nullptr;
    if (dual && (dst_rowq == nullptr || s_rowq == nullptr))
        return FP8LIN_ERR_NULL;
    if (kind == FP8LIN_SRC_FP8_ROWQ && dual)
        return FP8LIN_ERR_ARG;
    if (kind == FP8LIN_SRC_BF16 && src_scales != nullptr)
        return FP8LIN_ERR_ARG;
    if (T < 0 || C < 0 || T % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    if ((kind == FP8LIN_SRC_FP8_ROWQ || dual) && C % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    if (T / kGroup > kMaxGridY || (C + kGroup - 1) / kGroup > kMaxBlocks)
        return FP8LIN_ERR_SHAPE;
    const int64_t elem = kind == FP8LIN_SRC_BF16 ? 2 : 1;
    int64_t bsrc, bss = 0, bq, bs, bqr = 0, bsr = 0;
    if (!bytes_of(T, C, elem, &bsrc) || !bytes_of(T, C, 1, &bq) || !bytes_of(C, T / kGroup, 4, &bs))
        return FP8LIN_ERR_SHAPE;
    if (kind == FP8LIN_SRC_FP8_ROWQ) {
        if (src_scales == nullptr)
            return T * C == 0 ? FP8LIN_OK : FP8LIN_ERR_ARG;
        if (!bytes_of(T, C / kGroup, 4, &bss))
            return FP8LIN_ERR_SHAPE;
    }
    if (dual) {
        bqr = bq;
        if (!bytes_of(T, C / kGroup, 4, &bsr))
            return FP8LIN_ERR_SHAPE;
    }
    const Buf in[] = {{src, bsrc}, {src_scales, bss}};
    const Buf out[] = {{dstT, bq}, {sT, bs}, {dst_rowq, bqr}, {s_rowq, bsr}};
    fp8lin_status s = check_buffers(in, 2, out, 4);
    if (s != FP8LIN_OK)
        return s;
    if (bq == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    if (kind == FP8LIN_SRC_BF16)
        fp8lin::launch_quant_transpose_bf16(src, T, C, dstT, sT, dual ? dst_rowq : nullptr,
                                            dual ? s_rowq : nullptr, as_stream(stream));
    else
        fp8lin::launch_quant_transpose_fp8(static_cast<const uint8_t*>(src), src_scales, T, C, dstT, sT,
                                           as_stream(stream));
    return end_launch();
}

// Shared checks of the three GEMMs.  C = sum over Kc of A [M,Kc] x B.
static fp8lin_status gemm_common(const Buf* in, int64_t M, int64_t N, int64_t Kc, void* c, int64_t* bc)
{
    int64_t tm = (M + 127) / 128, tn = (N + 127) / 128, nb;
    if (!mul_ok(tm, tn, &nb) || nb > kMaxBlocks)
        return FP8LIN_ERR_SHAPE;
    if (!bytes_of(M, N, 2, bc))
        return FP8LIN_ERR_SHAPE;
    (void)Kc;
    const Buf out[] = {{c, *bc}};
    return check_buffers(in, 4, out, 1);
}

fp8lin_status fp8_gemm_fwd(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                           int64_t N, int64_t K, void* y, void* stream)
{
    if (M < 0 || N < 0 || K < 0 || N % kGroup != 0 || K % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    int64_t bx, bsx, bw, bsw, by;
    if (!bytes_of(M, K, 1, &bx) || !bytes_of(M, K / kGroup, 4, &bsx) || !bytes_of(N, K, 1, &bw) ||
        !bytes_of(N / kGroup, K / kGroup, 4, &bsw))
        return FP8LIN_ERR_SHAPE;
    if (M == 0 || N == 0)
        bx = bsx = bw = bsw = 0;
    const Buf in[] = {{xq, bx}, {sx, bsx}, {wq, bw}, {sw, bsw}};
    fp8lin_status s = gemm_common(in, M, N, K, y, &by);
    if (s != FP8LIN_OK)
        return s;
    if (by == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    if (K == 0)
        fp8lin::launch_fill_zero_bf16(y, M * N, as_stream(stream));
    else
        fp8lin::launch_gemm_fwd(xq, sx, wq, sw, M, N, K, y, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_mxfp4_quant_weight(const void* w, int64_t N, int64_t K, uint8_t* codes, uint8_t* scales,
                                     void* stream)
{
    if (N < 0 || K < 0 || K % 32 != 0)
        return FP8LIN_ERR_SHAPE;
    int64_t bw, bc, bs, nb;
    if (!bytes_of(N, K, 2, &bw) || !bytes_of(N, K / 2, 1, &bc) || !bytes_of(N, K / 32, 1, &bs))
        return FP8LIN_ERR_SHAPE;
    if (!mul_ok(N, K / 8, &nb) || (nb + 255) / 256 > kMaxBlocks)     // four threads per 32-block
        return FP8LIN_ERR_SHAPE;
    const Buf in[] = {{w, bw}};
    const Buf out[] = {{codes, bc}, {scales, bs}};
    fp8lin_status s = check_buffers(in, 1, out, 2);
    if (s != FP8LIN_OK)
        return s;
    if (bc == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_mxfp4_quant(w, N, K, codes, scales, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_gemm_fwd_w4(const uint8_t* xq, const float* sx, const uint8_t* codes, const uint8_t* scales,
                              int64_t M, int64_t N, int64_t K, void* y, void* stream)
{
    if (M < 0 || N < 0 || K < 0 || K % kGroup != 0 || K > fp8lin::gemm_w4_max_k())
        return FP8LIN_ERR_SHAPE;
    if ((M + 63) / 64 > kMaxGridY || (N + 63) / 64 > kMaxBlocks)
        return FP8LIN_ERR_SHAPE;
    int64_t bx, bsx, bc, bs, by;
    if (!bytes_of(M, K, 1, &bx) || !bytes_of(M, K / kGroup, 4, &bsx) || !bytes_of(N, K / 2, 1, &bc) ||
        !bytes_of(N, K / 32, 1, &bs) || !bytes_of(M, N, 2, &by))
        return FP8LIN_ERR_SHAPE;
    if (M == 0 || N == 0)
        bx = bsx = bc = bs = 0;
    const Buf in[] = {{xq, bx}, {sx, bsx}, {codes, bc}, {scales, bs}};
    const Buf out[] = {{y, by}};
    fp8lin_status s = check_buffers(in, 4, out, 1);
    if (s != FP8LIN_OK)
        return s;
    if (by == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    if (K == 0)
        fp8lin::launch_fill_zero_bf16(y, M * N, as_stream(stream));
    else
        fp8lin::launch_gemm_fwd_w4(xq, sx, codes, scales, M, N, K, y, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_gemm_fwd_unified(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                   int64_t M, int64_t N, int64_t K, void* y, void* stream)
{
    if (M < 0 || N < 0 || K < 0 || N % kGroup != 0 || K % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    int64_t bx, bsx, bw, bsw, by;
    if (!bytes_of(M, K, 1, &bx) || !bytes_of(M, K / kGroup, 4, &bsx) || !bytes_of(N, K, 1, &bw) ||
        !bytes_of(N / kGroup, K / kGroup, 4, &bsw))
        return FP8LIN_ERR_SHAPE;
    if (M == 0 || N == 0)
        bx = bsx = bw = bsw = 0;
    const Buf in[] = {{xq, bx}, {sx, bsx}, {wq, bw}, {sw, bsw}};
    fp8lin_status s = gemm_common(in, M, N, K, y, &by);
    if (s != FP8LIN_OK)
        return s;
    if (by == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    if (K == 0)
        fp8lin::launch_fill_zero_bf16(y, M * N, as_stream(stream));
    else
        fp8lin::launch_gemm_fwd_unified(xq, sx, wq, sw, M, N, K, y, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_weight_pack(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wqp, void* stream)
{
    if (N < 0 || K < 0 || N % kGroup != 0 || K % (2 * kGroup) != 0)
        return FP8LIN_ERR_SHAPE;
    int64_t bq;
    if (!bytes_of(N, K, 1, &bq))
        return FP8LIN_ERR_SHAPE;
    const Buf in[] = {{wq, bq}};
    const Buf out[] = {{wqp, bq}};
    fp8lin_status s = check_buffers(in, 1, out, 1);
    if (s != FP8LIN_OK)
        return s;
    if (bq == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_pack_decode(wq, N, K, wqp, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_gemm_fwd_packed(const uint8_t* xq, const float* sx, const uint8_t* wqp, const float* sw,
                                  int64_t M, int64_t N, int64_t K, void* y, void* stream)
{
    if (M < 0 || M > 64 || N < 0 || K < 0 || N % kGroup != 0 || K % (2 * kGroup) != 0 || K > 128 * kGroup)
        return FP8LIN_ERR_SHAPE;
    int64_t bx, bsx, bw, bsw, by;
    if (!bytes_of(M, K, 1, &bx) || !bytes_of(M, K / kGroup, 4, &bsx) || !bytes_of(N, K, 1, &bw) ||
        !bytes_of(N / kGroup, K / kGroup, 4, &bsw))
        return FP8LIN_ERR_SHAPE;
    if (M == 0 || N == 0)
        bx = bsx = bw = bsw = 0;
    const Buf in[] = {{xq, bx}, {sx, bsx}, {wqp, bw}, {sw, bsw}};
    fp8lin_status s = gemm_common(in, M, N, K, y, &by);
    if (s != FP8LIN_OK)
        return s;
    if (by == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    if (K == 0)
        fp8lin::launch_fill_zero_bf16(y, M * N, as_stream(stream));
    else
        fp8lin::launch_gemm_fwd_packed(xq, sx, wqp, sw, M, N, K, y, as_stream(stream));
    return end_launch();
}

int64_t fp8_gemm_fwd_packed_splitk_workspace(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || M > 64 || N < 0 || K < 0 || N % kGroup != 0 || K % (2 * kGroup) != 0 || K > 128 * kGroup)
        return -1;
    if (M == 0 || N == 0 || K == 0)
        return 0;
    const int64_t S = fp8lin::splitk_splits(N, K);
    return S > 1 ? S * M * N * 4 : 0;
}

fp8lin_status fp8_gemm_fwd_packed_splitk(const uint8_t* xq, const float* sx, const uint8_t* wqp, const float* sw,
                                         int64_t M, int64_t N, int64_t K, void* y, float* workspace,
                                         int64_t workspace_bytes, void* stream)
{
    const int64_t need = fp8_gemm_fwd_packed_splitk_workspace(M, N, K);
    if (need < 0)
        return FP8LIN_ERR_SHAPE;
    if (workspace_bytes < need)
        return FP8LIN_ERR_ARG;
    int64_t bx, bsx, bw, bsw, by;
    if (!bytes_of(M, K, 1, &bx) || !bytes_of(M, K / kGroup, 4, &bsx) || !bytes_of(N, K, 1, &bw) ||
        !bytes_of(N / kGroup, K / kGroup, 4, &bsw) || !bytes_of(M, N, 2, &by))
        return FP8LIN_ERR_SHAPE;
    if (M == 0 || N == 0)
        bx = bsx = bw = bsw = 0;
    const Buf in[] = {{xq, bx}, {sx, bsx}, {wqp, bw}, {sw, bsw}};
    const Buf out[] = {{y, by}, {workspace, need}};
    fp8lin_status s = check_buffers(in, 4, out, 2);
    if (s != FP8LIN_OK)
        return s;
    if (by == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    if (K == 0)
        fp8lin::launch_fill_zero_bf16(y, M * N, as_stream(stream));
    else
        fp8lin::launch_gemm_fwd_packed_splitk(xq, sx, wqp, sw, M, N, K, y, workspace, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_gemm_fwd_packed_splitk_noalloc(const uint8_t* xq, const float* sx, const uint8_t* wqp,
                                                 const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                                                 void* stream)
{
    const int64_t need = fp8_gemm_fwd_packed_splitk_workspace(M, N, K);
    if (need < 0)
        return FP8LIN_ERR_SHAPE;
    if (need > FP8LIN_SPLITK_SCRATCH_BYTES)
        return FP8LIN_ERR_SCRATCH;
    int64_t bx, bsx, bw, bsw, by;
    if (!bytes_of(M, K, 1, &bx) || !bytes_of(M, K / kGroup, 4, &bsx) || !bytes_of(N, K, 1, &bw) ||
        !bytes_of(N / kGroup, K / kGroup, 4, &bsw) || !bytes_of(M, N, 2, &by))
        return FP8LIN_ERR_SHAPE;
    if (M == 0 || N == 0)
        bx = bsx = bw = bsw = 0;
    const Buf in[] = {{xq, bx}, {sx, bsx}, {wqp, bw}, {sw, bsw}};
    const Buf out[] = {{y, by}};
    fp8lin_status s = check_buffers(in, 4, out, 1);
    if (s != FP8LIN_OK)
        return s;
    if (by == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = fp8lin::splitk_scratch(&ws);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            g_last_hip_error = (int)e;
            return FP8LIN_ERR_HIP;
        }
    }
    if (K == 0)
        fp8lin::launch_fill_zero_bf16(y, M * N, as_stream(stream));
    else
        fp8lin::launch_gemm_fwd_packed_splitk(xq, sx, wqp, sw, M, N, K, y, static_cast<float*>(ws),
                                              as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_linear_fwd(const void* x, const uint8_t* wq, const float* sw, int64_t M, int64_t N, int64_t K,
                             uint8_t* xq, float* sx, void* y, void* stream)
{
    if (M < 0 || N < 0 || K < 0 || N % kGroup != 0 || K % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    int64_t bx, bq, bsx, bw, bsw, by;
    if (!bytes_of(M, K, 2, &bx) || !bytes_of(M, K, 1, &bq) || !bytes_of(M, K / kGroup, 4, &bsx) ||
        !bytes_of(N, K, 1, &bw) || !bytes_of(N / kGroup, K / kGroup, 4, &bsw) || !bytes_of(M, N, 2, &by))
        return FP8LIN_ERR_SHAPE;
    int64_t tm = (M + 127) / 128, tn = (N + 127) / 128, nb;
    if (!mul_ok(tm, tn, &nb) || nb > kMaxBlocks)
        return FP8LIN_ERR_SHAPE;
    if (by == 0)
        bw = bsw = 0;
    const Buf in[] = {{x, bx}, {wq, bw}, {sw, bsw}};
    const Buf out[] = {{xq, bq}, {sx, bsx}, {y, by}};
    fp8lin_status s = check_buffers(in, 3, out, 3);
    if (s != FP8LIN_OK)
        return s;
    if (bq == 0 && by == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    const hipStream_t st = as_stream(stream);
    if (bq > 0)
        fp8lin::launch_quant_rowgroup(x, M * (K / kGroup), xq, sx, st);
    if (by > 0) {
        if (K == 0)
            fp8lin::launch_fill_zero_bf16(y, M * N, st);
        else
            fp8lin::launch_gemm_fwd(xq, sx, wq, sw, M, N, K, y, st);
    }
    return end_launch();
}

fp8lin_status fp8_rmsnorm_quant(const void* x, const void* gamma, int64_t M, int64_t K, float eps,
                                uint8_t* xq, float* sx, float* rstd, void* stream)
{
    if (M < 0 || K < 0 || K % kGroup != 0 || K > 16384 || (M + 3) / 4 > kMaxBlocks)
        return FP8LIN_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 3.4028234663852886e38f)
        return FP8LIN_ERR_ARG;
    int64_t bx, bq, bs, br, bg;
    if (!bytes_of(M, K, 2, &bx) || !bytes_of(M, K, 1, &bq) || !bytes_of(M, K / kGroup, 4, &bs) ||
        !bytes_of(M, 1, 4, &br) || !bytes_of(K, 1, 2, &bg))
        return FP8LIN_ERR_SHAPE;
    if (bq == 0)
        bg = br = 0;
    const Buf in[] = {{x, bx}, {gamma, bg}};
    const Buf out[] = {{xq, bq}, {sx, bs}, {rstd, rstd ? br : 0}};
    fp8lin_status s = check_buffers(in, 2, out, 3);
    if (s != FP8LIN_OK)
        return s;
    if (bq == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_rmsnorm_quant(x, gamma, M, K, eps, xq, sx, rstd, as_stream(stream));
    return end_launch();
}

int64_t fp8_rmsnorm_bwd_workspace(int64_t M, int64_t K)
{
    if (M < 0 || K < 0 || K % kGroup != 0 || K > 16384)
        return -1;
    int64_t b;
    if (!bytes_of((M + kGroup - 1) / kGroup, K, 8, &b))
        return -1;
    return b;
}

fp8lin_status fp8_rmsnorm_bwd(const void* x, const void* gamma, const float* rstd, const void* dy, int64_t M,
                              int64_t K, void* dx, float* dgamma, double* workspace, int64_t workspace_bytes,
                              void* stream)
{
    const int64_t need = fp8_rmsnorm_bwd_workspace(M, K);
    if (need < 0 || M > kMaxBlocks || (M + kGroup - 1) / kGroup > kMaxGridY)
        return FP8LIN_ERR_SHAPE;
    const int64_t wneed = dgamma ? need : 0;
    if (workspace_bytes < wneed)
        return FP8LIN_ERR_ARG;
    int64_t bx, bg, br, bdg;
    if (!bytes_of(M, K, 2, &bx) || !bytes_of(K, 1, 2, &bg) || !bytes_of(M, 1, 4, &br) || !bytes_of(K, 1, 4, &bdg))
        return FP8LIN_ERR_SHAPE;
    if (bx == 0)
        return FP8LIN_OK;
    const Buf in[] = {{x, bx}, {gamma, bg}, {rstd, br}, {dy, bx}};
    const Buf out[] = {{dx, bx}, {dgamma, dgamma ? bdg : 0}, {workspace, wneed}};
    fp8lin_status s = check_buffers(in, 4, out, 3);
    if (s != FP8LIN_OK)
        return s;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_rmsnorm_bwd(x, gamma, rstd, dy, M, K, dx, dgamma, workspace, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_swiglu_quant(const void* gate, const void* up, int64_t ld, int64_t M, int64_t F,
                               uint8_t* hq, float* sh, void* stream)
{
    if (M < 0 || F < 0 || F % kGroup != 0 || ld < F)
        return FP8LIN_ERR_SHAPE;
    int64_t bq, bs, ng, span;
    if (!bytes_of(M, F, 1, &bq) || !bytes_of(M, F / kGroup, 4, &bs) || !mul_ok(M, F / kGroup, &ng) ||
        ng >= ((int64_t)1 << 32))
        return FP8LIN_ERR_SHAPE;
    if (bq == 0)
        return FP8LIN_OK;
    if (!mul_ok(M - 1, ld, &span) || span > INT64_MAX / 2 - F)
        return FP8LIN_ERR_SHAPE;
    const int64_t bin = (span + F) * 2;
    if (ld % 8 != 0)
        return FP8LIN_ERR_ALIGN;
    const Buf in[] = {{gate, bin}, {up, bin}};
    const Buf out[] = {{hq, bq}, {sh, bs}};
    fp8lin_status s = check_buffers(in, 2, out, 2);
    if (s != FP8LIN_OK)
        return s;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_swiglu_quant(gate, up, ld, M, F, hq, sh, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_swiglu_bwd(const void* gate, const void* up, int64_t ld, const void* dh, int64_t M, int64_t F,
                             void* dgu, void* stream)
{
    if (M < 0 || F < 0 || F % kGroup != 0 || ld < F)
        return FP8LIN_ERR_SHAPE;
    int64_t bdh, bout, span;
    if (!bytes_of(M, F, 2, &bdh) || !bytes_of(M, 2 * F, 2, &bout))
        return FP8LIN_ERR_SHAPE;
    if (bdh == 0)
        return FP8LIN_OK;
    if (!mul_ok(M - 1, ld, &span) || span > INT64_MAX / 2 - F)
        return FP8LIN_ERR_SHAPE;
    const int64_t bin = (span + F) * 2;
    if (ld % 8 != 0)
        return FP8LIN_ERR_ALIGN;
    const Buf in[] = {{gate, bin}, {up, bin}, {dh, bdh}};
    const Buf out[] = {{dgu, bout}};
    fp8lin_status s = check_buffers(in, 3, out, 1);
    if (s != FP8LIN_OK)
        return s;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_swiglu_bwd(gate, up, ld, dh, M, F, dgu, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_swiglu_bwd_quant(const void* gate, const void* up, int64_t ld, const void* dh, int64_t T, int64_t F,
                                   uint8_t* dguq, float* sdgu, uint8_t* dguTq, float* sdguT, void* stream)
{
    if (T < 0 || F < 0 || T % kGroup != 0 || F % kGroup != 0 || ld < F || T / kGroup > kMaxGridY)
        return FP8LIN_ERR_SHAPE;
    int64_t F2, bdh, bq, bs, bsT, span;
    if (!mul_ok(F, 2, &F2) || !bytes_of(T, F, 2, &bdh) || !bytes_of(T, F2, 1, &bq) ||
        !bytes_of(T, F2 / kGroup, 4, &bs) || !bytes_of(F2, T / kGroup, 4, &bsT))
        return FP8LIN_ERR_SHAPE;
    if (bq == 0)
        return FP8LIN_OK;
    if (!mul_ok(T - 1, ld, &span) || span > INT64_MAX / 2 - F)
        return FP8LIN_ERR_SHAPE;
    const int64_t bin = (span + F) * 2;
    if (ld % 8 != 0)
        return FP8LIN_ERR_ALIGN;
    const Buf in[] = {{gate, bin}, {up, bin}, {dh, bdh}};
    const Buf out[] = {{dguq, bq}, {sdgu, bs}, {dguTq, bq}, {sdguT, bsT}};
    fp8lin_status s = check_buffers(in, 3, out, 4);
    if (s != FP8LIN_OK)
        return s;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_swiglu_bwd_quant(gate, up, ld, dh, T, F, dguq, sdgu, dguTq, sdguT, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_mlp_fwd(const void* x, const void* gamma, float eps, const uint8_t* wgu, const float* sgu,
                          const uint8_t* wdown, const float* sdown, int64_t T, int64_t K, int64_t F, uint8_t* xq,
                          float* sx, float* rstd, void* gu, uint8_t* hq, float* sh, void* y, void* stream)
{
    if (T < 0 || K < 0 || F < 0 || K % kGroup != 0 || F % kGroup != 0 || K > 16384 || (T + 3) / 4 > kMaxBlocks)
        return FP8LIN_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 3.4028234663852886e38f)
        return FP8LIN_ERR_ARG;
    int64_t F2, bx, bg, bxq, bsx, br, bwgu, bsgu, bwd, bsd, bgu, bhq, bsh, by, ng, nb1, nb2;
    if (!mul_ok(F, 2, &F2) || !bytes_of(T, K, 2, &bx) || !bytes_of(K, 1, 2, &bg) || !bytes_of(T, K, 1, &bxq) ||
        !bytes_of(T, K / kGroup, 4, &bsx) || !bytes_of(T, 1, 4, &br) || !bytes_of(F2, K, 1, &bwgu) ||
        !bytes_of(F2 / kGroup, K / kGroup, 4, &bsgu) || !bytes_of(K, F, 1, &bwd) ||
        !bytes_of(K / kGroup, F / kGroup, 4, &bsd) || !bytes_of(T, F2, 2, &bgu) || !bytes_of(T, F, 1, &bhq) ||
        !bytes_of(T, F / kGroup, 4, &bsh) || !bytes_of(T, K, 2, &by) || !mul_ok(T, F / kGroup, &ng) ||
        ng >= ((int64_t)1 << 32) || !mul_ok((T + 127) / 128, (F2 + 127) / 128, &nb1) || nb1 > kMaxBlocks ||
        !mul_ok((T + 127) / 128, (K + 127) / 128, &nb2) || nb2 > kMaxBlocks)
        return FP8LIN_ERR_SHAPE;
    if (T == 0 || K == 0 || F == 0) {
        // nothing to compute except y = 0 when the intermediate width is 0
        if (T == 0 || K == 0)
            return FP8LIN_OK;
        const Buf in0[] = {{x, bx}};
        const Buf out0[] = {{y, by}};
        fp8lin_status s0 = check_buffers(in0, 1, out0, 1);
        if (s0 != FP8LIN_OK)
            return s0;
        if ((s0 = begin_launch()) != FP8LIN_OK)
            return s0;
        fp8lin::launch_fill_zero_bf16(y, T * K, as_stream(stream));
        return end_launch();
    }
    const Buf in[] = {{x, bx}, {gamma, bg}, {wgu, bwgu}, {sgu, bsgu}, {wdown, bwd}, {sdown, bsd}};
    const Buf out[] = {{xq, bxq}, {sx, bsx}, {rstd, rstd ? br : 0}, {gu, bgu}, {hq, bhq}, {sh, bsh}, {y, by}};
    fp8lin_status s = check_buffers(in, 6, out, 7);
    if (s != FP8LIN_OK)
        return s;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    const hipStream_t st = as_stream(stream);
    const uint16_t* gup = static_cast<const uint16_t*>(gu);
    fp8lin::launch_rmsnorm_quant(x, gamma, T, K, eps, xq, sx, rstd, st);
    fp8lin::launch_gemm_fwd(xq, sx, wgu, sgu, T, F2, K, gu, st);
    fp8lin::launch_swiglu_quant(gup, gup + F, F2, T, F, hq, sh, st);
    fp8lin::launch_gemm_fwd(hq, sh, wdown, sdown, T, K, F, y, st);
    return end_launch();
}

fp8lin_status fp8_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw, int64_t T,
                             int64_t N, int64_t K, void* dx, void* stream)
{
    if (T < 0 || N < 0 || K < 0 || N % kGroup != 0 || K % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    int64_t bdy, bsdy, bw, bsw, bdx;
    if (!bytes_of(T, N, 1, &bdy) || !bytes_of(T, N / kGroup, 4, &bsdy) || !bytes_of(N, K, 1, &bw) ||
        !bytes_of(N / kGroup, K / kGroup, 4, &bsw))
        return FP8LIN_ERR_SHAPE;
    if (T == 0 || K == 0)
        bdy = bsdy = bw = bsw = 0;
    const Buf in[] = {{dyq, bdy}, {sdy, bsdy}, {wq, bw}, {sw, bsw}};
    fp8lin_status s = gemm_common(in, T, K, N, dx, &bdx);
    if (s != FP8LIN_OK)
        return s;
    if (bdx == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    if (N == 0)
        fp8lin::launch_fill_zero_bf16(dx, T * K, as_stream(stream));
    else
        fp8lin::launch_gemm_dgrad(dyq, sdy, wq, sw, T, N, K, dx, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8_gemm_dgrad_t(const uint8_t* dyq, const float* sdy, const uint8_t* wqT, const float* swT,
                               int64_t T, int64_t N, int64_t K, void* dx, void* stream)
{
    // the forward product of dY [T,N] with the rows of W^T [K,N]
    return fp8_gemm_fwd(dyq, sdy, wqT, swT, T, K, N, dx, stream);
}

fp8lin_status fp8_gemm_wgrad(const uint8_t* dyTq, const float* sdyT, const uint8_t* xTq, const float* sxT,
                             int64_t N, int64_t K, int64_t T, void* dw, void* stream)
{
    if (N < 0 || K < 0 || T < 0 || T % kGroup != 0)
        return FP8LIN_ERR_SHAPE;
    int64_t bdy, bsdy, bx, bsx, bdw;
    if (!bytes_of(N, T, 1, &bdy) || !bytes_of(N, T / kGroup, 4, &bsdy) || !bytes_of(K, T, 1, &bx) ||
        !bytes_of(K, T / kGroup, 4, &bsx))
        return FP8LIN_ERR_SHAPE;
    if (N == 0 || K == 0)
        bdy = bsdy = bx = bsx = 0;
    const Buf in[] = {{dyTq, bdy}, {sdyT, bsdy}, {xTq, bx}, {sxT, bsx}};
    fp8lin_status s = gemm_common(in, N, K, T, dw, &bdw);
    if (s != FP8LIN_OK)
        return s;
    if (bdw == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    if (T == 0)
        fp8lin::launch_fill_zero_bf16(dw, N * K, as_stream(stream));
    else
        fp8lin::launch_gemm_wgrad(dyTq, sdyT, xTq, sxT, N, K, T, dw, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8lin_encode_e4m3(const float* in, int64_t n, uint8_t* out, int method, void* stream)
{
    if (n < 0)
        return FP8LIN_ERR_SHAPE;
    if (method < 0 || method > 2)
        return FP8LIN_ERR_ARG;
    int64_t bi;
    if (!mul_ok(n, 4, &bi) || n / 1024 + 1 > kMaxBlocks)
        return FP8LIN_ERR_SHAPE;
    const Buf ib[] = {{in, bi}};
    const Buf ob[] = {{out, n}};
    fp8lin_status s = check_buffers(ib, 1, ob, 1);
    if (s != FP8LIN_OK)
        return s;
    if (n == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_encode_probe(in, n, out, method, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8lin_gemm_fwd_mfma_probe(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                         int64_t M, int64_t N, int64_t K, float* y, int form, void* stream)
{
    if (M < 0 || N < 0 || K <= 0 || N % kGroup != 0 || K % kGroup != 0 || M / 16 >= kMaxGridY)
        return FP8LIN_ERR_SHAPE;
    if (form < 0 || form > 4)
        return FP8LIN_ERR_ARG;
    int64_t bx, bsx, bw, bsw, by;
    if (!bytes_of(M, K, 1, &bx) || !bytes_of(M, K / kGroup, 4, &bsx) || !bytes_of(N, K, 1, &bw) ||
        !bytes_of(N / kGroup, K / kGroup, 4, &bsw) || !bytes_of(M, N, 4, &by))
        return FP8LIN_ERR_SHAPE;
    if (M == 0 || N == 0)
        return FP8LIN_OK;
    const Buf in[] = {{xq, bx}, {sx, bsx}, {wq, bw}, {sw, bsw}};
    const Buf out[] = {{y, by}};
    fp8lin_status s = check_buffers(in, 4, out, 1);
    if (s != FP8LIN_OK)
        return s;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_gemm_fwd_mfma_probe(xq, sx, wq, sw, M, N, K, y, form, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8lin_math_probe(const float* in, int64_t n, float* out, int fn, void* stream)
{
    if (n < 0)
        return FP8LIN_ERR_SHAPE;
    if (fn < 0 || fn > 3)
        return FP8LIN_ERR_ARG;
    int64_t b;
    if (!mul_ok(n, 4, &b))
        return FP8LIN_ERR_SHAPE;
    const Buf ib[] = {{in, b}};
    const Buf ob[] = {{out, b}};
    fp8lin_status s = check_buffers(ib, 1, ob, 1);
    if (s != FP8LIN_OK)
        return s;
    if (n == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_math_probe(in, n, out, fn, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8lin_flag_probe(const float* v, int64_t n, float lim, float* out, void* stream)
{
    if (n < 0)
        return FP8LIN_ERR_SHAPE;
    int64_t b;
    if (!mul_ok(n, 4, &b))
        return FP8LIN_ERR_SHAPE;
    const Buf ib[] = {{v, b}};
    const Buf ob[] = {{out, b}};
    fp8lin_status s = check_buffers(ib, 1, ob, 1);
    if (s != FP8LIN_OK)
        return s;
    if (n == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_flag_probe(v, n, lim, out, as_stream(stream));
    return end_launch();
}

fp8lin_status fp8lin_decode_e4m3(const uint8_t* in, int64_t n, float* out, int method, void* stream)
{
    if (n < 0)
        return FP8LIN_ERR_SHAPE;
    if (method < 0 || method > 2)
        return FP8LIN_ERR_ARG;
    int64_t bo;
    if (!mul_ok(n, 4, &bo) || n / 1024 + 1 > kMaxBlocks)
        return FP8LIN_ERR_SHAPE;
    const Buf ib[] = {{in, n}};
    const Buf ob[] = {{out, bo}};
    fp8lin_status s = check_buffers(ib, 1, ob, 1);
    if (s != FP8LIN_OK)
        return s;
    if (n == 0)
        return FP8LIN_OK;
    if ((s = begin_launch()) != FP8LIN_OK)
        return s;
    fp8lin::launch_decode_probe(in, n, out, method, as_stream(stream));
    return end_launch();
}

}  // extern "C"
