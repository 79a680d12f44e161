/*
 * fp8lin.h -- C ABI of libfp8lin, the FP8 block-scaled quantized linear layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the Jet-RL technical summary (gist.science, paper
 * 2601.14243):
 *   - section "Quantization scheme": activations are quantized per group of
 *     1x128, weights per block of 128x128; activations kept for the backward
 *     pass are stored in FP8; gradients handed between operators stay BF16;
 *     the backward GEMMs (DGrad and WGrad) run in FP8, WGrad with 1x128 and
 *     128x1 groupings;
 *   - section "Core architecture": rollout and the training forward pass use
 *     one and the same FP8 quantization flow (so both call the functions
 *     below), with BF16 master weights re-quantized from BF16.
 * The pages name the format only as "FP8"; this library fixes it as OCP E4M3FN
 * (max 448), the scale of a group as fp32(amax / 448), codes as
 * E4M3(fp32(x / scale)) with round-to-nearest-even and saturation, fp32
 * accumulation with one scale product per 128-wide contraction group, and
 * BF16 (round-to-nearest-even) GEMM outputs.
 *
 * Conventions for every call:
 *   - All tensors are dense, row-major, on the current HIP device, allocated
 *     and owned by the caller.  No call allocates memory or keeps a caller's
 *     pointer after it returns.  The only mutable global state is per-device
 *     values cached on first use (the architecture check, and the address of
 *     the device array of fp8_gemm_fwd_packed_splitk_noalloc); calls are
 *     thread-safe, apart from that entry point's documented sharing of its
 *     array.
 *   - BF16 tensors are passed as void* (2 bytes per element); FP8 codes as
 *     uint8_t (one E4M3FN code per byte); scales as float.
 *   - "1x128 scales of an [R,C] tensor" are float [R][C/128]; "128x128 scales"
 *     are float [R/128][C/128].  Groups are aligned at index 0.
 *   - The dimension along which 128-groups run must be a multiple of 128;
 *     other dimensions are free (ragged tails are handled).  Sizes are
 *     int64_t and must be >= 0.
 *   - Every base pointer must be 16-byte aligned.  Outputs must not overlap
 *     inputs or each other.  A required pointer may be NULL only when the
 *     call has nothing to read or write.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work and return; there is no host synchronisation.
 *     Buffers must stay valid until the enqueued work has finished.
 *   - Errors: argument errors are detected on the host before anything is
 *     enqueued and the outputs are left untouched.  FP8LIN_ERR_DEVICE means
 *     the current device is not a gfx950 (or there is none).  FP8LIN_ERR_HIP
 *     means a HIP runtime call or launch failed; fp8lin_last_hip_error()
 *     returns that hipError_t for the calling thread.  Nothing aborts or
 *     throws across this boundary.
 *   - An all-zero group gets scale 0 and signed-zero codes (0x00 / 0x80).
 *     Non-finite inputs are outside the contract.
 */
#ifndef FP8LIN_H
#define FP8LIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8LIN_VERSION 1
#define FP8LIN_GROUP 128

typedef enum fp8lin_status {
    FP8LIN_OK = 0,
    FP8LIN_ERR_NULL = 1,   /* a required pointer is NULL                          */
    FP8LIN_ERR_SHAPE = 2,  /* negative size, 128-group dim not a multiple of 128,
                              or a size whose byte count overflows int64          */
    FP8LIN_ERR_ALIGN = 3,  /* a base pointer is not 16-byte aligned              */
    FP8LIN_ERR_ALIAS = 4,  /* an output overlaps an input or another output      */
    FP8LIN_ERR_DEVICE = 5, /* no HIP device, or the current device is not gfx950 */
    FP8LIN_ERR_HIP = 6,    /* a HIP call or kernel launch failed                 */
    FP8LIN_ERR_ARG = 7,    /* an enum argument is out of range, or an option is
                              not available for the chosen source kind           */
    FP8LIN_ERR_SCRATCH = 8 /* the shape needs more than the static device scratch
                              of an allocation-free entry point holds            */
} fp8lin_status;

/* Source kinds of fp8_quant_transpose. */
typedef enum fp8lin_src_kind {
    FP8LIN_SRC_BF16 = 0,     /* src is BF16 [T,C]                                       */
    FP8LIN_SRC_FP8_ROWQ = 1  /* src is E4M3 codes [T,C] with 1x128 scales [T][C/128]:   */
                             /* the FP8 activations saved by the forward pass           */
} fp8lin_src_kind;

/* Library version (FP8LIN_VERSION of the build). */
int fp8lin_version(void);

/* Static, human-readable text for a status value (never NULL). */
const char* fp8lin_status_string(int status);

/* hipError_t behind the calling thread's most recent FP8LIN_ERR_HIP (0 if none). */
int fp8lin_last_hip_error(void);

/*
 * Activation quantization, 1x128 groups (forward, rollout and reference-model
 * activations; also the output gradient dY before DGrad).
 * Jet-RL summary, "Quantization scheme": per-group 1x128 activations.
 *   x   : BF16 [M,K]            (input)
 *   xq  : uint8 E4M3 [M,K]      (output)
 *   sx  : float [M][K/128]      (output) sx[m][g] = fp32(max_{k in g}|x[m,k]| / 448)
 * K % 128 == 0.  M == 0 or K == 0 is an OK no-op.
 * Rows are independent: quantizing any subset of rows gives identical codes
 * and scales, which is what keeps rollout and training on one flow.
 */
fp8lin_status fp8_quant_act(const void* x, int64_t M, int64_t K,
                            uint8_t* xq, float* sx, void* stream);

/*
 * Weight quantization, 128x128 blocks (from the BF16 master weights, once per
 * optimizer step).  Jet-RL summary, "Quantization scheme" (128x128 per-block
 * weights) and "Core architecture" (BF16 master weights).
 *   w   : BF16 [N,K]                (input)
 *   wq  : uint8 E4M3 [N,K]          (output)
 *   sw  : float [N/128][K/128]      (output) one scale per block
 * N % 128 == 0 and K % 128 == 0.  N == 0 or K == 0 is an OK no-op.
 */
fp8lin_status fp8_quant_weight(const void* w, int64_t N, int64_t K,
                               uint8_t* wq, float* sw, void* stream);

/*
 * Transposed copy of a quantized weight, for DGrad (once per optimizer step,
 * next to fp8_quant_weight).  Jet-RL summary, "Quantization scheme" (DGrad
 * in FP8 on the 128x128-quantized weight) and "Implementation" (custom
 * transposition kernels).  A 128x128 block has one scale whichever way it is
 * read, so the copy is exact:
 *   wq  : uint8 [N,K], sw : float [N/128][K/128]   (input, fp8_quant_weight)
 *   wqT : uint8 [K,N], swT : float [K/128][N/128]  (output)
 *   wqT[k][n] = wq[n][k], swT[j][i] = sw[i][j].
 * With it, fp8_gemm_dgrad_t(dyq, sdy, wqT, swT, T, N, K, dx) computes the
 * same sums as fp8_gemm_dgrad(dyq, sdy, wq, sw, T, N, K, dx) (up to fp32
 * summation order) as the forward GEMM on the transposed weight, with both
 * operands contiguous along the contraction.
 * N % 128 == 0 and K % 128 == 0.  N == 0 or K == 0 is an OK no-op.
 */
fp8lin_status fp8_weight_transpose(const uint8_t* wq, const float* sw, int64_t N, int64_t K,
                                   uint8_t* wqT, float* swT, void* stream);

/*
 * Transpose-quantization along tokens, 128x1 groups (WGrad operands).
 * Jet-RL summary, "Quantization scheme" (WGrad uses 1x128 and 128x1
 * quantization) and "Implementation" (custom transposition kernels).
 * For each column c and each run of 128 consecutive rows t, one scale and 128
 * codes are produced and written transposed, so the outputs are the 1x128
 * row-group quantization of the transposed tensor:
 *   kind == FP8LIN_SRC_BF16:
 *     src        : BF16 [T,C];  src_scales must be NULL
 *   kind == FP8LIN_SRC_FP8_ROWQ:
 *     src        : uint8 E4M3 [T,C];  src_scales : float [T][C/128]
 *     values are first dequantized exactly as v = fp32(dec(src) * scale)
 *   dstT  : uint8 E4M3 [C,T]      (output)
 *   sT    : float [C][T/128]      (output)
 *   dst_rowq, s_rowq : optional second output (both NULL, or both set;
 *     BF16 source only): the 1x128 activation quantization of src,
 *     [T,C] codes and [T][C/128] scales, bit-identical to fp8_quant_act on
 *     src, produced from the same read of src.
 * T % 128 == 0.  C % 128 == 0 for the FP8 source and for the dual output;
 * otherwise C >= 0 is free.  T == 0 or C == 0 is an OK no-op.
 * Returns FP8LIN_ERR_ARG for an unknown kind, a FP8 source with dual output
 * or with src_scales == NULL, or a BF16 source with src_scales != NULL.
 */
fp8lin_status fp8_quant_transpose(int kind, const void* src, const float* src_scales,
                                  int64_t T, int64_t C,
                                  uint8_t* dstT, float* sT,
                                  uint8_t* dst_rowq, float* s_rowq, void* stream);

/*
 * Forward / rollout GEMM (NT):  Y = X W^T.
 * Jet-RL summary, "Quantization scheme" and "Core architecture": FP8 GEMM on
 * 1x128-quantized activations and 128x128-quantized weights, identical for
 * rollout and training.
 *   Y[m,n] = sum_g sx[m][g] * sw[n/128][g] * sum_{k in g} dec(xq[m,k]) dec(wq[n,k])
 *   xq : [M,K], sx : [M][K/128], wq : [N,K], sw : [N/128][K/128]
 *   y  : BF16 [M,N] (output), fp32 accumulation, round-to-nearest-even.
 * N % 128 == 0 and K % 128 == 0; M >= 0 is free.  M == 0 or N == 0 is an OK
 * no-op; K == 0 writes zeros.
 */
fp8lin_status fp8_gemm_fwd(const uint8_t* xq, const float* sx,
                           const uint8_t* wq, const float* sw,
                           int64_t M, int64_t N, int64_t K,
                           void* y, void* stream);

/*
 * Decode layout of a quantized weight (once per optimizer step, next to
 * fp8_quant_weight), for rollout GEMMs with at most 64 rows.  Jet-RL
 * summary, "Core architecture" (rollout on the same FP8 weights as
 * training; only the byte order of the codes changes, not a value).
 *   wq  : uint8 [N,K]  (input, fp8_quant_weight's codes)
 *   wqp : uint8, N*K bytes (output): for each 64-row block, each 256-column
 *         chunk and each of the 8 matrix waves of the decode kernel, the 2 KB
 *         that wave multiplies, in the order its lanes load them.
 * The scales are not moved (fp8_gemm_fwd_packed takes fp8_quant_weight's sw).
 * N % 128 == 0 and K % 256 == 0.  N == 0 or K == 0 is an OK no-op.
 */
fp8lin_status fp8_weight_pack(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wqp, void* stream);

/*
 * Forward / rollout GEMM on the decode layout:  Y = X W^T, exactly the sums
 * (and bits) of fp8_gemm_fwd on the unpacked codes, for M <= 64.  Each
 * matrix wave loads its weight fragments with fully coalesced loads straight
 * into registers instead of staging them through LDS.
 *   xq : [M,K], sx : [M][K/128], wqp : fp8_weight_pack of wq [N,K],
 *   sw : [N/128][K/128], y : BF16 [M,N] (output).
 * 0 <= M <= 64, N % 128 == 0, K % 256 == 0 and K <= 16384
 * (FP8LIN_ERR_SHAPE otherwise).  M == 0 or N == 0 is an OK no-op; K == 0
 * writes zeros.
 */
fp8lin_status fp8_gemm_fwd_packed(const uint8_t* xq, const float* sx,
                                  const uint8_t* wqp, const float* sw,
                                  int64_t M, int64_t N, int64_t K,
                                  void* y, void* stream);

/*
 * One forward / rollout linear step from BF16 activations, in one call:
 *   fp8_quant_act(x) -> (xq, sx), then y = fp8_gemm_fwd(xq, sx, wq, sw),
 * enqueued as those two kernels on the stream.
 * Jet-RL summary, "Quantization scheme" and "Core architecture": the
 * activation of a linear layer is quantized 1x128 right before its FP8 GEMM,
 * the same way for rollout and training; xq / sx are also the FP8 copy of the
 * activation that the backward pass keeps.
 *   x    : BF16 [M,K]                              (input)
 *   wq   : uint8 [N,K], sw : float [N/128][K/128]  (input, fp8_quant_weight)
 *   xq   : uint8 [M,K], sx : float [M][K/128]      (output)
 *   y    : BF16 [M,N]                              (output)
 * Outputs are bit-identical to the two separate calls.
 * N % 128 == 0 and K % 128 == 0; M >= 0 is free.  M == 0 is an OK no-op;
 * N == 0 only quantizes; K == 0 writes zeros to y.
 */
fp8lin_status fp8_linear_fwd(const void* x, const uint8_t* wq, const float* sw,
                             int64_t M, int64_t N, int64_t K,
                             uint8_t* xq, float* sx, void* y, void* stream);

/*
 * RMSNorm fused with the 1x128 activation quantization of its output (the
 * operator in front of the attention / MLP input projections).  Jet-RL
 * summary, "Quantization scheme" (FP8 activations saved for the backward pass,
 * produced fused with the previous operator) and "Implementation" (fused
 * RMSNorm kernels).  The pages define no RMSNorm arithmetic; this call fixes
 * it as:
 *   ss[m]   = sum_k x[m,k]^2 in fp64, each 128-group summed as a balanced
 *             binary tree and the group sums added in ascending order;
 *   rstd[m] = fp32(1 / sqrt(ss[m] / K + eps)) (fp64 operations);
 *   y[m,k]  = bf16(fp32(fp32(x[m,k] * rstd[m]) * gamma[k])), round to nearest even;
 * and writes xq, sx = fp8_quant_act(y) without ever storing y.
 *   x     : BF16 [M,K]              (input)
 *   gamma : BF16 [K]                (input)
 *   eps   : finite, >= 0
 *   xq    : uint8 E4M3 [M,K]        (output)
 *   sx    : float [M][K/128]        (output)
 *   rstd  : float [M]               (output, may be NULL; kept for RMSNorm's backward)
 * K % 128 == 0 and K <= 16384 (a row is held in registers), else
 * FP8LIN_ERR_SHAPE; eps negative or not finite: FP8LIN_ERR_ARG.  M == 0 or
 * K == 0 is an OK no-op.  A row with ss / K + eps == 0 (all zeros with
 * eps == 0) is outside the contract.  Rows are independent.
 */
fp8lin_status fp8_rmsnorm_quant(const void* x, const void* gamma, int64_t M, int64_t K, float eps,
                                uint8_t* xq, float* sx, float* rstd, void* stream);

/*
 * Backward of fp8_rmsnorm_quant's RMSNorm, y = x * r * gamma with r = the
 * rstd the forward returned (the rounding of y and its quantization are
 * passed straight through; gradients stay BF16, Jet-RL summary,
 * "Quantization scheme").  With g = gamma * dy and c = sum_i g_i x_i:
 *   dx[m,j]  = bf16(r g_j - x_j (((r r) r) (c / K)))      one rounding
 *   dgamma_k = fp32(sum_t (dy[t,k] x[t,k]) r_t)
 * in fp64; c is summed in fp8_rmsnorm_quant's order for the sum of squares
 * (each 128-group a balanced binary tree, groups ascending); dgamma adds the
 * tokens of each block of 128 rows in ascending order, then the blocks in
 * ascending order.  Every output bit is fixed by these rules.
 *   x, dy  : BF16 [M,K] (input; x the forward's input)
 *   gamma  : BF16 [K];  rstd : float [M] (fp8_rmsnorm_quant's)
 *   dx     : BF16 [M,K] (output)
 *   dgamma : float [K] (output, may be NULL: then no workspace is needed)
 *   workspace : double, fp8_rmsnorm_bwd_workspace(M, K) bytes (ceil(M/128) x K
 *               block sums), caller-owned, contents ignored on entry; calls
 *               sharing it must be ordered on one stream
 * K % 128 == 0 and K <= 16384, else FP8LIN_ERR_SHAPE; workspace_bytes too
 * small: FP8LIN_ERR_ARG.  M == 0 or K == 0 is an OK no-op (dgamma untouched).
 */
int64_t fp8_rmsnorm_bwd_workspace(int64_t M, int64_t K);   /* -1: invalid shape */
fp8lin_status fp8_rmsnorm_bwd(const void* x, const void* gamma, const float* rstd, const void* dy,
                              int64_t M, int64_t K, void* dx, float* dgamma,
                              double* workspace, int64_t workspace_bytes, void* stream);

/*
 * SwiGLU fused with the 1x128 activation quantization of its output (the
 * input of the MLP down projection).  Jet-RL summary, "Quantization scheme"
 * and "Implementation" (fused activation kernels).  The pages define no
 * activation arithmetic; this call fixes it as
 *   h[m,f] = bf16(silu(gate[m,f]) * up[m,f]),  silu(g) = g / (1 + exp(-g)),
 * evaluated in fp64 and rounded once to BF16 (nearest even), and writes
 * hq, sh = fp8_quant_act(h) without ever storing h.
 *   gate, up : BF16, rows of F elements at row stride ld (elements), so they
 *              may be two tensors or the two halves of one [M, 2F] tensor
 *   hq       : uint8 E4M3 [M,F]     (output, dense)
 *   sh       : float [M][F/128]     (output)
 * F % 128 == 0, ld >= F, M * F / 128 < 2^32, else FP8LIN_ERR_SHAPE;
 * ld % 8 != 0 (rows not 16-byte aligned): FP8LIN_ERR_ALIGN.  gate and up
 * may overlap each other, not the outputs.  M == 0 or F == 0 is an OK no-op.
 */
fp8lin_status fp8_swiglu_quant(const void* gate, const void* up, int64_t ld, int64_t M, int64_t F,
                               uint8_t* hq, float* sh, void* stream);

/*
 * Backward of SwiGLU h = silu(gate) * up, BF16 in and out (Jet-RL summary,
 * "Quantization scheme": gradients handed between operators stay BF16; the
 * FP8 quantization of the result for the gate/up DGrad and WGrad GEMMs is
 * fp8_quant_transpose's dual output).  With s = 1 / (1 + exp(-g)):
 *   d_up[m,f]   = bf16(dh * (g * s))
 *   d_gate[m,f] = bf16(((dh * up) * s) * (1 + g * (1 - s)))
 * evaluated in fp64 in that order and rounded once to nearest even.
 *   gate, up : BF16, rows of F elements at row stride ld (e.g. the halves of
 *              the block's saved gate/up output [M, 2F])
 *   dh       : BF16 [M,F] (input, dense)
 *   dgu      : BF16 [M,2F] (output): d_gate in columns [0,F), d_up in [F,2F),
 *              the layout of the fused gate/up projection's output gradient
 * F % 128 == 0 and ld >= F, else FP8LIN_ERR_SHAPE; ld % 8 != 0:
 * FP8LIN_ERR_ALIGN.  M == 0 or F == 0 is an OK no-op.
 */
fp8lin_status fp8_swiglu_bwd(const void* gate, const void* up, int64_t ld, const void* dh,
                             int64_t M, int64_t F, void* dgu, void* stream);

/*
 * SwiGLU backward fused with the FP8 quantization of its result for the
 * gate/up projection's DGrad and WGrad (Jet-RL summary, "Quantization
 * scheme": FP8 backward GEMMs with 1x128 and 128x1 groups; "Implementation":
 * fused activation kernels).  The BF16 gradient dgu = [d_gate | d_up] of
 * fp8_swiglu_bwd is computed tile by tile in registers and never stored;
 * the outputs are bit-identical to fp8_quant_transpose(dgu, dual):
 *   gate, up : BF16, rows of F elements at row stride ld; dh : BF16 [T,F]
 *   dguq  : uint8 [T,2F],  sdgu  : float [T][2F/128]   (1x128 row groups)
 *   dguTq : uint8 [2F,T],  sdguT : float [2F][T/128]   (128-along-T groups, transposed)
 * T % 128 == 0, F % 128 == 0, ld >= F, T / 128 <= 65535, else
 * FP8LIN_ERR_SHAPE; ld % 8 != 0: FP8LIN_ERR_ALIGN.  T == 0 or F == 0 is an
 * OK no-op.
 */
fp8lin_status fp8_swiglu_bwd_quant(const void* gate, const void* up, int64_t ld, const void* dh,
                                   int64_t T, int64_t F, uint8_t* dguq, float* sdgu,
                                   uint8_t* dguTq, float* sdguT, void* stream);

/*
 * Forward pass of an FP8 MLP block (RMSNorm, gate/up projection, SwiGLU,
 * down projection) in one call: the unified FP8 flow of the Jet-RL summary
 * ("Core architecture": rollout and training forward share it; "Quantization
 * scheme": FP8 GEMMs with 1x128 activation and 128x128 weight quantization,
 * FP8 activations saved for the backward pass, produced fused with the
 * operator before each linear layer).  Enqueues, in order:
 *   fp8_rmsnorm_quant(x, gamma, eps)           -> xq, sx, rstd
 *   fp8_gemm_fwd(xq, sx, wgu, sgu)             -> gu  = [gate | up], BF16 [T, 2F]
 *   fp8_swiglu_quant(gu[:, :F], gu[:, F:])     -> hq, sh
 *   fp8_gemm_fwd(hq, sh, wdown, sdown)         -> y, BF16 [T, K]
 * and its outputs are bit-identical to those four calls.
 *   x      : BF16 [T,K] (input);  gamma : BF16 [K];  eps : finite, >= 0
 *   wgu    : uint8 [2F,K], sgu : float [2F/128][K/128]  (rows 0..F-1 gate, F..2F-1 up)
 *   wdown  : uint8 [K,F],  sdown : float [K/128][F/128]
 *   xq, sx, rstd (may be NULL) : as fp8_rmsnorm_quant (saved for the backward pass)
 *   gu     : BF16 [T,2F] (output; kept for SwiGLU's backward)
 *   hq, sh : uint8 [T,F], float [T][F/128] (output; saved FP8 input of the down projection)
 *   y      : BF16 [T,K] (output)
 * K % 128 == 0, K <= 16384, F % 128 == 0, else FP8LIN_ERR_SHAPE; eps as
 * fp8_rmsnorm_quant.  T == 0 or K == 0 is an OK no-op; F == 0 writes y = 0.
 */
fp8lin_status fp8_mlp_fwd(const void* x, const void* gamma, float eps,
                          const uint8_t* wgu, const float* sgu, const uint8_t* wdown, const float* sdown,
                          int64_t T, int64_t K, int64_t F,
                          uint8_t* xq, float* sx, float* rstd, void* gu, uint8_t* hq, float* sh,
                          void* y, void* stream);

/*
 * Rollout GEMM on the decode layout, split over the contraction for weights
 * with few output columns (the MLP down projection and attention projections
 * of a decode step: N / 64 column blocks leave most CUs idle).  Same product,
 * arguments, layouts and limits as fp8_gemm_fwd_packed (Jet-RL summary,
 * "Quantization scheme": 1x128 activations, 128x128 weights), plus a
 * caller-owned device workspace for fp32 partial sums:
 *   workspace       : float, at least fp8_gemm_fwd_packed_splitk_workspace(M, N, K)
 *                     bytes (0: may be NULL), 16-byte aligned, not overlapping
 *                     any argument; its contents on entry are ignored and on
 *                     return are unspecified.  Calls that share a workspace
 *                     must be ordered on one stream.
 * When the weight has at least 128 column blocks (N >= 8192) no split is made
 * and the result is bit-identical to fp8_gemm_fwd_packed; otherwise the S
 * partial products (S workgroups per 64-column block) are added in ascending
 * split order: deterministic, rows independent of the other rows, within the
 * accuracy metric of fp8_gemm_fwd_packed but not bit-identical to it.
 * Errors as fp8_gemm_fwd_packed; workspace_bytes too small: FP8LIN_ERR_ARG.
 */
int64_t fp8_gemm_fwd_packed_splitk_workspace(int64_t M, int64_t N, int64_t K);   /* -1: invalid shape */
fp8lin_status fp8_gemm_fwd_packed_splitk(const uint8_t* xq, const float* sx,
                                         const uint8_t* wqp, const float* sw,
                                         int64_t M, int64_t N, int64_t K, void* y,
                                         float* workspace, int64_t workspace_bytes, void* stream);

/*
 * fp8_gemm_fwd_packed_splitk without a workspace argument, for callers that
 * cannot allocate device memory or hand one in: code under HIP graph capture,
 * tight serving loops, and harnesses that forbid allocation.  It performs no
 * allocation (no hipMalloc, hipFree or allocating library routine): the fp32
 * partial sums live in a device array inside the library, one copy per GPU,
 * FP8LIN_SPLITK_SCRATCH_BYTES long, held until the process ends.
 *   Arguments, layouts, limits and results as fp8_gemm_fwd_packed_splitk
 *   (bit-identical to it for the same inputs).
 *   The caller still passes every input and the output y.
 *   A shape whose split needs more than FP8LIN_SPLITK_SCRATCH_BYTES
 *   (fp8_gemm_fwd_packed_splitk_workspace(M, N, K) above it) returns
 *   FP8LIN_ERR_SCRATCH before anything is enqueued.  The 8B MLP down
 *   projection at 64 tokens (M = 64, N = 4096, K = 14336: 4 MiB) fits.
 *   All calls on one GPU share its array and each leaves its partial sums
 *   there: calls that may overlap on one GPU (different streams, or several
 *   host threads without ordering) race and must not be issued; calls on one
 *   stream are ordered and safe.
 *   The first call on a device looks up that device's array address
 *   (hipGetSymbolAddress, no allocation); a failure there is FP8LIN_ERR_HIP.
 */
#define FP8LIN_SPLITK_SCRATCH_BYTES (4 << 20)
fp8lin_status fp8_gemm_fwd_packed_splitk_noalloc(const uint8_t* xq, const float* sx,
                                                 const uint8_t* wqp, const float* sw,
                                                 int64_t M, int64_t N, int64_t K, void* y,
                                                 void* stream);

/*
 * Forward GEMM with rollout and training on one kernel: the same product as
 * fp8_gemm_fwd (same arguments, layouts, errors), computed for every M by
 * the kernel fp8_gemm_fwd uses above 64 rows (with 64 x 64 tiles for
 * M <= 64, whose every output element runs the same instruction sequence as
 * in the 128 x 128 tiles).  Jet-RL summary, "Core
 * architecture": rollout must run the training forward's quantization flow
 * at the same granularity and precision; this call goes further and makes a
 * row's output bits independent of the batch it is computed in, so a
 * decode-sized rollout call and a prefill/training call give bit-identical
 * rows (fp8_gemm_fwd's decode kernels, used up to 64 rows, sum the groups in
 * another order and agree with it only within the accuracy metric).  It is
 * slower than fp8_gemm_fwd for M <= 64.
 */
fp8lin_status fp8_gemm_fwd_unified(const uint8_t* xq, const float* sx,
                                   const uint8_t* wq, const float* sw,
                                   int64_t M, int64_t N, int64_t K, void* y, void* stream);

/*
 * DGrad GEMM (NN):  dX = dY W, contracted over W's row dimension N.
 * Jet-RL summary, "Quantization scheme": the backward DGrad GEMM runs in FP8.
 *   dX[t,k] = sum_g sdy[t][g] * sw[g][k/128] * sum_{n in g} dec(dyq[t,n]) dec(wq[n,k])
 *   dyq : [T,N], sdy : [T][N/128] (1x128 quantization of dY, fp8_quant_act),
 *   wq : [N,K], sw : [N/128][K/128] (the forward's weight quantization)
 *   dx  : BF16 [T,K] (output).
 * N % 128 == 0 and K % 128 == 0; T >= 0 is free.  T == 0 or K == 0 is an OK
 * no-op; N == 0 writes zeros.
 */
fp8lin_status fp8_gemm_dgrad(const uint8_t* dyq, const float* sdy,
                             const uint8_t* wq, const float* sw,
                             int64_t T, int64_t N, int64_t K,
                             void* dx, void* stream);

/*
 * DGrad on the transposed weight (the fast path):  dX = dY W from
 * fp8_weight_transpose's copy, the same sums as fp8_gemm_dgrad with both
 * operands contiguous along the contraction.
 *   dX[t,k] = sum_g sdy[t][g] * swT[k/128][g] * sum_{n in g} dec(dyq[t,n]) dec(wqT[k,n])
 *   dyq : [T,N], sdy : [T][N/128];  wqT : [K,N], swT : [K/128][N/128]
 *   dx  : BF16 [T,K] (output).
 * Shapes, errors and empty cases as fp8_gemm_dgrad.
 */
fp8lin_status fp8_gemm_dgrad_t(const uint8_t* dyq, const float* sdy,
                               const uint8_t* wqT, const float* swT,
                               int64_t T, int64_t N, int64_t K,
                               void* dx, void* stream);

/*
 * WGrad GEMM (NT over tokens):  dW = dY^T X.
 * Jet-RL summary, "Quantization scheme": WGrad in FP8 with both operands
 * grouped 128-along-tokens, which fp8_quant_transpose produces.
 *   dW[n,k] = sum_g sdyT[n][g] * sxT[k][g] * sum_{t in g} dec(dyTq[n,t]) dec(xTq[k,t])
 *   dyTq : [N,T], sdyT : [N][T/128], xTq : [K,T], sxT : [K][T/128]
 *   dw   : BF16 [N,K] (output).
 * T % 128 == 0; N >= 0 and K >= 0 are free.  N == 0 or K == 0 is an OK no-op;
 * T == 0 writes zeros.
 */
fp8lin_status fp8_gemm_wgrad(const uint8_t* dyTq, const float* sdyT,
                             const uint8_t* xTq, const float* sxT,
                             int64_t N, int64_t K, int64_t T,
                             void* dw, void* stream);

/*
 * 4-bit weights for the rollout GEMM: MXFP4 quantization of BF16 weights
 * (once per optimizer step).  The QeRL page ("QeRL: Beyond Efficiency --
 * Quantization-enhanced Reinforcement Learning for LLMs", abstract) runs the
 * rollout on 4-bit NVFP4 weights without giving the format; it is read here as
 * OCP MX v1.0 MXFP4, the 4-bit format gfx950 converts natively:
 *   w      : BF16 [N,K]                (input)
 *   codes  : uint8 [N][K/2]            (output) E2M1 codes, two per byte, the
 *            even k in the low nibble (sign bit 3, exponent bits 2..1 with
 *            bias 1, mantissa bit 0)
 *   scales : uint8 [N][K/32]           (output) E8M0 = E + 127 per block of 32
 *            consecutive k, E = floor(log2(amax)) - 2 clamped to [-127, 127],
 *            -127 for an all-zero block
 * An element is the E2M1 value nearest to w / 2^E, ties to the even code,
 * magnitudes past 6 saturate to 6, the sign is kept.  Inputs must be finite.
 * K % 32 == 0.  N == 0 or K == 0 is an OK no-op.
 */
fp8lin_status fp8_mxfp4_quant_weight(const void* w, int64_t N, int64_t K,
                                     uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Rollout GEMM on 4-bit weights (NT):  Y = X W^T, with the activations in the
 * flow's FP8 1x128 groups (fp8_quant_act) and W from fp8_mxfp4_quant_weight.
 * The QeRL page ("QeRL: Beyond Efficiency -- Quantization-enhanced
 * Reinforcement Learning for LLMs", abstract): 4-bit weights for the rollout.
 *   Y[m,n] = sum_g sx[m][g] * sum_{k in g} dec(xq[m,k]) * e2m1(w[n,k]) * 2^E[n][k/32]
 *   xq : [M,K], sx : [M][K/128], codes : [N][K/2], scales : [N][K/32]
 *   y  : BF16 [M,N] (output), fp32 accumulation, round-to-nearest-even.
 * The codes are multiplied exactly on the fp16 matrix core; a 32-block more
 * than 2^23 below the largest block of its column's 128-group is rounded in
 * fp16.  Any M (64-row slabs); best for M <= 64.
 * K % 128 == 0 and K <= 16384; M, N >= 0 free.  M == 0 or N == 0 is an OK
 * no-op; K == 0 writes zeros.
 */
fp8lin_status fp8_gemm_fwd_w4(const uint8_t* xq, const float* sx,
                              const uint8_t* codes, const uint8_t* scales,
                              int64_t M, int64_t N, int64_t K,
                              void* y, void* stream);

/*
 * Diagnostics: the device's fp32 -> E4M3 encoder and E4M3 -> fp32 decoder on n
 * values, so that tests can check them against the definition on every input
 * (all 2^32 fp32 bit patterns, all 256 codes).
 *   method 0: the conversion the kernels use;
 *   method 1: the gfx950 hardware conversion instruction
 *             (v_cvt_pk_fp8_f32 / v_cvt_pk_f32_fp8), inputs as given;
 *   method 2: the integer (bit-manipulation) conversion.
 * The encoders round to nearest even; methods 0 and 2 saturate to +-448 and
 * keep the input's sign.  NaN/Inf inputs and the NaN codes give unspecified
 * results.  Buffers are device memory: in/out float [n] and uint8 [n].
 * FP8LIN_ERR_ARG for a method outside 0..2.
 */
fp8lin_status fp8lin_encode_e4m3(const float* in, int64_t n, uint8_t* out, int method, void* stream);
fp8lin_status fp8lin_decode_e4m3(const uint8_t* in, int64_t n, float* out, int method, void* stream);

/*
 * Diagnostic: the fp32 hardware functions that the SwiGLU kernels
 * (fp8_swiglu_quant, fp8_swiglu_bwd, fp8_swiglu_bwd_quant) evaluate the
 * logistic function with, and the division-free functions every quantizer
 * forms its group scale and reciprocal with, applied to each of n values, so
 * that tests can check them on every argument the kernels pass (the SwiGLU
 * kernels re-evaluate in fp64 every result that the first two functions'
 * error could round to a different BF16; the last two must equal the
 * correctly rounded quotient):
 *   fn 0: v_exp_f32, out = 2^in;   fn 1: v_rcp_f32, out = 1 / in;
 *   fn 2: out = fp32(in / 448) for in in [2^-100, 2^128);
 *   fn 3: out = fp32(1 / in) for in in [2^-92, 2^120).
 * Buffers are device memory, float [n] each.  n < 0: FP8LIN_ERR_SHAPE;
 * fn outside 0..3: FP8LIN_ERR_ARG; n == 0 is an OK no-op.
 */
fp8lin_status fp8lin_math_probe(const float* in, int64_t n, float* out, int fn, void* stream);

/*
 * Diagnostic: the test by which the SwiGLU kernels decide to re-evaluate an
 * fp32 result in fp64, applied to each of n values v with one bound lim (in
 * fp32 ulps), so that tests can check it against its definition on every bit
 * pattern: out[i] = 1.0 when a BF16 rounding midpoint lies within lim ulps of
 * v[i] (|low 16 bits of v[i] - 0x8000| <= lim) or |v[i]| is outside
 * [2^-100, 2^101) (NaN included), else 0.0.
 * Buffers are device memory, float [n] each.  n < 0: FP8LIN_ERR_SHAPE;
 * n == 0 is an OK no-op.
 */
fp8lin_status fp8lin_flag_probe(const float* v, int64_t n, float lim, float* out, void* stream);

/*
 * Diagnostic: the forward product of fp8_gemm_fwd (Jet-RL summary,
 * "Quantization scheme": FP8 codes, one scale per 128-wide contraction group
 * from 1x128 activation and 128x128 weight quantization) computed by a plain
 * one-wave-per-tile kernel on a chosen matrix-core instruction, written as
 * fp32 sums, so that tests can record how accurate each instruction is:
 *   form 0: v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 operands, unit scales)
 *   form 1: v_mfma_scale_f32_32x32x64_f8f6f4
 *   form 2: v_mfma_f32_16x16x32_fp8_fp8
 *   form 3: v_mfma_f32_32x32x16_fp8_fp8
 *   form 4: v_mfma_f32_32x32x16_f16 on the codes converted exactly to fp16
 *           (the instruction of the library's GEMMs), as the control.
 * Each 128-group's partial product is one chain of the form's instructions
 * from zero, added into the fp32 sum times sx * sw with one fused
 * multiply-add, groups in ascending order; only the instruction differs
 * between forms.  Not tuned for speed.
 *   xq, sx, wq, sw : as fp8_gemm_fwd;  y : float [M,N] (output)
 * N % 128 == 0, K % 128 == 0, K > 0, M >= 0 (M/16 < 65535), else FP8LIN_ERR_SHAPE;
 * form outside 0..4: FP8LIN_ERR_ARG.  M == 0 or N == 0 is an OK no-op.
 */
fp8lin_status fp8lin_gemm_fwd_mfma_probe(const uint8_t* xq, const float* sx,
                                         const uint8_t* wq, const float* sw,
                                         int64_t M, int64_t N, int64_t K,
                                         float* y, int form, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8LIN_H */
