/*
 * libfp8rl: fine-grained FP8 (E4M3) quantization and block-scaled FP8 GEMMs for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages describing the method), cited by title and section:
 *   [SkyRL-FP8] "Anyscale、SkyRL で FP8 学習・ロールアウトをサポートし一貫性を維持"
 *               (news.ainew.jp translation of the Anyscale/SkyRL FP8 article)
 *   [AIS]       "AIS: Adaptive Importance Sampling for Quantized RL" (kasblo.com explainer)
 *   [Jet-RL]    "Jet-RL: Enabling On-Policy FP8 Reinforcement Learning with Unified
 *               Training and Rollout Precision Flow" (gist.science summary)
 *
 * Conventions for every entry point:
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library keeps no
 *     pointer after returning and allocates no memory.
 *   - Tensors are row-major and contiguous. bf16 tensors are passed as uint16_t bit
 *     patterns. FP8 payloads are E4M3 "FN" bytes (bias 7, max 448, NaN 0x7F/0xFF).
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the legacy default
 *     stream). No synchronization, no host<->device copies; group offsets are read on the
 *     device.
 *   - All arguments are validated before any HIP call is made. Invalid arguments return a
 *     status code and enqueue nothing. A call whose work is empty (a zero-sized dimension)
 *     returns FP8RL_OK without touching the device.
 *   - Data pointers must be 16-byte aligned (FP8RL_ERR_ALIGN otherwise); scale pointers
 *     4-byte aligned (fp32) or 1-byte (E8M0).
 *   - Sizes: every matrix holds at most 2^40 elements, and a GEMM's reduction length (K for
 *     the forward and grouped GEMMs, N for DGrad, the token count M for WGrad) is at most
 *     2^23 (FP8RL_ERR_SHAPE otherwise).
 *   - FP8RL_ERR_DEVICE: the current device is not gfx950. FP8RL_ERR_LAUNCH: the kernel
 *     launch was rejected by the runtime. Faults inside a kernel surface at the caller's
 *     next synchronization with the stream, as for any HIP kernel.
 *   - Results are deterministic: no atomics, a fixed reduction order, and the same bytes
 *     from run to run and across output modes.
 *   - Calls that share no output buffer may run concurrently on different streams.
 */
#ifndef FP8RL_H
#define FP8RL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8RL_OK = 0,
  FP8RL_ERR_NULL = 1,      /* a required pointer is NULL, or an optional output pair is half given */
  FP8RL_ERR_SHAPE = 2,     /* a dimension is negative or breaks the granularity rules of the call */
  FP8RL_ERR_ALIGN = 3,     /* a pointer is not suitably aligned */
  FP8RL_ERR_RECIPE = 4,    /* unknown / unsupported recipe or dtype, or install descriptors disagree */
  FP8RL_ERR_DEVICE = 5,    /* current HIP device is not gfx950, or it could not be queried */
  FP8RL_ERR_LAUNCH = 6,    /* kernel launch failed */
  FP8RL_ERR_WORKSPACE = 7, /* workspace missing or smaller than fp8rl_fwd_workspace_bytes(), or that size
                              exceeds FP8RL_NOALLOC_SCRATCH_BYTES in the allocation-free call */
  FP8RL_ERR_VALUE = 8      /* a scalar argument is out of range (e.g. eps not positive and finite) */
} fp8rl_status;

/* Scaling recipes ([SkyRL-FP8] TL;DR and "Deep dive: FP8 quantization with FP32 and
 * power-of-two block scales": blockwise FP32 scales on Hopper, MXFP8 power-of-two scales
 * on Blackwell; the recipe is always chosen explicitly by the caller here). */
typedef enum {
  FP8RL_RECIPE_BLOCK128 = 0,   /* fp32 scale per 1x128 (activations) / 128x128 (weights) */
  FP8RL_RECIPE_MXFP8 = 1       /* E8M0 (power-of-two) scale byte per 1x32 along K */
} fp8rl_recipe;

typedef enum {
  FP8RL_OUT_BF16 = 0,          /* round-to-nearest-even of the fp32 accumulator */
  FP8RL_OUT_F32 = 1
} fp8rl_out;

/* Payload layouts of an installed weight (see fp8_weight_install). */
typedef enum {
  FP8RL_LAYOUT_ROWS = 0,       /* row-major [rows][cols]: the layout every quantizer writes */
  FP8RL_LAYOUT_DECODE = 1      /* BLOCK128 only: the same bytes regrouped for the decode GEMM */
} fp8rl_layout;

/* ABI version of this header. */
#define FP8RL_ABI_VERSION 7
int fp8rl_abi_version(void);
/* Text of a status code; any int is accepted ("unknown status" outside the enum). */
const char* fp8rl_status_str(int status);

/* ---------------------------------------------------------------------------------------
 * Quantizers. The quantizer is the symmetric one of [AIS] (quantizer equation), with the
 * E4M3 grid: s = fl32(amax / 448) per group (an IEEE fp32 division), q = E4M3(fl32(x / s))
 * with round-to-nearest-even and saturation to +-448, the sign of zero kept. A group whose
 * amax is 0 gets s = 1.0. Bytes and scales are bit-identical to the CPU oracle.
 * ------------------------------------------------------------------------------------- */

/* Activation quantization, 1x128 groups along K and/or 128x1 groups along M
 * ([Jet-RL] "Quantization scheme": activations 1x128; WGrad operands 1x128 and 128x1;
 * [SkyRL-FP8] "Performance analysis": row-wise plus transposed FP8 copies for backward).
 *   x   : bf16 [M][K]
 *   q,s : row-wise output, q uint8 [M][K], s fp32 [M][K/128]   (both NULL: not produced)
 *   qt,st: column-wise output written transposed: qt uint8 [K][M], st fp32 [K][M/128];
 *          qt[k][m] quantizes x[m][k] within the group of 128 consecutive rows m.
 *          (both NULL: not produced)
 * Rules: K % 128 == 0; M % 128 == 0 when qt is requested; at least one output pair. */
fp8rl_status fp8_quant_act_1x128(const uint16_t* x, int64_t M, int64_t K,
                                 uint8_t* q, float* s, uint8_t* qt, float* st, void* stream);

/* Weight quantization, one fp32 scale per 128x128 block ([SkyRL-FP8] "Why FP8 matters for
 * RL", "When independent quantization breaks policy consistency"; [Jet-RL]).
 *   w  : bf16 [N][K];  q uint8 [N][K];  s fp32 [N/128][K/128]
 *   qt : optional (NULL allowed) byte transpose of q, uint8 [K][N] (the DGrad operand;
 *        a 128x128 block stays a 128x128 block, so s is reused unchanged).
 * Rules: N % 128 == 0, K % 128 == 0. */
fp8rl_status fp8_quant_w_128x128(const uint16_t* w, int64_t N, int64_t K,
                                 uint8_t* q, float* s, uint8_t* qt, void* stream);

/* The same two quantizers with power-of-two block scales ([SkyRL-FP8] "Deep dive: FP8
 * quantization with FP32 and power-of-two block scales": exponent-only scales at the same
 * block granularity). Per group: s = 2^e with e the smallest integer such that
 * amax <= 448 * 2^e, clamped to [-127, 127] (e = 0 for an all-zero group); s is stored as an
 * fp32 value (2^-127 as the fp32 subnormal); q = E4M3(x * 2^-e), exact scaling that never
 * saturates. Arguments, layouts and rules are those of the calls above; bytes and scales
 * are bit-identical to the CPU oracle. The _pow2 GEMMs below take these scales. */
fp8rl_status fp8_quant_act_1x128_pow2(const uint16_t* x, int64_t M, int64_t K,
                                      uint8_t* q, float* s, uint8_t* qt, float* st, void* stream);
fp8rl_status fp8_quant_w_128x128_pow2(const uint16_t* w, int64_t N, int64_t K,
                                      uint8_t* q, float* s, uint8_t* qt, void* stream);

/* fp8_param requantization ([SkyRL-FP8] "Deep dive: FP8 quantization with FP32 and
 * power-of-two block scales": the optimizer updates an FP32 master copy and the FP8
 * parameter storage is recomputed from it after each step). 128x128 blocks quantized from
 * fp32 values: s = fl32(amax / 448) (pow2_scales == 0) or the power-of-two rule of
 * fp8_quant_w_128x128_pow2 (pow2_scales != 0); q = E4M3(fl32(w / s)) with an IEEE fp32
 * division (exact scaling for power-of-two scales). A block amax so small that
 * fl32(amax / 448) rounds to zero (below about 224 * 2^-149) gets s = 2^-149, the smallest
 * positive fp32 value, and a quotient beyond 448 (possible only with a subnormal s of a few
 * significant bits) saturates to +-448; neither case arises for bf16-representable values.
 *   w  : fp32 [N][K], finite;  q uint8 [N][K];  s fp32 [N/128][K/128]
 *   qt : optional (NULL allowed) byte transpose of q, uint8 [K][N] (the DGrad operand).
 * Rules: N % 128 == 0, K % 128 == 0. Bytes and scales are bit-identical to the CPU oracle. */
fp8rl_status fp8_quant_w_128x128_f32(const float* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                     int pow2_scales, void* stream);

/* MXFP8 quantization, one E8M0 scale per 1x32 group along K ([SkyRL-FP8] "When
 * independent quantization breaks policy consistency": one scale per 1x32 block; "Deep
 * dive": power-of-two, exponent-only scales). The exponent is the smallest e with
 * amax <= 448 * 2^e (clamped to [-127, 127]; amax 0 gives e = 0); byte = e + 127;
 * q = E4M3(x * 2^-e) (exact scaling, never saturates).
 *   x : bf16 [R][K];  q uint8 [R][K];  e8m0 uint8 [R][K/32].   Rules: K % 32 == 0. */
fp8rl_status mxfp8_quant_1x32(const uint16_t* x, int64_t R, int64_t K,
                              uint8_t* q, uint8_t* e8m0, void* stream);

/* MXFP8 activation quantization with 1x32 row groups and/or 32x1 column groups written
 * transposed: the operands of an MXFP8 linear layer's backward, whose GEMMs contract over
 * the token (or output-feature) dimension ([SkyRL-FP8] "When independent quantization
 * breaks policy consistency": 1x32 blocks; the MXFP8 recipe for the linear layers). Same
 * scale rule and encoding as mxfp8_quant_1x32.
 *   x : bf16 [R][K]
 *   q, e8m0   : rows: uint8 [R][K], E8M0 uint8 [R][K/32]             (both NULL: not produced)
 *   qt, e8m0t : columns, transposed: uint8 [K][R], E8M0 uint8 [K][R/32]; qt[k][r] quantizes
 *               x[r][k] within the group of 32 consecutive rows r     (both NULL: not produced)
 * Rules: K % 32 == 0; R % 128 == 0 and K % 128 == 0 when qt is requested; at least one pair. */
fp8rl_status mxfp8_quant_act_1x32(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e8m0,
                                  uint8_t* qt, uint8_t* e8m0t, void* stream);

/* ---------------------------------------------------------------------------------------
 * Fused producers ([Jet-RL] "Quantization scheme": the FP8 activations a linear layer
 * consumes are produced by the operator before it, fused with the quantization, so no bf16
 * copy goes through memory). Each computes the bf16 value a bf16 framework stores and
 * quantizes it exactly as fp8_quant_act_1x128 (or its _pow2 form, pow2_scales != 0) would:
 * the bytes equal those of the unfused pair of calls. The _bf16 calls are the unfused
 * producers (same values, stored as bf16).
 * ------------------------------------------------------------------------------------- */

/* SwiGLU. gu: bf16 [M][2F], the fused gate/up output: gate in columns [0, F), up in
 * columns [F, 2F). h[m][f] = bf16(fl32(bf16(silu(gate)) * up)) with silu(g) = g/(1+e^-g)
 * rounded once (nearest even) from its exact value. fp8_swiglu_bf16 writes h: bf16 [M][F].
 * fp8_swiglu_quant_1x128 quantizes h: q,s / qt,st as in fp8_quant_act_1x128 with K = F.
 * Rules: F % 128 == 0; M % 128 == 0 when qt is requested; at least one output pair for
 * the quantizing form. Non-finite inputs, and products beyond the bf16 range, are outside
 * the contract. */
fp8rl_status fp8_swiglu_bf16(const uint16_t* gu, int64_t M, int64_t F, uint16_t* h, void* stream);
fp8rl_status fp8_swiglu_quant_1x128(const uint16_t* gu, int64_t M, int64_t F,
                                    uint8_t* q, float* s, uint8_t* qt, float* st,
                                    int pow2_scales, void* stream);

/* RMSNorm. x: bf16 [M][K]; gamma: bf16 [K]; eps: positive, finite (FP8RL_ERR_VALUE).
 * r[m] = fl32(1 / sqrt(mean_k x[m][k]^2 + eps)) (rounded once from the exact value, up to
 * fp64 evaluation error), written to rstd fp32 [M] (required: the backward pass keeps it);
 * y[m][k] = bf16(fl32(gamma[k] * bf16(fl32(x[m][k] * r[m])))).
 * fp8_rmsnorm_bf16 writes y: bf16 [M][K]. fp8_rmsnorm_quant_1x128 quantizes y: q,s / qt,st
 * as in fp8_quant_act_1x128.
 * Rules: K % 128 == 0, K <= 65536; M % 128 == 0 when qt is requested; at least one output
 * pair for the quantizing form. gamma[k] * sqrt(K) beyond the bf16 range is outside the
 * contract. */
fp8rl_status fp8_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                              uint16_t* y, float* rstd, void* stream);
fp8rl_status fp8_rmsnorm_quant_1x128(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                                     float* rstd, uint8_t* q, float* s, uint8_t* qt, float* st,
                                     int pow2_scales, void* stream);

/* ---------------------------------------------------------------------------------------
 * Block-scaled GEMMs (FP8 operands, fp32 accumulation). Each is the product of the
 * dequantized operands, dequantized value = E4M3 value * scale of its group/block
 * ([SkyRL-FP8] TL;DR: FP8 linear-layer GEMMs; [Jet-RL] "Quantization scheme").
 * ------------------------------------------------------------------------------------- */

/* Forward: Y[M][N] = deq(X) . deq(W)^T.
 *   X given EITHER quantized (xq uint8 [M][K] + sx fp32 [M][K/128], x_bf16 = NULL)
 *   OR as bf16 (x_bf16 [M][K], xq = sx = NULL): then X is quantized 1x128 on the device
 *   inside this call ([SkyRL-FP8] "Performance analysis", generation: activations quantized
 *   on the fly in the GEMM path while weights and scales stay fixed), into the caller's
 *   workspace, with bytes identical to fp8_quant_act_1x128 (a quantizer launch, then the
 *   GEMM launch, on the given stream).
 *   wq uint8 [N][K], sw fp32 [N/128][K/128] (as produced by fp8_quant_w_128x128 or
 *   installed by fp8_weight_install).
 *   y: [M][N], bf16 or fp32 per y_dtype.
 *   workspace/workspace_bytes: only for the bf16-input form; at least
 *   fp8rl_fwd_workspace_bytes(M, K) bytes, 16-byte aligned, any contents (the call overwrites
 *   it with quantized X). Ignored otherwise (may be NULL). Calls that run at the same time
 *   must not share a workspace.
 * Rules: K % 128 == 0, N % 128 == 0, M >= 0 (any M); M * K < 2^32 for the bf16-input form. */
fp8rl_status fp8_gemm_blockscaled_fwd(const uint8_t* xq, const float* sx, const uint16_t* x_bf16,
                                      const uint8_t* wq, const float* sw,
                                      int64_t M, int64_t N, int64_t K,
                                      void* y, int y_dtype,
                                      void* workspace, size_t workspace_bytes, void* stream);
size_t fp8rl_fwd_workspace_bytes(int64_t M, int64_t K);

/* Forward with the weight in the decode layout (FP8RL_LAYOUT_DECODE, written by
 * fp8_weight_install): the same product, arguments and rules as fp8_gemm_blockscaled_fwd,
 * with wq the decode-layout payload of W[N][K] (N * K bytes) and sw W's block scales
 * [N/128][K/128]. The output is bit-identical to fp8_gemm_blockscaled_fwd on the row-major
 * payload for M <= 256. Made for decode-shaped calls (few rows, weight-stream bound); any M
 * is accepted. Extra rule: M * K < 2^32 and N * K < 2^32. */
fp8rl_status fp8_gemm_blockscaled_fwd_decode_layout(const uint8_t* xq, const float* sx, const uint16_t* x_bf16,
                                                    const uint8_t* wq, const float* sw,
                                                    int64_t M, int64_t N, int64_t K,
                                                    void* y, int y_dtype,
                                                    void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free variant of fp8_gemm_blockscaled_fwd_decode_layout, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same product, arguments and rules without the workspace. The
 * bf16-input form quantizes X into a device array built into the library (the library's own
 * scratch, FP8RL_NOALLOC_SCRATCH_BYTES on every GPU it runs on, held until the process
 * ends), so the call allocates nothing. FP8RL_ERR_WORKSPACE when
 * fp8rl_fwd_workspace_bytes(M, K) exceeds FP8RL_NOALLOC_SCRATCH_BYTES. All calls on one GPU
 * share that array: calls that may overlap on one GPU (different streams, or host threads)
 * race and must be serialised by the caller; calls in order on one stream are safe. */
#define FP8RL_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
fp8rl_status fp8_gemm_blockscaled_fwd_decode_layout_noalloc(const uint8_t* xq, const float* sx,
                                                            const uint16_t* x_bf16,
                                                            const uint8_t* wq, const float* sw,
                                                            int64_t M, int64_t N, int64_t K,
                                                            void* y, int y_dtype, void* stream);

/* DGrad: dX[M][K] = deq(dY) . deq(W)  ([Jet-RL] "Quantization scheme": DGrad in FP8).
 *   dyq uint8 [M][N], sdy fp32 [M][N/128]  (dY quantized 1x128 along N)
 *   wqt uint8 [K][N]: byte transpose of W's payload (fp8_quant_w_128x128's qt)
 *   sw  fp32 [N/128][K/128]: W's block scales, NOT transposed.
 *   dx: [M][K], bf16 or fp32.   Rules: N % 128 == 0, K % 128 == 0, M >= 0. */
fp8rl_status fp8_gemm_blockscaled_dgrad(const uint8_t* dyq, const float* sdy,
                                        const uint8_t* wqt, const float* sw,
                                        int64_t M, int64_t N, int64_t K,
                                        void* dx, int dx_dtype, void* stream);

/* WGrad: dW[N][K] = deq(dY)^T . deq(X), both operands grouped 128x1 along the M tokens
 * ([Jet-RL] "Quantization scheme": WGrad with 1x128 and 128x1 groups), i.e. the
 * column-wise outputs of fp8_quant_act_1x128:
 *   dyqt uint8 [N][M], sdyt fp32 [N][M/128];  xqt uint8 [K][M], sxt fp32 [K][M/128].
 *   dw fp32 [N][K]; accumulate != 0 adds the product to the existing dw contents.
 * Rules: M % 128 == 0, N % 128 == 0, K % 128 == 0. */
fp8rl_status fp8_gemm_blockscaled_wgrad(const uint8_t* dyqt, const float* sdyt,
                                        const uint8_t* xqt, const float* sxt,
                                        int64_t M, int64_t N, int64_t K,
                                        float* dw, int accumulate, void* stream);

/* Forward, DGrad and WGrad for power-of-two block scales (the _pow2 quantizers' output):
 * the same products, layouts and rules as fp8_gemm_blockscaled_fwd (FP8 X only: xq, sx),
 * _dgrad and _wgrad, but the scaled MFMA applies each block's 2^e itself, taken from the
 * exponent field of the fp32 scale, so there is no per-block rescale step ([SkyRL-FP8]
 * "Deep dive": power-of-two scales are applied by the hardware's block-scaled matrix
 * instructions). Precondition: every scale is a power of two in [2^-127, 2^127]; for any
 * other value only its exponent field is used (the mantissa is ignored). Any M is served
 * by the tiled kernel (there is no few-row form). */
fp8rl_status fp8_gemm_blockscaled_pow2_fwd(const uint8_t* xq, const float* sx,
                                           const uint8_t* wq, const float* sw,
                                           int64_t M, int64_t N, int64_t K,
                                           void* y, int y_dtype, void* stream);
fp8rl_status fp8_gemm_blockscaled_pow2_dgrad(const uint8_t* dyq, const float* sdy,
                                             const uint8_t* wqt, const float* sw,
                                             int64_t M, int64_t N, int64_t K,
                                             void* dx, int dx_dtype, void* stream);
fp8rl_status fp8_gemm_blockscaled_pow2_wgrad(const uint8_t* dyqt, const float* sdyt,
                                             const uint8_t* xqt, const float* sxt,
                                             int64_t M, int64_t N, int64_t K,
                                             float* dw, int accumulate, void* stream);

/* MXFP8 dense linear layer ([SkyRL-FP8]: the MXFP8 recipe for the linear layers, one E8M0
 * scale per 1x32 block along each GEMM's contraction dimension). The scaled MFMA applies
 * the E8M0 scales; fp32 accumulation.
 *   forward: Y[M][N] = deq(X) . deq(W)^T; xq [M][K], ex [M][K/32]; wq [N][K], ew [N][K/32];
 *            y bf16 or fp32 [M][N].                Rules: K % 128 == 0, N % 128 == 0, any M.
 *   DGrad  : dX[M][K] = deq(dY) . deq(W); dyq [M][N], edy [M][N/32]; W as its 32x1 copy
 *            (mxfp8_quant_act_1x32's qt of W): wqt [K][N], ewt [K][N/32];
 *            dx bf16 or fp32 [M][K].               Rules: N % 128 == 0, K % 128 == 0, any M.
 *   WGrad  : dW[N][K] = deq(dY)^T . deq(X) from the 32x1 copies dyqt [N][M], edyt [N][M/32],
 *            xqt [K][M], ext [K][M/32]; dw fp32 [N][K]; accumulate != 0 adds to dw.
 *                                                  Rules: M, N, K % 128 == 0.
 * E8M0 arrays must be 4-byte aligned (their rows are read as dwords of 4 bytes). */
fp8rl_status fp8_gemm_mxfp8_fwd(const uint8_t* xq, const uint8_t* ex, const uint8_t* wq, const uint8_t* ew,
                                int64_t M, int64_t N, int64_t K, void* y, int y_dtype, void* stream);
fp8rl_status fp8_gemm_mxfp8_dgrad(const uint8_t* dyq, const uint8_t* edy, const uint8_t* wqt, const uint8_t* ewt,
                                  int64_t M, int64_t N, int64_t K, void* dx, int dx_dtype, void* stream);
fp8rl_status fp8_gemm_mxfp8_wgrad(const uint8_t* dyqt, const uint8_t* edyt, const uint8_t* xqt, const uint8_t* ext,
                                  int64_t M, int64_t N, int64_t K, float* dw, int accumulate, void* stream);

/* Grouped GEMM for mixture-of-experts ([SkyRL-FP8] MoE: routed experts hold most
 * parameters; MXFP8 recipe, or the blockwise recipe of the dense layers). Routed rows are
 * grouped by expert; rows offsets[e] .. offsets[e+1]-1 belong to expert e:
 *   Y[t][n] = sum_k deq(X)[t][k] * deq(W[e])[n][k].
 *   recipe FP8RL_RECIPE_MXFP8:    xq uint8 [T][K], sx = E8M0 uint8 [T][K/32],
 *                                 wq uint8 [E][N][K], sw = E8M0 uint8 [E][N][K/32].
 *   recipe FP8RL_RECIPE_BLOCK128: xq uint8 [T][K], sx = fp32 [T][K/128] (1x128 groups, as
 *                                 from fp8_quant_act_1x128), wq uint8 [E][N][K],
 *                                 sw = fp32 [E][N/128][K/128] (each expert's 128x128
 *                                 blocks, as from fp8_quant_w_128x128 of its [N][K] slice).
 *   offsets: DEVICE int32 [E+1], expected 0 = offsets[0] <= ... <= offsets[E] = T. The
 *   kernel clamps every offset into [0, T] and treats a decreasing step as an empty
 *   expert, so malformed offsets never cause an out-of-bounds access; rows not covered by
 *   any expert are left unwritten. If clamped ranges overlap, the experts' 256-row tiles
 *   can outnumber the T/256 + E the launch provides for; the tiles past that are skipped.
 *   y: [T][N], bf16 or fp32.
 * Rules: K % 128 == 0, N % 16 == 0 (MXFP8) or N % 128 == 0 (BLOCK128), E >= 1; pointers
 * 16-byte aligned (scales and offsets 4-byte). Any other recipe -> FP8RL_ERR_RECIPE. */
fp8rl_status fp8_grouped_gemm(int recipe, const uint8_t* xq, const void* sx,
                              const uint8_t* wq, const void* sw, const int32_t* offsets,
                              int64_t T, int64_t E, int64_t N, int64_t K,
                              void* y, int y_dtype, void* stream);

/* ---------------------------------------------------------------------------------------
 * Zero-requantization weight install ([SkyRL-FP8] "On-Policy FP8 weight sync", Fig. 3:
 * the rollout side installs the trainer's FP8 payload and block scales without a
 * quantizer of its own, so both sides hold bit-identical weights).
 * ------------------------------------------------------------------------------------- */
typedef struct {
  int recipe;        /* fp8rl_recipe */
  int64_t rows;      /* N (for MXFP8 expert stacks: E*N) */
  int64_t cols;      /* K */
  uint8_t* q;        /* payload, rows * cols bytes in the descriptor's layout */
  void* s;           /* BLOCK128: fp32 [rows/128][cols/128];  MXFP8: E8M0 uint8 [rows][cols/32] */
  int layout;        /* fp8rl_layout of q (FP8RL_LAYOUT_ROWS = 0 when zero-initialised) */
} fp8rl_weight;

/* Installs src's payload and scales into dst's buffers without any quantizer: the scales
 * are copied verbatim, and so is the payload when both layouts agree. With src row-major
 * and dst FP8RL_LAYOUT_DECODE (BLOCK128), the payload bytes are regrouped for the decode
 * GEMM (fp8_gemm_blockscaled_fwd_decode_layout): for 16-row group f and 128-column block
 * kb, the 2048 bytes at (f * cols/128 + kb) * 2048 hold, for i = 0..63, bytes
 * kb*128 + 16*(i/16) .. +15 of row 16 f + i%16 at 16 i and bytes kb*128 + 64 + 16*(i/16) .. +15
 * of that row at 1024 + 16 i -- the order in which the matrix instruction takes them; every
 * byte keeps its value ([SkyRL-FP8] practical findings: one configuration fixes values,
 * scales and layout conversions for both engines).
 * The descriptors must agree on recipe, rows and cols; a DECODE dst needs a ROWS or DECODE
 * src (FP8RL_ERR_RECIPE otherwise: the library never requantizes).
 * Rules: BLOCK128: rows % 128 == 0, cols % 128 == 0; MXFP8: cols % 32 == 0, ROWS layout
 * only. src and dst buffers must not overlap. */
fp8rl_status fp8_weight_install(const fp8rl_weight* src, const fp8rl_weight* dst, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP8RL_H */
