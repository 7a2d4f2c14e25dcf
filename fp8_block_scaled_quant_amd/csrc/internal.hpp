// Internal launch interface between the C ABI layer (abi.hip) and the kernel files.
// Launchers assume validated arguments: non-empty shapes that satisfy each call's rules.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8rl {

// pow2: power-of-two group scales (exponent rule of MXFP8) instead of fl32(amax / 448).
hipError_t launch_quant_rows_1x128(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, bool pow2,
                                   hipStream_t stream);
hipError_t launch_quant_act_tile(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                 float* st, bool pow2, hipStream_t stream);
hipError_t launch_quant_w_128x128(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                  bool pow2, hipStream_t stream);
// fp8_param: 128x128-block quantization of an fp32 master W[N][K] (fp8_param.hip).
hipError_t launch_quant_w_f32(const float* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt, bool pow2,
                              hipStream_t stream);
// Fused producers (producers.hip). gu is [M][2F] = [gate | up]; rstd [M].
hipError_t launch_swiglu_bf16(const uint16_t* gu, int64_t M, int64_t F, uint16_t* h, hipStream_t stream);
hipError_t launch_swiglu_quant(const uint16_t* gu, int64_t M, int64_t F, uint8_t* q, float* s, uint8_t* qt,
                               float* st, bool pow2, hipStream_t stream);
hipError_t launch_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                               uint16_t* y, float* rstd, hipStream_t stream);
hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                                float* rstd, uint8_t* q, float* s, uint8_t* qt, float* st, bool pow2,
                                hipStream_t stream);
// MXFP8 1x32 rows and/or 32x1 columns (written transposed) of X[R][K], R % 128 == K % 128 == 0.
hipError_t launch_quant_mx_tile(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e8m0, uint8_t* qt,
                                uint8_t* e8m0t, hipStream_t stream);
hipError_t launch_quant_mx_1x32(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e8m0,
                                hipStream_t stream);

// C[m][n] = sum_kb sA[m * sa_ld + kb] * sB(n, kb) * sum_{k in kb} A[m][k] * B[n][k]
//   row-scaled B : sB(n, kb) = sB[n * sb_ld_n + kb]
//   block-scaled B: sB(n, kb) = sB[(n / 128) * sb_ld_n + kb * sb_ld_k]
struct GemmParams {
  const uint8_t* A;
  const uint8_t* B;
  const float* sA;
  const float* sB;
  void* C;
  int64_t M, N, K;
  int64_t sa_ld, sb_ld_n, sb_ld_k, ldc;
  int accumulate;
  // Grouped (MoE) form only: rows of A grouped by expert, expert e owning rows
  // [offsets[e], offsets[e + 1]) of [0, M); B and sB advance by b_stride bytes and sb_stride
  // dwords per expert.
  const int32_t* offsets;
  int64_t E, b_stride, sb_stride;
};
// pow2: every scale is a power of two (the pow2 quantizers' output); the scaled MFMA then
// applies them (their fp32 exponent fields) and no rescale step is needed.
hipError_t launch_gemm_blockscaled(const GemmParams& p, bool row_scale_b, bool f32, bool pow2, hipStream_t stream);
// MXFP8 TN GEMM: sA / sB are E8M0 bytes [rows][K/32] (passed as float* to dwords of 4 bytes).
hipError_t launch_gemm_mx(const GemmParams& p, bool f32, hipStream_t stream);
// Few-row forward GEMM (decode.hip), M <= 256, block-scaled B [N][K] with fp32 scales
// sB[(n / 128) * sb_ld_n + kb * sb_ld_k]. A is addressed through strides: element (m, k) at
// A[m * a_ld + (k / 128) * a_kb + k % 128], its scale at sA[m * sa_ld + (k / 128) * sa_kb];
// row-major A: (a_ld, a_kb) = (K, 128), (sa_ld, sa_kb) = (K / 128, 1); K-block-major:
// (128, 128 M) and (1, M). C [M][ldc], bf16 or fp32 (no accumulation).
// tiled_b: B in the decode layout (launch_decode_layout) instead of row-major.
struct DecodeParams {
  const uint8_t* A;
  const float* sA;
  const uint8_t* B;
  const float* sB;
  void* C;
  int64_t M, N, K;
  int64_t a_ld, a_kb, sa_ld, sa_kb, sb_ld_n, sb_ld_k, ldc;
  int tiled_b;
};
hipError_t launch_gemm_decode(const DecodeParams& p, bool f32, hipStream_t stream);
// 1x128 quantization of bf16 X [M][K] into the K-block-major copy q [K/128][M][128], s
// [K/128][M] (decode.hip); same bytes and scales as launch_quant_rows_1x128, permuted.
hipError_t launch_quant_kbmajor(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, hipStream_t stream);
// Row-major FP8 weight [N][K] -> decode layout (decode.hip), N % 16 == 0, K % 128 == 0.
hipError_t launch_decode_layout(const uint8_t* src, uint8_t* dst, int64_t N, int64_t K, hipStream_t stream);

// Scales: MXFP8 = E8M0 bytes Xs [T][K/32], Ws [E][N][K/32]; blockwise = fp32
// Xs [T][K/128] (1x128 groups), Ws [E][N/128][K/128] (128x128 blocks per expert).
struct GroupedParams {
  const uint8_t* X;     // [T][K]
  const uint8_t* Xs;
  const uint8_t* W;     // [E][N][K]
  const uint8_t* Ws;
  const int32_t* offsets;
  void* Y;              // [T][N]
  int64_t T, E, N, K;
};
hipError_t launch_grouped_mx(const GroupedParams& p, bool f32, hipStream_t stream);
hipError_t launch_grouped_block(const GroupedParams& p, bool f32, hipStream_t stream);

hipError_t launch_copy(const uint8_t* src_q, uint8_t* dst_q, int64_t qbytes, const uint8_t* src_s, uint8_t* dst_s,
                       int64_t sbytes, hipStream_t stream);

}  // namespace fp8rl
