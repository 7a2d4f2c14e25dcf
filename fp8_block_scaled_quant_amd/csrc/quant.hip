// FP8 quantizer kernels: 1x128 rows, 128x1 columns (transposed output), 128x128 blocks,
// and MXFP8 1x32 groups. The blockwise kernels take kPow2 = true for power-of-two scales
// ([SkyRL-FP8] "Deep dive": exponent-only block scales; MX exponent rule per group). Method: [AIS] symmetric quantizer equation on the E4M3 grid;
// granularities from [Jet-RL] "Quantization scheme" and [SkyRL-FP8] (block and MXFP8
// recipes). Each kernel is a single pass over its bf16 input: coalesced 16-byte loads,
// group amax by lane shuffles (or LDS for 128x1 / 128x128), and E4M3 conversion.
#include "device.hpp"
#include "internal.hpp"
#include "quant_kernels.hpp"

namespace fp8rl {

// ---------------------------------------------------------------------------------------
// MXFP8 1x32 groups: 2 lanes per group, 16 elements (32 bytes) per lane. Group g starts
// at element g * 32; its E8M0 byte is e8m0[g] (row-major [R][K/32]).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_mx_1x32(const uint16_t* __restrict__ x,
                                                       uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ e8m0,
                                                       int64_t ngroups) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t g = t >> 1;
  const int part = (int)(t & 1);
  const bool valid = g < ngroups;
  uint4 a = make_uint4(0, 0, 0, 0), b = a;
  if (valid) {
    const uint16_t* src = x + g * 32 + part * 16;
    a = ntload16(src);
    b = ntload16(src + 8);
  }
  const float amax = group_amax<2>(pk_max_u16(mag8(a), mag8(b)));
  const int e = mx_exponent(amax);
  if (valid) {
    // x * 2^-e is exact (v_ldexp_f32) and |x * 2^-e| <= 448 by the choice of e.
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack4_e4m3(ldexpf(bf16_lo(w[2 * i]), -e), ldexpf(bf16_hi(w[2 * i]), -e),
                        ldexpf(bf16_lo(w[2 * i + 1]), -e), ldexpf(bf16_hi(w[2 * i + 1]), -e));
    *reinterpret_cast<uint4*>(q + g * 32 + part * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    if (part == 0) e8m0[g] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------------------------------
// Launchers (argument validation happens in the C ABI layer before these are called).
// ---------------------------------------------------------------------------------------
hipError_t launch_quant_rows_1x128(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, bool pow2,
                                   hipStream_t stream) {
  const int64_t ngroups = M * (K / 128);
  const int64_t threads = ngroups * 8;
  const int64_t blocks = (threads + 255) / 256;
  const PlainSrc src{x, K};
  if (pow2)
    hipLaunchKernelGGL((k_quant_rows_1x128<PlainSrc, true>), dim3((unsigned)blocks), dim3(256), 0, stream, src, q, s,
                       ngroups);
  else
    hipLaunchKernelGGL((k_quant_rows_1x128<PlainSrc, false>), dim3((unsigned)blocks), dim3(256), 0, stream, src, q, s,
                       ngroups);
  return hipGetLastError();
}

hipError_t launch_quant_act_tile(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                 float* st, bool pow2, hipStream_t stream) {
  const dim3 grid((unsigned)((K / 128) * (M / 128)));
  const PlainSrc src{x, K};
  if (pow2)
    hipLaunchKernelGGL((k_quant_tile<PlainSrc, false, true>), grid, dim3(512), 0, stream, src, M, K, q, s, qt, st);
  else
    hipLaunchKernelGGL((k_quant_tile<PlainSrc, false, false>), grid, dim3(512), 0, stream, src, M, K, q, s, qt, st);
  return hipGetLastError();
}

hipError_t launch_quant_w_128x128(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                  bool pow2, hipStream_t stream) {
  const dim3 grid((unsigned)((K / 128) * (N / 128)));
  const PlainSrc src{w, K};
  if (pow2)
    hipLaunchKernelGGL((k_quant_tile<PlainSrc, true, true>), grid, dim3(512), 0, stream, src, N, K, q, s, qt,
                       (float*)nullptr);
  else
    hipLaunchKernelGGL((k_quant_tile<PlainSrc, true, false>), grid, dim3(512), 0, stream, src, N, K, q, s, qt,
                       (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_quant_mx_tile(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e8m0, uint8_t* qt,
                                uint8_t* e8m0t, hipStream_t stream) {
  const dim3 grid((unsigned)((K / 128) * (R / 128)));
  const PlainSrc src{x, K};
  hipLaunchKernelGGL((k_quant_tile<PlainSrc, false, true, 32>), grid, dim3(512), 0, stream, src, R, K, q, e8m0, qt,
                     e8m0t);
  return hipGetLastError();
}

hipError_t launch_quant_mx_1x32(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e8m0,
                                hipStream_t stream) {
  const int64_t ngroups = R * (K / 32);
  const int64_t blocks = (ngroups * 2 + 255) / 256;
  hipLaunchKernelGGL(k_quant_mx_1x32, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, e8m0, ngroups);
  return hipGetLastError();
}

}  // namespace fp8rl
