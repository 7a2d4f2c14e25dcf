// fp8_param requantization: FP8 parameter storage Q(W_t) recomputed from the FP32 master
// copy after each optimizer step ([SkyRL-FP8] "Deep dive: FP8 quantization with FP32 and
// power-of-two block scales": the optimizer updates the FP32 master and the FP8 storage is
// requantized from it, with fp32 or power-of-two block scales). One 128x128 block per
// workgroup: s = fl32(amax / 448) (or the power-of-two rule), q = E4M3(fl32(w / s)) with an
// IEEE fp32 division (the master has 24 significant bits, so the quotient is formed
// exactly as defined rather than through a reciprocal), and optionally the byte transpose
// of the block (the DGrad operand) through LDS.
#include "device.hpp"
#include "internal.hpp"

namespace fp8rl {

// Thread t owns rows 4*(t/16) .. +3, columns 8*(t%16) .. +7 of the block: each wave load
// reads 4 whole 512-byte row segments and each row store writes whole 128-byte lines.
template <bool kPow2>
__global__ __launch_bounds__(512) void k_quant_w_f32(const float* __restrict__ w, int64_t N, int64_t K,
                                                     uint8_t* __restrict__ q, float* __restrict__ s,
                                                     uint8_t* __restrict__ qt) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[128 * 32];   // codes, [column][128 rows]
  __shared__ float red[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 15, rg = tid >> 4;
  const int64_t ncb = K / 128;
  const int64_t cb = blockIdx.x % ncb, rb = blockIdx.x / ncb;

  float4 v[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4* p = reinterpret_cast<const float4*>(w + (rb * 128 + 4 * rg + i) * K + cb * 128 + c * 8);
    v[i][0] = p[0];
    v[i][1] = p[1];
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      a = fmaxf(a, fmaxf(fmaxf(fabsf(v[i][h].x), fabsf(v[i][h].y)), fmaxf(fabsf(v[i][h].z), fabsf(v[i][h].w))));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
  if (lane == 0) red[wave] = a;
  __syncthreads();
  a = fmaxf(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7])));

  float sv;
  int e = 0;
  if constexpr (kPow2) {
    e = mx_exponent(a);
    sv = ldexpf(1.0f, e);
  } else {
    sv = (a == 0.0f) ? 1.0f : a / kE4M3Max;
    // An amax below about 224 * 2^-149 gives a scale that rounds to zero: it is raised to
    // the smallest positive fp32 value, so every quotient stays finite.
    if (sv == 0.0f) sv = __uint_as_float(1u);
  }
  if (tid == 0) s[rb * ncb + cb] = sv;
  // fl32(x / s): exact scaling by 2^-e (at most 448 in magnitude), or an IEEE division. A
  // subnormal scale with few significant bits can give quotients up to 512, which the
  // non-saturating converter would turn into NaN: they are clamped to +-448 first, the
  // saturation of the E4M3 encoding (values in (448, 464) round to 448 anyway).
  auto quo = [&](float x) __attribute__((always_inline)) {
    if constexpr (kPow2) return ldexpf(x, -e);
    else return fminf(fmaxf(x / sv, -kE4M3Max), kE4M3Max);
  };

  uint2 code[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    code[i].x = pack4_e4m3(quo(v[i][0].x), quo(v[i][0].y), quo(v[i][0].z), quo(v[i][0].w));
    code[i].y = pack4_e4m3(quo(v[i][1].x), quo(v[i][1].y), quo(v[i][1].z), quo(v[i][1].w));
    *reinterpret_cast<uint2*>(q + (rb * 128 + 4 * rg + i) * K + cb * 128 + c * 8) = code[i];
  }
  if (qt == nullptr) return;

  // Column 8c + j gets the 4 bytes of rows 4rg .. 4rg+3: one dword at [column][rg].
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int sh = 8 * (j & 3);
    const uint32_t b0 = ((j < 4 ? code[0].x : code[0].y) >> sh) & 0xffu;
    const uint32_t b1 = ((j < 4 ? code[1].x : code[1].y) >> sh) & 0xffu;
    const uint32_t b2 = ((j < 4 ? code[2].x : code[2].y) >> sh) & 0xffu;
    const uint32_t b3 = ((j < 4 ? code[3].x : code[3].y) >> sh) & 0xffu;
    tile[(8 * c + j) * 32 + rg] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
  }
  __syncthreads();
  // 128 columns x 128 bytes = 1024 chunks of 16 bytes; 8 lanes write one 128-byte line of qt.
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int idx = tid + 512 * r;
    const int col = idx >> 3, part = idx & 7;
    const uint4 chunk = *reinterpret_cast<const uint4*>(tile + col * 32 + part * 4);
    *reinterpret_cast<uint4*>(qt + (cb * 128 + col) * N + rb * 128 + part * 16) = chunk;
  }
}

hipError_t launch_quant_w_f32(const float* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt, bool pow2,
                              hipStream_t stream) {
  const dim3 grid((unsigned)((K / 128) * (N / 128)));
  if (pow2)
    hipLaunchKernelGGL(k_quant_w_f32<true>, grid, dim3(512), 0, stream, w, N, K, q, s, qt);
  else
    hipLaunchKernelGGL(k_quant_w_f32<false>, grid, dim3(512), 0, stream, w, N, K, q, s, qt);
  return hipGetLastError();
}

}  // namespace fp8rl
