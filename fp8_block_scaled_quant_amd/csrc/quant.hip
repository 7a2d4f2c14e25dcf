// FP8 quantizer kernels: 1x128 rows, 128x1 columns (transposed output), 128x128 blocks,
// and MXFP8 1x32 groups. Method: [AIS] symmetric quantizer equation on the E4M3 grid;
// granularities from [Jet-RL] "Quantization scheme" and [SkyRL-FP8] (block and MXFP8
// recipes). Each kernel is a single pass over its bf16 input: coalesced 16-byte loads,
// group amax by lane shuffles (or LDS for 128x1 / 128x128), and E4M3 conversion.
#include "device.hpp"
#include "internal.hpp"

namespace fp8rl {

// ---------------------------------------------------------------------------------------
// 1x128 row groups. The groups of X[M][K] tile each row exactly, so group g starts at
// element g * 128 and its scale is s[g] (row-major [M][K/128]). 8 lanes per group, 16
// elements (32 bytes) per lane; one wave covers 8 consecutive groups = 2 KB of input.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_rows_1x128(const uint16_t* __restrict__ x,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ s,
                                                          int64_t ngroups) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t g = t >> 3;
  const int part = (int)(t & 7);
  const bool valid = g < ngroups;
  uint4 a = make_uint4(0, 0, 0, 0), b = a;
  if (valid) {
    const uint4* src = reinterpret_cast<const uint4*>(x + g * 128 + part * 16);
    a = src[0];
    b = src[1];
  }
  float amax = fmaxf(fmaxf(fmaxf(absmax2(a.x), absmax2(a.y)), fmaxf(absmax2(a.z), absmax2(a.w))),
                     fmaxf(fmaxf(absmax2(b.x), absmax2(b.y)), fmaxf(absmax2(b.z), absmax2(b.w))));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  const BlockScale bs = block_scale(amax);
  if (valid) {
    const uint2 lo = quant8(a.x, a.y, a.z, a.w, bs.r);
    const uint2 hi = quant8(b.x, b.y, b.z, b.w, bs.r);
    *reinterpret_cast<uint4*>(q + g * 128 + part * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    if (part == 0) s[g] = bs.s;
  }
}

// ---------------------------------------------------------------------------------------
// 128 x 128 tile kernel, 256 threads.
//   kBlock = false: activation mode. Row output = 1x128 groups (q [R][C], s [R][C/128]),
//                   column output = 128x1 groups written transposed (qt [C][R], st [C][R/128]).
//   kBlock = true : weight mode. One scale for the whole 128x128 block (s [R/128][C/128]);
//                   qt, if requested, is the byte transpose of q (same scale, same bytes).
// Grid: one workgroup per tile, blockIdx.x = rb * (C/128) + cb.
// Thread t loads row t/2, columns (t%2)*64 .. +64 (8 x 16-byte loads). For the column pass
// the tile goes through LDS; wave w then reads rows 32w .. 32w+31 of the column pair
// (2l, 2l+1) held in 32-bit word l (conflict-free: a wave reads 64 consecutive words).
// ---------------------------------------------------------------------------------------
template <bool kBlock>
__global__ __launch_bounds__(256) void k_quant_tile(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                    uint8_t* __restrict__ q, float* __restrict__ s,
                                                    uint8_t* __restrict__ qt, float* __restrict__ st) {
  constexpr int LDW = 68;  // LDS row stride in words (64 + 4 keeps 16-byte row writes conflict-free)
  __shared__ __attribute__((aligned(16))) uint32_t tile[128 * LDW];
  __shared__ float red[4 * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t ncb = C / 128;
  const int64_t cb = blockIdx.x % ncb, rb = blockIdx.x / ncb;
  const int r = tid >> 1, h = tid & 1;
  const bool want_rows = q != nullptr, want_cols = qt != nullptr;

  const uint4* src = reinterpret_cast<const uint4*>(x + (rb * 128 + r) * C + cb * 128 + h * 64);
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = src[i];

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    amax = fmaxf(amax, fmaxf(fmaxf(absmax2(v[i].x), absmax2(v[i].y)), fmaxf(absmax2(v[i].z), absmax2(v[i].w))));

  BlockScale row_bs;
  if (kBlock) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    row_bs = block_scale(amax);
    if (tid == 0) s[rb * (C / 128) + cb] = row_bs.s;
  } else {
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    row_bs = block_scale(amax);
    if (want_rows && h == 0) s[(rb * 128 + r) * (C / 128) + cb] = row_bs.s;
  }

  if (want_rows) {
    uint4* dst = reinterpret_cast<uint4*>(q + (rb * 128 + r) * C + cb * 128 + h * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 lo = quant8(v[2 * i].x, v[2 * i].y, v[2 * i].z, v[2 * i].w, row_bs.r);
      const uint2 hi = quant8(v[2 * i + 1].x, v[2 * i + 1].y, v[2 * i + 1].z, v[2 * i + 1].w, row_bs.r);
      dst[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
  if (!want_cols) return;

  uint4* trow = reinterpret_cast<uint4*>(tile + r * LDW + h * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) trow[i] = v[i];
  __syncthreads();

  uint32_t col[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) col[i] = tile[(32 * wave + i) * LDW + lane];

  double r0, r1;
  if (kBlock) {
    r0 = r1 = row_bs.r;
  } else {
    float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      m0 = fmaxf(m0, fabsf(bf16_lo(col[i])));
      m1 = fmaxf(m1, fabsf(bf16_hi(col[i])));
    }
    red[wave * 128 + 2 * lane] = m0;
    red[wave * 128 + 2 * lane + 1] = m1;
    __syncthreads();
    m0 = fmaxf(fmaxf(red[2 * lane], red[128 + 2 * lane]), fmaxf(red[256 + 2 * lane], red[384 + 2 * lane]));
    m1 = fmaxf(fmaxf(red[2 * lane + 1], red[128 + 2 * lane + 1]),
               fmaxf(red[256 + 2 * lane + 1], red[384 + 2 * lane + 1]));
    const BlockScale b0 = block_scale(m0), b1 = block_scale(m1);
    r0 = b0.r;
    r1 = b1.r;
    if (wave == 0) {
      st[(cb * 128 + 2 * lane) * (R / 128) + rb] = b0.s;
      st[(cb * 128 + 2 * lane + 1) * (R / 128) + rb] = b1.s;
    }
  }
  // column c = 2*lane (low halves) and 2*lane+1 (high halves), rows 32*wave .. +31
  uint32_t o0[8], o1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o0[i] = pack4_e4m3(scaled(bf16_lo(col[4 * i]), r0), scaled(bf16_lo(col[4 * i + 1]), r0),
                       scaled(bf16_lo(col[4 * i + 2]), r0), scaled(bf16_lo(col[4 * i + 3]), r0));
    o1[i] = pack4_e4m3(scaled(bf16_hi(col[4 * i]), r1), scaled(bf16_hi(col[4 * i + 1]), r1),
                       scaled(bf16_hi(col[4 * i + 2]), r1), scaled(bf16_hi(col[4 * i + 3]), r1));
  }
  uint4* d0 = reinterpret_cast<uint4*>(qt + (cb * 128 + 2 * lane) * R + rb * 128 + 32 * wave);
  uint4* d1 = reinterpret_cast<uint4*>(qt + (cb * 128 + 2 * lane + 1) * R + rb * 128 + 32 * wave);
  d0[0] = make_uint4(o0[0], o0[1], o0[2], o0[3]);
  d0[1] = make_uint4(o0[4], o0[5], o0[6], o0[7]);
  d1[0] = make_uint4(o1[0], o1[1], o1[2], o1[3]);
  d1[1] = make_uint4(o1[4], o1[5], o1[6], o1[7]);
}

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
    const uint4* src = reinterpret_cast<const uint4*>(x + g * 32 + part * 16);
    a = src[0];
    b = src[1];
  }
  float amax = fmaxf(fmaxf(fmaxf(absmax2(a.x), absmax2(a.y)), fmaxf(absmax2(a.z), absmax2(a.w))),
                     fmaxf(fmaxf(absmax2(b.x), absmax2(b.y)), fmaxf(absmax2(b.z), absmax2(b.w))));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
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
hipError_t launch_quant_rows_1x128(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                   hipStream_t stream) {
  const int64_t ngroups = M * (K / 128);
  const int64_t threads = ngroups * 8;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(k_quant_rows_1x128, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, s, ngroups);
  return hipGetLastError();
}

hipError_t launch_quant_act_tile(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                 float* st, hipStream_t stream) {
  hipLaunchKernelGGL(k_quant_tile<false>, dim3((unsigned)((K / 128) * (M / 128))), dim3(256), 0, stream, x, M, K,
                     q, s, qt, st);
  return hipGetLastError();
}

hipError_t launch_quant_w_128x128(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(k_quant_tile<true>, dim3((unsigned)((K / 128) * (N / 128))), dim3(256), 0, stream, w, N, K,
                     q, s, qt, (float*)nullptr);
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
