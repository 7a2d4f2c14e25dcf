// Fused FP8 producers: SwiGLU(gate, up) -> FP8 and RMSNorm -> FP8 ([Jet-RL] "Quantization
// scheme": the FP8 activations a linear layer consumes come straight out of the operator
// before it, so no bf16 copy goes through memory; [SkyRL-FP8] "Performance analysis" on
// the cost of separate quantization passes). Both compute the bf16 value a bf16 framework
// would store, then quantize it exactly as the plain quantizers do (same kernels, through
// a source that computes the values instead of loading them):
//   SwiGLU : h = bf16(fl32(bf16(silu(g)) * u)),   GU[M][2F] = [gate | up];
//   RMSNorm: y = bf16(fl32(gamma * bf16(fl32(x * r)))),
//            r = fl32(1 / sqrt(mean(x^2) + eps)) per row (also returned).
// bf16(silu(g)) is the correctly rounded bf16 of the exact silu(g): an fp32 evaluation
// with a rounding-ambiguity test, an fp64 fallback for the inputs it cannot settle, and
// the series g/2 + g^2/4 for tiny g (where g/2 can sit exactly on a bf16 tie).
#include <algorithm>

#include "device.hpp"
#include "internal.hpp"
#include "quant_kernels.hpp"

namespace fp8rl {

// bf16(silu(g)) for 2^-16 <= |g| < 64, generated at build time by gen_silu_lut.py.
#include "silu_lut.inc"

// bf16 bits of the nearest-even rounding of an fp64 value: round to odd at fp32 precision
// (16 bits more than bf16, also in the subnormal range), then to nearest even.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double d) {
  float f = __double2float_rz(d);
  if ((double)f != d) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f32_to_bf16_bits(f);
}

__device__ __noinline__ uint32_t silu_bf16_bits_f64(float g) {
  const double x = g;
  double v;
  if (x >= 0.0) {
    v = x / (1.0 + exp(-x));
  } else {
    const double e = exp(x);
    v = x * e / (1.0 + e);
  }
  return f64_to_bf16_bits(v);
}

// bf16 bits of silu(g) for a bf16 value g, fast path. `slow` is set when the fp32 value
// cannot settle the rounding (then silu_bf16_bits_f64 must be used).
//  - |g| < 2^-100: silu(g) = g/2 + g^2/4 + O(g^3). g/2 is exact in fp32; it is a bf16 tie
//    only below 2^-125, where the g^2/4 term decides: up in magnitude for g > 0, down for
//    g < 0.
//  - otherwise, with e = exp(-|g|) in (0, 1]: v = g / (1 + e) for g >= 0, g e / (1 + e)
//    for g < 0. exp(-|g|) = 2^(-|g| Lh) 2^(-|g| Ll) with log2(e) = Lh + Ll and Lh of 15
//    significant bits, so |g| Lh is exact for a bf16 g; v_exp_f32 gives the first factor
//    and one FMA the second (1 - |g| Ll ln2). The quotient uses v_rcp_f32 and a Newton
//    step. v is then within a few fp32 ulps of silu(g); when it lies within 16 ulps of a
//    bf16 rounding midpoint, or g < -80 (exp(g) near the fp32 subnormal range), the fp64
//    path decides.
__device__ __forceinline__ uint32_t silu_bf16_bits_fast(float g, bool& slow) {
  constexpr float kLog2eHi = 1.44268798828125f;           // log2(e) to 15 significant bits
  constexpr float kNegLn2Log2eLo = -4.888495368504664e-06f; // -ln(2) * (log2(e) - kLog2eHi)
  const float ag = fabsf(g);
  const uint32_t ut = __float_as_uint(g * 0.5f);
  const uint32_t lowt = ut & 0xffffu;
  const uint32_t tiny_bits = (ut >> 16) + ((lowt > 0x8000u || (lowt == 0x8000u && g > 0.0f)) ? 1u : 0u);
  const float e0 = __builtin_amdgcn_exp2f(-(ag * kLog2eHi));
  const float e = __builtin_fmaf(e0, ag * kNegLn2Log2eLo, e0);
  const float d = 1.0f + e;
  const float num = g >= 0.0f ? g : g * e;
  const float r = __builtin_amdgcn_rcpf(d);
  const float v0 = num * r;
  const float v = __builtin_fmaf(__builtin_fmaf(-d, v0, num), r, v0);
  const uint32_t bits = __float_as_uint(v);
  const bool tiny = ag < 0x1p-100f;
  slow = !tiny && ((((bits & 0xffffu) - 0x7ff0u) <= 0x20u) || g < -80.0f);
  return tiny ? tiny_bits : f32_to_bf16_bits(v);
}

// bf16 bits of silu(g) computed (for the bf16 values outside the table).
__device__ __forceinline__ uint32_t silu_bf16_bits_computed(float g) {
  bool slow;
  const uint32_t b = silu_bf16_bits_fast(g, slow);
  return slow ? silu_bf16_bits_f64(g) : b;
}

// Eight SwiGLU outputs h = bf16(fl32(bf16(silu(g)) * u)) from eight gate and eight up values
// (bf16 pairs in words). bf16(silu(g)) comes from the LDS table for 2^-16 <= |g| < 64
// (almost every gate value); the others are computed after the table lookups.
__device__ __forceinline__ uint4 swiglu8(uint4 gw, uint4 uw, const uint16_t* lut) {
  const uint32_t gs[4] = {gw.x, gw.y, gw.z, gw.w}, us[4] = {uw.x, uw.y, uw.z, uw.w};
  uint32_t sb[8];
  uint32_t miss = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t p = (j & 1) ? (gs[j >> 1] >> 16) : (gs[j >> 1] & 0xffffu);
    const uint32_t off = (p & 0x7fffu) - FP8RL_SILU_LUT_LO;
    const bool in = off < FP8RL_SILU_LUT_N;
    sb[j] = lut[in ? off + (p >> 15) * FP8RL_SILU_LUT_N : 0u];
    miss |= (in ? 0u : 1u) << j;
  }
  if (miss != 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((miss >> j) & 1u) {
        const uint32_t w = gs[j >> 1];
        sb[j] = silu_bf16_bits_computed((j & 1) ? bf16_hi(w) : bf16_lo(w));
      }
  }
  uint32_t h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = us[j];
    h[j] = bf16x2_bits(__uint_as_float(sb[2 * j] << 16) * bf16_lo(w), __uint_as_float(sb[2 * j + 1] << 16) * bf16_hi(w));
  }
  return make_uint4(h[0], h[1], h[2], h[3]);
}

// SwiGLU of GU[M][2F], presented as h[M][F].
struct SwigluSrc {
  struct Raw {
    uint4 g, u;
  };
  static constexpr int kLdsBytes = (int)(2 * FP8RL_SILU_LUT_N * sizeof(uint16_t));
  const uint16_t* gu;
  int64_t F;
  uint32_t gpr;   // 1x128 groups per row = F / 128
  __device__ __forceinline__ Raw fetch8(int64_t row, int64_t col) const {
    const uint16_t* p = gu + row * 2 * F + col;
    return Raw{*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + F)};
  }
  __device__ __forceinline__ void fetch16(int64_t g, int part, Raw& a, Raw& b) const {
    const int64_t row = (int64_t)((uint64_t)g / gpr);
    const int64_t col = (g - row * gpr) * 128 + part * 16;
    a = fetch8(row, col);
    b = fetch8(row, col + 8);
  }
  __device__ __forceinline__ void prepare(void* lds, int tid, int nt) const {
    const uint4* src = reinterpret_cast<const uint4*>(kSiluLut);
    uint4* dst = reinterpret_cast<uint4*>(lds);
    for (int i = tid; i < kLdsBytes / 16; i += nt) dst[i] = src[i];
  }
  __device__ __forceinline__ uint4 make(const Raw& r, const void* lds) const {
    return swiglu8(r.g, r.u, reinterpret_cast<const uint16_t*>(lds));
  }
};

// RMSNorm output for two x values and two gamma values (bf16 pairs in words).
__device__ __forceinline__ uint32_t rms2(uint32_t xw, uint32_t gw, float r) {
  const uint32_t t = bf16x2_bits(bf16_lo(xw) * r, bf16_hi(xw) * r);
  return bf16x2_bits(bf16_lo(gw) * bf16_lo(t), bf16_hi(gw) * bf16_hi(t));
}
__device__ __forceinline__ uint4 rms8(uint4 x, uint4 g, float r) {
  return make_uint4(rms2(x.x, g.x, r), rms2(x.y, g.y, r), rms2(x.z, g.z, r), rms2(x.w, g.w, r));
}

// RMSNorm of X[M][K] with per-row r (already computed), presented as y[M][K].
struct RmsSrc {
  struct Raw {
    uint4 x, g;
    float r;
  };
  static constexpr int kLdsBytes = 0;
  const uint16_t* x;
  const uint16_t* gamma;
  const float* rstd;
  int64_t C;
  uint32_t gpr;
  __device__ __forceinline__ Raw fetch8(int64_t row, int64_t col) const {
    return Raw{*reinterpret_cast<const uint4*>(x + row * C + col), *reinterpret_cast<const uint4*>(gamma + col),
               rstd[row]};
  }
  __device__ __forceinline__ void fetch16(int64_t g, int part, Raw& a, Raw& b) const {
    const int64_t row = (int64_t)((uint64_t)g / gpr);
    const int64_t col = (g - row * gpr) * 128 + part * 16;
    a = fetch8(row, col);
    b = fetch8(row, col + 8);
  }
  __device__ __forceinline__ void prepare(void*, int, int) const {}
  __device__ __forceinline__ uint4 make(const Raw& r, const void*) const { return rms8(r.x, r.g, r.r); }
};

// h[M][F] in bf16 (the unfused SwiGLU): 8 outputs per thread and step, grid-stride.
__global__ __launch_bounds__(256) void k_swiglu_bf16(SwigluSrc src, uint16_t* __restrict__ h, int64_t n8) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[SwigluSrc::kLdsBytes];
  src.prepare(lds, threadIdx.x, 256);
  __syncthreads();
  const int64_t per_row = src.F / 8;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n8; t += (int64_t)gridDim.x * 256) {
    const int64_t row = t / per_row;
    const int64_t col = (t - row * per_row) * 8;
    *reinterpret_cast<uint4*>(h + row * src.F + col) = src.make(src.fetch8(row, col), lds);
  }
}

// Workgroups for the grid-stride kernels that fill an LDS table first: enough to fill the
// chip several times over, few enough that the table copies stay small.
constexpr int64_t kTableGrid = 256 * 8;

// One workgroup (256 threads) per row of X[M][K]; thread t holds the 16-value chunks
// t, t + 256, ... (NCH of them, K <= NCH * 4096). The sum of squares is exact per element
// in fp64 and reduced in a fixed order, so every launch of this kernel gives the same r.
//   kMode 1: r and y (bf16);  2: r and the 1x128 FP8 rows of y.
template <int NCH, int kMode, bool kPow2>
__global__ __launch_bounds__(256) void k_rmsnorm_rows(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ gamma, int64_t K, float eps,
                                                      float* __restrict__ rstd, uint16_t* __restrict__ y,
                                                      uint8_t* __restrict__ q, float* __restrict__ s) {
  __shared__ double red[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (int)(K / 16);
  const uint16_t* xr = x + row * K;
  uint4 a[NCH], b[NCH];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + 256 * i;
    a[i] = make_uint4(0, 0, 0, 0);
    b[i] = a[i];
    if (c < nch) {
      const uint4* p = reinterpret_cast<const uint4*>(xr + c * 16);
      a[i] = p[0];
      b[i] = p[1];
    }
    const uint32_t w[8] = {a[i].x, a[i].y, a[i].z, a[i].w, b[i].x, b[i].y, b[i].z, b[i].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
      ss = __builtin_fma(lo, lo, ss);
      ss = __builtin_fma(hi, hi, ss);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
  if (tid == 0) rstd[row] = r;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + 256 * i;
    const bool valid = c < nch;
    uint4 ya = make_uint4(0, 0, 0, 0), yb = ya;
    if (valid) {
      const uint4* gp = reinterpret_cast<const uint4*>(gamma + c * 16);
      ya = rms8(a[i], gp[0], r);
      yb = rms8(b[i], gp[1], r);
    }
    if constexpr (kMode == 1) {
      if (valid) {
        uint4* yp = reinterpret_cast<uint4*>(y + row * K + c * 16);
        yp[0] = ya;
        yp[1] = yb;
      }
    } else {
      // 8 consecutive lanes hold one 1x128 group; every lane takes part in the shuffles.
      const float amax = group_amax<8>(pk_max_u16(mag8(ya), mag8(yb)));
      const BlockScale bs = group_scale<kPow2>(amax);
      if (valid) {
        const uint2 lo = quant8<kPow2>(ya.x, ya.y, ya.z, ya.w, bs);
        const uint2 hi = quant8<kPow2>(yb.x, yb.y, yb.z, yb.w, bs);
        *reinterpret_cast<uint4*>(q + row * K + c * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        if ((c & 7) == 0) s[row * (K / 128) + c / 8] = bs.s;
      }
    }
  }
}

// r only (the first launch of the column-wise form): one wave per row, four rows per
// workgroup. Lane l sums the squares of the 8-value chunks l, l + 64, ... of its row in
// fp64 (each square of a bf16 value is exact), then the wave reduces by a fixed butterfly,
// so every launch gives the same r (within 2^-41 of the exact sum's, far inside the margin
// the oracle's ambiguity test leaves).
__global__ __launch_bounds__(256) void k_rmsnorm_r(const uint16_t* __restrict__ x, int64_t M, int64_t K, float eps,
                                                   float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;                                              // whole wave
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * K);
  const int nch = (int)(K / 8);
  double ss = 0.0;
#pragma unroll 8
  for (int c = lane; c < nch; c += 64) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
      ss = __builtin_fma(lo, lo, ss);
      ss = __builtin_fma(hi, hi, ss);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) rstd[row] = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
}

// ---------------------------------------------------------------------------------------
// Launchers (arguments validated by the C ABI layer).
// ---------------------------------------------------------------------------------------
hipError_t launch_swiglu_bf16(const uint16_t* gu, int64_t M, int64_t F, uint16_t* h, hipStream_t stream) {
  const SwigluSrc src{gu, F, (uint32_t)(F / 128)};
  const int64_t n8 = M * F / 8;
  const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, kTableGrid);
  hipLaunchKernelGGL(k_swiglu_bf16, dim3((unsigned)blocks), dim3(256), 0, stream, src, h, n8);
  return hipGetLastError();
}

hipError_t launch_swiglu_quant(const uint16_t* gu, int64_t M, int64_t F, uint8_t* q, float* s, uint8_t* qt,
                               float* st, bool pow2, hipStream_t stream) {
  const SwigluSrc src{gu, F, (uint32_t)(F / 128)};
  if (qt == nullptr) {
    const int64_t ngroups = M * (F / 128);
    const dim3 grid((unsigned)std::min<int64_t>((ngroups * 8 + 255) / 256, kTableGrid));
    if (pow2)
      hipLaunchKernelGGL((k_quant_rows_1x128<SwigluSrc, true>), grid, dim3(256), 0, stream, src, q, s, ngroups);
    else
      hipLaunchKernelGGL((k_quant_rows_1x128<SwigluSrc, false>), grid, dim3(256), 0, stream, src, q, s, ngroups);
  } else {
    const dim3 grid((unsigned)((F / 128) * (M / 128)));
    if (pow2)
      hipLaunchKernelGGL((k_quant_tile<SwigluSrc, false, true>), grid, dim3(512), 0, stream, src, M, F, q, s, qt, st);
    else
      hipLaunchKernelGGL((k_quant_tile<SwigluSrc, false, false>), grid, dim3(512), 0, stream, src, M, F, q, s, qt,
                         st);
  }
  return hipGetLastError();
}

template <int kMode, bool kPow2>
static hipError_t launch_rms_rows(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                                  float* rstd, uint16_t* y, uint8_t* q, float* s, hipStream_t stream) {
  const dim3 grid((unsigned)M), block(256);
  const int64_t nch = K / 16;
  if (nch <= 256)
    hipLaunchKernelGGL((k_rmsnorm_rows<1, kMode, kPow2>), grid, block, 0, stream, x, gamma, K, eps, rstd, y, q, s);
  else if (nch <= 512)
    hipLaunchKernelGGL((k_rmsnorm_rows<2, kMode, kPow2>), grid, block, 0, stream, x, gamma, K, eps, rstd, y, q, s);
  else if (nch <= 1024)
    hipLaunchKernelGGL((k_rmsnorm_rows<4, kMode, kPow2>), grid, block, 0, stream, x, gamma, K, eps, rstd, y, q, s);
  else if (nch <= 2048)
    hipLaunchKernelGGL((k_rmsnorm_rows<8, kMode, kPow2>), grid, block, 0, stream, x, gamma, K, eps, rstd, y, q, s);
  else
    hipLaunchKernelGGL((k_rmsnorm_rows<16, kMode, kPow2>), grid, block, 0, stream, x, gamma, K, eps, rstd, y, q, s);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                               uint16_t* y, float* rstd, hipStream_t stream) {
  return launch_rms_rows<1, false>(x, gamma, M, K, eps, rstd, y, nullptr, nullptr, stream);
}

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                                float* rstd, uint8_t* q, float* s, uint8_t* qt, float* st, bool pow2,
                                hipStream_t stream) {
  if (qt == nullptr)
    return pow2 ? launch_rms_rows<2, true>(x, gamma, M, K, eps, rstd, nullptr, q, s, stream)
                : launch_rms_rows<2, false>(x, gamma, M, K, eps, rstd, nullptr, q, s, stream);
  // Column-wise groups need 128 whole rows per tile: r first, then the tile kernel.
  hipLaunchKernelGGL(k_rmsnorm_r, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream, x, M, K, eps, rstd);
  if (hipError_t e = hipGetLastError()) return e;
  const RmsSrc src{x, gamma, rstd, K, (uint32_t)(K / 128)};
  const dim3 grid((unsigned)((K / 128) * (M / 128)));
  if (pow2)
    hipLaunchKernelGGL((k_quant_tile<RmsSrc, false, true>), grid, dim3(512), 0, stream, src, M, K, q, s, qt, st);
  else
    hipLaunchKernelGGL((k_quant_tile<RmsSrc, false, false>), grid, dim3(512), 0, stream, src, M, K, q, s, qt, st);
  return hipGetLastError();
}

}  // namespace fp8rl
