// Block-scaled FP8 GEMM on gfx950 MFMA: C[m][n] = sum_kb sA[m,kb] * sB(n,kb) * sum_{k in kb} A[m][k] B[n][k]
// with A[M][K], B[N][K] both K-contiguous ("TN"), fp32 accumulation.
//   forward : A = X (1x128 scales per row), B = W (128x128 block scales)
//   DGrad   : A = dY (1x128), B = W^T bytes (block scales read transposed)
//   WGrad   : A = dY^T, B = X^T (both 128x1 groups: one scale per row per 128 tokens)
// ([SkyRL-FP8] TL;DR: FP8 linear-layer GEMMs; [Jet-RL] "Quantization scheme": forward,
// DGrad and WGrad in FP8 with 1x128 / 128x128 / 128x1 groups.)
//
// Design (gfx950):
// * One v_mfma_scale_f32_16x16x128_f8f6f4 (neutral E8M0 scales) consumes exactly one
//   128-wide K block of a 16x16 output tile, starting from a zero accumulator. Its fp32
//   partial is then folded into the running sum with one FMA per output:
//   acc += P * (sA * sB).
// * Tiles are computed transposed (MFMA first operand = B rows n, second = A rows m), so
//   the 4 outputs a lane holds share one m and four consecutive n inside one 128-row
//   block of B: one scale product per lane per K block for the forward/DGrad recipe.
// * Per K block, the workgroup stages BM x 128 bytes of A, BN x 128 bytes of B and their
//   scales in LDS with direct global->LDS loads (no VGRP staging), double-buffered so
//   the loads of block kb+1 overlap the MFMAs of block kb; one barrier per K block.
//   The two stages are distinct LDS objects and the K loop is unrolled by two, so each
//   compute phase reads a statically known stage.
// * Rows are 128 bytes with a 16-byte-chunk XOR swizzle to keep fragment reads
//   bank-conflict free.
// * Workgroups are mapped to tiles XCD-aware (contiguous tile ranges per XCD) and in
//   groups of 8 m-tiles, so concurrently running tiles share operand rows in L2.
// Deterministic: fixed K order, no atomics; bf16 output is the RNE rounding of the same
// fp32 accumulator the fp32 output mode stores.
#include "device.hpp"
#include "internal.hpp"

namespace fp8rl {

template <int BM, int BN, int WM, int WN, bool kRowB, bool kF32>
__global__ __launch_bounds__(WM* WN * 64) void k_gemm_blockscaled(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int NSB = kRowB ? BN : 64;                       // B scale slots per stage
  constexpr int OFF_B = BM * 128;
  constexpr int OFF_SA = OFF_B + BN * 128;
  constexpr int OFF_SB = OFF_SA + BM * 4;
  constexpr int STAGE = OFF_SB + NSB * 4;
  static_assert(BM % WM == 0 && BN % WN == 0 && TM % 16 == 0 && TN % 16 == 0, "tile shape");
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "load split");
  static_assert(NT >= BM + NSB, "one scale load per wave");
  static_assert(kRowB || TN <= 128, "a wave's n range must sit inside one 128-row scale block");
  __shared__ __attribute__((aligned(16))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave % WM) * TM;
  const int wn0 = (wave / WM) * TN;

  const int64_t M = p.M, N = p.N, K = p.K;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  constexpr int GM = 8;
  const int group = L / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_group = L - group * GM * tiles_n;
  const int64_t m0 = (int64_t)(first_m + in_group % gsz) * BM;
  const int64_t n0 = (int64_t)(in_group / gsz) * BN;
  const int nkb = (int)(K / 128);
  const int64_t nb0 = n0 >> 7;                                  // first 128-row B block of the tile
  const int64_t nbl = (N - 1) >> 7;                             // last B block

  // Staged loads go through raw buffer descriptors whose range ends at the last valid row
  // of the tile, so rows past the end of A / B (and their scales) read as zero without a
  // memory access; their results are never stored. Per lane: one 32-bit offset per load.
  constexpr int LA = BM * 8 / NT, LB = BN * 8 / NT;
  const int64_t rows_a = min((int64_t)BM, M - m0), rows_b = min((int64_t)BN, N - n0);
  uint32_t offA[LA], offB[LB];
#pragma unroll
  for (int it = 0; it < LA; ++it) {
    const int Lc = it * NT + tid, r = Lc >> 3;
    offA[it] = (uint32_t)(r * K) + (uint32_t)(swz(r, Lc & 7) << 4);
  }
#pragma unroll
  for (int it = 0; it < LB; ++it) {
    const int Lc = it * NT + tid, r = Lc >> 3;
    offB[it] = (uint32_t)(r * K) + (uint32_t)(swz(r, Lc & 7) << 4);
  }
  const uint32_t bytesA = (uint32_t)((rows_a - 1) * K + 128), bytesB = (uint32_t)((rows_b - 1) * K + 128);
  // Scale loads: waves [0, BM/64) fetch sA of the tile rows, the next NSB/64 waves fetch sB.
  const bool sa_wave = wave < BM / 64;
  const bool sb_wave = !sa_wave && wave < BM / 64 + NSB / 64;
  const float* baseS;
  uint32_t offS, bytesS;
  int64_t sstep;  // floats per K block
  if (sa_wave) {
    baseS = p.sA + m0 * p.sa_ld;
    offS = (uint32_t)((wave * 64 + lane) * p.sa_ld * 4);
    bytesS = (uint32_t)((rows_a - 1) * p.sa_ld * 4 + 4);
    sstep = 1;
  } else if (kRowB) {
    baseS = p.sB + n0 * p.sb_ld_n;
    offS = (uint32_t)(((wave - BM / 64) * 64 + lane) * p.sb_ld_n * 4);
    bytesS = (uint32_t)((rows_b - 1) * p.sb_ld_n * 4 + 4);
    sstep = 1;
  } else {
    baseS = p.sB + nb0 * p.sb_ld_n;
    offS = (uint32_t)(lane * p.sb_ld_n * 4);
    bytesS = (uint32_t)((nbl - nb0) * p.sb_ld_n * 4 + 4);
    sstep = p.sb_ld_k;
  }
  const int s_lds = sa_wave ? OFF_SA + wave * 256 : OFF_SB + (wave - BM / 64) * 256;

  auto issue = [&](int kb, uint8_t* sm) {
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + m0 * K + kb * 128, bytesA);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + n0 * K + kb * 128, bytesB);
#pragma unroll
    for (int it = 0; it < LA; ++it) buf2lds16(ra, offA[it], sm + (it * NT + wave * 64) * 16);
#pragma unroll
    for (int it = 0; it < LB; ++it) buf2lds16(rb, offB[it], sm + OFF_B + (it * NT + wave * 64) * 16);
    if (sa_wave || sb_wave) buf2lds4(make_rsrc(baseS + kb * sstep, bytesS), offS, sm + s_lds);
  };

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* sm) {
    const float* scA = reinterpret_cast<const float*>(sm + OFF_SA);
    const float* scB = reinterpret_cast<const float*>(sm + OFF_SB);
    v8i af[FM];
    float sa[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      af[j] = load_frag(sm, wm0 + 16 * j, lane);
      sa[j] = scA[wm0 + 16 * j + (lane & 15)];
    }
    float prod[FM];
    if (!kRowB) {
      const float sb = scB[((n0 + wn0) >> 7) - nb0];
#pragma unroll
      for (int j = 0; j < FM; ++j) prod[j] = sa[j] * sb;
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const v8i bfr = load_frag(sm + OFF_B, wn0 + 16 * i, lane);
      float4 sb4;
      if (kRowB) sb4 = *reinterpret_cast<const float4*>(scB + wn0 + 16 * i + 4 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const v4f pr = mfma_fp8(bfr, af[j], v4f{0.f, 0.f, 0.f, 0.f}, 127, 127);
        if (kRowB) {
          acc[i][j][0] = __builtin_fmaf(pr[0], sa[j] * sb4.x, acc[i][j][0]);
          acc[i][j][1] = __builtin_fmaf(pr[1], sa[j] * sb4.y, acc[i][j][1]);
          acc[i][j][2] = __builtin_fmaf(pr[2], sa[j] * sb4.z, acc[i][j][2]);
          acc[i][j][3] = __builtin_fmaf(pr[3], sa[j] * sb4.w, acc[i][j][3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[r], prod[j], acc[i][j][r]);
        }
      }
    }
  };

  // K loop over pairs of blocks (stage 0 then stage 1) with a single exit, and a peeled
  // last block when the count is odd.
  issue(0, sm0);
  int kb = 0;
  for (; kb + 2 <= nkb; kb += 2) {
    wait_vmem();
    __syncthreads();
    issue(kb + 1, sm1);
    compute(sm0);
    wait_vmem();
    __syncthreads();
    if (kb + 2 < nkb) issue(kb + 2, sm0);
    compute(sm1);
  }
  if (kb < nkb) {
    wait_vmem();
    __syncthreads();
    compute(sm0);
  }

  // Epilogue: lane holds C[m][n .. n+3] of each 16x16 tile.
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t m = m0 + wm0 + 16 * j + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int64_t n = n0 + wn0 + 16 * i + 4 * (lane >> 4);
      if (n >= N) continue;
      if (kF32) {
        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + m * p.ldc + n);
        float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        if (p.accumulate) {
          const float4 o = *dst;
          v.x += o.x;
          v.y += o.y;
          v.z += o.z;
          v.w += o.w;
        }
        *dst = v;
      } else {
        uint2 v;
        v.x = f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16);
        v.y = f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + m * p.ldc + n) = v;
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool kRowB>
static hipError_t launch_cfg(const GemmParams& p, bool f32, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(WM * WN * 64);
  if (f32)
    hipLaunchKernelGGL((k_gemm_blockscaled<BM, BN, WM, WN, kRowB, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_blockscaled<BM, BN, WM, WN, kRowB, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

// Tile choice: 256x256 tiles (8 waves, 64x128 per wave) when there are enough of them to
// fill the 256 CUs; 128x128 tiles (4 waves, 64x64 per wave) otherwise.
hipError_t launch_gemm_blockscaled(const GemmParams& p, bool row_scale_b, bool f32, hipStream_t stream) {
  const int64_t big_tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
  const bool big = big_tiles >= 256;
  if (row_scale_b) {
    return big ? launch_cfg<256, 256, 4, 2, true>(p, f32, stream) : launch_cfg<128, 128, 2, 2, true>(p, f32, stream);
  }
  return big ? launch_cfg<256, 256, 4, 2, false>(p, f32, stream) : launch_cfg<128, 128, 2, 2, false>(p, f32, stream);
}

}  // namespace fp8rl
