// Block-scaled FP8 GEMM for few rows (M <= 256): the rollout decode shape, where 256 token
// rows meet a large weight and the weight stream from HBM sets the pace ([SkyRL-FP8]
// "Performance analysis": decode is memory-bound on the weight reads; activation groups
// 1x128, weight blocks 128x128 as for the training GEMMs).
//   C[m][n] = sum_kb sA[m * sa_ld + kb] * sB[(n / 128) * sb_ld_n + kb * sb_ld_k]
//             * sum_{k in kb} A[m][k] * B[n][k]
//
// Design (gfx950):
// * Every workgroup takes all M rows (up to 256, rows past M read as zero) and a contiguous
//   run of F 16-row fragments of B, so a launch of N / (16 F) workgroups (256 for the
//   decode shapes) puts one workgroup on every CU and streams each weight byte once.
// * NW waves (4 in use); wave w owns A rows (256/NW) w .. (256/NW)(w+1)-1 against all F
//   fragments of B. With 4 waves a wave reads 4 A and F B fragments from LDS per K block
//   (about 80 KB per workgroup for F = 6) against 4 F MFMAs.
// * Three LDS stages filled by direct global->LDS copies: the copies of K blocks kb+1 and
//   kb+2 are in flight while kb is computed.
// * Scales: one fp32 per A row per K block, and one per B fragment per K block (a 16-row
//   fragment never straddles a 128-row block, so a run of fragments may). The product of
//   each 16x16x128 MFMA (neutral E8M0 scales) is folded into the fp32 accumulator with one
//   FMA per output, kLag MFMAs after it was issued.
// Deterministic: fixed K order, no atomics.
#include "device.hpp"
#include "internal.hpp"

namespace fp8rl {

namespace {

constexpr int kSkinnyM = 256;   // rows per workgroup (all of M)
constexpr int kSkinnyLag = 3;

template <int F, int NW>
struct SkinnyShape {
  static constexpr int NT = NW * 64;
  static constexpr int FM = kSkinnyM / (16 * NW);     // A fragments per wave
  static constexpr int BN = 16 * F;
  static constexpr int CR = NT / 8;                   // rows per copy (8 lanes per 128-byte row)
  static constexpr int LA = kSkinnyM / CR;            // A copies per thread
  static constexpr int LB = (BN + CR - 1) / CR;       // B copies per thread
  static constexpr int OFF_B = kSkinnyM * 128;
  static constexpr int OFF_SA = OFF_B + LB * CR * 128;
  // one 64-float scale slot per wave for sA (rows 0..255 are slots 0..3) and for sB: every
  // wave's copy lands in its own slot, even an empty one (which writes zeros)
  static constexpr int OFF_SB = OFF_SA + NW * 256;
  static constexpr int STAGE = OFF_SB + NW * 256;
  static constexpr int LDS = 3 * STAGE;
  static_assert(CR % 16 == 0, "swizzle phase must repeat across copies");
};

}  // namespace

template <int F, int NW, bool kF32>
__global__ __launch_bounds__(NW * 64) void k_gemm_skinny(GemmParams p) {
  using S = SkinnyShape<F, NW>;
  constexpr int FM = S::FM;
  constexpr int WR = 16 * FM;                           // A rows per wave
  static_assert(S::LDS <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t n0 = (int64_t)blockIdx.x * S::BN;
  const int nkb = (int)(K / 128);
  const int64_t rows_a = M < kSkinnyM ? M : kSkinnyM;
  const int64_t rows_b = (N - n0) < S::BN ? (N - n0) : S::BN;
  const int fvalid = (int)(rows_b / 16);                // fragments inside N (N % 16 == 0)

  // Operand copies: thread t moves 16 bytes of row t/8 (+CR per copy), chunk t%8 swizzled.
  const int lr = tid >> 3;
  const uint32_t off0 = (uint32_t)(lr * K) + (uint32_t)(swz(lr, tid & 7) << 4);
  const uint32_t bytesA = (uint32_t)((rows_a - 1) * K + 128), bytesB = (uint32_t)((rows_b - 1) * K + 128);
  // Scale copies: waves 0..3 fetch sA of rows 64w + lane; wave 0 also fetches the F fragment
  // scales of B (lanes past the last valid fragment repeat it); every other copy goes
  // through an empty descriptor, so that every wave counts the same number of copies.
  const uint32_t offSA = (uint32_t)(((wave & 3) * 64 + lane) * p.sa_ld * 4);
  const uint32_t bytesSA = wave < 4 ? (uint32_t)((rows_a - 1) * p.sa_ld * 4 + 4) : 0u;
  const int fl = lane < fvalid ? lane : fvalid - 1;
  const uint32_t offSB = (uint32_t)(((n0 + 16 * fl) >> 7) * p.sb_ld_n * 4);
  const uint32_t bytesSB = wave == 0 ? (uint32_t)(((N - 1) >> 7) * p.sb_ld_n * 4 + 4) : 0u;

  auto issue = [&](int kb, uint32_t st) __attribute__((always_inline)) {
    const bool live = kb < nkb;
    const int kbc = live ? kb : 0;
#pragma unroll
    for (int it = 0; it < S::LA; ++it) {
      const int64_t r0 = (int64_t)it * S::CR;
      const uint32_t nb = (live && bytesA > r0 * K) ? (uint32_t)(bytesA - r0 * K) : 0u;
      dma16(make_rsrc(p.A + r0 * K + kbc * 128, nb), off0, st + (it * S::NT + wave * 64) * 16);
    }
#pragma unroll
    for (int it = 0; it < S::LB; ++it) {
      const int64_t r0 = (int64_t)it * S::CR;
      const uint32_t nb = (live && bytesB > r0 * K) ? (uint32_t)(bytesB - r0 * K) : 0u;
      dma16(make_rsrc(p.B + (n0 + r0) * K + kbc * 128, nb), off0, st + S::OFF_B + (it * S::NT + wave * 64) * 16);
    }
    dma4(make_rsrc(p.sA + kbc, live ? bytesSA : 0u), offSA, st + S::OFF_SA + wave * 256);
    dma4(make_rsrc(p.sB + (int64_t)kbc * p.sb_ld_k, live ? bytesSB : 0u), offSB, st + S::OFF_SB + wave * 256);
  };
  constexpr int kCopies = S::LA + S::LB + 2;            // copies per wave per stage

  v4f acc[F][FM];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const FragOffsets fa = frag_offsets(wave * WR, lane), fb = frag_offsets(0, lane);
  const uint32_t o_sa = S::OFF_SA + (wave * WR + (lane & 15)) * 4;

  auto compute = [&](uint32_t st) __attribute__((always_inline)) {
    const uint32_t a_lo = st + fa.lo, a_hi = st + fa.hi;
    const uint32_t b_lo = st + S::OFF_B + fb.lo, b_hi = st + S::OFF_B + fb.hi;
    const uint32_t sa_ad = st + o_sa, sb_ad = st + S::OFF_SB;
    v4i alo[FM], ahi[FM];
    float sa[FM], sb[F];
    static_for<0, FM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      alo[j] = ds_read16<j * 2048>(a_lo);
      ahi[j] = ds_read16<j * 2048>(a_hi);
      sa[j] = ds_read4f<j * 64>(sa_ad);
    });
    static_for<0, F>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      sb[i] = ds_read4f<i * 4>(sb_ad);
    });
    v4i blo = ds_read16<0>(b_lo), bhi = ds_read16<0>(b_hi);
    lds_wait<0>();
    v8i af[FM];
    static_for<0, FM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      hold(alo[j]);
      hold(ahi[j]);
      hold(sa[j]);
      af[j] = join(alo[j], ahi[j]);
    });
    static_for<0, F>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      hold(sb[i]);
    });
    hold(blo);
    hold(bhi);
    v4f pipe[kSkinnyLag + 1];
    auto fold = [&](int u) __attribute__((always_inline)) {
      const int i = u / FM, j = u % FM;
      const float sc = sa[j] * sb[i];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pipe[u % (kSkinnyLag + 1)][r], sc, acc[i][j][r]);
    };
    static_for<0, F>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      v4i nlo, nhi;
      if constexpr (i + 1 < F) {
        nlo = ds_read16<(i + 1) * 2048>(b_lo);
        nhi = ds_read16<(i + 1) * 2048>(b_hi);
      }
      const v8i bf = join(blo, bhi);
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int t = i * FM + j;
        pipe[t % (kSkinnyLag + 1)] = mfma_fp8(bf, af[j], v4f{0.f, 0.f, 0.f, 0.f}, 127, 127);
        if (t >= kSkinnyLag) fold(t - kSkinnyLag);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (i + 1 < F) {
        __builtin_amdgcn_sched_barrier(0);
        lds_wait<0>();
        hold(nlo);
        hold(nhi);
        blo = nlo;
        bhi = nhi;
      }
    });
#pragma unroll
    for (int u = (F * FM > kSkinnyLag ? F * FM - kSkinnyLag : 0); u < F * FM; ++u) fold(u);
  };

  // K loop over three stages: before computing block kb, wait until this wave's copies of
  // kb have landed (those of kb+1 may still be in flight), barrier (every wave's copies of
  // kb landed; every wave is done with kb-1, whose stage is refilled next), then start
  // copying kb+2 and compute kb.
  const uint32_t base = lds_addr(smem);
  issue(0, base);
  issue(1, base + S::STAGE);
  uint32_t cur = base, nxt2 = base + 2 * S::STAGE;
  for (int kb = 0; kb < nkb; ++kb) {
    wait_vmem_n<kCopies>();
    __syncthreads();
    issue(kb + 2, nxt2);
    compute(cur);
    nxt2 = cur;
    cur = (cur + S::STAGE == base + 3 * S::STAGE) ? base : cur + S::STAGE;
  }
  wait_vmem();   // drain the empty copies issued past the last K block

  // Epilogue: lane holds C[m][n .. n+3] of each 16x16 tile.
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t m = wave * WR + 16 * j + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < F; ++i) {
      const int64_t n = n0 + 16 * i + 4 * (lane >> 4);
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

// 4 waves of 64 rows: measured faster than 8 waves of 32 rows for every decode shape.
constexpr int kSkinnyWaves = 4;

template <int F>
static hipError_t launch_skinny_f(const GemmParams& p, bool f32, hipStream_t stream) {
  constexpr int NW = kSkinnyWaves;
  const int64_t blocks = (p.N + 16 * F - 1) / (16 * F);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (f32)
    hipLaunchKernelGGL((k_gemm_skinny<F, NW, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_skinny<F, NW, false>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

// F = fragments per workgroup: the smallest of 1, 2, 3, 4, 6, 8 that needs at most 256
// workgroups (one per CU), 8 beyond that.
hipError_t launch_gemm_skinny(const GemmParams& p, bool f32, hipStream_t stream) {
  const int64_t frags = p.N / 16;
  if (frags <= 256) return launch_skinny_f<1>(p, f32, stream);
  if (frags <= 512) return launch_skinny_f<2>(p, f32, stream);
  if (frags <= 768) return launch_skinny_f<3>(p, f32, stream);
  if (frags <= 1024) return launch_skinny_f<4>(p, f32, stream);
  if (frags <= 1536) return launch_skinny_f<6>(p, f32, stream);
  return launch_skinny_f<8>(p, f32, stream);
}

}  // namespace fp8rl
