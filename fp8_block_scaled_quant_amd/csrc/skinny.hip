// Block-scaled FP8 GEMM for few rows (M <= 256): the rollout decode shape, where 256 token
// rows meet a large weight and the weight stream from HBM sets the pace ([SkyRL-FP8]
// "Performance analysis": decode is memory-bound on the weight reads; activation groups
// 1x128, weight blocks 128x128 as for the training GEMMs).
//   C[m][n] = sum_kb sA[m * sa_ld + kb] * sB[(n / 128) * sb_ld_n + kb * sb_ld_k]
//             * sum_{k in kb} A[m][k] * B[n][k]
//
// Design (gfx950):
// * Every workgroup takes MR of the rows (MR = 256, 128 or 64; rows past M read as zero)
//   and a contiguous run of F 16-row fragments of B; the launch holds ceil(M / MR) row
//   parts times N / (16 F) fragment runs, 256 workgroups for the decode shapes (one per
//   CU). Every workgroup copies its MR x 128 slice of A from L2 per K block, and each
//   fragment run is read by all row parts, so MR trades the replicated A reads (MR x 128
//   bytes per CU per K block) against B's (16 F x 128): a 4096-column weight takes
//   MR = 64, F = 4 (16 KB per CU per K block instead of 34 KB with MR = 256, F = 1). The
//   row parts of one fragment run go to the same XCD, one after another, so B comes from
//   HBM once and from that XCD's L2 after.
// * NW waves (4 in use); wave w owns A rows (MR/NW) w .. (MR/NW)(w+1)-1 against all F
//   fragments of B, i.e. reads MR/64 A and F B fragments from LDS per K block against
//   F MR/64 MFMAs.
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

constexpr int kSkinnyLag = 3;

template <int F, int NW, int MR>
struct SkinnyShape {
  static constexpr int NT = NW * 64;
  static constexpr int FM = MR / (16 * NW);           // A fragments per wave
  static constexpr int BN = 16 * F;
  static constexpr int CR = NT / 8;                   // rows per copy (8 lanes per 128-byte row)
  static constexpr int LA = MR / CR;                  // A copies per thread
  static constexpr int LB = (BN + CR - 1) / CR;       // B copies per thread
  static constexpr int OFF_B = MR * 128;
  static constexpr int OFF_SA = OFF_B + LB * CR * 128;
  // one 64-float scale slot per wave for sA (rows 0..255 are slots 0..3) and for sB: every
  // wave's copy lands in its own slot, even an empty one (which writes zeros)
  static constexpr int OFF_SB = OFF_SA + NW * 256;
  static constexpr int STAGE = OFF_SB + NW * 256;
  static constexpr int LDS = 3 * STAGE;
  static_assert(CR % 16 == 0, "swizzle phase must repeat across copies");
  static_assert(FM >= 1 && MR % CR == 0 && MR <= 256, "row part shape");
  static_assert(F <= 64, "one B fragment scale per lane of wave 0");
};

}  // namespace

template <int F, int NW, int MR, bool kF32>
__global__ __launch_bounds__(NW * 64) void k_gemm_skinny(GemmParams p) {
  using S = SkinnyShape<F, NW, MR>;
  constexpr int FM = S::FM;
  constexpr int WR = 16 * FM;                           // A rows per wave
  static_assert(S::LDS <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t M = p.M, N = p.N, K = p.K;
  // Workgroup b: XCD b % 8; its row part is (b / 8) % ms and its fragment run
  // 8 ((b / 8) / ms) + b % 8, so the ms row parts of a run share an XCD and follow each
  // other in dispatch order. The grid is rounded up to whole groups of 8 runs.
  const int64_t ms = (M + MR - 1) / MR;
  const int64_t q8 = blockIdx.x >> 3;
  const int64_t mpart = q8 % ms, run = (q8 / ms) * 8 + (blockIdx.x & 7);
  const int64_t n0 = run * S::BN, m0 = mpart * MR;
  if (n0 >= N) return;                                  // uniform: a padding workgroup
  const int nkb = (int)(K / 128);
  const int64_t rows_a = (M - m0) < MR ? (M - m0) : MR;
  const int64_t rows_b = (N - n0) < S::BN ? (N - n0) : S::BN;
  const int fvalid = (int)(rows_b / 16);                // fragments inside N (N % 16 == 0)

  // Operand copies: thread t moves 16 bytes of row t/8 (+CR per copy), chunk t%8 swizzled.
  const int lr = tid >> 3;
  const uint32_t off0 = (uint32_t)(lr * K) + (uint32_t)(swz(lr, tid & 7) << 4);
  const uint32_t bytesA = (uint32_t)((rows_a - 1) * K + 128), bytesB = (uint32_t)((rows_b - 1) * K + 128);
  // Scale copies: waves 0..3 fetch sA of rows 64w + lane; wave 0 also fetches the F fragment
  // scales of B (lanes past the last valid fragment repeat it); every other copy goes
  // through an empty descriptor, so that every wave counts the same number of copies.
  const uint8_t* Ap = p.A + m0 * K;
  const float* sAp = p.sA + m0 * p.sa_ld;
  const uint32_t offSA = (uint32_t)(((wave & 3) * 64 + lane) * p.sa_ld * 4);
  const uint32_t bytesSA = wave < 4 ? (uint32_t)((rows_a - 1) * p.sa_ld * 4 + 4) : 0u;
  const int fl = lane < fvalid ? lane : fvalid - 1;
  const uint32_t offSB = (uint32_t)(((n0 + 16 * fl) >> 7) * p.sb_ld_n * 4);
  const uint32_t bytesSB = wave == 0 ? (uint32_t)(((N - 1) >> 7) * p.sb_ld_n * 4 + 4) : 0u;

  auto issue = [&](int kb, uint32_t st) __attribute__((always_inline)) {
    const bool live = kb < nkb;
    const int kbc = live ? kb : 0;
    // One descriptor per operand and K block; copy `it` adds its first row to the lane
    // offset, and lanes whose offset passes the descriptor's range read zeros.
    const v4i ra = make_rsrc(Ap + kbc * 128, live ? bytesA : 0u);
#pragma unroll
    for (int it = 0; it < S::LA; ++it)
      dma16(ra, off0 + (uint32_t)(it * S::CR) * (uint32_t)K, st + (it * S::NT + wave * 64) * 16);
    const v4i rb = make_rsrc(p.B + n0 * K + kbc * 128, live ? bytesB : 0u);
#pragma unroll
    for (int it = 0; it < S::LB; ++it)
      dma16(rb, off0 + (uint32_t)(it * S::CR) * (uint32_t)K, st + S::OFF_B + (it * S::NT + wave * 64) * 16);
    dma4(make_rsrc(sAp + kbc, live ? bytesSA : 0u), offSA, st + S::OFF_SA + wave * 256);
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
    const int64_t m = m0 + wave * WR + 16 * j + (lane & 15);
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

template <int MR, int F>
static hipError_t launch_skinny_f(const GemmParams& p, bool f32, hipStream_t stream) {
  constexpr int NW = kSkinnyWaves;
  const int64_t runs = (p.N + 16 * F - 1) / (16 * F), ms = (p.M + MR - 1) / MR;
  const int64_t blocks = (runs + 7) / 8 * 8 * ms;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (f32)
    hipLaunchKernelGGL((k_gemm_skinny<F, NW, MR, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_skinny<F, NW, MR, false>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

// The (MR, F) configurations built, in the order they are considered.
struct SkinnyCfg {
  int mr, f;
  hipError_t (*launch)(const GemmParams&, bool, hipStream_t);
};
static const SkinnyCfg kSkinnyCfgs[] = {
    {256, 1, launch_skinny_f<256, 1>},  {256, 2, launch_skinny_f<256, 2>},  {256, 3, launch_skinny_f<256, 3>},
    {256, 4, launch_skinny_f<256, 4>},  {256, 6, launch_skinny_f<256, 6>},  {256, 8, launch_skinny_f<256, 8>},
    {128, 2, launch_skinny_f<128, 2>},  {128, 3, launch_skinny_f<128, 3>},  {128, 4, launch_skinny_f<128, 4>},
    {128, 6, launch_skinny_f<128, 6>},  {128, 8, launch_skinny_f<128, 8>},  {128, 12, launch_skinny_f<128, 12>},
    {64, 4, launch_skinny_f<64, 4>},    {64, 6, launch_skinny_f<64, 6>},    {64, 8, launch_skinny_f<64, 8>},
    {64, 12, launch_skinny_f<64, 12>},  {64, 16, launch_skinny_f<64, 16>},
};

// For each row-part size MR: the smallest F that needs at most 256 workgroups (one per
// CU), else its largest F. Among those, the least copy traffic per CU per K block over
// the launch (rounds of 256 workgroups x (min(MR, M) rows of A + 16 F rows of B)), then
// the fewest padded rows (MR x row parts), then the larger MR.
hipError_t launch_gemm_skinny(const GemmParams& p, bool f32, hipStream_t stream) {
  const int64_t frags = (p.N + 15) / 16;
  const SkinnyCfg* best = nullptr;
  int64_t best_cost = 0, best_pad = 0;
  for (int mr : {256, 128, 64}) {
    const SkinnyCfg* pick = nullptr;
    const int64_t ms = (p.M + mr - 1) / mr;
    for (const SkinnyCfg& c : kSkinnyCfgs) {
      if (c.mr != mr) continue;
      pick = &c;
      if ((frags + c.f - 1) / c.f * ms <= 256) break;
    }
    const int64_t wgs = (frags + pick->f - 1) / pick->f * ms;
    const int64_t cost = (wgs + 255) / 256 * ((p.M < mr ? p.M : mr) + 16 * pick->f), pad = mr * ms;
    if (best == nullptr || cost < best_cost || (cost == best_cost && pad < best_pad)) {
      best = pick;
      best_cost = cost;
      best_pad = pad;
    }
  }
  return best->launch(p, f32, stream);
}

}  // namespace fp8rl
