// Block-scaled FP8 GEMM for the decode shape: few activation rows (256 token rows in the
// rollout) against a large installed weight, where the weight stream from HBM sets the
// pace ([SkyRL-FP8] "Performance analysis": generation is memory-bound on the weight reads,
// activations are quantized on the fly while weights and scales stay fixed; activation
// groups 1x128 and weight blocks 128x128, as for the training GEMMs).
//   C[m][n] = sum_kb sA(m, kb) * sB[(n / 128) * sb_ld_n + kb * sb_ld_k]
//             * sum_{k in kb} A(m, k) * B(n, k)
// A (the quantized activations) is addressed with a row stride and a K-block stride, so it
// may be row-major ([M][K]: strides K and 128) or K-block-major ([K/128][M][128]: strides
// 128 and 128 M, each K block's slice contiguous); its scales likewise.
// B is row-major [N][K], or in the decode layout (see k_decode_layout below): every
// 16-row x 128-byte tile stored in the order the matrix instruction reads it, so that every
// load instruction of the weight stream reads 1 KB of consecutive bytes.
//
// Design (gfx950):
// * Every weight byte is used by exactly one wave, so the weights bypass LDS: wave w loads
//   its FW 16-row fragments of B for K block kb straight into VGPRs (two 16-byte buffer
//   loads per lane and fragment, in the operand layout of the MFMA), P K blocks ahead of
//   the block it computes.
// * The activations are shared by all waves of the workgroup: the MT x 128 bytes of A and
//   the MT row scales of K block kb go to LDS by direct global->LDS copies, into one of P + 1
//   stages, also P K blocks ahead; so are the F = NW FW fragment scales of B.
// * Workgroup = MT rows (a row part) x a run of F fragments; a launch has ceil(M / MT) row
//   parts times N / (16 F) runs. Consecutive workgroups b go to XCD b % 8; the row parts of a
//   run share an XCD and run together, so B comes from HBM once and from that XCD's L2 for
//   the other row parts.
// * One v_mfma_scale_f32_16x16x128_f8f6f4 (neutral E8M0 scales) per 16x16 tile and K block,
//   computed transposed (first operand: 16 rows of B, second: 16 rows of A), so a lane's four
//   outputs share one row m and one 128-row block of B; its fp32 product is folded into the
//   accumulator with one FMA per output, kLag MFMAs after it was issued.
// * K loop: wait for this wave's loads of kb (those of kb+1 .. kb+P-1 stay in flight),
//   barrier (every wave's copies of kb landed; every wave is done with kb-1, whose stage and
//   register set are refilled next), issue kb+P, compute kb. Past the last K block the loads
//   go through empty descriptors (zeros, no memory access), so every step counts the same.
// * bf16 X: a first launch quantizes X 1x128 into a K-block-major copy in the caller's
//   workspace (k_quant_kbmajor: one workgroup per K block x 32 rows), and the GEMM reads that
//   copy, each K block's MT rows one contiguous run. Quantizing inside the GEMM launch instead
//   needs a device-scope hand-over between workgroups (release, counter, acquire), and on a
//   chip whose eight L2s are not coherent with each other every such fence writes back or
//   invalidates an L2: measured, that costs 20 to 45 us per call against a few us for the
//   second launch.
// Deterministic: fixed K order, no atomics.
#include "device.hpp"
#include "internal.hpp"

namespace fp8rl {

namespace {

constexpr int kDecodeLag = 3;
// Every load and copy of the K loop is inline assembly, and every wait for them is explicit:
// the compiler inserts no wait of its own in the loop. (With the loads expressed as compiler
// intrinsics, its wait analysis merged the states of the loop's guarded steps and of the
// loop back-edge, and in some unrolled steps waited for the next K block's loads as well,
// i.e. ran without prefetch.) A weight register is therefore written by the hardware after
// the compiler believes it holds its value; the kernel reads it only after the wait for
// its K block, and the register must not be moved, copied, spilled or reused before then.
// The kernel is built for at most 256 VGPRs and no AGPRs (two waves per SIMD), and a test
// scans the compiled code of every configuration for any access to a weight register
// between its load and the wait that covers it.
template <int OFF>
__device__ __forceinline__ v4i wload16(v4i rsrc, uint32_t voff) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate buffer offset");
  v4i r;
  // s_nop 4: wait states after a VALU write of the descriptor's SGPRs (see dma16).
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2, 0 offen offset:%3"
               : "=v"(r)
               : "v"(voff), "s"(rsrc), "i"(OFF)
               : "memory");
  return r;
}
// Workgroup barrier with no wait of its own (__syncthreads() would also wait for every
// copy in flight, prefetches included); the K loop waits for exactly the copies it needs
// before it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

template <int MT, int NW, int FW, int P>
struct DecodeShape {
  static constexpr int NT = NW * 64;
  static constexpr int F = NW * FW;                  // B fragments per workgroup
  static constexpr int BN = 16 * F;
  static constexpr int XF = MT / 16;                 // A fragments
  static constexpr int NS = P + 1;                   // stages / register sets
  static constexpr int LX = MT * 8 / NT;             // A copies (16 B per lane) per wave per K block
  static constexpr int OFF_SA = MT * 128;
  static constexpr int OFF_SB = OFF_SA + MT * 4;
  static constexpr int OFF_NIL = OFF_SB + 256;       // scale copies of waves that have none
  static constexpr int STAGE = OFF_NIL + 256;
  static constexpr int LDS = NS * STAGE;
  static constexpr int SA_WAVES = (MT + 63) / 64;    // waves that copy A's row scales
  static constexpr int SB_WAVE = SA_WAVES % NW;      // the wave that copies B's fragment scales
  static constexpr int OPS = MT * 8 / NT + 2 + 2 * FW; // vector-memory operations per wave and K block
  static_assert(MT % 64 == 0 && MT <= 256, "row part");
  static_assert((MT * 8) % NT == 0 && (NT / 8) % 16 == 0, "A copy split keeps the swizzle phase");
  static_assert(F <= 64, "one B fragment scale per lane");
  static_assert(P >= 1 && P <= 8, "prefetch distance");
};

}  // namespace

// 1x128 quantization of bf16 X[M][K] into the K-block-major copy: workgroup u covers K block
// kb = u / mch and rows 32 (u % mch) .. +31 (mch = ceil(M / 32)); group (m, kb) -> payload
// q[(kb M + m) * 128 ..], scale s[kb M + m]. 256 threads, 8 lanes per group, 16 elements
// each. Bytes and scales equal those of the row-major 1x128 quantizer ([AIS] quantizer
// equation; [Jet-RL] 1x128 groups).
__global__ __launch_bounds__(256) void k_quant_kbmajor(const uint16_t* __restrict__ x, int M, int64_t K, int mch,
                                                       uint8_t* __restrict__ q, float* __restrict__ s) {
  const int tid = threadIdx.x;
  const int u = (int)blockIdx.x;
  const int kb = u / mch;
  const int m = (u - kb * mch) * 32 + (tid >> 3);
  const int part = tid & 7;
  const bool valid = m < M;
  uint4 a = make_uint4(0, 0, 0, 0), b = a;
  if (valid) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)m * K + (int64_t)kb * 128 + part * 16);
    a = src[0];
    b = src[1];
  }
  const float amax = group_amax<8>(pk_max_u16(mag8(a), mag8(b)));
  const BlockScale bs = block_scale(amax);
  if (valid) {
    const int64_t g = (int64_t)kb * M + m;
    const uint2 lo = quant8<false>(a.x, a.y, a.z, a.w, bs);
    const uint2 hi = quant8<false>(b.x, b.y, b.z, b.w, bs);
    *reinterpret_cast<uint4*>(q + g * 128 + part * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    if (part == 0) s[g] = bs.s;
  }
}

hipError_t launch_quant_kbmajor(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, hipStream_t stream) {
  const int64_t mch = (M + 31) / 32, units = (K / 128) * mch;
  if (units > 0x7fffffff || M > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quant_kbmajor, dim3((unsigned)units), dim3(256), 0, stream, x, (int)M, K, (int)mch, q, s);
  return hipGetLastError();
}

// kTiledB: B is in the decode layout.
template <int MT, int NW, int FW, int P, bool kF32, bool kTiledB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_decode(DecodeParams p) {
  using S = DecodeShape<MT, NW, FW, P>;
  constexpr int NT = S::NT, XF = S::XF, NS = S::NS, LX = S::LX;
  static_assert(S::LDS <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = (int)p.M;
  const int64_t N = p.N, K = p.K;
  const int nkb = (int)(K / 128);
  const int ms = (M + MT - 1) / MT;
  const int q8 = (int)(blockIdx.x >> 3);
  const int mpart = q8 % ms, run = (q8 / ms) * 8 + (int)(blockIdx.x & 7);
  const int64_t n0 = (int64_t)run * S::BN;
  const int m0 = mpart * MT;
  if (n0 >= N) return;                                 // padding workgroup (uniform)

  const int64_t rows_b = (N - n0) < S::BN ? (N - n0) : S::BN;
  const int fvalid = (int)(rows_b / 16);

  // A copies: thread t moves 16 bytes of tile row t/8 (+ NT/8 per copy), LDS chunk t%8,
  // global chunk swz(row, t%8) (see frag_offsets). Rows past M read zeros (row-major) or
  // another K block's rows (K-block-major); their results are never stored.
  const int lr = tid >> 3;
  const uint32_t offA = (uint32_t)((int64_t)(m0 + lr) * p.a_ld) + (uint32_t)(swz(lr, tid & 7) << 4);
  const uint64_t a_total = (uint64_t)M * (uint64_t)K;
  // A's row scales: wave w < SA_WAVES copies rows 64 w + lane.
  const bool cA = wave < S::SA_WAVES;
  const uint32_t offSA = (uint32_t)((int64_t)(m0 + (wave & 3) * 64 + lane) * p.sa_ld * 4);
  const uint64_t sa_total = (uint64_t)M * (uint64_t)nkb * 4;
  // B's fragment scales: lane f holds fragment f's block scale (lanes past the last valid
  // fragment repeat it).
  const bool cB = wave == S::SB_WAVE;
  const int fl = lane < fvalid ? lane : fvalid - 1;
  const uint32_t offSB = (uint32_t)(((n0 + 16 * fl) >> 7) * p.sb_ld_n * 4);
  const uint64_t sb_total = (uint64_t)(((N - 1) >> 7) * p.sb_ld_n + (int64_t)(nkb - 1) * p.sb_ld_k + 1) * 4;
  // B fragments. Row-major: lane l reads row (l & 15) of the fragment, bytes 16 g and
  // 64 + 16 g of the K block (g = l >> 4), the operand layout of the MFMA. Decode layout:
  // the fragment's tile for K block kb is 2 KB at (fragment * nkb + kb) * 2048; lane l reads
  // bytes 16 l (first half) and 1024 + 16 l (second half).
  const uint32_t offB = kTiledB ? (uint32_t)((int64_t)wave * FW * 16 * K + 16 * lane)
                                : (uint32_t)((int64_t)(wave * FW * 16 + (lane & 15)) * K + 16 * (lane >> 4));
  const uint32_t bytesB = (uint32_t)(kTiledB ? rows_b * K : (rows_b - 1) * K + 128);
  const uint8_t* Bp = p.B + n0 * K;

  auto rng = [](uint64_t total, uint64_t used) __attribute__((always_inline)) -> uint32_t {
    const uint64_t r = total - used;
    return r > 0xffffffffull ? 0xffffffffu : (uint32_t)r;
  };

  v4i wlo[NS][FW], whi[NS][FW];
  // The weight loads of K block kb into register set `set`.
  auto issue_b = [&](int kb, auto setc) __attribute__((always_inline)) {
    constexpr int set = decltype(setc)::value;
    const bool live = kb < nkb;
    const int kbc = live ? kb : 0;
    const v4i rb = make_rsrc(Bp + (kTiledB ? 0 : kbc * 128), live ? bytesB : 0u);
    const uint32_t ok = kTiledB ? (uint32_t)kbc * 2048u : 0u;
#pragma unroll
    for (int i = 0; i < FW; ++i) {
      const uint32_t o = offB + ok + (uint32_t)(i * 16) * (uint32_t)K;
      wlo[set][i] = wload16<0>(rb, o);
      whi[set][i] = wload16<kTiledB ? 1024 : 64>(rb, o);
    }
  };
  // The activation and scale copies of K block kb into stage `set`. Every wave issues both
  // scale copies; a wave without scales to copy issues them through empty descriptors (no
  // memory access) into the stage's unused slot, so that every wave has the same number of
  // operations in flight and one wait count serves all.
  const uint32_t st0 = lds_addr(smem);
  const uint32_t dSA = cA ? S::OFF_SA + wave * 256 : S::OFF_NIL;
  const uint32_t dSB = cB ? S::OFF_SB : S::OFF_NIL;
  auto issue_a = [&](int kb, auto setc) __attribute__((always_inline)) {
    constexpr int set = decltype(setc)::value;
    const uint32_t st = st0 + set * S::STAGE;
    const bool live = kb < nkb;
    const int64_t kbc = live ? kb : 0;
    const v4i ra = make_rsrc(p.A + kbc * p.a_kb, live ? rng(a_total, (uint64_t)(kbc * p.a_kb)) : 0u);
#pragma unroll
    for (int it = 0; it < LX; ++it)
      dma16(ra, offA + (uint32_t)(it * (NT / 8)) * (uint32_t)p.a_ld, st + (it * NT + wave * 64) * 16);
    dma4(make_rsrc(p.sA + kbc * p.sa_kb, live && cA ? rng(sa_total, (uint64_t)(kbc * p.sa_kb) * 4) : 0u), offSA,
         st + dSA);
    dma4(make_rsrc(p.sB + kbc * p.sb_ld_k, live && cB ? rng(sb_total, (uint64_t)(kbc * p.sb_ld_k) * 4) : 0u), offSB,
         st + dSB);
  };
  // Operations per wave and K block: LX activation copies, 2 scale copies, 2 FW weight
  // loads (OPS). At the wait of K block kb those of kb+1 .. kb+P-1 stay outstanding.
  static_assert((P - 1) * S::OPS <= 63, "vmcnt range");
  auto wait_block = [&]() __attribute__((always_inline)) { wait_vmem_n<(P - 1) * S::OPS>(); };

  v4f acc[FW][XF];
#pragma unroll
  for (int i = 0; i < FW; ++i)
#pragma unroll
    for (int j = 0; j < XF; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const FragOffsets fa = frag_offsets(0, lane);
  const uint32_t o_sa = S::OFF_SA + (lane & 15) * 4;

  auto compute = [&](auto setc) __attribute__((always_inline)) {
    constexpr int set = decltype(setc)::value;
    const uint32_t st = st0 + set * S::STAGE;
    const uint32_t a_lo = st + fa.lo, a_hi = st + fa.hi, sa_ad = st + o_sa;
    const uint32_t sb_ad = st + S::OFF_SB + wave * FW * 4;
    float sb[FW];
    static_for<0, FW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      sb[i] = ds_read4f<i * 4>(sb_ad);
    });
    // Every X fragment of the K block (and its row scale) is requested at once; fragment j
    // is then awaited alone (LDS reads complete in issue order), so the reads of the later
    // fragments overlap the MFMAs of the earlier ones.
    v4i xlo[XF], xhi[XF];
    float sx[XF];
    static_for<0, XF>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      xlo[j] = ds_read16<j * 2048>(a_lo);
      xhi[j] = ds_read16<j * 2048>(a_hi);
      sx[j] = ds_read4f<j * 64>(sa_ad);
    });
    v8i bf[FW];
    v4f pipe[kDecodeLag + 1];
    float prod[kDecodeLag + 1];
    auto fold = [&](int u) __attribute__((always_inline)) {
      const int j = u / FW, i = u % FW;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[i][j][r] = __builtin_fmaf(pipe[u % (kDecodeLag + 1)][r], prod[u % (kDecodeLag + 1)], acc[i][j][r]);
    };
    static_for<0, XF>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      lds_wait<3 * (XF - 1 - j)>();     // 3 reads per later fragment may still be in flight
      hold(xlo[j]);
      hold(xhi[j]);
      hold(sx[j]);
      if constexpr (j == 0) {
        static_for<0, FW>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          hold(sb[i]);
          bf[i] = join(wlo[set][i], whi[set][i]);
        });
      }
      const v8i xf = join(xlo[j], xhi[j]);
#pragma unroll
      for (int i = 0; i < FW; ++i) {
        const int t = j * FW + i;
        pipe[t % (kDecodeLag + 1)] = mfma_fp8(bf[i], xf, v4f{0.f, 0.f, 0.f, 0.f}, 127, 127);
        prod[t % (kDecodeLag + 1)] = sx[j] * sb[i];
        if (t >= kDecodeLag) fold(t - kDecodeLag);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
#pragma unroll
    for (int u = (XF * FW > kDecodeLag ? XF * FW - kDecodeLag : 0); u < XF * FW; ++u) fold(u);
    // Tie the accumulators to this point: the MFMAs and folds of K block kb stay ahead of the
    // next step's wait and barrier. (Without it the compiler sinks them below the wait for
    // K block kb + 1, so each block's arithmetic waits for the next block's loads.)
#pragma unroll
    for (int i = 0; i < FW; ++i)
#pragma unroll
      for (int j = 0; j < XF; ++j) hold(acc[i][j]);
  };

  {
    // Prologue: K blocks 0 .. P-1 in the loop's own order (copies, then weights), so the
    // first step's wait is the same as every other step's. The loop issues loads and copies
    // in every step, also in the at most NS - 1 steps past the last K block (empty
    // descriptors); only the compute is skipped there. Every path through the loop thus
    // issues the same operations and the wait counts hold on all of them.
    static_for<0, P>([&](auto sc) {
      issue_a(decltype(sc)::value, sc);
      issue_b(decltype(sc)::value, sc);
    });
    for (int kb0 = 0; kb0 < nkb; kb0 += NS) {
      static_for<0, NS>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        const int kb = kb0 + s;
        wait_block();
        barrier_only();
        constexpr auto nxt = std::integral_constant<int, (s + P) % NS>{};
        issue_a(kb + P, nxt);
        issue_b(kb + P, nxt);
        if (kb < nkb) compute(sc);
      });
    }
    // The loads of the last P steps (past the last K block: zeros) are never read; they still
    // write their registers when they complete. Tying every weight register to this wait keeps
    // the compiler from giving any of them to another value before then.
    wait_vmem();
    static_for<0, NS>([&](auto sc) {
      static_for<0, FW>([&](auto ic) {
        hold(wlo[decltype(sc)::value][decltype(ic)::value]);
        hold(whi[decltype(sc)::value][decltype(ic)::value]);
      });
    });

    // Epilogue: lane holds C[m][n .. n+3] for m = m0 + 16 j + (lane & 15) and
    // n = n0 + 16 (wave FW + i) + 4 (lane >> 4).
#pragma unroll
    for (int j = 0; j < XF; ++j) {
      const int m = m0 + 16 * j + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < FW; ++i) {
        const int64_t n = n0 + 16 * (wave * FW + i) + 4 * (lane >> 4);
        if (n >= N) continue;
        if constexpr (kF32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + (int64_t)m * p.ldc + n) =
              make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
          uint2 v;
          v.x = f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16);
          v.y = f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc + n) = v;
        }
      }
    }
  }
}

// The same product, restructured around what bounds the kernel above on the decode shapes.
// Per-step timestamps of a probe build showed the waves waiting for their loads only about a
// tenth of each K step; most of a step went to issuing the step's copies and loads (every wave
// of the CU issued them in one burst right after the barrier and stalled in the texture unit's
// queue), then to the MFMAs, one after the other; a quarter of the issued operations were
// scale copies, most of them through empty descriptors.
// * Every row scale of A and fragment scale of B for the whole K range goes to LDS once,
//   before the K loop (at most KPRE K blocks, for M K < 2^32); no scale copies per step.
// * The copies and loads of K block kb + P are issued between the MFMAs of K block kb, a few
//   before each X fragment, from descriptors made once per launch (the K block's offset goes
//   into the instruction's scalar offset, which the hardware range check includes).
// * Every step runs the same code, the steps past the last K block included: their loads and
//   copies go through an empty descriptor (no memory access; registers get zeros, a stage
//   keeps zeros or an earlier K block's codes), so every operand is finite, and their scales are
//   read from a zero-filled LDS slot: each fold is fma(P, 0, acc) = acc (acc is never -0), and
//   the results do not change. With no branch in the K loop every path issues the same loads
//   into the same registers.
// Measured against k_gemm_decode on the rollout decode shapes (M = 256, K = 4096, weights in
// the decode layout streamed from HBM): 20% faster at N = 4096, 8% at N = 12288, 6% at
// N = 24576; at N = 24576 the form with two row parts per workgroup and the weights staged in
// LDS (WL) is another 4% (back-to-back launches) to 10% (kernel trace) faster. With the
// copies moved to two copy waves (NP = 2), which leaves the compute waves nothing to issue
// but LDS reads and MFMAs, the decode-layout launches were faster again, in three interleaved
// rounds of back-to-back launches: N = 4096 (one row part, FW = 1) 5% with the weights in
// the last-level cache and 1.5% streamed from HBM, N = 12288 (one row part, FW = 3) 10% and
// 4%, N = 24576 (two row parts) 6% and 3%; four copy waves were no faster than two.
constexpr int KPRE = 64;

template <int OFF>
__device__ __forceinline__ v4i wload16s(v4i rsrc, uint32_t voff, uint32_t soff) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate buffer offset");
  v4i r;
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4"
               : "=v"(r)
               : "v"(voff), "s"(rsrc), "s"(soff), "i"(OFF)
               : "memory");
  return r;
}
// dma16 (device.hpp) with a scalar byte offset.
__device__ __forceinline__ void dma16s(v4i rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
               : "memory", "m0");
}

// MT rows per wave, NW fragment groups of FW fragments, RP row parts per workgroup: the
// workgroup's NW RP waves cover MTW = MT RP rows x F = NW FW fragments, wave w taking rows
// MT (w / NW) .. + MT - 1 and fragment group w % NW. WL (decode layout only): the
// workgroup's weight tiles are copied into the stage once and every wave reads its fragments
// from there, instead of each wave loading its fragments into registers (with RP = 2 this
// halves the weight bytes a CU moves). NP > 0 (with WL): NP further copy waves issue every
// copy of the stage and the NW RP compute waves issue none, so that no compute wave stalls
// on the texture unit's queue between its MFMAs.
template <int MT, int NW, int FW, int P, int RP = 1, bool WL = false, int NP = 0>
struct PreShape {
  static constexpr int NWT = NW * RP;                // compute waves per workgroup
  static constexpr int NT = NWT * 64;
  static constexpr int NPT = NP * 64;                // copy-wave threads
  static constexpr int NTA = NT + NPT;
  static constexpr int MTW = MT * RP;                // activation rows per workgroup
  static constexpr int F = NW * FW;                  // B fragments per workgroup
  static constexpr int BN = 16 * F;
  static constexpr int XF = MT / 16;                 // A fragments per wave
  static constexpr int NS = P + 1;                   // stages / register sets
  static constexpr int LX = MTW * 8 / NT;            // A copies (16 B per lane) per wave and K block
  static constexpr int LW = WL ? 2 * F / NWT : 0;    // B copies (1 KB halves of fragment tiles) per wave
  static constexpr int XS = MTW * 128;               // A bytes per K block
  static constexpr int STAGE = XS + (WL ? F * 2048 : 0);
  static constexpr int ZB = MTW * 4 > 256 ? MTW * 4 : 256;
  static constexpr int OFF_ZERO = NS * STAGE;        // ZB zero bytes: the scales of dead K blocks
  static constexpr int OFF_PA = OFF_ZERO + ZB;       // A's row scales [KPRE][MTW]
  static constexpr int SBW = WL ? 16 : 64;           // B fragment scales per K block
  static constexpr int OFF_PB = OFF_PA + KPRE * MTW * 4;  // B's fragment scales [KPRE][SBW]
  static constexpr int LDS = OFF_PB + KPRE * SBW * 4;
  static constexpr int OPS = NP ? 0 : LX + (WL ? LW : 2 * FW);  // operations per compute wave and K block
  static constexpr int LXP = NP ? MTW * 8 / (NP * 64) : 0;   // A copies per copy wave and K block
  static constexpr int LWP = NP ? 2 * F / NP : 0;            // B copies per copy wave and K block
  static constexpr int OPSP = LXP + LWP;
  static constexpr int SA_COPIES = MTW / 64;         // 64-row scale copies per K block
  static_assert(MTW % 64 == 0 && MTW <= 256 && (MTW * 8) % NT == 0 && (NT / 8) % 16 == 0, "row part");
  static_assert(MT % 16 == 0 && F <= SBW && SA_COPIES <= NWT, "fragments");
  static_assert(!WL || (2 * F) % NWT == 0, "B copies split evenly over the waves");
  static_assert(P >= 1 && (P - 1) * OPS <= 63 && (P - 1) * OPSP <= 63, "vmcnt range");
  static_assert(NP == 0 || (WL && NP % 2 == 0 && (MTW * 8) % NPT == 0 && (2 * F) % NP == 0), "copy waves");
  static_assert(LDS <= (WL ? 160 : 80) * 1024, "LDS budget (two workgroups per CU without WL)");
};

template <int MT, int NW, int FW, int P, int RP, bool WL, int NP, bool kF32, bool kTiledB>
__global__ __launch_bounds__((NW * RP + NP) * 64) __attribute__((amdgpu_waves_per_eu(NP ? 3 : 2))) void k_gemm_decode_pre(DecodeParams p) {
  using S = PreShape<MT, NW, FW, P, RP, WL, NP>;
  constexpr int NT = S::NT, XF = S::XF, NS = S::NS, LX = S::LX, MTW = S::MTW;
  static_assert(!WL || kTiledB, "weights through LDS need the decode layout");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rp = wave / NW, wf = wave - rp * NW;     // row part, fragment group
  const int M = (int)p.M;
  const int64_t N = p.N, K = p.K;
  const int nkb = (int)(K / 128);
  const int ms = (M + MTW - 1) / MTW;
  const int q8 = (int)(blockIdx.x >> 3);
  const int mpart = q8 % ms, run = (q8 / ms) * 8 + (int)(blockIdx.x & 7);
  const int64_t n0 = (int64_t)run * S::BN;
  const int m0 = mpart * MTW;
  if (n0 >= N) return;                                 // padding workgroup (uniform)
  const int64_t rows_b = (N - n0) < S::BN ? (N - n0) : S::BN;
  const int fvalid = (int)(rows_b / 16);
  const uint32_t st0 = lds_addr(smem);

  auto rng = [](uint64_t total, uint64_t used) __attribute__((always_inline)) -> uint32_t {
    const uint64_t r = total - used;
    return r > 0xffffffffull ? 0xffffffffu : (uint32_t)r;
  };

  // Zero the stages and the dead-block scale slot before any copy writes LDS.
  for (int o = tid * 16; o < S::OFF_PA; o += S::NTA * 16) *reinterpret_cast<uint4*>(smem + o) = make_uint4(0, 0, 0, 0);
  __syncthreads();

  // Scales of the whole K range: A's rows [kb][m] (one copy of 64 rows per K block and 64-row
  // part) and B's fragment scales [kb][f] (lane f < SBW: fragment f's block scale; lanes past the
  // last valid fragment repeat it), spread over the waves. The K loop's waits bound only the newest
  // operations, so these older copies are complete at its first wait.
  {
    const uint64_t sa_total = (uint64_t)M * (uint64_t)nkb * 4;
    const uint64_t sb_total = (uint64_t)(((N - 1) >> 7) * p.sb_ld_n + (int64_t)(nkb - 1) * p.sb_ld_k + 1) * 4;
    const int fl = lane < fvalid ? lane : fvalid - 1;
    const uint32_t offSB = (uint32_t)(((n0 + 16 * fl) >> 7) * p.sb_ld_n * 4);
    const int nA = nkb * S::SA_COPIES, ncp = nA + nkb;
    for (int c = wave; c < ncp; c += S::NWT + NP) {
      if (c < nA) {
        const int kb = c / S::SA_COPIES, w = c - kb * S::SA_COPIES;
        const uint64_t used = (uint64_t)((int64_t)kb * p.sa_kb) * 4;
        dma4(make_rsrc(p.sA + (int64_t)kb * p.sa_kb, rng(sa_total, used)),
             (uint32_t)((int64_t)(m0 + w * 64 + lane) * p.sa_ld * 4), st0 + S::OFF_PA + (uint32_t)((kb * MTW + w * 64) * 4));
      } else if (lane < S::SBW) {
        const int kb = c - nA;
        const uint64_t used = (uint64_t)((int64_t)kb * p.sb_ld_k) * 4;
        dma4(make_rsrc(p.sB + (int64_t)kb * p.sb_ld_k, rng(sb_total, used)), offSB,
             st0 + S::OFF_PB + (uint32_t)(kb * S::SBW * 4));
      }
    }
  }

  // Descriptors for the whole launch. A copies: thread t moves 16 bytes of row t/8 (+ NT/8 per
  // copy), LDS chunk t%8, global chunk swz(row, t%8); rows past M read zeros in every K block.
  // B fragments: as in k_gemm_decode. The range of B's descriptor is the run's rows, all of K.
  const v4i rA = make_rsrc(p.A, (uint32_t)((uint64_t)M * (uint64_t)K));
  const v4i rZ = make_rsrc(p.A, 0u);
  const uint8_t* Bp = p.B + n0 * K;
  const v4i rB = make_rsrc(Bp, (uint32_t)(rows_b * K));
  const int lr = tid >> 3;
  const uint32_t offA = (uint32_t)((int64_t)(m0 + lr) * p.a_ld) + (uint32_t)(swz(lr, tid & 7) << 4);
  const uint32_t offB = kTiledB ? (uint32_t)((int64_t)wf * FW * 16 * K + 16 * lane)
                                : (uint32_t)((int64_t)(wf * FW * 16 + (lane & 15)) * K + 16 * (lane >> 4));
  // WL: copy c of wave w moves half h = w + c NWT of the workgroup's fragment tiles (fragment
  // h / 2, bytes 1024 (h % 2) .. + 1023 of its 2 KB tile) to the same place in the stage.
  uint32_t offW[S::LW > 0 ? S::LW : 1], ldsW[S::LW > 0 ? S::LW : 1];
#pragma unroll
  for (int c = 0; c < S::LW; ++c) {
    const int h = wave + c * S::NWT;
    offW[c] = (uint32_t)((int64_t)(h >> 1) * 16 * K) + (uint32_t)((h & 1) * 1024 + 16 * lane);
    ldsW[c] = (uint32_t)(S::XS + (h >> 1) * 2048 + (h & 1) * 1024);
  }

  // Copy waves: copy c of copy wave w moves A copies as the compute waves' copies do, with the
  // NP copy waves' threads in place of the compute threads, and B halves h = w + c NP. Each
  // K step: wait for this wave's copies of the current K block, meet the compute waves at the
  // barrier, issue the copies of K block kb + P into the stage refilled next. Same barriers and
  // stage protocol as the compute waves, which issue no copies.
  if constexpr (NP > 0) {
    if (wave >= S::NWT) {
      const int pt = tid - NT, pw = wave - S::NWT, plr = pt >> 3;
      const uint32_t poffA = (uint32_t)((int64_t)(m0 + plr) * p.a_ld) + (uint32_t)(swz(plr, pt & 7) << 4);
      uint32_t poffW[S::LWP], pldsW[S::LWP];
#pragma unroll
      for (int c = 0; c < S::LWP; ++c) {
        const int h = pw + c * NP;
        poffW[c] = (uint32_t)((int64_t)(h >> 1) * 16 * K) + (uint32_t)((h & 1) * 1024 + 16 * lane);
        pldsW[c] = (uint32_t)(S::XS + (h >> 1) * 2048 + (h & 1) * 1024);
      }
      auto pissue = [&](auto oc, auto setc, int kb) __attribute__((always_inline)) {
        constexpr int o = decltype(oc)::value, set = decltype(setc)::value;
        const bool live = kb < nkb;
        if constexpr (o < S::LXP) {
          const uint32_t soff = live ? (uint32_t)((int64_t)kb * p.a_kb) : 0u;
          dma16s(live ? rA : rZ, poffA + (uint32_t)(o * (S::NPT / 8)) * (uint32_t)p.a_ld, soff,
                 st0 + set * S::STAGE + (o * S::NPT + pw * 64) * 16);
        } else {
          dma16s(live ? rB : rZ, poffW[o - S::LXP], live ? (uint32_t)kb * 2048u : 0u, st0 + set * S::STAGE + pldsW[o - S::LXP]);
        }
      };
      static_for<0, P>([&](auto sc) {
        static_for<0, S::OPSP>([&](auto oc) { pissue(oc, sc, decltype(sc)::value); });
      });
      for (int kb0 = 0; kb0 < nkb; kb0 += NS) {
        static_for<0, NS>([&](auto sc) {
          constexpr int c = decltype(sc)::value;
          wait_vmem_n<(P - 1) * S::OPSP>();
          barrier_only();
          static_for<0, S::OPSP>([&](auto oc) { pissue(oc, std::integral_constant<int, (c + P) % NS>{}, kb0 + c + P); });
        });
      }
      wait_vmem();                                   // no LDS write outlives the workgroup
      return;
    }
  }

  v4i wlo[WL ? 1 : NS][FW], whi[WL ? 1 : NS][FW];
  // Operation o of K block kb into stage / register set `set`: the LX activation copies, then
  // the FW pairs of weight loads.
  auto issue_op = [&](auto oc, auto setc, int kb) __attribute__((always_inline)) {
    constexpr int o = decltype(oc)::value, set = decltype(setc)::value;
    const bool live = kb < nkb;
    if constexpr (o < LX) {
      const uint32_t soff = live ? (uint32_t)((int64_t)kb * p.a_kb) : 0u;
      dma16s(live ? rA : rZ, offA + (uint32_t)(o * (NT / 8)) * (uint32_t)p.a_ld, soff,
             st0 + set * S::STAGE + (o * NT + wave * 64) * 16);
    } else if constexpr (WL) {
      dma16s(live ? rB : rZ, offW[o - LX], live ? (uint32_t)kb * 2048u : 0u, st0 + set * S::STAGE + ldsW[o - LX]);
    } else {
      constexpr int i = (o - LX) / 2;
      const uint32_t soff = live ? (uint32_t)kb * (kTiledB ? 2048u : 128u) : 0u;
      const uint32_t off = offB + (uint32_t)(i * 16) * (uint32_t)K;
      if constexpr ((o - LX) % 2 == 0) wlo[set][i] = wload16s<0>(live ? rB : rZ, off, soff);
      else whi[set][i] = wload16s<kTiledB ? 1024 : 64>(live ? rB : rZ, off, soff);
    }
  };

  v4f acc[FW][XF];
#pragma unroll
  for (int i = 0; i < FW; ++i)
#pragma unroll
    for (int j = 0; j < XF; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const FragOffsets fa = frag_offsets(0, lane);

  // K block kb from stage / register set `set`, issuing K block kb + P's operations into set
  // `nset` between its MFMAs (OPS of them over the XF fragment slots).
  auto step = [&](auto setc, auto nsetc, int kb) __attribute__((always_inline)) {
    constexpr int set = decltype(setc)::value;
    const uint32_t st = st0 + set * S::STAGE;
    const uint32_t a_lo = st + (uint32_t)(rp * MT * 128) + fa.lo, a_hi = st + (uint32_t)(rp * MT * 128) + fa.hi;
    const bool live = kb < nkb;
    const uint32_t sa_ad = st0 + (live ? S::OFF_PA + (uint32_t)(kb * MTW * 4) : S::OFF_ZERO) + (uint32_t)((rp * MT + (lane & 15)) * 4);
    const uint32_t sb_ad = st0 + (live ? S::OFF_PB + (uint32_t)(kb * S::SBW * 4) : S::OFF_ZERO) + (uint32_t)(wf * FW * 4);
    float sb[FW];
    static_for<0, FW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      sb[i] = ds_read4f<i * 4>(sb_ad);
    });
    v4i blo[FW], bhi[FW];                 // WL: the wave's fragment tiles from the stage
    if constexpr (WL) {
      const uint32_t w_ad = st + S::XS + (uint32_t)(wf * FW * 2048 + 16 * lane);
      static_for<0, FW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        blo[i] = ds_read16<i * 2048>(w_ad);
        bhi[i] = ds_read16<i * 2048 + 1024>(w_ad);
      });
    }
    // A fragment j (rows 16 j ..) and its row scales, XD fragments in flight (3 LDS reads
    // each; lgkmcnt counts up to 15).
    constexpr int XD = (15 - FW - (WL ? 2 * FW : 0)) / 3 < XF ? (15 - FW - (WL ? 2 * FW : 0)) / 3 : XF;
    static_assert(XD >= 1, "LDS read window");
    v4i xlo[XF], xhi[XF];
    float sx[XF];
    auto read_x = [&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      xlo[j] = ds_read16<j * 2048>(a_lo);
      xhi[j] = ds_read16<j * 2048>(a_hi);
      sx[j] = ds_read4f<j * 64>(sa_ad);
    };
    static_for<0, XD>(read_x);
    v8i bf[FW];
    v4f pipe[kDecodeLag + 1];
    float prod[kDecodeLag + 1];
    auto fold = [&](int t) __attribute__((always_inline)) {
      const int j = t / FW, i = t % FW;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[i][j][r] = __builtin_fmaf(pipe[t % (kDecodeLag + 1)][r], prod[t % (kDecodeLag + 1)], acc[i][j][r]);
    };
    static_for<0, XF>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      // this slot's share of the next K block's operations
      static_for<j * S::OPS / XF, (j + 1) * S::OPS / XF>([&](auto oc) { issue_op(oc, nsetc, kb + P); });
      constexpr int later = (XF - 1 - j) < (XD - 1) ? (XF - 1 - j) : (XD - 1);
      lds_wait<3 * later>();
      hold(xlo[j]);
      hold(xhi[j]);
      hold(sx[j]);
      if constexpr (j == 0) {
        static_for<0, FW>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          hold(sb[i]);
          if constexpr (WL) {
            hold(blo[i]);
            hold(bhi[i]);
            bf[i] = join(blo[i], bhi[i]);
          } else {
            bf[i] = join(wlo[set][i], whi[set][i]);
          }
        });
      }
      const v8i xf = join(xlo[j], xhi[j]);
#pragma unroll
      for (int i = 0; i < FW; ++i) {
        const int t = j * FW + i;
        pipe[t % (kDecodeLag + 1)] = mfma_fp8(bf[i], xf, v4f{0.f, 0.f, 0.f, 0.f}, 127, 127);
        prod[t % (kDecodeLag + 1)] = sx[j] * sb[i];
        if (t >= kDecodeLag) fold(t - kDecodeLag);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (j + XD < XF) read_x(std::integral_constant<int, j + XD>{});
    });
#pragma unroll
    for (int t = (XF * FW > kDecodeLag ? XF * FW - kDecodeLag : 0); t < XF * FW; ++t) fold(t);
    // The MFMAs and folds of this K block stay ahead of the next step's wait and barrier.
#pragma unroll
    for (int i = 0; i < FW; ++i)
#pragma unroll
      for (int j = 0; j < XF; ++j) hold(acc[i][j]);
  };

  {
    static_for<0, P>([&](auto sc) {
      static_for<0, S::OPS>([&](auto oc) { issue_op(oc, sc, decltype(sc)::value); });
    });
    for (int kb0 = 0; kb0 < nkb; kb0 += NS) {
      static_for<0, NS>([&](auto sc) {
        constexpr int c = decltype(sc)::value;
        wait_vmem_n<(P - 1) * S::OPS>();             // this wave's operations of K block kb0 + c
        barrier_only();                              // every wave's copies; every wave done with the set refilled next
        step(sc, std::integral_constant<int, (c + P) % NS>{}, kb0 + c);
      });
    }
    // The loads of the last P steps (past the last K block: zeros) are never read; they still
    // write their registers when they complete. Tying every weight register to this wait keeps
    // the compiler from giving any of them to another value before then.
    wait_vmem();
    if constexpr (!WL) {
      static_for<0, NS>([&](auto sc) {
        static_for<0, FW>([&](auto ic) {
          hold(wlo[decltype(sc)::value][decltype(ic)::value]);
          hold(whi[decltype(sc)::value][decltype(ic)::value]);
        });
      });
    }

#pragma unroll
    for (int j = 0; j < XF; ++j) {
      const int m = m0 + MT * rp + 16 * j + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < FW; ++i) {
        const int64_t n = n0 + 16 * (wf * FW + i) + 4 * (lane >> 4);
        if (n >= N) continue;
        if constexpr (kF32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + (int64_t)m * p.ldc + n) =
              make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
          uint2 v;
          v.x = f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16);
          v.y = f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc + n) = v;
        }
      }
    }
  }
}

// Decode layout of a row-major FP8 weight W[N][K] (N % 16 == 0, K % 128 == 0): for 16-row
// fragment f and K block kb, the 2 KB tile at (f * (K / 128) + kb) * 2048 holds, for lane
// l = 0..63, row 16 f + (l & 15), bytes kb * 128 + 16 (l >> 4) .. + 15 at 16 l and bytes
// kb * 128 + 64 + 16 (l >> 4) .. + 15 at 1024 + 16 l. A permutation of each fragment's
// 16 K bytes: the values are the trainer's bytes, unchanged. Thread t moves 16 bytes.
__global__ __launch_bounds__(256) void k_decode_layout(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                       int64_t N, int64_t K) {
  const int64_t nkb = K / 128;
  const int64_t chunks = N * K / 16;
  for (int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x; d < chunks; d += (int64_t)gridDim.x * 256) {
    const int64_t tile = d >> 7;                       // 128 chunks of 16 bytes per tile
    const int in = (int)(d & 127), h = in >> 6, l = in & 63;
    const int64_t f = tile / nkb, kb = tile - f * nkb;
    const uint4* s = reinterpret_cast<const uint4*>(src + (f * 16 + (l & 15)) * K + kb * 128 + h * 64 + 16 * (l >> 4));
    reinterpret_cast<uint4*>(dst)[d] = *s;
  }
}

hipError_t launch_decode_layout(const uint8_t* src, uint8_t* dst, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t chunks = N * K / 16;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_decode_layout, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, N, K);
  return hipGetLastError();
}

template <int MT, int NW, int FW, int P>
static hipError_t launch_decode_cfg(const DecodeParams& p, bool f32, hipStream_t stream) {
  using S = DecodeShape<MT, NW, FW, P>;
  const int64_t runs = (p.N + S::BN - 1) / S::BN, ms = (p.M + MT - 1) / MT;
  const int64_t blocks = (runs + 7) / 8 * 8 * ms;
  if (blocks > 0x7fffffff || p.M > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), b(NW * 64);
#define FP8RL_DECODE_LAUNCH(F32, TILED) \
  hipLaunchKernelGGL((k_gemm_decode<MT, NW, FW, P, F32, TILED>), g, b, 0, stream, p)
  if (f32) {
    if (p.tiled_b) FP8RL_DECODE_LAUNCH(true, true); else FP8RL_DECODE_LAUNCH(true, false);
  } else {
    if (p.tiled_b) FP8RL_DECODE_LAUNCH(false, true); else FP8RL_DECODE_LAUNCH(false, false);
  }
#undef FP8RL_DECODE_LAUNCH
  return hipGetLastError();
}

template <int MT, int NW, int FW, int P, int RP = 1, bool WL = false, int NP = 0>
static hipError_t launch_decode_pre_cfg(const DecodeParams& p, bool f32, hipStream_t stream) {
  using S = PreShape<MT, NW, FW, P, RP, WL, NP>;
  const int64_t runs = (p.N + S::BN - 1) / S::BN, ms = (p.M + S::MTW - 1) / S::MTW;
  const int64_t blocks = (runs + 7) / 8 * 8 * ms;
  if (blocks > 0x7fffffff || p.M > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), b(S::NTA);
#define FP8RL_DECODE_PRE_LAUNCH(F32, TILED) \
  hipLaunchKernelGGL((k_gemm_decode_pre<MT, NW, FW, P, RP, WL, NP, F32, TILED>), g, b, 0, stream, p)
  if constexpr (WL) {
    if (f32) FP8RL_DECODE_PRE_LAUNCH(true, true); else FP8RL_DECODE_PRE_LAUNCH(false, true);
  } else if (f32) {
    if (p.tiled_b) FP8RL_DECODE_PRE_LAUNCH(true, true); else FP8RL_DECODE_PRE_LAUNCH(true, false);
  } else {
    if (p.tiled_b) FP8RL_DECODE_PRE_LAUNCH(false, true); else FP8RL_DECODE_PRE_LAUNCH(false, false);
  }
#undef FP8RL_DECODE_PRE_LAUNCH
  return hipGetLastError();
}

// Row part MT = 64 and 4 waves; fragments per wave FW = 1, 2 or 3 with the prefetch distance
// that measured fastest for it. On the rollout decode shapes (M = 256, K = 4096,
// N = 4096 / 12288 / 24576, weights in the decode layout and streamed from HBM): for
// k_gemm_decode (P = 3, 2, 2) a row part of 128, four fragments per wave or deeper prefetch
// were slower or equal, and with more than three fragments per wave (or 128 rows and three)
// the kernel no longer fits in 256 VGPRs; for k_gemm_decode_pre P = 3, 3, 2, and two K blocks
// per barrier were no faster. Each register-weight configuration fits two workgroups per CU
// (registers and LDS); the staged forms (decode-layout weights copied into LDS by two copy
// waves) fit one, so they are used only where the grid is at most one workgroup per CU. For
// FW = 2 the staged form was slower (its grid starts at 256 workgroups).
using DecodeLaunch = hipError_t (*)(const DecodeParams&, bool, hipStream_t);
struct DecodeCfg {
  int fw;
  DecodeLaunch launch;
  DecodeLaunch staged;   // decode-layout weights through LDS, or null
};
static const DecodeCfg kDecodeCfgs[] = {
    {3, launch_decode_cfg<64, 4, 3, 2>, nullptr},
    {2, launch_decode_cfg<64, 4, 2, 2>, nullptr},
    {1, launch_decode_cfg<64, 4, 1, 3>, nullptr},
};
static const DecodeCfg kDecodePreCfgs[] = {
    {3, launch_decode_pre_cfg<64, 4, 3, 2>, launch_decode_pre_cfg<64, 4, 3, 2, 1, true, 2>},
    {2, launch_decode_pre_cfg<64, 4, 2, 3>, nullptr},
    {1, launch_decode_pre_cfg<64, 4, 1, 3>, launch_decode_pre_cfg<64, 4, 1, 3, 1, true, 2>},
};

// Kernel: k_gemm_decode_pre when its scale tables hold the K range (K / 128 <= KPRE) and the
// activations fit its 32-bit offsets; k_gemm_decode otherwise. Configuration: the most
// fragments per wave (the longest weight run per copied activation row) whose grid still has
// a workgroup for every one of the 256 CUs; one fragment per wave when none has. On the
// decode shapes this picks the fastest measured configuration for every N: FW = 1 at
// N = 4096, FW = 3 at N = 12288 and 24576.
hipError_t launch_gemm_decode(const DecodeParams& p, bool f32, hipStream_t stream) {
  const bool pre = p.K / 128 <= KPRE && (uint64_t)p.M * (uint64_t)p.K <= 0xffffffffull;
  if (pre && p.tiled_b) {
    // Decode-layout weights: two row parts per workgroup sharing one LDS copy of the weights,
    // when that grid still has a workgroup for every CU (the N = 24576 decode shape); else one
    // row part, as below.
    using SW = PreShape<64, 4, 3, 2, 2, true, 2>;
    if ((p.N + SW::BN - 1) / SW::BN * ((p.M + SW::MTW - 1) / SW::MTW) >= 256)
      return launch_decode_pre_cfg<64, 4, 3, 2, 2, true, 2>(p, f32, stream);
  }
  const DecodeCfg* cfgs = pre ? kDecodePreCfgs : kDecodeCfgs;
  const int64_t ms = (p.M + 63) / 64;
  for (int i = 0; i < 3; ++i) {
    const DecodeCfg& c = cfgs[i];
    const int64_t runs = (p.N + 64 * c.fw - 1) / (64 * c.fw);
    if (ms * runs >= 256 || c.fw == 1)
      return (p.tiled_b && c.staged && ms * runs <= 256 ? c.staged : c.launch)(p, f32, stream);
  }
  return hipErrorInvalidValue;   // not reached: the last configuration always applies
}

}  // namespace fp8rl
