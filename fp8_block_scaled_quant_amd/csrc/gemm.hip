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
//   acc += P * (sA * sB), kLag MFMAs later so the wave does not wait on the result.
// * Tiles are computed transposed (MFMA first operand = B rows n, second = A rows m), so
//   the 4 outputs a lane holds share one m and four consecutive n inside one 128-row
//   block of B: one scale product per lane per K block for the forward/DGrad recipe.
// * Per K block, the workgroup stages BM x 128 bytes of A, BN x 128 bytes of B and their
//   scales in LDS with direct global->LDS loads (no VGRP staging), double-buffered so
//   the loads of block kb+1 overlap the MFMAs of block kb; one barrier per K block.
//   The two stages are distinct LDS objects and the K loop is unrolled by two, so each
//   compute phase reads a statically known stage.
// * Row scales (1x128 / 128x1 groups: one fp32 or E8M0 dword per row per K block) come SK
//   K blocks at a time (SK = 8, or 4 when B's row scales come too) into a double-buffered
//   LDS ring: one cache-line request per row per SK K blocks instead of one per row per K
//   block. Those 4-byte loads were a third of the kernel's L2 read requests, and the
//   number of requests in flight per CU is what limits the operand copies.
// * Rows are 128 bytes with a 16-byte-chunk XOR swizzle to keep fragment reads
//   bank-conflict free.
// * Workgroups are mapped to tiles XCD-aware (contiguous tile ranges per XCD) and in
//   groups of 8 m-tiles, so concurrently running tiles share operand rows in L2.
// Deterministic: fixed K order, no atomics; bf16 output is the RNE rounding of the same
// fp32 accumulator the fp32 output mode stores.
#include "device.hpp"
#include "internal.hpp"

namespace fp8rl {

// Distance, in MFMA tiles, between an MFMA and the FMAs that fold its result.
constexpr int kLag = 3;
// Largest K / 128 of the ring configuration (its B block-scale table holds 2 x kMaxKb floats).
constexpr int kMaxKb = 1024;

// kScale: 0 = fp32 scales (each 128-K block product folded in with one FMA),
//         1 = power-of-two fp32 scales (their exponent fields go to the scaled MFMA),
//         2 = MXFP8: each scale dword holds the 4 E8M0 bytes of a row's 128-K block, one per
//             32-wide part; lane l hands the MFMA the byte of part l >> 4.
// SK: 1 = every scale is loaded per K block into the stage; otherwise A's row scales (and
//     B's, when they are row scales applied by the MFMA: SK = 4) come SK K blocks at a time
//     through the ring, and K / 128 must be a multiple of SK.
// kGroup: the grouped (MoE) form; each workgroup resolves its expert, row range and the
//     expert's B and sB from the device offsets (see below); everything else is shared.
template <int BM, int BN, int WM, int WN, bool kRowB, bool kF32, int kScale, int SK, bool kGroup = false>
// At most two waves per SIMD, so at most 256 VGPRs: the compiler then keeps MFMA results in
// VGPRs (no accumulator-register reads before the fold). The 256x256 kernels are there anyway
// (8 waves, one workgroup per CU); the 128x128 ones ran 5% faster on the gate/up shape.
__global__ __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_blockscaled(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int NSB = kRowB ? BN : 64;                       // B scale slots per stage
  constexpr int OFF_B = BM * 128;
  constexpr int OFF_SA = OFF_B + BN * 128;
  constexpr int OFF_SB = OFF_SA + BM * 4;
  constexpr int STAGE = OFF_SA + NT * 4;   // one 64-float scale slot per wave (A, B, then unused)
  static_assert(BM % WM == 0 && BN % WN == 0 && TM % 16 == 0 && TN % 16 == 0, "tile shape");
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "load split");
  static_assert(NT >= BM + NSB, "one scale load per wave");
  static_assert(OFF_SB + NSB * 4 <= STAGE, "scale slots");
  static_assert(kRowB || TN <= 128, "a wave's n range must sit inside one 128-row scale block");
  static_assert(kLag < FM, "a folded tile is at most one B fragment behind");
  constexpr bool kChunkB = SK > 1 && kRowB;                  // B's row scales come through the ring
  constexpr int CROWS = BM + (kChunkB ? BN : 0);               // ring rows: A's, then B's
  constexpr int CBUF = CROWS * SK * 4;                         // bytes per ring buffer
  constexpr int LPR = SK > 4 ? SK / 4 : 1;                     // ring lanes per row, 16 bytes each
  // With SK > 1 and 128x128 block scales on B, the tile's B scales (2 block rows x K / 128)
  // are loaded into an LDS table once, before the K loop (at most kMaxKb K blocks).
  constexpr bool kPreB = SK > 1 && !kRowB;
  constexpr int kPreFloats = kPreB ? 2 * kMaxKb : 1;
  static_assert(LPR >= 1, "LPR divides lane indices");
  static_assert(SK == 1 || (SK == (kChunkB ? 4 : 8) && CROWS * LPR == NT), "every lane loads one ring piece");
  __shared__ __attribute__((aligned(16))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t scr[SK > 1 ? 2 * CBUF : 16];
  __shared__ __attribute__((aligned(16))) float sbk[kPreFloats];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Wave grid position. The grouped form puts the wave rows across SIMDs (wave w runs on
  // SIMD w % 4): wave row w / WN, so the two waves sharing a SIMD own rows TM * (w % 4 / WN)
  // and 2 TM further. A wave whose rows all lie past the expert's last row skips its
  // MFMAs, which then halves the SIMD time of an m-tile with at most 2 TM rows.
  const int wmi = kGroup ? wave / WN : wave % WM;
  const int wm0 = wmi * TM;
  const int wn0 = (kGroup ? wave % WN : wave / WM) * TN;

  const int64_t M = p.M, N = p.N, K = p.K;
  const int tiles_n = (int)((N + BN - 1) / BN);
  int64_t m0, n0, m_end;                 // tile origin; A rows of this tile end before m_end
  const uint8_t* Bp = p.B;
  const float* sBp = p.sB;
  if constexpr (kGroup) {
    // Expert e owns ceil(count_e / BM) m-tiles. A wave-level prefix sum over the experts
    // (64 per step) gives the total, then the expert owning m-tile mt. Offsets are clamped
    // into [0, M] and a decreasing step is an empty expert, so no access leaves the
    // buffers whatever they hold. Only the real tiles are mapped (XCD-aware, n fastest, so
    // an XCD's concurrent tiles share A rows and the expert's B); the grid's spare
    // workgroups exit here.
    auto rows_of = [&](int64_t e, int64_t& beg) __attribute__((always_inline)) -> int64_t {
      const int64_t a = min(max((int64_t)p.offsets[e], (int64_t)0), M);
      const int64_t b = min(max((int64_t)p.offsets[e + 1], (int64_t)0), M);
      beg = a;
      return b > a ? b - a : 0;
    };
    int64_t total = 0;
    for (int64_t c0 = 0; c0 < p.E; c0 += 64) {
      int64_t beg, t = 0;
      if (c0 + lane < p.E) t = (rows_of(c0 + lane, beg) + BM - 1) / BM;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
      total += t;
    }
    // Offsets that do not partition [0, M] can give more tiles than the grid holds: only the
    // first gridDim.x of them are computed, and every index stays in range.
    const int64_t G = min(total * tiles_n, (int64_t)gridDim.x);
    if ((int64_t)blockIdx.x >= G) return;   // uniform across the workgroup
    const int L = xcd_remap(blockIdx.x, (int)G);
    const int64_t mt = L / tiles_n;
    n0 = (int64_t)(L % tiles_n) * BN;
    int64_t base = 0, expert = -1, row_beg = 0, row_cnt = 0;
    m0 = 0;
    for (int64_t c0 = 0; c0 < p.E && expert < 0; c0 += 64) {
      const int64_t e = c0 + lane;
      int64_t beg = 0, cnt = 0;
      if (e < p.E) cnt = rows_of(e, beg);
      const int64_t tiles = (cnt + BM - 1) / BM;
      int64_t incl = tiles;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int64_t v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      const int64_t excl = incl - tiles;
      const uint64_t hit = __ballot(e < p.E && mt >= base + excl && mt < base + incl);
      if (hit) {
        const int src = __ffsll((unsigned long long)hit) - 1;
        expert = c0 + src;
        row_beg = __shfl(beg, src);
        row_cnt = __shfl(cnt, src);
        m0 = row_beg + (mt - base - __shfl(excl, src)) * BM;
      }
      base += __shfl(incl, 63);
    }
    if (expert < 0) return;                 // not reached for mt < total; uniform
    m_end = row_beg + row_cnt;
    Bp += expert * p.b_stride;
    sBp += expert * p.sb_stride;
  } else {
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    constexpr int GM = 8;
    const int group = L / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int in_group = L - group * GM * tiles_n;
    m0 = (int64_t)(first_m + in_group % gsz) * BM;
    n0 = (int64_t)(in_group / gsz) * BN;
    m_end = M;
  }
  const int nkb = (int)(K / 128);
  const int64_t nb0 = n0 >> 7;                                  // first 128-row B block of the tile
  const int64_t nbl = (N - 1) >> 7;                             // last B block

  // Staged loads go through raw buffer descriptors whose range ends at the last valid row
  // of the tile, so rows past the end of A / B (and their scales) read as zero without a
  // memory access; their results are never stored. One descriptor per operand and K block
  // (base: the tile's first row at column kb * 128) serves all of the operand's loads.
  constexpr int LA = BM * 8 / NT, LB = BN * 8 / NT;
  // Load `it` covers tile rows it * NT/8 .. : its lane offset is the first load's plus
  // it * (NT/8) * K bytes, and NT/8 is a multiple of 16, so the row swizzle phase
  // ((r >> 1) & 7) is the same for every load.
  static_assert((NT / 8) % 16 == 0, "swizzle phase must repeat across loads");
  const int64_t rows_a = min((int64_t)BM, m_end - m0), rows_b = min((int64_t)BN, N - n0);
  const int lr = tid >> 3;
  const uint32_t off0 = (uint32_t)(lr * K) + (uint32_t)(swz(lr, tid & 7) << 4);
  const uint32_t bytesA = (uint32_t)((rows_a - 1) * K + 128), bytesB = (uint32_t)((rows_b - 1) * K + 128);
  // Scale loads: waves [0, BM/64) fetch sA of the tile rows, the next NSB/64 waves fetch
  // sB; every other wave issues the same per-K-block instruction through an empty
  // descriptor (no memory access) into its own unused slot, which keeps that part of the K
  // step branch-free. With SK > 1 only B's scales that do not go through the ring are
  // loaded per K block.
  const bool sa_wave = wave < BM / 64;
  const bool sb_wave = !sa_wave && wave < BM / 64 + NSB / 64;
  // Per-K-block scale loads (SK == 1 only): every wave, with empty descriptors for waves
  // without scales.
  // Ring loads: lane idx = wave * 64 + lane loads 16 bytes (4 K blocks) of ring row
  // idx / LPR (A's rows, then B's), piece idx % LPR; the ring row r, K block kb % SK sits at
  // byte (r * SK + kb % SK) * 4 of a buffer, which is where the lane-ordered LDS write puts it.
  const int cidx = wave * 64 + lane;
  const int crow = cidx / LPR;
  const bool c_a = crow < BM;                                    // wave-uniform
  const float* cbase = c_a ? p.sA + m0 * p.sa_ld : sBp + n0 * p.sb_ld_n;
  const int64_t cld = c_a ? p.sa_ld : p.sb_ld_n;
  const uint32_t coff = (uint32_t)(((c_a ? crow : crow - BM) * cld + (cidx % LPR) * 4) * 4);
  // Rows past the tile's last valid row read as zero; nkb % SK == 0 keeps every load of a
  // valid row inside that row's scales.
  const uint32_t cbytes = (uint32_t)(((c_a ? rows_a : rows_b) - 1) * cld * 4 + nkb * 4);
  const uint32_t scr0 = lds_addr(scr);
  const float* baseS;
  uint32_t offS, bytesS;
  int64_t sstep;  // floats per K block
  if (sa_wave) {
    baseS = p.sA + m0 * p.sa_ld;
    offS = (uint32_t)((wave * 64 + lane) * p.sa_ld * 4);
    bytesS = (uint32_t)((rows_a - 1) * p.sa_ld * 4 + 4);
    sstep = 1;
  } else if (kRowB) {
    baseS = sBp + n0 * p.sb_ld_n;
    offS = (uint32_t)(((wave - BM / 64) * 64 + lane) * p.sb_ld_n * 4);
    bytesS = sb_wave ? (uint32_t)((rows_b - 1) * p.sb_ld_n * 4 + 4) : 0u;
    sstep = 1;
  } else {
    baseS = sBp + nb0 * p.sb_ld_n;
    offS = (uint32_t)(lane * p.sb_ld_n * 4);
    bytesS = sb_wave ? (uint32_t)((nbl - nb0) * p.sb_ld_n * 4 + 4) : 0u;
    sstep = p.sb_ld_k;
  }

  // Stage the operands of K block kb into the stage at LDS address st: operand copy `part`
  // (A's loads, then B's), and the scale copies. For kb >= nkb every descriptor is empty:
  // the loads write zeros without touching memory.
  constexpr int NPART = LA + LB;
  auto issue_part = [&](int kb, uint32_t st, auto partc) __attribute__((always_inline)) {
    constexpr int part = decltype(partc)::value;
    const bool live = kb < nkb;
    const int kbc = live ? kb : 0;
    if constexpr (part < LA) {
      dma16(make_rsrc(p.A + m0 * K + kbc * 128, live ? bytesA : 0u), off0 + (uint32_t)(part * (NT / 8)) * (uint32_t)K,
            st + (part * NT + wave * 64) * 16);
    } else {
      dma16(make_rsrc(Bp + n0 * K + kbc * 128, live ? bytesB : 0u), off0 + (uint32_t)((part - LA) * (NT / 8)) * (uint32_t)K,
            st + OFF_B + ((part - LA) * NT + wave * 64) * 16);
    }
  };
  auto issue_scales = [&](int kb, uint32_t st) __attribute__((always_inline)) {
    const bool live = kb < nkb;
    const int kbc = live ? kb : 0;
    if constexpr (SK == 1) {
      dma4(make_rsrc(baseS + kbc * sstep, live ? bytesS : 0u), offS, st + OFF_SA + wave * 256);
    } else {
      // Only the K blocks that start a ring chunk issue a scale copy: an instruction with an
      // empty descriptor or exec = 0 still costs the texture unit the time of a real one.
      // At kb % SK == 0: row scales of K blocks kb .. kb + SK - 1 into ring buffer
      // (kb / SK) & 1, whose previous contents were read by K blocks that every wave
      // finished before the barrier preceding this issue.
      dma16_if(make_rsrc(cbase, cbytes), coff + (uint32_t)(kbc * 4), scr0 + ((kb / SK) & 1) * CBUF + wave * 1024,
               (uint32_t)(live && kb % SK == 0));
    }
  };
  auto issue = [&](int kb, uint32_t st) __attribute__((always_inline)) {
    static_for<0, NPART>([&](auto pc) { issue_part(kb, st, pc); });
    issue_scales(kb, st);
  };
  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Per-lane LDS byte offsets inside a stage (fragment rows, scale slots).
  const FragOffsets fa = frag_offsets(wm0, lane), fb = frag_offsets(wn0, lane);
  const uint32_t o_sa = OFF_SA + (wm0 + (lane & 15)) * 4;
  const uint32_t o_sb = kRowB ? OFF_SB + (wn0 + 4 * (lane >> 4)) * 4 : OFF_SB + (uint32_t)(((n0 + wn0) >> 7) - nb0) * 4;
  const uint32_t o_sbr = OFF_SB + (wn0 + (lane & 15)) * 4;     // row (lane & 15) of each B fragment
  const uint32_t sbk_w = lds_addr(sbk) + (uint32_t)((((n0 + wn0) >> 7) - nb0) * nkb) * 4;

  // One K block from the stage at st. A fragments stay in registers for the whole block; B
  // fragments are double-buffered (fragment i+1 is read while fragment i feeds the MFMAs);
  // the FMAs that fold tile t-1 into the accumulators follow the MFMA of tile t
  // (t = i * FM + j), so one MFMA result is in flight while the previous one is folded.
  auto compute = [&](uint32_t st, int kb) __attribute__((always_inline)) {
    const uint32_t a_lo = st + fa.lo, a_hi = st + fa.hi;
    const uint32_t b_lo = st + OFF_B + fb.lo, b_hi = st + OFF_B + fb.hi;
    // Ring slot of K block kb: row r's scale sits at byte (r * SK + kb % SK) * 4 of the buffer.
    const uint32_t cb = scr0 + ((kb / SK) & 1) * CBUF + (kb % SK) * 4;
    const uint32_t sa_ad = SK > 1 ? cb + (wm0 + (lane & 15)) * SK * 4 : st + o_sa;
    // B's block scale of this wave's 128 columns: its table entry, or the stage slot.
    const uint32_t sb_ad = kPreB ? sbk_w + kb * 4 : st + o_sb;
    v4i alo[FM], ahi[FM];
    float sa[FM];
    static_for<0, FM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      alo[j] = ds_read16<j * 2048>(a_lo);
      ahi[j] = ds_read16<j * 2048>(a_hi);
      sa[j] = ds_read4f<j * 16 * SK * 4>(sa_ad);
    });
    float sb = 0.f;
    v4i sbv;
    // The fold's B row scales of B-fragment step i: rows wn0 + 16 i + 4 (lane >> 4) .. + 3,
    // contiguous in the stage slot; 16 bytes apart in the ring.
    const uint32_t sbv_ad = kChunkB ? cb + (BM + wn0 + 4 * (lane >> 4)) * SK * 4 : sb_ad;
    auto read_sbv = [&](auto ic) __attribute__((always_inline)) -> v4i {
      constexpr int i = decltype(ic)::value;
      if constexpr (kChunkB) {
        const uint32_t a = sbv_ad + i * 16 * SK * 4;
        const v2i lo = ds_read2_b32<0, SK>(a), hi = ds_read2_b32<2 * SK, 3 * SK>(a);
        return v4i{lo.x, lo.y, hi.x, hi.y};
      } else {
        return ds_read16<i * 64>(sb_ad);
      }
    };
    if (!kRowB) sb = ds_read4f<0>(sb_ad);
    else if (kScale == 0) sbv = read_sbv(std::integral_constant<int, 0>{});
    v4i blo = ds_read16<0>(b_lo), bhi = ds_read16<0>(b_hi);
    lds_wait<0>();
    v8i af[FM];
    float prod[FM];
    static_for<0, FM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      hold(alo[j]);
      hold(ahi[j]);
      hold(sa[j]);
      af[j] = join(alo[j], ahi[j]);
    });
    hold(sb);
    hold(sbv);
    hold(blo);
    hold(bhi);
    if constexpr (kScale != 0) {
      // Power-of-two scales: the scaled MFMA applies 2^(e_a + e_b) itself (E8M0 bytes are
      // the scales' fp32 exponent fields; 2^-127, an fp32 subnormal, gives byte 0), so the
      // products accumulate directly. Lane l supplies the scale of row l & 15 for all four
      // 32-wide parts of the K block. MXFP8: lane l supplies the E8M0 byte of row l & 15
      // for 32-wide part l >> 4 (the MFMA reads the low byte of the operand).
      const int esh = kScale == 2 ? 8 * (lane >> 4) : 23;
      int ua[FM];
#pragma unroll
      for (int j = 0; j < FM; ++j) ua[j] = (int)(__float_as_uint(sa[j]) >> esh);
      int ubr[FN];
      if constexpr (kRowB) {
        // The LDS reads land only at the wait: take the exponents after it.
        float sbr[FN];
        const uint32_t sbr_ad = kChunkB ? cb + (BM + wn0 + (lane & 15)) * SK * 4 : st + o_sbr;
        static_for<0, FN>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          sbr[i] = ds_read4f<i * 16 * (kChunkB ? SK : 1) * 4>(sbr_ad);
        });
        lds_wait<0>();
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          hold(sbr[i]);
          ubr[i] = (int)(__float_as_uint(sbr[i]) >> esh);
        }
      }
      const int ub = kRowB ? 0 : (int)(__float_as_uint(sb) >> esh);
      static_for<0, FN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        v4i nlo, nhi;
        if constexpr (i + 1 < FN) {
          nlo = ds_read16<(i + 1) * 2048>(b_lo);
          nhi = ds_read16<(i + 1) * 2048>(b_hi);
        }
        const v8i bf = join(blo, bhi);
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = mfma_fp8(bf, af[j], acc[i][j], kRowB ? ubr[i] : ub, ua[j]);
        if constexpr (i + 1 < FN) {
          __builtin_amdgcn_sched_barrier(0);
          lds_wait<0>();
          hold(nlo);
          hold(nhi);
          blo = nlo;
          bhi = nhi;
        }
      });
    } else {
      if (!kRowB) {
#pragma unroll
        for (int j = 0; j < FM; ++j) prod[j] = sa[j] * sb;
      }
      // Tiles run in the order t = i * FM + j; the FMAs that fold tile t - kLag into the
      // accumulators follow the MFMA of tile t, so the wave never stalls on a fresh MFMA
      // result. `pipe` holds the kLag + 1 most recent MFMA results.
      v4f pipe[kLag + 1];
      v4i sbprev = sbv;
      auto fold = [&](int i, int j, const v4f& pr, const v4i& sbw) __attribute__((always_inline)) {
        if (kRowB) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] = __builtin_fmaf(pr[r], sa[j] * __int_as_float(sbw[r]), acc[i][j][r]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[r], prod[j], acc[i][j][r]);
        }
      };
      static_for<0, FN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        v4i nlo, nhi, nsb;
        if constexpr (i + 1 < FN) {
          nlo = ds_read16<(i + 1) * 2048>(b_lo);
          nhi = ds_read16<(i + 1) * 2048>(b_hi);
          if (kRowB) nsb = read_sbv(std::integral_constant<int, i + 1>{});
        }
        const v8i bf = join(blo, bhi);
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int t = i * FM + j;
          pipe[t % (kLag + 1)] = mfma_fp8(bf, af[j], v4f{0.f, 0.f, 0.f, 0.f}, 127, 127);
          if (t >= kLag) {
            const int u = t - kLag;
            fold(u / FM, u % FM, pipe[u % (kLag + 1)], (u / FM == i) ? sbv : sbprev);
          }
          __builtin_amdgcn_sched_barrier(0);   // keep the MFMA / fold interleave as written
        }
        sbprev = sbv;
        if constexpr (i + 1 < FN) {
          __builtin_amdgcn_sched_barrier(0);   // this step's MFMAs stay ahead of the wait
          lds_wait<0>();
          hold(nlo);
          hold(nhi);
          blo = nlo;
          bhi = nhi;
          if (kRowB) {
            hold(nsb);
            sbv = nsb;
          }
        }
      });
#pragma unroll
      for (int u = FN * FM - kLag; u < FN * FM; ++u) fold(u / FM, u % FM, pipe[u % (kLag + 1)], sbprev);
    }
  };

  // K loop. Each step: wait until this wave's copies into the current stage have landed,
  // barrier (all waves' copies landed, and everyone is done reading the other stage),
  // start copying K block kb+1 into the other stage, then compute on the current one.
  const uint32_t st0 = lds_addr(sm0), st1 = lds_addr(sm1);
  const uint32_t sbk0 = lds_addr(sbk);
  if constexpr (kPreB) {
    // Entry e of the table is B block row e / nkb (of the tile's two), K block e % nkb; the
    // descriptor's range ends at the last valid entry, so entries of a block row past the
    // end of B read as zero or as other scales of B (never used). Entries past 2 * nkb read
    // as zero. The K loop's first wait and barrier cover these copies.
    const int ne = 2 * nkb;
    const v4i rs = make_rsrc(sBp + nb0 * p.sb_ld_n,
                             (uint32_t)(((nbl - nb0) * p.sb_ld_n + (int64_t)(nkb - 1) * p.sb_ld_k + 1) * 4));
    for (int e0 = 0; e0 < ne; e0 += NT) {
      const int e = e0 + wave * 64 + lane;
      const int r = e / nkb, k = e - r * nkb;
      const uint32_t off = e < ne ? (uint32_t)((r * p.sb_ld_n + (int64_t)k * p.sb_ld_k) * 4) : 0xfffffff0u;
      dma4(rs, off, sbk0 + (e0 + wave * 64) * 4);
    }
  }
  // Grouped form: a wave with no rows of the expert computes nothing (wave-uniform).
  const bool busy = !kGroup || m0 + wm0 < m_end;
  issue(0, st0);
  int kb = 0;
  for (; kb + 2 <= nkb; kb += 2) {
    wait_vmem();
    __syncthreads();
    issue(kb + 1, st1);
    if (busy) compute(st0, kb);
    wait_vmem();
    __syncthreads();
    issue(kb + 2, st0);
    if (busy) compute(st1, kb + 1);
  }
  if (kb < nkb) {
    wait_vmem();
    __syncthreads();
    if (busy) compute(st0, kb);
  }

  // Epilogue. The tile goes out through LDS (the stages are free after the K loop), so that
  // every global store instruction writes whole 128-byte lines instead of 16-byte (fp32) or
  // 8-byte (bf16) pieces of 16 rows; lane l holds C[m][n .. n+3] of each 16x16 tile.
  // fp32: one wave row (TM rows) at a time, read back and added to when accumulating.
  // bf16: the whole tile at once, rows [0, BM/2) in sm0 and the rest in sm1.
  wait_vmem();  // the empty copy issued past the last K block still writes (zeros) to a stage
  if constexpr (kF32) {
    constexpr int ROWF = BN * 4 + 16;                // staged row stride in bytes
    constexpr int CPR = BN * 4 / 16;                 // 16-byte chunks per row
    constexpr int RPP = NT / CPR;                    // rows per pass
    static_assert(TM * ROWF <= STAGE && NT % CPR == 0 && TM % RPP == 0, "fp32 staging");
    const int cr = tid / CPR, cc = tid % CPR;
    const int64_t n = n0 + cc * 4;
#pragma unroll
    for (int q = 0; q < WM; ++q) {
      uint8_t* buf = (q & 1) ? sm1 : sm0;
      __syncthreads();                               // the stage is free (K loop / previous chunk)
      if (wmi == q) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          uint8_t* rowp = buf + (16 * j + (lane & 15)) * ROWF;
#pragma unroll
          for (int i = 0; i < FN; ++i)
            *reinterpret_cast<float4*>(rowp + (wn0 + 16 * i + 4 * (lane >> 4)) * 4) =
                make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int r0 = 0; r0 < TM; r0 += RPP) {
        const int r = r0 + cr;
        const int64_t m = m0 + q * TM + r;
        float4 v = *reinterpret_cast<const float4*>(buf + r * ROWF + cc * 16);
        if (m < m_end && n < N) {
          float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + m * p.ldc + n);
          if (p.accumulate) {
            const float4 o = *dst;
            v.x += o.x;
            v.y += o.y;
            v.z += o.z;
            v.w += o.w;
          }
          *dst = v;
        }
      }
    }
  } else {
    constexpr int ROW = BN * 2 + 16;                 // staged row stride in bytes
    constexpr int HALF = BM / 2;
    static_assert(HALF * ROW <= STAGE, "half a bf16 tile fits in one stage");
    __syncthreads();                                 // every wave is done reading the stages
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int r = wm0 + 16 * j + (lane & 15);
      uint8_t* rowp = (r < HALF ? sm0 : sm1) + (r % HALF) * ROW;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int c = wn0 + 16 * i + 4 * (lane >> 4);
        uint2 v;
        v.x = f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16);
        v.y = f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(rowp + c * 2) = v;
      }
    }
    __syncthreads();
    constexpr int CPR = BN * 2 / 16;                 // 16-byte chunks per row
    constexpr int RPP = NT / CPR;                    // rows per pass
    static_assert(NT % CPR == 0 && BM % RPP == 0, "copy-out split");
    const int cr = tid / CPR, cc = tid % CPR;
    const int64_t n = n0 + cc * 8;
#pragma unroll
    for (int r0 = 0; r0 < BM; r0 += RPP) {
      const int r = r0 + cr;
      const int64_t m = m0 + r;
      const uint4 v = *reinterpret_cast<const uint4*>((r < HALF ? sm0 : sm1) + (r % HALF) * ROW + cc * 16);
      if (m < m_end && n < N) *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.C) + m * p.ldc + n) = v;
    }
  }
}

template <int BM, int BN, int WM, int WN, bool kRowB, int kScale, int SK, bool kGroup = false>
static hipError_t launch_sk(const GemmParams& p, bool f32, int64_t tiles, hipStream_t stream) {
  const dim3 grid((unsigned)tiles), block(WM * WN * 64);
  if (f32)
    hipLaunchKernelGGL((k_gemm_blockscaled<BM, BN, WM, WN, kRowB, true, kScale, SK, kGroup>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_blockscaled<BM, BN, WM, WN, kRowB, false, kScale, SK, kGroup>), grid, block, 0, stream, p);
  return hipGetLastError();
}

// 256x256 tiles take their row scales through the ring whenever K / 128 is a multiple of SK.
template <int BM, int BN, int WM, int WN, bool kRowB, int kScale>
static hipError_t launch_cfg(const GemmParams& p, bool f32, hipStream_t stream) {
  constexpr int SK = kRowB ? 4 : 8;
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if constexpr (BM == 256)
    if ((p.K / 128) % SK == 0 && p.K / 128 <= kMaxKb)
      return launch_sk<BM, BN, WM, WN, kRowB, kScale, SK>(p, f32, tiles, stream);
  return launch_sk<BM, BN, WM, WN, kRowB, kScale, 1>(p, f32, tiles, stream);
}

// Tile choice: at most 256 rows with block-scaled fp32 scales go to the decode kernel
// (decode.hip; A row-major); otherwise 256x256 tiles (8 waves, 64x128 per wave) when there
// are enough of them to fill the 256 CUs, else 128x128 tiles (4 waves, 64x64 per wave).
hipError_t launch_gemm_blockscaled(const GemmParams& p, bool row_scale_b, bool f32, bool pow2, hipStream_t stream) {
  if (!pow2 && !row_scale_b && p.M <= 256 && !p.accumulate) {
    DecodeParams d{};
    d.A = p.A;
    d.sA = p.sA;
    d.B = p.B;
    d.sB = p.sB;
    d.C = p.C;
    d.M = p.M;
    d.N = p.N;
    d.K = p.K;
    d.a_ld = p.K;
    d.a_kb = 128;
    d.sa_ld = p.sa_ld;
    d.sa_kb = 1;
    d.sb_ld_n = p.sb_ld_n;
    d.sb_ld_k = p.sb_ld_k;
    d.ldc = p.ldc;
    return launch_gemm_decode(d, f32, stream);
  }
  const int64_t big_tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
  const bool big = big_tiles >= 256;
  if (pow2) {
    if (row_scale_b)
      return big ? launch_cfg<256, 256, 4, 2, true, 1>(p, f32, stream) : launch_cfg<128, 128, 2, 2, true, 1>(p, f32, stream);
    return big ? launch_cfg<256, 256, 4, 2, false, 1>(p, f32, stream) : launch_cfg<128, 128, 2, 2, false, 1>(p, f32, stream);
  }
  if (row_scale_b)
    return big ? launch_cfg<256, 256, 4, 2, true, 0>(p, f32, stream) : launch_cfg<128, 128, 2, 2, true, 0>(p, f32, stream);
  return big ? launch_cfg<256, 256, 4, 2, false, 0>(p, f32, stream) : launch_cfg<128, 128, 2, 2, false, 0>(p, f32, stream);
}

// MXFP8: both operands carry one E8M0 byte per row per 32 K (sA / sB point at those bytes,
// sa_ld = sb_ld_n = K / 128 dwords per row).
hipError_t launch_gemm_mx(const GemmParams& p, bool f32, hipStream_t stream) {
  const bool big = ((p.M + 255) / 256) * ((p.N + 255) / 256) >= 256;
  return big ? launch_cfg<256, 256, 4, 2, true, 2>(p, f32, stream) : launch_cfg<128, 128, 2, 2, true, 2>(p, f32, stream);
}

// Grouped GEMMs (MoE): the kernels above with grouped tile resolution, 256x256 tiles
// (measured faster than 128x128 / 128x256 / 256x128 tiles on the routed-MoE shapes even
// though ragged experts leave more of their last m-tile empty). X rows are grouped by
// expert; W is [E][N][K]. The grid is an upper bound
// on the tiles (sum_e ceil(c_e / 256) <= T / 256 + E for offsets that partition [0, T]);
// its spare workgroups exit at once.
static GemmParams grouped_params(const GroupedParams& g) {
  GemmParams p{};
  p.A = g.X;
  p.B = g.W;
  p.sA = reinterpret_cast<const float*>(g.Xs);
  p.sB = reinterpret_cast<const float*>(g.Ws);
  p.C = g.Y;
  p.M = g.T;
  p.N = g.N;
  p.K = g.K;
  p.sa_ld = p.sb_ld_n = g.K / 128;   // MXFP8: dwords of 4 E8M0 bytes per row; blockwise: K blocks
  p.sb_ld_k = 1;
  p.ldc = g.N;
  p.offsets = g.offsets;
  p.E = g.E;
  p.b_stride = g.N * g.K;
  return p;
}

static int64_t grouped_tiles(const GroupedParams& g) { return ((g.T + 255) / 256 + g.E) * ((g.N + 255) / 256); }

hipError_t launch_grouped_mx(const GroupedParams& g, bool f32, hipStream_t stream) {
  GemmParams p = grouped_params(g);
  p.sb_stride = g.N * (g.K / 128);
  const int64_t tiles = grouped_tiles(g);
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  if ((g.K / 128) % 4 == 0 && g.K / 128 <= kMaxKb) return launch_sk<256, 256, 4, 2, true, 2, 4, true>(p, f32, tiles, stream);
  return launch_sk<256, 256, 4, 2, true, 2, 1, true>(p, f32, tiles, stream);
}

// Blockwise grouped GEMM: the fp32-scale forward kernel (1x128 row scales of X through the
// ring, the expert's 128x128 block scales preloaded per tile) with grouped tile resolution;
// expert e's block scales start sb_stride = (N/128)(K/128) floats after expert e-1's.
hipError_t launch_grouped_block(const GroupedParams& g, bool f32, hipStream_t stream) {
  GemmParams p = grouped_params(g);
  p.sb_stride = (g.N / 128) * (g.K / 128);
  const int64_t tiles = grouped_tiles(g);
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  if ((g.K / 128) % 8 == 0 && g.K / 128 <= kMaxKb)
    return launch_sk<256, 256, 4, 2, false, 0, 8, true>(p, f32, tiles, stream);
  return launch_sk<256, 256, 4, 2, false, 0, 1, true>(p, f32, tiles, stream);
}

}  // namespace fp8rl
