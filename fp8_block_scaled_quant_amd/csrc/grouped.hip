// MXFP8 grouped GEMM for mixture-of-experts layers: routed rows grouped by expert,
// Y[t][n] = sum_k deq(X)[t][k] * deq(W[e])[n][k] for rows t of expert e, with one E8M0
// scale per 1x32 group on both operands ([SkyRL-FP8] MoE: routed experts hold most
// parameters; MXFP8 recipe with power-of-two 1x32 scales).
//
// gfx950 design: v_mfma_scale_f32_16x16x128_f8f6f4 takes the E8M0 scales of both operands
// per lane (lane i + 16b: row i, K block [32b, 32b+32)) and applies them inside the matrix
// core, so the K loop is pure MFMA accumulation with no VALU rescaling. Operands and the
// scale bytes of each 128-wide K chunk (one dword = 4 E8M0 bytes per row) are staged in
// LDS with direct global->LDS loads, double-buffered as in the dense GEMM.
// Work split: the per-expert row counts come from the device offsets; every workgroup
// derives its (expert, m-tile) by a wave-level prefix sum over ceil(count_e / BM), so no
// host round trip is needed and ragged experts get only the tiles they need. Offsets are
// clamped into [0, T] (a decreasing step is an empty expert), so no access leaves the
// buffers whatever the offsets hold.
#include "device.hpp"
#include "internal.hpp"

namespace fp8rl {

template <int BM, int BN, int WM, int WN, bool kF32>
__global__ __launch_bounds__(WM* WN * 64) void k_grouped_mx(GroupedParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int OFF_B = BM * 128;
  constexpr int OFF_SA = OFF_B + BN * 128;
  constexpr int OFF_SB = OFF_SA + BM * 4;
  constexpr int STAGE = OFF_SA + NT * 4;   // one 64-dword scale slot per wave (X, W, then unused)
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0 && NT >= BM + BN, "load split");
  __shared__ __attribute__((aligned(16))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave % WM) * TM;
  const int wn0 = (wave / WM) * TN;
  const int64_t T = p.T, E = p.E, N = p.N, K = p.K;
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int mt = (int)(blockIdx.x / tiles_n);
  const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;

  // Locate the expert owning global m-tile `mt`.
  int64_t row_beg = 0, row_end = 0, expert = -1;
  int local_tile = 0;
  int64_t base = 0;
  for (int64_t c0 = 0; c0 < E; c0 += 64) {
    const int64_t e = c0 + lane;
    int64_t beg = 0, cnt = 0;
    if (e < E) {
      const int64_t a = min(max((int64_t)p.offsets[e], (int64_t)0), T);
      const int64_t b = min(max((int64_t)p.offsets[e + 1], (int64_t)0), T);
      beg = a;
      cnt = b > a ? b - a : 0;
    }
    const int64_t tiles = (cnt + BM - 1) / BM;
    int64_t incl = tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    const int64_t excl = incl - tiles;
    const bool hit = (e < E) && (mt >= base + excl) && (mt < base + incl);
    const uint64_t mask = __ballot(hit);
    if (mask) {
      const int src = __ffsll((unsigned long long)mask) - 1;
      expert = c0 + src;
      local_tile = (int)(mt - base - __shfl(excl, src));
      row_beg = __shfl(beg, src);
      row_end = row_beg + __shfl(cnt, src);
      break;
    }
    base += __shfl(incl, 63);
  }
  if (expert < 0) return;  // beyond the last tile (uniform across the workgroup)

  const int64_t m0 = row_beg + (int64_t)local_tile * BM;
  const uint8_t* Wb = p.W + expert * N * K;
  const uint8_t* Wsb = p.Ws + expert * N * (K / 32);
  const int nkc = (int)(K / 128);

  // Raw buffer descriptors end at the expert's last row / at N, so rows past them read as
  // zero without a memory access (see the dense GEMM); one per-lane offset per operand.
  constexpr int LA = BM * 8 / NT, LB = BN * 8 / NT;
  static_assert((NT / 8) % 16 == 0, "swizzle phase must repeat across loads");
  const int64_t rows_a = min((int64_t)BM, row_end - m0), rows_b = min((int64_t)BN, N - n0);
  const int lr = tid >> 3;
  const uint32_t off0 = (uint32_t)(lr * K) + (uint32_t)(swz(lr, tid & 7) << 4);
  const uint32_t bytesA = (uint32_t)((rows_a - 1) * K + 128), bytesB = (uint32_t)((rows_b - 1) * K + 128);
  // Scale dwords (4 E8M0 bytes of one row for one 128-wide K chunk): waves [0, BM/64)
  // fetch X's, the next BN/64 waves W's, the rest issue an empty load into a spare slot.
  const bool sa_wave = wave < BM / 64;
  const bool sb_wave = !sa_wave && wave < (BM + BN) / 64;
  const uint8_t* baseS;
  uint32_t offS, bytesS;
  if (sa_wave) {
    baseS = p.Xs + m0 * (K / 32);
    offS = (uint32_t)((wave * 64 + lane) * (K / 32));
    bytesS = (uint32_t)((rows_a - 1) * (K / 32) + 4);
  } else {
    baseS = Wsb + n0 * (K / 32);
    offS = (uint32_t)(((wave - BM / 64) * 64 + lane) * (K / 32));
    bytesS = sb_wave ? (uint32_t)((rows_b - 1) * (K / 32) + 4) : 0u;
  }

  auto issue = [&](int kc, uint32_t st) __attribute__((always_inline)) {
    const bool live = kc < nkc;
    const int kcc = live ? kc : 0;
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      const int64_t r0 = (int64_t)it * (NT / 8);
      const uint32_t nb = (live && bytesA > r0 * K) ? (uint32_t)(bytesA - r0 * K) : 0u;
      dma16(make_rsrc(p.X + (m0 + r0) * K + kcc * 128, nb), off0, st + (it * NT + wave * 64) * 16);
    }
#pragma unroll
    for (int it = 0; it < LB; ++it) {
      const int64_t r0 = (int64_t)it * (NT / 8);
      const uint32_t nb = (live && bytesB > r0 * K) ? (uint32_t)(bytesB - r0 * K) : 0u;
      dma16(make_rsrc(Wb + (n0 + r0) * K + kcc * 128, nb), off0, st + OFF_B + (it * NT + wave * 64) * 16);
    }
    dma4(make_rsrc(baseS + kcc * 4, live ? bytesS : 0u), offS, st + OFF_SA + wave * 256);
  };

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const FragOffsets fa = frag_offsets(wm0, lane), fb = frag_offsets(wn0, lane);
  const uint32_t o_sa = OFF_SA + (wm0 + (lane & 15)) * 4, o_sb = OFF_SB + (wn0 + (lane & 15)) * 4;
  const int bsh = 8 * (lane >> 4);  // this lane supplies the scale of 32-wide K block (lane >> 4)

  // One 128-wide K chunk: A fragments and their scale bytes stay in registers, B fragments
  // are double-buffered; the scaled MFMA accumulates directly (no VALU rescale).
  auto compute = [&](uint32_t st) __attribute__((always_inline)) {
    const uint32_t a_lo = st + fa.lo, a_hi = st + fa.hi;
    const uint32_t b_lo = st + OFF_B + fb.lo, b_hi = st + OFF_B + fb.hi;
    const uint32_t sa_ad = st + o_sa, sb_ad = st + o_sb;
    v4i alo[FM], ahi[FM];
    float uaf[FM];
    static_for<0, FM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      alo[j] = ds_read16<j * 2048>(a_lo);
      ahi[j] = ds_read16<j * 2048>(a_hi);
      uaf[j] = ds_read4f<j * 64>(sa_ad);
    });
    v4i blo = ds_read16<0>(b_lo), bhi = ds_read16<0>(b_hi);
    float ubf = ds_read4f<0>(sb_ad);
    lds_wait<0>();
    v8i af[FM];
    int ua[FM];
    static_for<0, FM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      hold(alo[j]);
      hold(ahi[j]);
      hold(uaf[j]);
      af[j] = join(alo[j], ahi[j]);
      ua[j] = (int)(__float_as_uint(uaf[j]) >> bsh);
    });
    hold(blo);
    hold(bhi);
    hold(ubf);
    static_for<0, FN>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      v4i nlo, nhi;
      float nub;
      if constexpr (i + 1 < FN) {
        nlo = ds_read16<(i + 1) * 2048>(b_lo);
        nhi = ds_read16<(i + 1) * 2048>(b_hi);
        nub = ds_read4f<(i + 1) * 64>(sb_ad);
      }
      const v8i bf = join(blo, bhi);
      const int ub = (int)(__float_as_uint(ubf) >> bsh);
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = mfma_fp8(bf, af[j], acc[i][j], ub, ua[j]);
      if constexpr (i + 1 < FN) {
        __builtin_amdgcn_sched_barrier(0);
        lds_wait<0>();
        hold(nlo);
        hold(nhi);
        hold(nub);
        blo = nlo;
        bhi = nhi;
        ubf = nub;
      }
    });
  };

  const uint32_t st0 = lds_addr(sm0), st1 = lds_addr(sm1);
  issue(0, st0);
  int kc = 0;
  for (; kc + 2 <= nkc; kc += 2) {
    wait_vmem();
    __syncthreads();
    issue(kc + 1, st1);
    compute(st0);
    wait_vmem();
    __syncthreads();
    issue(kc + 2, st0);
    compute(st1);
  }
  if (kc < nkc) {
    wait_vmem();
    __syncthreads();
    compute(st0);
  }

#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t m = m0 + wm0 + 16 * j + (lane & 15);
    if (m >= row_end) continue;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int64_t n = n0 + wn0 + 16 * i + 4 * (lane >> 4);
      if (n >= N) continue;
      if (kF32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.Y) + m * N + n) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
        uint2 v;
        v.x = f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16);
        v.y = f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.Y) + m * N + n) = v;
      }
    }
  }
}

// 256x256 tiles, 8 waves of 64x128 (the dense GEMM's large-tile shape): measured faster than
// 128x128 / 128x256 / 256x128 tiles on the routed-MoE shapes even though ragged experts
// leave more of the last m-tile empty.
hipError_t launch_grouped_mx(const GroupedParams& p, bool f32, hipStream_t stream) {
  constexpr int BM = 256, BN = 256, WM = 4, WN = 2;
  // Upper bound on m-tiles for well-formed offsets: sum_e ceil(c_e / BM) <= T / BM + E.
  const int64_t mtiles = (p.T + BM - 1) / BM + p.E;
  const int64_t grid = mtiles * ((p.N + BN - 1) / BN);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (f32)
    hipLaunchKernelGGL((k_grouped_mx<BM, BN, WM, WN, true>), dim3((unsigned)grid), dim3(WM * WN * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((k_grouped_mx<BM, BN, WM, WN, false>), dim3((unsigned)grid), dim3(WM * WN * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fp8rl
