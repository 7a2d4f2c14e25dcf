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
  constexpr int STAGE = OFF_SB + BN * 4;
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
  // zero without a memory access (see the dense GEMM).
  constexpr int LA = BM * 8 / NT, LB = BN * 8 / NT;
  const int64_t rows_a = min((int64_t)BM, row_end - m0), rows_b = min((int64_t)BN, N - n0);
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
    bytesS = (uint32_t)((rows_b - 1) * (K / 32) + 4);
  }
  const int s_lds = sa_wave ? OFF_SA + wave * 256 : OFF_SB + (wave - BM / 64) * 256;

  auto issue = [&](int kc, uint8_t* sm) {
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.X + m0 * K + kc * 128, bytesA);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Wb + n0 * K + kc * 128, bytesB);
#pragma unroll
    for (int it = 0; it < LA; ++it) buf2lds16(ra, offA[it], sm + (it * NT + wave * 64) * 16);
#pragma unroll
    for (int it = 0; it < LB; ++it) buf2lds16(rb, offB[it], sm + OFF_B + (it * NT + wave * 64) * 16);
    if (sa_wave || sb_wave) buf2lds4(make_rsrc(baseS + kc * 4, bytesS), offS, sm + s_lds);
  };

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int bsh = 8 * (lane >> 4);  // this lane supplies the scale of K block (lane >> 4)
  auto compute = [&](const uint8_t* sm) {
    const uint32_t* scA = reinterpret_cast<const uint32_t*>(sm + OFF_SA);
    const uint32_t* scB = reinterpret_cast<const uint32_t*>(sm + OFF_SB);
    v8i af[FM];
    int ua[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      af[j] = load_frag(sm, wm0 + 16 * j, lane);
      ua[j] = (int)(scA[wm0 + 16 * j + (lane & 15)] >> bsh);
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const v8i bfr = load_frag(sm + OFF_B, wn0 + 16 * i, lane);
      const int ub = (int)(scB[wn0 + 16 * i + (lane & 15)] >> bsh);
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = mfma_fp8(bfr, af[j], acc[i][j], ub, ua[j]);
    }
  };

  // K loop over pairs of blocks (stage 0 then stage 1) with a single exit, and a peeled
  // last block when the count is odd.
  issue(0, sm0);
  int kc = 0;
  for (; kc + 2 <= nkc; kc += 2) {
    wait_vmem();
    __syncthreads();
    issue(kc + 1, sm1);
    compute(sm0);
    wait_vmem();
    __syncthreads();
    if (kc + 2 < nkc) issue(kc + 2, sm0);
    compute(sm1);
  }
  if (kc < nkc) {
    wait_vmem();
    __syncthreads();
    compute(sm0);
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

hipError_t launch_grouped_mx(const GroupedParams& p, bool f32, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  // Upper bound on m-tiles for well-formed offsets: sum_e ceil(c_e / BM) <= T / BM + E.
  const int64_t mtiles = (p.T + BM - 1) / BM + p.E;
  const int64_t grid = mtiles * ((p.N + BN - 1) / BN);
  if (f32)
    hipLaunchKernelGGL((k_grouped_mx<BM, BN, 2, 2, true>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((k_grouped_mx<BM, BN, 2, 2, false>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fp8rl
