// The 1x128 row and 128x128 tile quantizer kernels, generic over where their bf16 input
// comes from. A source presents a virtual bf16 matrix [R][C] (C % 128 == 0) in two steps,
// so that a thread issues all of its loads before any of the arithmetic:
//   fetch8(row, col)        -> the raw inputs (Src::Raw) of the 8 values at (row, col .. col+7),
//                              col % 8 == 0;
//   fetch16(g, part, a, b)  -> those of the 16 values of 1x128 group g, part `part` (0..7),
//                              i.e. row g / (C/128), columns (g % (C/128)) * 128 + 16 * part ...;
//   make(raw, lds)          -> the 8 bf16 values (4 words) from their raw inputs.
// A source may keep a table in LDS: Src::kLdsBytes bytes, filled by prepare(lds, tid, nt)
// (all threads of the workgroup, then a barrier) before the first make().
// Plain quantization reads the matrix from memory; the fused producers compute it from
// their own inputs (SwiGLU of the gate/up output, RMSNorm of the residual stream), so the
// bf16 values never go through memory. Method: [AIS] symmetric quantizer equation on the
// E4M3 grid; granularities from [Jet-RL] "Quantization scheme".
#pragma once

#include "device.hpp"

namespace fp8rl {

// 16-byte non-temporal load (global_load_dwordx4 ... nt).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ntload16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 matrix [R][C] in memory, row-major. The quantizers read their input once, so the
// loads are non-temporal: they do not displace lines the last-level cache holds for
// others, such as the dirty output of the GEMM that ran before (which the loads would
// otherwise have to evict).
struct PlainSrc {
  typedef uint4 Raw;
  static constexpr int kLdsBytes = 0;
  const uint16_t* x;
  int64_t C;
  __device__ __forceinline__ Raw fetch8(int64_t row, int64_t col) const { return ntload16(x + row * C + col); }
  // Groups tile the rows exactly, so group g starts at element g * 128.
  __device__ __forceinline__ void fetch16(int64_t g, int part, Raw& a, Raw& b) const {
    const uint16_t* p = x + g * 128 + part * 16;
    a = ntload16(p);
    b = ntload16(p + 8);
  }
  __device__ __forceinline__ void prepare(void*, int, int) const {}
  __device__ __forceinline__ uint4 make(const Raw& r, const void*) const { return r; }
};

// LDS for a source's table (at least 16 bytes so that the declaration is valid).
template <class Src>
struct SrcLds {
  static constexpr int kBytes = Src::kLdsBytes > 0 ? Src::kLdsBytes : 16;
};

// ---------------------------------------------------------------------------------------
// 1x128 row groups. The groups of X[M][K] tile each row exactly, so group g starts at
// element g * 128 and its scale is s[g] (row-major [M][K/128]). 8 lanes per group, 16
// elements (32 bytes) per lane; one wave covers 8 consecutive groups = 2 KB of input.
// ---------------------------------------------------------------------------------------
template <class Src, bool kPow2>
__global__ __launch_bounds__(256) void k_quant_rows_1x128(Src src, uint8_t* __restrict__ q, float* __restrict__ s,
                                                          int64_t ngroups) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[SrcLds<Src>::kBytes];
  if constexpr (Src::kLdsBytes > 0) {
    src.prepare(lds, threadIdx.x, 256);
    __syncthreads();
  }
  const int part = (int)(threadIdx.x & 7);
  // Each workgroup takes 32 consecutive groups per step (one step when the grid covers
  // all groups, as for plain quantization).
  for (int64_t g0 = (int64_t)blockIdx.x * 32; g0 < ngroups; g0 += (int64_t)gridDim.x * 32) {
    const int64_t g = g0 + (threadIdx.x >> 3);
    const bool valid = g < ngroups;
    uint4 a = make_uint4(0, 0, 0, 0), b = a;
    if (valid) {
      typename Src::Raw ra, rb;
      src.fetch16(g, part, ra, rb);
      a = src.make(ra, lds);
      b = src.make(rb, lds);
    }
    const float amax = group_amax<8>(pk_max_u16(mag8(a), mag8(b)));
    const BlockScale bs = group_scale<kPow2>(amax);
    if (valid) {
      const uint2 lo = quant8<kPow2>(a.x, a.y, a.z, a.w, bs);
      const uint2 hi = quant8<kPow2>(b.x, b.y, b.z, b.w, bs);
      *reinterpret_cast<uint4*>(q + g * 128 + part * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
      if (part == 0) s[g] = bs.s;
    }
  }
}

// ---------------------------------------------------------------------------------------
// 128 x 128 tile kernel, 512 threads (8 waves), one tile per workgroup.
//   kBlock = false: activation mode. Row output = 1x128 groups (q [R][C], s [R][C/128]),
//                   column output = 128x1 groups written transposed (qt [C][R], st [C][R/128]).
//   kBlock = true : weight mode. One scale for the whole 128x128 block (s [R/128][C/128]);
//                   qt, if requested, is the byte transpose of q (same scale, same bytes).
//   kG = 32 (with kPow2): MXFP8 mode. Row output = 1x32 groups, column output = 32x1
//                   groups written transposed; the scales are E8M0 bytes (e + 127, the
//                   exponent field of the power-of-two scale) [R][C/32] and [C][R/32].
// Grid: one workgroup per tile, (R/128) * (C/128) of them (tile order below).
// Thread t owns the 4x8 sub-block rows 4*(t/16) .. +3, columns 8*(t%16) .. +7. Each wave
// load instruction then reads 4 whole 256-byte row segments, and each row-output store
// writes whole 128-byte lines. Row amax: max over the 16 lanes sharing a row.
// Column pass: each thread transposes its sub-block in registers (byte permutes) into a
// column-major LDS tile, [column][128 rows of bf16], whose 16-byte chunks (8 rows) are
// XOR-swizzled by column/8 so that neither the writes nor the reads conflict. Eight lanes
// then own one column (16 rows each): column amax over those 8 lanes, and each store
// instruction writes 8 whole 128-byte lines of qt.
// ---------------------------------------------------------------------------------------
// Store a group scale: fp32 for 128-wide groups, the E8M0 byte for 32-wide (MX) groups.
template <int kG>
__device__ __forceinline__ void store_scale(void* p, int64_t i, const BlockScale& bs) {
  if constexpr (kG == 32)
    reinterpret_cast<uint8_t*>(p)[i] = (uint8_t)(__float_as_uint(bs.s) >> 23);
  else
    reinterpret_cast<float*>(p)[i] = bs.s;
}

template <class Src, bool kBlock, bool kPow2, int kG = 128>
__global__ __launch_bounds__(512) void k_quant_tile(Src src, int64_t R, int64_t C, uint8_t* __restrict__ q,
                                                    void* __restrict__ s, uint8_t* __restrict__ qt,
                                                    void* __restrict__ st) {
  static_assert(kG == 128 || (kG == 32 && kPow2 && !kBlock), "MX groups take power-of-two scales");
  __shared__ __attribute__((aligned(16))) uint32_t tile[128 * 64];   // [column][row pair]
  __shared__ float red[8];
  __shared__ __attribute__((aligned(16))) uint8_t src_lds[SrcLds<Src>::kBytes];
  // fp32 scales of the row and column groups (several per thread) come from a table
  constexpr bool kTab = !kBlock && !kPow2;
  __shared__ float2 stab[kTab ? 128 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 15, rg = tid >> 4;                               // rg: 0..31
  // The grid has (R/128) (C/128) < 2^32 workgroups, so tile indices fit in 32 bits.
  const uint32_t ncb = (uint32_t)(C / 128), bid = blockIdx.x;
  // Tile order: the hardware deals consecutive workgroups to the 8 XCDs in turn. When the
  // column blocks split evenly, XCD x takes the column blocks [x w, (x+1) w), w = ncb / 8,
  // row block by row block. The tiles in flight still cover a few whole block rows (the
  // read stream keeps its locality), and each XCD's L2 sees fewer of the lines that
  // several tiles' 4-byte scale stores share.
  uint32_t cb, rb;
  if (ncb % 8 == 0) {
    const uint32_t w = ncb / 8, i = bid >> 3;
    cb = (bid & 7) * w + i % w;
    rb = i / w;
  } else {
    cb = bid % ncb;
    rb = bid / ncb;
  }
  const bool want_rows = q != nullptr, want_cols = qt != nullptr;
  // Element offsets: this thread's first row and column, and (column pass) its first column.
  const int64_t row0 = (int64_t)rb * 128 + 4 * rg, col0 = (int64_t)cb * 128 + c * 8;
  const int64_t qoff = row0 * C + col0;

  typename Src::Raw raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = src.fetch8(row0 + i, col0);
  if constexpr (Src::kLdsBytes > 0 || kTab) {
    if constexpr (Src::kLdsBytes > 0) src.prepare(src_lds, tid, 512);
    if constexpr (kTab) fill_scale_table(stab, tid);
    __syncthreads();
  }
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src.make(raw[i], src_lds);

  BlockScale bblk{1.0f, 1.0f, 0.0f};
  if (kBlock) {
    uint32_t m = pk_max_u16(pk_max_u16(mag8(v[0]), mag8(v[1])), pk_max_u16(mag8(v[2]), mag8(v[3])));
    m = group_max<16>(mag_fold(m));
    m = max(m, (uint32_t)__shfl_xor((int)m, 16));
    float a = mag_to_f32(max(m, (uint32_t)__shfl_xor((int)m, 32)));
    if (lane == 0) red[wave] = a;
    __syncthreads();
    a = fmaxf(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7])));
    bblk = group_scale<kPow2>(a);
    if (tid == 0) store_scale<128>(s, rb * ncb + cb, bblk);
    if (want_rows) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint2*>(q + qoff + i * C) = quant8<kPow2>(v[i].x, v[i].y, v[i].z, v[i].w, bblk);
    }
  } else if (want_rows) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m16 = group_max<kG / 8>(mag_fold(mag8(v[i])));
      BlockScale bs;
      if constexpr (kTab) bs = table_scale(m16, stab);
      else bs = group_scale<kPow2>(mag_to_f32(m16));
      constexpr int kLanes = kG / 8;                               // lanes of one row group
      if ((c & (kLanes - 1)) == 0) store_scale<kG>(s, (int64_t)((uint64_t)(qoff + i * C) / kG), bs);
      *reinterpret_cast<uint2*>(q + qoff + i * C) = quant8<kPow2>(v[i].x, v[i].y, v[i].z, v[i].w, bs);
    }
  }
  if (!want_cols) return;

  // Column 8c+j, rows 4rg..4rg+3 = 8 bytes: half (rg & 1) of the 16-byte chunk rg >> 1,
  // stored at chunk position (rg >> 1) ^ c.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;   // high or low bf16 of each word
    const int p = j >> 1;
    const uint32_t a0 = p == 0 ? v[0].x : p == 1 ? v[0].y : p == 2 ? v[0].z : v[0].w;
    const uint32_t a1 = p == 0 ? v[1].x : p == 1 ? v[1].y : p == 2 ? v[1].z : v[1].w;
    const uint32_t a2 = p == 0 ? v[2].x : p == 1 ? v[2].y : p == 2 ? v[2].z : v[2].w;
    const uint32_t a3 = p == 0 ? v[3].x : p == 1 ? v[3].y : p == 2 ? v[3].z : v[3].w;
    *reinterpret_cast<uint2*>(tile + (8 * c + j) * 64 + (((rg >> 1) ^ c) & 15) * 4 + (rg & 1) * 2) =
        make_uint2(__builtin_amdgcn_perm(a1, a0, sel), __builtin_amdgcn_perm(a3, a2, sel));
  }
  __syncthreads();

  // Wave w: columns 16w .. 16w+15, 8 per round; lane: column +lane/8, rows 16k .. 16k+15.
  // The two chunks are read in an order (odd first for half the lanes) that keeps every
  // group of 8 or 16 lanes on distinct banks.
  const int k = lane & 7;
  // qt [C][R]: this lane's first column is cb 128 + 16 wave + lane / 8, rows rb 128 + 16 k ...
  const int64_t qtoff = ((int64_t)cb * 128 + 16 * wave + (lane >> 3)) * R + (int64_t)rb * 128 + 16 * k;
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int col = 16 * wave + 8 * rd + (lane >> 3);
    const int sw = (2 * wave + rd) & 15;                            // = (col / 8) & 15
    const int a = 2 * k + ((k >> 2) ^ (col & 1));
    const uint4 A = *reinterpret_cast<const uint4*>(tile + col * 64 + ((a ^ sw) * 4));
    const uint4 B = *reinterpret_cast<const uint4*>(tile + col * 64 + (((a ^ 1) ^ sw) * 4));
    const bool even = (a & 1) == 0;
    const uint4 lo = even ? A : B, hi = even ? B : A;               // rows 16k..+7, 16k+8..+15
    BlockScale r = bblk;
    if (!kBlock) {
      const uint32_t m16 = group_max<kG / 16>(mag_fold(pk_max_u16(mag8(lo), mag8(hi))));
      BlockScale bs;
      if constexpr (kTab) bs = table_scale(m16, stab);
      else bs = group_scale<kPow2>(mag_to_f32(m16));
      r = bs;
      constexpr int kLanes = kG / 16;                              // lanes of one column group
      if ((k & (kLanes - 1)) == 0) store_scale<kG>(st, (int64_t)((uint64_t)(qtoff + 8 * rd * R) / kG), bs);
    }
    const uint2 o0 = quant8<kPow2>(lo.x, lo.y, lo.z, lo.w, r);
    const uint2 o1 = quant8<kPow2>(hi.x, hi.y, hi.z, hi.w, r);
    *reinterpret_cast<uint4*>(qt + qtoff + 8 * rd * R) = make_uint4(o0.x, o0.y, o1.x, o1.y);
  }
}

}  // namespace fp8rl
