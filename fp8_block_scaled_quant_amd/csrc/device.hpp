// Device helpers shared by the libfp8rl kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp8rl {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round an fp32 value to bf16 bits, nearest-even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two fp32 values -> their bf16 bits in one word (lo in bits 0..15), nearest-even: one
// v_cvt_pk_bf16_f32 on gfx950. For finite values the same bits as f32_to_bf16_bits (checked on
// the device over every bf16 high half with boundary, tie and subnormal low halves, and 4M
// random patterns).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// MXFP8 exponent for a group amax: the smallest integer e with amax <= 448 * 2^e, clamped
// to [-127, 127]; 0 for amax == 0. For amax = 1.m * 2^F (m the 23-bit field), 448 * 2^(F-8)
// = 1.75 * 2^F, so e = F - 8 when the mantissa field is <= 0x600000, else F - 7. A
// subnormal amax (< 2^-126) needs e <= -134, i.e. the clamp value -127.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.0f) return 0;
  const uint32_t u = __float_as_uint(amax);
  const int be = (int)((u >> 23) & 0xffu);
  if (be == 0) return -127;
  const int F = be - 127;
  int e = ((u & 0x7fffffu) <= 0x600000u) ? F - 8 : F - 7;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Scale of a 1x128 / 128x1 / 128x128 group: s = fl32(amax / 448) (IEEE division; hipcc's
// default fp32 division is correctly rounded), 1.0 for an all-zero group. `r` is the
// fp64 reciprocal used to form the scaled values (see scaled()).
struct BlockScale {
  float s;
  double r;
};

__device__ __forceinline__ BlockScale block_scale(float amax) {
  BlockScale b;
  b.s = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
  b.r = 1.0 / (double)b.s;
  return b;
}

// Power-of-two block scale: s = 2^e with the MX exponent rule (smallest e with
// amax <= 448 * 2^e, clamped to [-127, 127]; 2^-127 is an exact fp32 subnormal). The
// scaled value x * 2^-e is then exact (scaled() computes it without rounding) and at most
// 448 in magnitude.
__device__ __forceinline__ BlockScale block_scale_pow2(float amax) {
  const int e = mx_exponent(amax);
  BlockScale b;
  b.s = ldexpf(1.0f, e);
  b.r = ldexp(1.0, -e);
  return b;
}

template <bool kPow2>
__device__ __forceinline__ BlockScale group_scale(float amax) {
  if constexpr (kPow2) return block_scale_pow2(amax);
  else return block_scale(amax);
}

// The fp32 quotient fl32(x / s) for a bf16 value x with |x| <= amax, computed as
// fl32(x * fl64(1/s)). x has 8 significant bits and s 24, so x/s never lies within a
// relative 2^-49 of an fp32 rounding midpoint, while the fp64 product is within 2^-52 of
// x/s: both round to the same fp32 value. (An exhaustive CPU test over every bf16 pair
// (x, amax) checks this identity, and that |x/s| stays below 449.)
__device__ __forceinline__ float scaled(float x, double r) { return (float)((double)x * r); }

// Four fp32 values -> four E4M3 bytes, round to nearest even (v_cvt_pk_fp8_f32 under the
// default round-to-nearest-even mode). The converter does not saturate: it returns the
// max-magnitude code only for 448 < |v| < 464, which covers every quotient above, and NaN
// beyond; callers never pass |v| >= 464.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// Quantize 8 bf16 values held in 4 words (2 per word) with one group scale -> 8 E4M3 bytes.
__device__ __forceinline__ uint2 quant8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, double r) {
  uint2 o;
  o.x = pack4_e4m3(scaled(bf16_lo(w0), r), scaled(bf16_hi(w0), r), scaled(bf16_lo(w1), r), scaled(bf16_hi(w1), r));
  o.y = pack4_e4m3(scaled(bf16_lo(w2), r), scaled(bf16_hi(w2), r), scaled(bf16_lo(w3), r), scaled(bf16_hi(w3), r));
  return o;
}

// max(|lo|, |hi|) of the two bf16 values in a word.
__device__ __forceinline__ float absmax2(uint32_t w) {
  return fmaxf(fabsf(bf16_lo(w)), fabsf(bf16_hi(w)));
}


// Raw buffer descriptor over [base, base + bytes) as four SGPR words: loads at byte
// offsets >= bytes return zero instead of touching memory (the hardware range check of
// raw buffers, stride 0). The last word is the gfx9 buffer format word.
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t*)p);
}

// Direct buffer -> LDS copies (buffer_load_dword{,x4} ... lds): lane i's 16 (or 4) bytes
// from rsrc + voff land at LDS address lds + 16 * i (or 4 * i); lds must be wave-uniform.
// Issued as inline assembly on purpose: the copy's completion is awaited explicitly
// (wait_vmem() followed by a barrier before the stage is read), so the compiler must not
// insert its own conservative vmcnt waits in front of unrelated LDS reads. The copy
// instruction takes its LDS address in m0, which the asm sets and declares clobbered
// (the compiler warns that m0 is reserved); gfx950 code needs m0 for nothing else here,
// and the generated kernels contain no other access to it.
// Wait states (CDNA3/CDNA4 ISA, manually inserted wait states): a buffer instruction that
// reads an SGPR needs 5 wait states after a VALU instruction wrote that SGPR (the compiler
// often rebuilds a descriptor with v_readfirstlane right before the asm), and a copy to LDS
// needs 1 after an SALU write of m0. The compiler's hazard pass cannot see inside an asm
// statement, so every asm buffer instruction here pays for both itself: the s_nop 4 after
// the m0 write (or in front of the load) supplies the wait states. Without them the load may
// use the previous descriptor or m0, i.e. read another buffer or write another LDS slot.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(v4i rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

// dma16 when `on` (wave-uniform) is non-zero; otherwise the copy is skipped. The
// branch sits inside the one asm statement, so the compiler sees straight-line code (a
// branch around the copy in the K loop costs the register allocator ~40 VGPRs), and a
// skipped copy costs the texture unit nothing (unlike one issued with exec = 0 or an empty
// descriptor, which it processes like a real one).
__device__ __forceinline__ void dma16_if(v4i rsrc, uint32_t voff, uint32_t lds, uint32_t on) {
  asm volatile(
      "s_cmp_eq_u32 %3, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds\n"
      "1:"
      :
      : "v"(voff), "s"(rsrc), "s"(lds), "s"(__builtin_amdgcn_readfirstlane(on))
      : "memory", "m0", "scc");
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory operations of this wave are outstanding (they
// complete in issue order, so this waits for all but the N most recent).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Swizzled LDS layout for 128-byte rows of FP8 (one 128-wide K block per row): the 16-byte
// chunk c of row r is stored at chunk position c ^ ((r >> 1) & 7). With 64 banks of 4 bytes,
// 16 consecutive rows reading the same logical chunk then hit 16 distinct 16-byte bank
// groups.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// MFMA operand fragment for v_mfma_*_16x16x128_f8f6f4: lane l holds row (l & 15) of a
// 16 x 128 FP8 tile; lane group g = l >> 4 holds K bytes [16g, 16g+16) in bytes 0..15 and
// [64+16g, 64+16g+16) in bytes 16..31. In the swizzled 128-byte-row LDS tile, every
// fragment that starts on a multiple of 16 rows has the same swizzle phase, so a lane's
// two byte offsets are computed once (FragOffsets) and fragment f of a run of fragments
// is read at those offsets + f * 2048 (an immediate offset of the LDS read).
struct FragOffsets {
  uint32_t lo, hi;
};
__device__ __forceinline__ FragOffsets frag_offsets(int row0, int lane) {
  const int row = row0 + (lane & 15);   // row0 % 16 == 0
  const int g = lane >> 4;
  FragOffsets o;
  o.lo = (uint32_t)(row * 128 + (swz(row, g) << 4));
  o.hi = (uint32_t)(row * 128 + (swz(row, g + 4) << 4));
  return o;
}
// LDS reads issued in program order as inline assembly (the compiler neither hoists them
// nor inserts waits for them); the consumer calls lds_wait(...) on the destination
// registers, which orders every later use after the wait.
template <int OFF>
__device__ __forceinline__ v4i ds_read16(uint32_t addr) {
  v4i r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ float ds_read4f(uint32_t addr) {
  float r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Two dwords at addr + 4 * O0 and addr + 4 * O1 (offsets in dwords, at most 255).
template <int O0, int O1>
__device__ __forceinline__ v2i ds_read2_b32(uint32_t addr) {
  static_assert(O0 >= 0 && O0 <= 255 && O1 >= 0 && O1 <= 255, "ds_read2_b32 offsets");
  v2i r;
  asm volatile("ds_read2_b32 %0, %1 offset0:%2 offset1:%3" : "=v"(r) : "v"(addr), "i"(O0), "i"(O1));
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N)); }
// Tie a value to the preceding wait so no use of it can be scheduled before the wait.
template <typename T>
__device__ __forceinline__ void hold(T& v) { asm volatile("" : "+v"(v)); }

// Fragment f of a run (see FragOffsets) from the LDS tile at byte address `tile`.
template <int F>
__device__ __forceinline__ void read_frag(uint32_t tile, FragOffsets o, v4i& lo, v4i& hi) {
  lo = ds_read16<F * 2048>(tile + o.lo);
  hi = ds_read16<F * 2048>(tile + o.hi);
}
__device__ __forceinline__ v8i join(const v4i& lo, const v4i& hi) {
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}
// 16x16x128 FP8 MFMA (E4M3 x E4M3, cbsz = blgp = 0). Scales are E8M0 bytes; lane
// (i + 16 b) supplies the scale of row i for K block [32b, 32b+32). 127 = 1.0.
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b, v4f c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Logical tile index for workgroup `bid` of `nblocks`: the hardware deals workgroups to
// the 8 XCDs round-robin (bid % 8); this gives XCD x the contiguous logical range
// [start_x, start_x + count_x) so that neighbouring tiles, which share operand rows,
// run under the same L2. A bijection on [0, nblocks).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks >> 3, rem = nblocks & 7;
  const int x = bid & 7, idx = bid >> 3;
  return (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

}  // namespace fp8rl
