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
// default fp32 division is correctly rounded), 1.0 for an all-zero group. The scaled values
// x / s are formed without a division per value (quant8 below):
//  - fp32 scales: h = 1/s rounded toward zero, l = (1 - h s) h >= 0 (the residual 1 - h s is
//    exact in one fma), and q = fl32(x h + fl32(x l)): one multiply and one fma per value.
//    q can differ from fl32(x / s) in its last bit, but never so that its E4M3 code (or the
//    sign of a zero) changes: an exhaustive CPU check over every pair of bf16 values
//    (x, amax) with |x| <= amax and a normal s finds no pair whose code differs.
//  - a subnormal s (0 < amax < 448 * 2^-126) has no fp32 reciprocal; a wave with such a
//    group forms fl32(x * fl64(1/s)), which equals fl32(x / s) for every bf16 pair (the same
//    CPU check covers it).
//  - power-of-two scales: h = 2^-e, l = 0 and q = x h, exact whenever |q| is above the fp32
//    subnormal range; below it the E4M3 code is a zero of x's sign either way.
struct BlockScale {
  float s;
  float h, l;
};

__device__ __forceinline__ BlockScale block_scale(float amax) {
  BlockScale b;
  b.s = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
  float h = 1.0f / b.s;
  const float e0 = __builtin_fmaf(-h, b.s, 1.0f);
  h = e0 < 0.0f ? __uint_as_float(__float_as_uint(h) - 1u) : h;   // the float below 1/s
  b.h = h;
  b.l = __builtin_fmaf(-h, b.s, 1.0f) * h;
  return b;
}

// Power-of-two block scale: s = 2^e with the MX exponent rule (smallest e with
// amax <= 448 * 2^e, clamped to [-127, 127]; 2^-127 is an exact fp32 subnormal). The
// scaled value x * 2^-e is then exact (above the fp32 subnormal range) and at most 448 in
// magnitude.
__device__ __forceinline__ BlockScale block_scale_pow2(float amax) {
  const int e = mx_exponent(amax);
  BlockScale b;
  b.s = ldexpf(1.0f, e);
  b.h = ldexpf(1.0f, -e);
  b.l = 0.0f;
  return b;
}

template <bool kPow2>
__device__ __forceinline__ BlockScale group_scale(float amax) {
  if constexpr (kPow2) return block_scale_pow2(amax);
  else return block_scale(amax);
}

// Four fp32 values -> four E4M3 bytes, round to nearest even (v_cvt_pk_fp8_f32 under the
// default round-to-nearest-even mode). The converter does not saturate: it returns the
// max-magnitude code only for 448 < |v| < 464, which covers every quotient above (below 449),
// and NaN beyond; callers never pass |v| >= 464.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// Quantize 8 bf16 values held in 4 words (2 per word) with one group scale -> 8 E4M3 bytes.
// kPow2 names the scale kind (compile time); the fp64 form is chosen per wave, so the branch
// is uniform.
template <bool kPow2>
__device__ __forceinline__ uint2 quant8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, const BlockScale& b) {
  const float x[8] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1),
                      bf16_lo(w2), bf16_hi(w2), bf16_lo(w3), bf16_hi(w3)};
  float q[8];
  if constexpr (kPow2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = x[i] * b.h;
  } else if (__builtin_amdgcn_ballot_w64(!(b.s >= 0x1p-126f)) == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_fmaf(x[i], b.h, x[i] * b.l);
  } else {
    const double r = 1.0 / (double)b.s;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = (float)((double)x[i] * r);
  }
  return make_uint2(pack4_e4m3(q[0], q[1], q[2], q[3]), pack4_e4m3(q[4], q[5], q[6], q[7]));
}

// Group amax in the integer domain. For finite bf16 values the order of the magnitude bits
// (the value with its sign bit cleared) is the numeric order of |x|, so the max needs no
// float compare (and no NaN canonicalization of its operands). mag8() gives, per 16-bit
// half, the largest magnitude among the 8 values in four words (one v_and and one
// v_pk_max_u16 per word); mag_fold() takes the larger half; mag_to_f32() turns magnitude
// bits back into the fp32 value (exact).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b)));
}
__device__ __forceinline__ uint32_t mag8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  constexpr uint32_t k = 0x7fff7fffu;
  return pk_max_u16(pk_max_u16(w0 & k, w1 & k), pk_max_u16(w2 & k, w3 & k));
}
__device__ __forceinline__ uint32_t mag8(const uint4& v) { return mag8(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ uint32_t mag_fold(uint32_t m) { return max(m & 0xffffu, m >> 16); }
__device__ __forceinline__ float mag_to_f32(uint32_t m) { return __uint_as_float(m << 16); }

// Max over aligned groups of kLanes consecutive lanes (2, 4, 8 or 16), every lane of a group
// receiving it, by DPP lane moves: swaps within a quad (lanes i ^ 1, then i ^ 2), then the
// half-row mirror (lane i with 7 - i within 8) and the row mirror (i with 15 - i within 16).
// Every lane of the wave must be active.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kCtrl, 0xf, 0xf, true));
}
template <int kLanes>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  static_assert(kLanes == 2 || kLanes == 4 || kLanes == 8 || kLanes == 16, "group of 2-16 lanes");
  v = dpp_max<0xB1>(v);                                // quad_perm [1, 0, 3, 2]
  if constexpr (kLanes >= 4) v = dpp_max<0x4E>(v);     // quad_perm [2, 3, 0, 1]
  if constexpr (kLanes >= 8) v = dpp_max<0x141>(v);    // row_half_mirror
  if constexpr (kLanes >= 16) v = dpp_max<0x140>(v);   // row_mirror
  return v;
}

// amax of a group whose lanes hold 8 values each in (a, b) words: magnitude bits, group max.
template <int kLanes>
__device__ __forceinline__ float group_amax(uint32_t m) {
  return mag_to_f32(group_max<kLanes>(mag_fold(m)));
}

// fp32 group scales from a 1 KB per-workgroup table instead of two divisions per group. For
// the 128 bf16 mantissas of an amax in [1, 2) the table holds s_m = fl32(a / 448) and h_m =
// 1/s_m rounded toward zero. For an amax with biased exponent E and a normal s,
// fl32(amax / 448) = s_m 2^(E-127) and its rounded-down reciprocal is h_m 2^(127-E), exactly
// (a power-of-two factor commutes with both roundings while the results stay normal), so
// these scales equal block_scale()'s bit for bit. A subnormal s (amax below 448 * 2^-126,
// bf16 magnitude bits < 0x04E0) is divided for as in block_scale(); quant8() then takes the
// fp64 form for the wave.
__device__ __forceinline__ void fill_scale_table(float2* tab, int tid) {
  if (tid < 128) {
    const BlockScale b = block_scale(__uint_as_float(0x3F800000u | ((uint32_t)tid << 16)));
    tab[tid] = make_float2(b.s, b.h);
  }
}
__device__ __forceinline__ BlockScale table_scale(uint32_t m16, const float2* tab) {
  const float2 t = tab[m16 & 127u];
  const int E = (int)(m16 >> 7);
  BlockScale b;
  b.s = ldexpf(t.x, E - 127);
  b.h = ldexpf(t.y, 127 - E);
  b.l = __builtin_fmaf(-b.h, b.s, 1.0f) * b.h;
  if (m16 == 0) b = BlockScale{1.0f, 1.0f, 0.0f};
  const bool tiny = m16 != 0 && m16 < 0x04E0u;
  if (__builtin_amdgcn_ballot_w64(tiny) != 0 && tiny) b.s = mag_to_f32(m16) / kE4M3Max;
  return b;
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
