// Zero-requantization weight install: the FP8 payload and its scales are copied verbatim
// into the rollout-owned buffers ([SkyRL-FP8] "On-Policy FP8 weight sync", Fig. 3: the
// rollout engine installs the transferred representation without a quantizer of its own).
// One launch copies both buffers: 16-byte vector copies for the payload (its size is a
// multiple of 16 for both recipes), then the scale bytes.
#include "device.hpp"
#include "internal.hpp"

namespace fp8rl {

// Each thread copies 4 payload vectors (all loads issued before the stores), with
// non-temporal hints: the copy streams through once and should not displace cached data.
constexpr int kCopyUnroll = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_install_copy(const u32x4* __restrict__ src_q, u32x4* __restrict__ dst_q,
                                                      int64_t n16, const uint8_t* __restrict__ src_s,
                                                      uint8_t* __restrict__ dst_s, int64_t sbytes) {
  const int64_t base = (int64_t)blockIdx.x * 256 * kCopyUnroll + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < n16) v[u] = __builtin_nontemporal_load(src_q + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < n16) __builtin_nontemporal_store(v[u], dst_q + i);
  }
  // scales: dwords, then the byte tail, spread over the same grid
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t s4 = sbytes >> 2;
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src_s);
  uint32_t* d32 = reinterpret_cast<uint32_t*>(dst_s);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < s4; i += stride) d32[i] = s32[i];
  const int64_t tail = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tail < (sbytes & 3)) dst_s[s4 * 4 + tail] = src_s[s4 * 4 + tail];
}

hipError_t launch_copy(const uint8_t* src_q, uint8_t* dst_q, int64_t qbytes, const uint8_t* src_s, uint8_t* dst_s,
                       int64_t sbytes, hipStream_t stream) {
  const int64_t n16 = qbytes / 16;
  int64_t blocks = (n16 + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
  if (blocks < 1) blocks = 1;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_install_copy, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(src_q), reinterpret_cast<u32x4*>(dst_q), n16, src_s, dst_s,
                     sbytes);
  return hipGetLastError();
}

}  // namespace fp8rl
