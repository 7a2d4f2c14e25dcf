// Zero-requantization weight install: the FP8 payload and its scales are copied verbatim
// into the rollout-owned buffers ([SkyRL-FP8] "On-Policy FP8 weight sync", Fig. 3: the
// rollout engine installs the transferred representation without a quantizer of its own).
// One launch copies both buffers: 16-byte vector copies for the payload (its size is a
// multiple of 16 for both recipes), then the scale bytes.
#include "device.hpp"
#include "internal.hpp"

namespace fp8rl {

__global__ __launch_bounds__(256) void k_install_copy(const uint4* __restrict__ src_q, uint4* __restrict__ dst_q,
                                                      int64_t n16, const uint8_t* __restrict__ src_s,
                                                      uint8_t* __restrict__ dst_s, int64_t sbytes) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst_q[i] = src_q[i];
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
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;  // grid-stride beyond 1M lanes
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_install_copy, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(src_q), reinterpret_cast<uint4*>(dst_q), n16, src_s, dst_s,
                     sbytes);
  return hipGetLastError();
}

}  // namespace fp8rl
