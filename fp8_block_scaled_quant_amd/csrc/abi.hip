// C ABI of libfp8rl (declared in include/fp8rl.h). Every entry point validates all of its
// arguments on the host before making any HIP call, checks once per device that the
// current device is gfx950, then enqueues its kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/fp8rl.h"
#include "internal.hpp"

namespace {

using namespace fp8rl;

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

fp8rl_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8RL_ERR_DEVICE;
  int state = dev < kMaxDevices ? g_device_state[dev].load(std::memory_order_acquire) : 0;
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8RL_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (dev < kMaxDevices) g_device_state[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? FP8RL_OK : FP8RL_ERR_DEVICE;
}

fp8rl_status launched(hipError_t e) { return e == hipSuccess ? FP8RL_OK : FP8RL_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Grid-size guard: kernels index workgroups with 32-bit ids.
constexpr int64_t kMaxElems = (int64_t)1 << 40;

fp8rl_status check_dims(int64_t a, int64_t b) {
  if (a < 0 || b < 0) return FP8RL_ERR_SHAPE;
  if (a > 0 && b > kMaxElems / a) return FP8RL_ERR_SHAPE;
  return FP8RL_OK;
}

// GEMM reduction length: the kernels address up to 256 operand rows of one tile through a
// single buffer descriptor with 32-bit byte offsets, (256 - 1) * kred + 128 < 2^32.
constexpr int64_t kMaxRed = (int64_t)1 << 23;

fp8rl_status check_red(int64_t kred) { return kred > kMaxRed ? FP8RL_ERR_SHAPE : FP8RL_OK; }

// Scratch of the allocation-free forward (fp8_gemm_blockscaled_fwd_decode_layout_noalloc):
// the quantized X and its scales of one call, in a file-scope device array that every GPU
// the library runs on holds until the process ends. In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[FP8RL_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

fp8rl_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8RL_ERR_DEVICE;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FP8RL_ERR_DEVICE;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP8RL_OK;
}

}  // namespace

extern "C" {

int fp8rl_abi_version(void) { return FP8RL_ABI_VERSION; }

const char* fp8rl_status_str(int s) {
  switch (s) {
    case FP8RL_OK: return "ok";
    case FP8RL_ERR_NULL: return "required pointer is NULL (or an output pair is half given)";
    case FP8RL_ERR_SHAPE: return "invalid shape for this call's granularity rules";
    case FP8RL_ERR_ALIGN: return "pointer misaligned (data 16 bytes, fp32 scales 4 bytes)";
    case FP8RL_ERR_RECIPE: return "unsupported recipe/dtype or install descriptors disagree";
    case FP8RL_ERR_DEVICE: return "current HIP device is not gfx950";
    case FP8RL_ERR_LAUNCH: return "kernel launch failed";
    case FP8RL_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8RL_ERR_VALUE: return "scalar argument out of range";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

// Output-pair rules of the activation quantizers and the quantizing producers.
fp8rl_status check_act_outputs(int64_t M, uint8_t* q, float* s, uint8_t* qt, float* st) {
  if ((q == nullptr) != (s == nullptr) || (qt == nullptr) != (st == nullptr)) return FP8RL_ERR_NULL;
  if (q == nullptr && qt == nullptr) return FP8RL_ERR_NULL;
  if (qt != nullptr && M % 128 != 0) return FP8RL_ERR_SHAPE;
  return FP8RL_OK;
}

fp8rl_status quant_act_impl(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, uint8_t* qt, float* st,
                            bool pow2, void* stream) {
  if (fp8rl_status e = check_dims(M, K)) return e;
  if (K % 128 != 0) return FP8RL_ERR_SHAPE;
  if (M == 0 || K == 0) return FP8RL_OK;                     // empty work: outputs may be empty (NULL)
  if (fp8rl_status e = check_act_outputs(M, q, s, qt, st)) return e;
  if (x == nullptr) return FP8RL_ERR_NULL;
  if (!aligned(x, 16) || (q && !aligned(q, 16)) || (qt && !aligned(qt, 16)) || (s && !aligned(s, 4)) ||
      (st && !aligned(st, 4)))
    return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  if (qt == nullptr) return launched(launch_quant_rows_1x128(x, M, K, q, s, pow2, as_stream(stream)));
  return launched(launch_quant_act_tile(x, M, K, q, s, qt, st, pow2, as_stream(stream)));
}

bool act_outputs_aligned(uint8_t* q, float* s, uint8_t* qt, float* st) {
  return !((q && !aligned(q, 16)) || (qt && !aligned(qt, 16)) || (s && !aligned(s, 4)) || (st && !aligned(st, 4)));
}

fp8rl_status swiglu_check(const uint16_t* gu, int64_t M, int64_t F) {
  if (fp8rl_status e = check_dims(M, 2 * F)) return e;
  if (F % 128 != 0) return FP8RL_ERR_SHAPE;
  if (M > 0 && F > 0 && gu == nullptr) return FP8RL_ERR_NULL;
  if (gu != nullptr && !aligned(gu, 16)) return FP8RL_ERR_ALIGN;
  return FP8RL_OK;
}

fp8rl_status rms_check(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps, const float* rstd) {
  if (fp8rl_status e = check_dims(M, K)) return e;
  if (K % 128 != 0 || K > 65536 || M > INT32_MAX) return FP8RL_ERR_SHAPE;
  if (!(eps > 0.0f) || !(eps <= 3.4028235e38f)) return FP8RL_ERR_VALUE;
  if (M > 0 && K > 0 && (x == nullptr || gamma == nullptr || rstd == nullptr)) return FP8RL_ERR_NULL;
  if ((x && !aligned(x, 16)) || (gamma && !aligned(gamma, 16)) || (rstd && !aligned(rstd, 4))) return FP8RL_ERR_ALIGN;
  return FP8RL_OK;
}

fp8rl_status quant_w_impl(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt, bool pow2,
                          void* stream) {
  if (q == nullptr || s == nullptr) return FP8RL_ERR_NULL;
  if (fp8rl_status e = check_dims(N, K)) return e;
  if (N % 128 != 0 || K % 128 != 0) return FP8RL_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8RL_OK;
  if (w == nullptr) return FP8RL_ERR_NULL;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s, 4) || (qt && !aligned(qt, 16))) return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  return launched(launch_quant_w_128x128(w, N, K, q, s, qt, pow2, as_stream(stream)));
}

}  // namespace

extern "C" {

fp8rl_status fp8_quant_act_1x128(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                 float* st, void* stream) {
  return quant_act_impl(x, M, K, q, s, qt, st, false, stream);
}

fp8rl_status fp8_quant_act_1x128_pow2(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                      float* st, void* stream) {
  return quant_act_impl(x, M, K, q, s, qt, st, true, stream);
}

fp8rl_status fp8_quant_w_128x128_f32(const float* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                     int pow2_scales, void* stream) {
  if (q == nullptr || s == nullptr) return FP8RL_ERR_NULL;
  if (fp8rl_status e = check_dims(N, K)) return e;
  if (N % 128 != 0 || K % 128 != 0) return FP8RL_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8RL_OK;
  if (w == nullptr) return FP8RL_ERR_NULL;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s, 4) || (qt && !aligned(qt, 16))) return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  return launched(launch_quant_w_f32(w, N, K, q, s, qt, pow2_scales != 0, as_stream(stream)));
}

fp8rl_status fp8_swiglu_bf16(const uint16_t* gu, int64_t M, int64_t F, uint16_t* h, void* stream) {
  if (fp8rl_status e = swiglu_check(gu, M, F)) return e;
  if (M == 0 || F == 0) return FP8RL_OK;
  if (h == nullptr) return FP8RL_ERR_NULL;
  if (!aligned(h, 16)) return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  return launched(launch_swiglu_bf16(gu, M, F, h, as_stream(stream)));
}

fp8rl_status fp8_swiglu_quant_1x128(const uint16_t* gu, int64_t M, int64_t F, uint8_t* q, float* s, uint8_t* qt,
                                    float* st, int pow2_scales, void* stream) {
  if (fp8rl_status e = swiglu_check(gu, M, F)) return e;
  if (M == 0 || F == 0) return FP8RL_OK;
  if (fp8rl_status e = check_act_outputs(M, q, s, qt, st)) return e;
  if (!act_outputs_aligned(q, s, qt, st)) return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  return launched(launch_swiglu_quant(gu, M, F, q, s, qt, st, pow2_scales != 0, as_stream(stream)));
}

fp8rl_status fp8_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps, uint16_t* y,
                              float* rstd, void* stream) {
  if (fp8rl_status e = rms_check(x, gamma, M, K, eps, rstd)) return e;
  if (M == 0 || K == 0) return FP8RL_OK;
  if (y == nullptr) return FP8RL_ERR_NULL;
  if (!aligned(y, 16)) return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  return launched(launch_rmsnorm_bf16(x, gamma, M, K, eps, y, rstd, as_stream(stream)));
}

fp8rl_status fp8_rmsnorm_quant_1x128(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                                     float* rstd, uint8_t* q, float* s, uint8_t* qt, float* st, int pow2_scales,
                                     void* stream) {
  if (fp8rl_status e = rms_check(x, gamma, M, K, eps, rstd)) return e;
  if (M == 0 || K == 0) return FP8RL_OK;
  if (fp8rl_status e = check_act_outputs(M, q, s, qt, st)) return e;
  if (!act_outputs_aligned(q, s, qt, st)) return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  return launched(launch_rmsnorm_quant(x, gamma, M, K, eps, rstd, q, s, qt, st, pow2_scales != 0,
                                       as_stream(stream)));
}

fp8rl_status fp8_quant_w_128x128(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                 void* stream) {
  return quant_w_impl(w, N, K, q, s, qt, false, stream);
}

fp8rl_status fp8_quant_w_128x128_pow2(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s, uint8_t* qt,
                                      void* stream) {
  return quant_w_impl(w, N, K, q, s, qt, true, stream);
}

fp8rl_status mxfp8_quant_1x32(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e8m0, void* stream) {
  if (q == nullptr || e8m0 == nullptr) return FP8RL_ERR_NULL;
  if (fp8rl_status e = check_dims(R, K)) return e;
  if (K % 32 != 0) return FP8RL_ERR_SHAPE;
  if (R == 0 || K == 0) return FP8RL_OK;
  if (x == nullptr) return FP8RL_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16)) return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  return launched(launch_quant_mx_1x32(x, R, K, q, e8m0, as_stream(stream)));
}

fp8rl_status mxfp8_quant_act_1x32(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e8m0, uint8_t* qt,
                                  uint8_t* e8m0t, void* stream) {
  if (fp8rl_status e = check_dims(R, K)) return e;
  if (K % 32 != 0) return FP8RL_ERR_SHAPE;
  if (R == 0 || K == 0) return FP8RL_OK;
  if ((q == nullptr) != (e8m0 == nullptr) || (qt == nullptr) != (e8m0t == nullptr)) return FP8RL_ERR_NULL;
  if (q == nullptr && qt == nullptr) return FP8RL_ERR_NULL;
  if (qt != nullptr && (R % 128 != 0 || K % 128 != 0)) return FP8RL_ERR_SHAPE;
  if (x == nullptr) return FP8RL_ERR_NULL;
  if (!aligned(x, 16) || (q && !aligned(q, 16)) || (qt && !aligned(qt, 16))) return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  if (qt == nullptr) return launched(launch_quant_mx_1x32(x, R, K, q, e8m0, as_stream(stream)));
  return launched(launch_quant_mx_tile(x, R, K, q, e8m0, qt, e8m0t, as_stream(stream)));
}

// Forward workspace: the quantized X (row-major for the tiled GEMM, K-block-major for the
// decode kernel), then its scales.
size_t fp8rl_fwd_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 128 != 0 || check_dims(M, K) != FP8RL_OK) return 0;
  const size_t qbytes = (size_t)(M * K);
  const size_t qpad = (qbytes + 255) & ~(size_t)255;
  return qpad + (size_t)M * (size_t)(K / 128) * sizeof(float);
}

}  // extern "C"

namespace {

// The forward product for both weight layouts. tiled_b: W in the decode layout (decode
// kernel for every M). Otherwise M <= 256 goes to the decode kernel and larger M to the tiled
// GEMM. A bf16 X is first quantized into the workspace: K-block-major for the decode kernel,
// row-major for the tiled GEMM.
// noalloc: the workspace is the library's scratch array (workspace arguments ignored).
fp8rl_status fwd_impl(const uint8_t* xq, const float* sx, const uint16_t* x_bf16, const uint8_t* wq, const float* sw,
                      int64_t M, int64_t N, int64_t K, void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                      bool tiled_b, void* stream, bool noalloc = false) {
  const bool quantized = xq != nullptr || sx != nullptr;
  if (quantized && (xq == nullptr || sx == nullptr)) return FP8RL_ERR_NULL;
  if (quantized == (x_bf16 != nullptr)) return FP8RL_ERR_NULL;  // exactly one form of X
  if (wq == nullptr || sw == nullptr || y == nullptr) return FP8RL_ERR_NULL;
  if (y_dtype != FP8RL_OUT_BF16 && y_dtype != FP8RL_OUT_F32) return FP8RL_ERR_RECIPE;
  if (fp8rl_status e = check_dims(M, K)) return e;
  if (fp8rl_status e = check_dims(N, K)) return e;
  if (fp8rl_status e = check_dims(M, N)) return e;
  if (K % 128 != 0 || N % 128 != 0) return FP8RL_ERR_SHAPE;
  if (fp8rl_status e = check_red(K)) return e;
  const bool decode = tiled_b || M <= 256;
  // The decode kernel addresses A and B with 32-bit offsets and counts rows in int32.
  if (decode && (M * K >= ((int64_t)1 << 32) || N * K >= ((int64_t)1 << 32))) return FP8RL_ERR_SHAPE;
  if (!quantized && M * K >= ((int64_t)1 << 32)) return FP8RL_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8RL_OK;
  if (K == 0) return FP8RL_ERR_SHAPE;  // the product would be all zeros; not a supported call
  if (!aligned(wq, 16) || !aligned(sw, 4) || !aligned(y, 16)) return FP8RL_ERR_ALIGN;
  if (quantized && (!aligned(xq, 16) || !aligned(sx, 4))) return FP8RL_ERR_ALIGN;
  if (!quantized) {
    if (!aligned(x_bf16, 16)) return FP8RL_ERR_ALIGN;
    if (noalloc) {
      if (fp8rl_fwd_workspace_bytes(M, K) > FP8RL_NOALLOC_SCRATCH_BYTES) return FP8RL_ERR_WORKSPACE;
    } else {
      if (workspace == nullptr || workspace_bytes < fp8rl_fwd_workspace_bytes(M, K)) return FP8RL_ERR_WORKSPACE;
      if (!aligned(workspace, 16)) return FP8RL_ERR_ALIGN;
    }
  }
  if (fp8rl_status e = check_device()) return e;
  if (!quantized && noalloc) {
    if (fp8rl_status e = scratch_address(&workspace)) return e;
  }
  hipStream_t st = as_stream(stream);
  uint8_t* wsq = nullptr;
  float* wss = nullptr;
  if (!quantized) {
    const size_t qpad = ((size_t)(M * K) + 255) & ~(size_t)255;
    wsq = static_cast<uint8_t*>(workspace);
    wss = reinterpret_cast<float*>(wsq + qpad);
  }
  if (decode) {
    DecodeParams d{};
    d.B = wq;
    d.sB = sw;
    d.C = y;
    d.M = M;
    d.N = N;
    d.K = K;
    d.sb_ld_n = K / 128;
    d.sb_ld_k = 1;
    d.ldc = N;
    d.tiled_b = tiled_b ? 1 : 0;
    if (quantized) {
      d.A = xq;
      d.sA = sx;
      d.a_ld = K;
      d.a_kb = 128;
      d.sa_ld = K / 128;
      d.sa_kb = 1;
    } else {
      if (launch_quant_kbmajor(x_bf16, M, K, wsq, wss, st) != hipSuccess) return FP8RL_ERR_LAUNCH;
      d.A = wsq;
      d.sA = wss;
      d.a_ld = 128;
      d.a_kb = 128 * M;
      d.sa_ld = 1;
      d.sa_kb = M;
    }
    return launched(launch_gemm_decode(d, y_dtype == FP8RL_OUT_F32, st));
  }
  if (!quantized) {
    if (launch_quant_rows_1x128(x_bf16, M, K, wsq, wss, false, st) != hipSuccess) return FP8RL_ERR_LAUNCH;
    xq = wsq;
    sx = wss;
  }
  GemmParams p{};
  p.A = xq;
  p.B = wq;
  p.sA = sx;
  p.sB = sw;
  p.C = y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.sa_ld = K / 128;
  p.sb_ld_n = K / 128;
  p.sb_ld_k = 1;
  p.ldc = N;
  p.accumulate = 0;
  return launched(launch_gemm_blockscaled(p, false, y_dtype == FP8RL_OUT_F32, false, st));
}

}  // namespace

extern "C" {

fp8rl_status fp8_gemm_blockscaled_fwd(const uint8_t* xq, const float* sx, const uint16_t* x_bf16, const uint8_t* wq,
                                      const float* sw, int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(xq, sx, x_bf16, wq, sw, M, N, K, y, y_dtype, workspace, workspace_bytes, false, stream);
}

fp8rl_status fp8_gemm_blockscaled_fwd_decode_layout(const uint8_t* xq, const float* sx, const uint16_t* x_bf16,
                                                    const uint8_t* wq, const float* sw, int64_t M, int64_t N,
                                                    int64_t K, void* y, int y_dtype, void* workspace,
                                                    size_t workspace_bytes, void* stream) {
  return fwd_impl(xq, sx, x_bf16, wq, sw, M, N, K, y, y_dtype, workspace, workspace_bytes, true, stream);
}

fp8rl_status fp8_gemm_blockscaled_fwd_decode_layout_noalloc(const uint8_t* xq, const float* sx, const uint16_t* x_bf16,
                                                            const uint8_t* wq, const float* sw, int64_t M, int64_t N,
                                                            int64_t K, void* y, int y_dtype, void* stream) {
  return fwd_impl(xq, sx, x_bf16, wq, sw, M, N, K, y, y_dtype, nullptr, 0, true, stream, true);
}

fp8rl_status fp8_gemm_blockscaled_pow2_fwd(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                           int64_t M, int64_t N, int64_t K, void* y, int y_dtype, void* stream) {
  if (xq == nullptr || sx == nullptr || wq == nullptr || sw == nullptr || y == nullptr) return FP8RL_ERR_NULL;
  if (y_dtype != FP8RL_OUT_BF16 && y_dtype != FP8RL_OUT_F32) return FP8RL_ERR_RECIPE;
  if (fp8rl_status e = check_dims(M, K)) return e;
  if (fp8rl_status e = check_dims(N, K)) return e;
  if (fp8rl_status e = check_dims(M, N)) return e;
  if (K % 128 != 0 || N % 128 != 0) return FP8RL_ERR_SHAPE;
  if (fp8rl_status e = check_red(K)) return e;
  if (M == 0 || N == 0) return FP8RL_OK;
  if (K == 0) return FP8RL_ERR_SHAPE;
  if (!aligned(xq, 16) || !aligned(sx, 4) || !aligned(wq, 16) || !aligned(sw, 4) || !aligned(y, 16))
    return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  GemmParams p{};
  p.A = xq;
  p.B = wq;
  p.sA = sx;
  p.sB = sw;
  p.C = y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.sa_ld = K / 128;
  p.sb_ld_n = K / 128;
  p.sb_ld_k = 1;
  p.ldc = N;
  p.accumulate = 0;
  return launched(launch_gemm_blockscaled(p, false, y_dtype == FP8RL_OUT_F32, true, as_stream(stream)));
}

}  // extern "C"

namespace {

// MXFP8 TN GEMM C[ra][rb] = sum_k deq(A)[ra][k] deq(B)[rb][k], E8M0 bytes [rows][kred/32].
fp8rl_status mx_gemm_impl(const uint8_t* a, const uint8_t* ea, const uint8_t* b, const uint8_t* eb, int64_t ra,
                          int64_t rb, int64_t kred, void* c, bool f32, int accumulate, void* stream) {
  if (a == nullptr || ea == nullptr || b == nullptr || eb == nullptr || c == nullptr) return FP8RL_ERR_NULL;
  if (fp8rl_status e = check_dims(ra, kred)) return e;
  if (fp8rl_status e = check_dims(rb, kred)) return e;
  if (fp8rl_status e = check_dims(ra, rb)) return e;
  if (kred % 128 != 0 || rb % 128 != 0) return FP8RL_ERR_SHAPE;
  if (fp8rl_status e = check_red(kred)) return e;
  if (ra == 0 || rb == 0) return FP8RL_OK;
  if (kred == 0) return FP8RL_ERR_SHAPE;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(ea, 4) || !aligned(eb, 4) || !aligned(c, 16))
    return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  GemmParams p{};
  p.A = a;
  p.B = b;
  p.sA = reinterpret_cast<const float*>(ea);     // read as dwords: 4 E8M0 bytes per 128 K
  p.sB = reinterpret_cast<const float*>(eb);
  p.C = c;
  p.M = ra;
  p.N = rb;
  p.K = kred;
  p.sa_ld = kred / 128;
  p.sb_ld_n = kred / 128;
  p.sb_ld_k = 1;
  p.ldc = rb;
  p.accumulate = accumulate;
  return launched(launch_gemm_mx(p, f32, as_stream(stream)));
}

fp8rl_status dgrad_impl(const uint8_t* dyq, const float* sdy, const uint8_t* wqt, const float* sw, int64_t M,
                        int64_t N, int64_t K, void* dx, int dx_dtype, bool pow2, void* stream) {
  if (dyq == nullptr || sdy == nullptr || wqt == nullptr || sw == nullptr || dx == nullptr) return FP8RL_ERR_NULL;
  if (dx_dtype != FP8RL_OUT_BF16 && dx_dtype != FP8RL_OUT_F32) return FP8RL_ERR_RECIPE;
  if (fp8rl_status e = check_dims(M, N)) return e;
  if (fp8rl_status e = check_dims(N, K)) return e;
  if (fp8rl_status e = check_dims(M, K)) return e;
  if (N % 128 != 0 || K % 128 != 0) return FP8RL_ERR_SHAPE;
  if (fp8rl_status e = check_red(N)) return e;
  if (M == 0 || K == 0) return FP8RL_OK;
  if (N == 0) return FP8RL_ERR_SHAPE;
  if (!aligned(dyq, 16) || !aligned(wqt, 16) || !aligned(dx, 16) || !aligned(sdy, 4) || !aligned(sw, 4))
    return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  GemmParams p{};
  p.A = dyq;                 // [M][N]: contraction over N
  p.B = wqt;                 // [K][N]
  p.sA = sdy;
  p.sB = sw;                 // sw[N/128][K/128]: output block j = k/128, contraction block c = n/128
  p.C = dx;
  p.M = M;
  p.N = K;
  p.K = N;
  p.sa_ld = N / 128;
  p.sb_ld_n = 1;
  p.sb_ld_k = K / 128;
  p.ldc = K;
  p.accumulate = 0;
  return launched(launch_gemm_blockscaled(p, false, dx_dtype == FP8RL_OUT_F32, pow2, as_stream(stream)));
}

fp8rl_status wgrad_impl(const uint8_t* dyqt, const float* sdyt, const uint8_t* xqt, const float* sxt, int64_t M,
                        int64_t N, int64_t K, float* dw, int accumulate, bool pow2, void* stream) {
  if (dyqt == nullptr || sdyt == nullptr || xqt == nullptr || sxt == nullptr || dw == nullptr) return FP8RL_ERR_NULL;
  if (fp8rl_status e = check_dims(M, N)) return e;
  if (fp8rl_status e = check_dims(M, K)) return e;
  if (fp8rl_status e = check_dims(N, K)) return e;
  if (M % 128 != 0 || N % 128 != 0 || K % 128 != 0) return FP8RL_ERR_SHAPE;
  if (fp8rl_status e = check_red(M)) return e;
  if (N == 0 || K == 0) return FP8RL_OK;
  if (M == 0) return FP8RL_ERR_SHAPE;
  if (!aligned(dyqt, 16) || !aligned(xqt, 16) || !aligned(dw, 16) || !aligned(sdyt, 4) || !aligned(sxt, 4))
    return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  GemmParams p{};
  p.A = dyqt;                // [N][M]: contraction over the M tokens
  p.B = xqt;                 // [K][M]
  p.sA = sdyt;
  p.sB = sxt;
  p.C = dw;
  p.M = N;
  p.N = K;
  p.K = M;
  p.sa_ld = M / 128;
  p.sb_ld_n = M / 128;
  p.sb_ld_k = 1;
  p.ldc = K;
  p.accumulate = accumulate ? 1 : 0;
  return launched(launch_gemm_blockscaled(p, true, true, pow2, as_stream(stream)));
}

}  // namespace

extern "C" {

fp8rl_status fp8_gemm_blockscaled_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wqt, const float* sw,
                                        int64_t M, int64_t N, int64_t K, void* dx, int dx_dtype, void* stream) {
  return dgrad_impl(dyq, sdy, wqt, sw, M, N, K, dx, dx_dtype, false, stream);
}

fp8rl_status fp8_gemm_blockscaled_pow2_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wqt,
                                             const float* sw, int64_t M, int64_t N, int64_t K, void* dx,
                                             int dx_dtype, void* stream) {
  return dgrad_impl(dyq, sdy, wqt, sw, M, N, K, dx, dx_dtype, true, stream);
}

fp8rl_status fp8_gemm_blockscaled_wgrad(const uint8_t* dyqt, const float* sdyt, const uint8_t* xqt, const float* sxt,
                                        int64_t M, int64_t N, int64_t K, float* dw, int accumulate, void* stream) {
  return wgrad_impl(dyqt, sdyt, xqt, sxt, M, N, K, dw, accumulate, false, stream);
}

fp8rl_status fp8_gemm_blockscaled_pow2_wgrad(const uint8_t* dyqt, const float* sdyt, const uint8_t* xqt,
                                             const float* sxt, int64_t M, int64_t N, int64_t K, float* dw,
                                             int accumulate, void* stream) {
  return wgrad_impl(dyqt, sdyt, xqt, sxt, M, N, K, dw, accumulate, true, stream);
}

fp8rl_status fp8_gemm_mxfp8_fwd(const uint8_t* xq, const uint8_t* ex, const uint8_t* wq, const uint8_t* ew, int64_t M,
                                int64_t N, int64_t K, void* y, int y_dtype, void* stream) {
  if (y_dtype != FP8RL_OUT_BF16 && y_dtype != FP8RL_OUT_F32) return FP8RL_ERR_RECIPE;
  return mx_gemm_impl(xq, ex, wq, ew, M, N, K, y, y_dtype == FP8RL_OUT_F32, 0, stream);
}

fp8rl_status fp8_gemm_mxfp8_dgrad(const uint8_t* dyq, const uint8_t* edy, const uint8_t* wqt, const uint8_t* ewt,
                                  int64_t M, int64_t N, int64_t K, void* dx, int dx_dtype, void* stream) {
  if (dx_dtype != FP8RL_OUT_BF16 && dx_dtype != FP8RL_OUT_F32) return FP8RL_ERR_RECIPE;
  return mx_gemm_impl(dyq, edy, wqt, ewt, M, K, N, dx, dx_dtype == FP8RL_OUT_F32, 0, stream);
}

fp8rl_status fp8_gemm_mxfp8_wgrad(const uint8_t* dyqt, const uint8_t* edyt, const uint8_t* xqt, const uint8_t* ext,
                                  int64_t M, int64_t N, int64_t K, float* dw, int accumulate, void* stream) {
  if (M % 128 != 0) return FP8RL_ERR_SHAPE;
  if (N > 0 && K > 0 && M == 0) return FP8RL_ERR_SHAPE;
  return mx_gemm_impl(dyqt, edyt, xqt, ext, N, K, M, dw, true, accumulate ? 1 : 0, stream);
}

fp8rl_status fp8_grouped_gemm(int recipe, const uint8_t* xq, const void* sx, const uint8_t* wq, const void* sw,
                              const int32_t* offsets, int64_t T, int64_t E, int64_t N, int64_t K, void* y,
                              int y_dtype, void* stream) {
  if (recipe != FP8RL_RECIPE_MXFP8 && recipe != FP8RL_RECIPE_BLOCK128) return FP8RL_ERR_RECIPE;
  if (y_dtype != FP8RL_OUT_BF16 && y_dtype != FP8RL_OUT_F32) return FP8RL_ERR_RECIPE;
  if (xq == nullptr || sx == nullptr || wq == nullptr || sw == nullptr || offsets == nullptr || y == nullptr)
    return FP8RL_ERR_NULL;
  if (E < 1) return FP8RL_ERR_SHAPE;
  if (fp8rl_status e = check_dims(T, K)) return e;
  if (fp8rl_status e = check_dims(E * N, K)) return e;
  if (fp8rl_status e = check_dims(T, N)) return e;
  if (K % 128 != 0 || N % 16 != 0 || E > ((int64_t)1 << 24)) return FP8RL_ERR_SHAPE;
  if (recipe == FP8RL_RECIPE_BLOCK128 && N % 128 != 0) return FP8RL_ERR_SHAPE;   // whole 128-row weight blocks
  if (fp8rl_status e = check_red(K)) return e;
  if (T == 0 || N == 0) return FP8RL_OK;
  if (K == 0) return FP8RL_ERR_SHAPE;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(y, 16) || !aligned(sx, 4) || !aligned(sw, 4) ||
      !aligned(offsets, 4))
    return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  GroupedParams p{};
  p.X = xq;
  p.Xs = static_cast<const uint8_t*>(sx);
  p.W = wq;
  p.Ws = static_cast<const uint8_t*>(sw);
  p.offsets = offsets;
  p.Y = y;
  p.T = T;
  p.E = E;
  p.N = N;
  p.K = K;
  const bool f32 = y_dtype == FP8RL_OUT_F32;
  return launched(recipe == FP8RL_RECIPE_MXFP8 ? launch_grouped_mx(p, f32, as_stream(stream))
                                               : launch_grouped_block(p, f32, as_stream(stream)));
}

fp8rl_status fp8_weight_install(const fp8rl_weight* src, const fp8rl_weight* dst, void* stream) {
  if (src == nullptr || dst == nullptr) return FP8RL_ERR_NULL;
  if (src->recipe != dst->recipe || src->rows != dst->rows || src->cols != dst->cols) return FP8RL_ERR_RECIPE;
  if ((src->layout != FP8RL_LAYOUT_ROWS && src->layout != FP8RL_LAYOUT_DECODE) ||
      (dst->layout != FP8RL_LAYOUT_ROWS && dst->layout != FP8RL_LAYOUT_DECODE))
    return FP8RL_ERR_RECIPE;
  // A decode-layout payload is never turned back into rows; MXFP8 has no decode layout.
  if (src->layout == FP8RL_LAYOUT_DECODE && dst->layout != FP8RL_LAYOUT_DECODE) return FP8RL_ERR_RECIPE;
  if (dst->layout == FP8RL_LAYOUT_DECODE && src->recipe != FP8RL_RECIPE_BLOCK128) return FP8RL_ERR_RECIPE;
  const int64_t rows = src->rows, cols = src->cols;
  if (fp8rl_status e = check_dims(rows, cols)) return e;
  int64_t sbytes;
  if (src->recipe == FP8RL_RECIPE_BLOCK128) {
    if (rows % 128 != 0 || cols % 128 != 0) return FP8RL_ERR_SHAPE;
    sbytes = (rows / 128) * (cols / 128) * 4;
  } else if (src->recipe == FP8RL_RECIPE_MXFP8) {
    if (cols % 32 != 0) return FP8RL_ERR_SHAPE;
    sbytes = rows * (cols / 32);
  } else {
    return FP8RL_ERR_RECIPE;
  }
  if (rows == 0 || cols == 0) return FP8RL_OK;
  if (src->q == nullptr || src->s == nullptr || dst->q == nullptr || dst->s == nullptr) return FP8RL_ERR_NULL;
  if (!aligned(src->q, 16) || !aligned(dst->q, 16) || !aligned(src->s, 4) || !aligned(dst->s, 4))
    return FP8RL_ERR_ALIGN;
  if (fp8rl_status e = check_device()) return e;
  hipStream_t st = as_stream(stream);
  if (src->layout == dst->layout)
    return launched(launch_copy(src->q, dst->q, rows * cols, static_cast<const uint8_t*>(src->s),
                                static_cast<uint8_t*>(dst->s), sbytes, st));
  // Rows -> decode layout: the payload is regrouped, the scales copied verbatim.
  if (launch_decode_layout(src->q, dst->q, rows, cols, st) != hipSuccess) return FP8RL_ERR_LAUNCH;
  return launched(launch_copy(nullptr, nullptr, 0, static_cast<const uint8_t*>(src->s),
                              static_cast<uint8_t*>(dst->s), sbytes, st));
}

}  // extern "C"
