// nvfp4_quantize_linear_noalloc: nvfp4_quantize_linear for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  The workspace the call needs (the
// activation quantizer's sync record, the split-K arrival counters and the
// split-K partial sums) lives in a library-owned device array instead of a
// caller-supplied buffer; the call allocates nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/nvfp4.h"
#include "launch.hpp"

namespace nvfp4 {
nvfp4_status record_hip_error(hipError_t e);   // abi.cpp: keeps nvfp4_last_hip_error
}

// The scratch workspace, one copy per device, held until the process ends.
// Host code never passes this name to a kernel: its host-side symbol is only
// a stand-in, so the device address is taken once per device with
// hipGetSymbolAddress and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::atomic<int> g_ready[kMaxDevices];
std::mutex g_init_mu;

// The current device's scratch address.  The first call on a device (with
// that device current) takes the array's device address and zeroes the array
// with a fill kernel on `stream`, ordered before the call's own kernels; the
// counters and the sync record inside it return to zero at the end of every
// call, so later calls need no clearing.
nvfp4_status scratch_for_current_device(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return nvfp4::record_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
  if (g_ready[dev].load(std::memory_order_acquire)) {
    *out = g_scratch[dev];
    return NVFP4_OK;
  }
  std::lock_guard<std::mutex> lock(g_init_mu);
  if (!g_ready[dev].load(std::memory_order_relaxed)) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return nvfp4::record_hip_error(e);
    if (!p) return NVFP4_ERR_HIP;
    const nvfp4_status st = nvfp4_workspace_init(p, NVFP4_NOALLOC_SCRATCH_BYTES, stream);
    if (st != NVFP4_OK) return st;
    g_scratch[dev] = p;
    g_ready[dev].store(1, std::memory_order_release);
  }
  *out = g_scratch[dev];
  return NVFP4_OK;
}

}  // namespace

extern "C" nvfp4_status nvfp4_quantize_linear_noalloc(
    int M, int64_t N, int64_t K, const uint16_t* x_bf16, int64_t ldx, const uint8_t* w_codes,
    const uint8_t* w_scales, const float* w_gscale, void* y, int out_dtype, uint8_t* x_codes,
    uint8_t* x_scales, float* x_gscale, void* stream) {
  const size_t need = nvfp4_quantize_linear_workspace_bytes(M, N, K);
  const bool args_ok = x_bf16 && w_codes && w_scales && w_gscale && y && x_codes && x_scales &&
                       x_gscale && ldx >= K && ldx % 8 == 0 &&
                       (out_dtype == NVFP4_OUT_F32 || out_dtype == NVFP4_OUT_BF16);
  if (need == 0 || !args_ok) {
    // arguments nvfp4_quantize_linear rejects: its own checks return the
    // error before any HIP call
    return nvfp4_quantize_linear(M, N, K, x_bf16, ldx, w_codes, w_scales, w_gscale, y, out_dtype,
                                 x_codes, x_scales, x_gscale, nullptr, 0, stream);
  }
  if (need > NVFP4_NOALLOC_SCRATCH_BYTES) return NVFP4_ERR_WORKSPACE;
  void* ws = nullptr;
  const nvfp4_status st = scratch_for_current_device(stream, &ws);
  if (st != NVFP4_OK) return st;
  return nvfp4_quantize_linear(M, N, K, x_bf16, ldx, w_codes, w_scales, w_gscale, y, out_dtype,
                               x_codes, x_scales, x_gscale, ws, NVFP4_NOALLOC_SCRATCH_BYTES, stream);
}
