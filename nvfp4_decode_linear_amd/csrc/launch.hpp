// Host-side launchers of the NVFP4 kernels.  Called by the C ABI layer
// (abi.cpp) after it has validated every argument; each returns the
// hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

struct GemvPlan {
  int kc;        // K_pad / 64 chunks
  int tiles;     // N_pad / 32 row tiles
  int cpw;       // chunks per wavefront (multiple of 4)
  int waves;     // wavefronts per workgroup
  int cps;       // chunks per K slice (= cpw * waves)
  int splits;    // K slices
  int nontemporal;
  size_t ws_partials;  // bytes of split-K partials in the workspace
  size_t ws_bytes;     // total workspace bytes
};

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

hipError_t launch_quantize_act(const uint16_t* x, int M, int K, int64_t ldx, uint8_t* codes,
                               uint8_t* scales, float* gscale, hipStream_t s);

hipError_t launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* codes, uint8_t* scales, float* gscale, hipStream_t s);

hipError_t launch_unpack_weight(const uint8_t* codes, const uint8_t* scales, int64_t N,
                                int64_t K, uint8_t* codes_rm, uint8_t* scales_rm, hipStream_t s);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

hipError_t launch_gemv_valu(const GemvPlan& p, int M, int64_t N, int64_t K,
                            const uint8_t* xc, const uint8_t* xs, const float* xg,
                            const uint8_t* wc, const uint8_t* ws, const float* wg, void* y,
                            int out_bf16, void* workspace, hipStream_t s);

}  // namespace nvfp4
