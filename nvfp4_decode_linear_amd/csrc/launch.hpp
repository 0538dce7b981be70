// Host-side launchers of the NVFP4 kernels.  Called by the C ABI layer
// (abi.cpp) after it has validated every argument; each returns the
// hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// Split-K arrival counters: one per row tile, in a fixed region at the start
// of every workspace.  Shapes with more row tiles never split K.
constexpr int kMaxCounterTiles = 16384;
constexpr size_t kCounterBytes = (size_t)kMaxCounterTiles * 4;

enum GemvKind { kGemvStream = 0, kGemvSplit = 1, kGemvMfma = 2 };

// Dynamic LDS bytes of a streaming workgroup (VALU or MFMA variant) with
// `waves` wavefronts, before the reservation that keeps one workgroup per CU.
inline size_t stream_lds_need(int M, int kc, int waves, bool mfma) {
  const size_t act = mfma ? (size_t)M * kc * 32 + (size_t)kc * 4 * M * 4   // codes + scales
                          : (size_t)M * kc * 128;                          // f16 x~
  return act + (size_t)2 * waves * M * 32 * 4;
}

struct GemvPlan {
  int kind;      // kGemvStream: persistent VALU, whole K per workgroup, no workspace
                 // kGemvMfma: the same with the dot on FP4 MFMA
                 // kGemvSplit: one workgroup per (tile, K slice), split-K tail
  int kc;        // K_pad / 64 chunks
  int tiles;     // N_pad / 32 row tiles
  int cpw;       // chunks per wavefront (per tile and slice; multiple of 4)
  int waves;     // wavefronts per workgroup
  int cps;       // chunks per K slice (= cpw * waves; split kernel)
  int splits;    // K slices (split kernel; 1 for the stream kernel)
  int depth;     // weight records in flight per wavefront (stream kernel)
  int grid;      // workgroups launched
  int nontemporal;
  size_t ws_partials;  // bytes of split-K partials (after the counter region)
  size_t ws_bytes;     // total workspace bytes (0 without split-K)
};

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

hipError_t launch_quantize_act(const uint16_t* x, int M, int K, int64_t ldx, uint8_t* codes,
                               uint8_t* scales, float* gscale, hipStream_t s);

hipError_t launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* codes, uint8_t* scales, float* gscale, hipStream_t s);

hipError_t launch_unpack_weight(const uint8_t* codes, const uint8_t* scales, int64_t N,
                                int64_t K, uint8_t* codes_rm, uint8_t* scales_rm, hipStream_t s);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

hipError_t launch_gemv_split(const GemvPlan& p, int M, int64_t N, int64_t K,
                             const uint8_t* xc, const uint8_t* xs, const float* xg,
                             const uint8_t* wc, const uint8_t* ws, const float* wg, void* y,
                             int out_bf16, void* workspace, hipStream_t s);

hipError_t launch_gemv_stream(const GemvPlan& p, int M, int64_t N, int64_t K,
                              const uint8_t* xc, const uint8_t* xs, const float* xg,
                              const uint8_t* wc, const uint8_t* ws, const float* wg, void* y,
                              int out_bf16, hipStream_t s);

}  // namespace nvfp4
