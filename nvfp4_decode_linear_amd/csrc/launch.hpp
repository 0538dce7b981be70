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
// LDS bytes of a streaming-kernel workgroup: the activation (MFMA: codes and
// f16 scales; VALU: f16 x~) plus `batch` item slots of per-wave partial sums.
inline size_t stream_act_lds(int M, int kc, bool mfma) {
  return mfma ? (size_t)M * (kc * 32 + 32) + ((size_t)kc * 4 * M + 1) / 2 * 4
              : (size_t)M * kc * 128;
}
inline size_t stream_lds_need(int M, int kc, int waves, bool mfma, int batch, int rows = 32) {
  return stream_act_lds(M, kc, mfma) + (size_t)batch * waves * M * rows * 4;
}

struct GemvPlan {
  int kind;      // kGemvStream: persistent VALU over (tile, K slice) items
                 // kGemvMfma: the same with the dot on FP4 MFMA
                 // kGemvSplit: one workgroup per (tile, K slice), split-K tail
  int kc;        // K_pad / 64 chunks
  int tiles;     // N_pad / 32 row tiles
  int cpw;       // chunks per wavefront (per tile and slice; multiple of 4)
  int waves;     // wavefronts per workgroup
  int cps;       // chunks per K slice (= cpw * waves)
  int splits;    // K slices per row tile (1 = no split-K tail, no workspace)
  int batch;     // streaming kernels: items whose partial sums share one barrier
  int h16;       // MFMA streaming kernel on 16-row half tiles (16x16x128 MFMA)
  int depth;     // weight records in flight per wavefront (stream kernel)
  int grid;      // workgroups launched
  int nontemporal;
  size_t ws_partials;  // bytes of split-K partials (after the counter region)
  size_t ws_bytes;     // total workspace bytes (0 without split-K)
};

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Activation quantizer launch: `groups` workgroups of 256 threads, each
// thread owning `bpt` (1, 2 or 4) blocks of 16.  Largest tensor: 256 * 256 *
// 4 blocks (kActMaxBlocks).
struct ActPlan {
  int groups;
  int bpt;
};
constexpr int64_t kActMaxBlocks = 256 * 256 * 4;
constexpr size_t kActSyncBytes = 16;
ActPlan act_plan(int M, int64_t K);

// sg_static: quantize with this device tensor scale instead of the tensor's
// own (gscale is then not written and sync not used).
hipError_t launch_quantize_act(const uint16_t* x, int M, int K, int64_t ldx, uint8_t* codes,
                               uint8_t* scales, float* gscale, uint32_t* sync, uint32_t spin_limit,
                               hipStream_t s, const float* sg_static = nullptr);

// The activation quantizer on a binary32 activation; amax_in: the record
// of per-workgroup maxima its producer wrote (kAmaxSlots), or null.
hipError_t launch_quantize_act_f32(const float* x, int M, int K, int64_t ldx,
                                   const uint32_t* amax_in, uint8_t* codes, uint8_t* scales,
                                   float* gscale, uint32_t* sync, uint32_t spin_limit,
                                   hipStream_t s);

// Fused stack quantizers (mode 0: RMS norm, 1: SiLU * mul), one workgroup
// per row of up to 2 * 1024 blocks, K <= kPrepMaxK.
constexpr int64_t kPrepMaxK = 32768;
hipError_t launch_prep_quantize(int mode, const uint16_t* x, int M, int K, int64_t ldx, float eps,
                                uint8_t* codes, uint8_t* scales, float* gscale, float* h_out,
                                uint32_t* sync, uint32_t spin_limit, hipStream_t s);

// gate_up_f > 0: the weight is a gate_up projection [2F][K] (F = gate_up_f)
// and the tiled rows interleave gate and up in groups of 16: tiled row 32t +
// r is source row 16t + r (r < 16) or F + 16t + r - 16 (r >= 16).
hipError_t launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* codes, uint8_t* scales, float* gscale, hipStream_t s,
                                  int64_t gate_up_f = 0);

hipError_t launch_unpack_weight(const uint8_t* codes, const uint8_t* scales, int64_t N,
                                int64_t K, uint8_t* codes_rm, uint8_t* scales_rm, hipStream_t s);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

// Exhaustive check of the instruction E2M1 encoder (out: 2 x u64).
hipError_t launch_e2m1_selftest(unsigned long long* out, hipStream_t s);

hipError_t launch_gemv_split(const GemvPlan& p, int M, int64_t N, int64_t K,
                             const uint8_t* xc, const uint8_t* xs, const float* xg,
                             const uint8_t* wc, const uint8_t* ws, const float* wg, void* y,
                             int out_bf16, void* workspace, hipStream_t s);

hipError_t launch_gemv_stream(const GemvPlan& p, int M, int64_t N, int64_t K,
                              const uint8_t* xc, const uint8_t* xs, const float* xg,
                              const uint8_t* wc, const uint8_t* ws, const float* wg, void* y,
                              int out_bf16, void* workspace, hipStream_t s,
                              const uint16_t* xb = nullptr, int64_t ldx = 0,
                              uint8_t* oc = nullptr, uint8_t* os = nullptr,
                              float* og = nullptr, int rms = 0, float eps = 0.0f,
                              float* ho = nullptr, const float* sgs = nullptr,
                              const float* xf = nullptr, const uint32_t* amax_in = nullptr,
                              int qslice = 0, uint32_t* amax_out = nullptr, int64_t ldh = 0,
                              uint16_t* gu = nullptr);

// ReSET temperature (reset.hip): per-row arrival counters (at most
// kResetMaxRows rows) at the start of the workspace, then the partial
// (max, sum, weighted sum) of every workgroup: [rows][groups][4] floats.
constexpr int kResetMaxRows = 256;
constexpr int64_t kResetMaxV = int64_t(1) << 20;   // 256 groups of 4096 logits per row
constexpr size_t kResetCounterBytes = (size_t)kResetMaxRows * 4;
int reset_groups_per_row(int64_t V);
hipError_t launch_reset_temperature(const float* z, int M, int64_t V, int64_t ldz, float t_low,
                                    float tau0, float t_base, float t_max, float* state,
                                    const int32_t* step_end, float* h_out, float* t_out,
                                    float* z_out, int64_t ldo, void* workspace, hipStream_t s);

// Per-workgroup maxima record of a binary32 activation (the SiLU * mul
// output of the gate_up GEMV): one |h| bit pattern per workgroup slot, zero
// past the grid; the tensor maximum is the largest entry.
constexpr int kAmaxSlots = 256;

// Largest M * K / 16 the MFMA streaming kernel quantizes in its prologue
// (4 bf16 blocks per thread, 8 with four or more rows; `four`: 4 per thread
// at any M, as binary32 blocks, which take twice the registers, need).
inline int64_t qa_max_blocks(int M, int waves, bool four = false) {
  return (int64_t)(M >= 4 && !four ? 8 : 4) * 64 * waves;
}

}  // namespace nvfp4
