// Layer-stack driver: one decode step of an L-layer stack of NVFP4 linears
// captured once into a HIP graph and replayed (the "ReSET" GitHub README's
// end-to-end figure, in the caption under its introduction, is a 1,500-token
// decode of Qwen3-32B at batch 1 with the decode step replayed as a graph).  Per layer, in stream order:
//
//   x -> RMS norm + quantize -> QKV -> quantize (first q_cols columns)
//     -> O -> RMS norm + quantize -> gate_up -> SiLU * mul + quantize
//     -> down -> x of the next layer
//
// With interleaved gate_up weights the SiLU * mul runs in the gate_up GEMV's
// epilogue (binary32 h and its maxima record) and its quantizer in the down
// GEMV's prologue; otherwise gate_up writes bf16 and the SiLU quantizer runs
// on its own.
// Every linear writes bf16.  There is no attention, residual or weighted
// norm: the stack exercises the linears and the quantizers between them at
// the model's shapes, the rest of a layer is out of scope.  The graph holds
// kernel nodes only (the workspace is zeroed once, before capture, by a fill
// kernel; the split-K counters and the quantizer's sync record reset
// themselves), so replays need no host work.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/nvfp4.h"

namespace nvfp4 {
nvfp4_status record_hip_error(hipError_t e);   // abi.cpp: keeps nvfp4_last_hip_error
bool silu_plan_ok(int M, int64_t F, int64_t K);  // abi.cpp: the fused gate_up has a plan
}

struct nvfp4_stack {
  nvfp4_stack_config cfg;
  std::vector<nvfp4_weight> w;          // [layers][4]
  int device = -1;
  const uint16_t* x_in = nullptr;       // [M][hidden] (the caller's)
  uint16_t* y_out = nullptr;            // [M][hidden] (the caller's)
  // device buffers (owned)
  uint16_t* h = nullptr;                // [M][hidden] inter-layer activation
  uint16_t* qkv = nullptr;              // [M][qkv_n]
  uint16_t* o = nullptr;                // [M][hidden]
  uint16_t* gu = nullptr;               // [M][2 ffn] (unfused SiLU * mul only)
  float* hf = nullptr;                  // [M][ffn] binary32 SiLU * mul output (fused)
  uint32_t* hamax = nullptr;            // its maxima record (fused)
  bool silu_fused = false;
  uint8_t* a_codes = nullptr;           // [M][kmax / 2]
  uint8_t* a_scales = nullptr;          // [M][kmax / 16]
  float* a_gscale = nullptr;            // 1 float (padded to 256 B)
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace {

enum { kQkv = 0, kO = 1, kGateUp = 2, kDown = 3 };

nvfp4_status hip_err(hipError_t e) { return nvfp4::record_hip_error(e); }

void free_all(nvfp4_stack* s) {
  if (s->exec) (void)hipGraphExecDestroy(s->exec);
  if (s->graph) (void)hipGraphDestroy(s->graph);
  void* bufs[] = {s->h,       s->qkv,      s->o,        s->gu, s->hf,
                  s->hamax,   s->a_codes,  s->a_scales, s->a_gscale, s->ws};
  for (void* p : bufs)
    if (p) (void)hipFree(p);
}

// One decode step, enqueued on `st` (eagerly or under capture).
nvfp4_status enqueue_step(nvfp4_stack* s, void* st) {
  const nvfp4_stack_config& c = s->cfg;
  const int M = c.M;
  nvfp4_status r = NVFP4_OK;
  auto lin = [&](const nvfp4_weight& w, int64_t N, int64_t K, void* y) {
    return nvfp4_linear(M, N, K, s->a_codes, s->a_scales, s->a_gscale, w.codes, w.scales,
                        w.gscale, y, NVFP4_OUT_BF16, s->ws, s->ws_bytes, st);
  };
  for (int l = 0; l < c.layers && r == NVFP4_OK; ++l) {
    const nvfp4_weight* w = &s->w[(size_t)l * 4];
    const uint16_t* xin = l == 0 ? s->x_in : s->h;
    uint16_t* xout = l == c.layers - 1 ? s->y_out : s->h;
    // RMS norm + quantize + QKV (one kernel when it fits)
    if ((r = nvfp4_rmsnorm_quantize_linear(M, c.qkv_n, c.hidden, xin, c.hidden, c.eps,
                                           w[kQkv].codes, w[kQkv].scales, w[kQkv].gscale, s->qkv,
                                           NVFP4_OUT_BF16, s->a_codes, s->a_scales, s->a_gscale,
                                           nullptr, s->ws, s->ws_bytes, st)) != NVFP4_OK)
      break;
    // quantize the q columns and apply O (one kernel when it fits)
    if ((r = nvfp4_quantize_linear(M, c.hidden, c.q_cols, s->qkv, c.qkv_n, w[kO].codes,
                                   w[kO].scales, w[kO].gscale, s->o, NVFP4_OUT_BF16, s->a_codes,
                                   s->a_scales, s->a_gscale, s->ws, s->ws_bytes, st)) != NVFP4_OK)
      break;
    if (s->silu_fused) {
      // RMS norm + quantize + gate_up + SiLU * mul, then quantize + down
      if ((r = nvfp4_quantize_linear_silu_mul(
               M, c.ffn, c.hidden, s->o, c.hidden, 1, c.eps, w[kGateUp].codes, w[kGateUp].scales,
               w[kGateUp].gscale, s->hf, c.ffn, s->hamax, nullptr, s->a_codes, s->a_scales,
               s->a_gscale, nullptr, s->ws, s->ws_bytes, st)) != NVFP4_OK)
        break;
      r = nvfp4_quantize_linear_f32(M, c.hidden, c.ffn, s->hf, c.ffn, s->hamax, w[kDown].codes,
                                    w[kDown].scales, w[kDown].gscale, xout, NVFP4_OUT_BF16,
                                    s->a_codes, s->a_scales, s->a_gscale, s->ws, s->ws_bytes, st);
      continue;
    }
    // RMS norm + quantize + gate_up (one kernel when it fits)
    if ((r = nvfp4_rmsnorm_quantize_linear(M, 2 * c.ffn, c.hidden, s->o, c.hidden, c.eps,
                                           w[kGateUp].codes, w[kGateUp].scales,
                                           w[kGateUp].gscale, s->gu, NVFP4_OUT_BF16, s->a_codes,
                                           s->a_scales, s->a_gscale, nullptr, s->ws, s->ws_bytes,
                                           st)) != NVFP4_OK)
      break;
    if ((r = nvfp4_silu_mul_quantize_act(s->gu, M, c.ffn, 2 * c.ffn, s->a_codes, s->a_scales,
                                         s->a_gscale, nullptr, s->ws, s->ws_bytes, st)) !=
        NVFP4_OK)
      break;
    r = lin(w[kDown], c.hidden, c.ffn, xout);
  }
  return r;
}

bool valid_config(const nvfp4_stack_config& c) {
  auto ok_dim = [](int64_t v) { return v >= 16 && v % 16 == 0 && v <= 32768; };
  return c.M >= 1 && c.M <= 8 && c.layers >= 1 && c.layers <= 4096 && ok_dim(c.hidden) &&
         ok_dim(c.q_cols) && ok_dim(c.ffn) && c.qkv_n >= c.q_cols && c.qkv_n % 8 == 0 &&
         c.qkv_n <= (int64_t(1) << 20) && c.eps >= 0.0f && c.eps < 1.0f &&
         (c.gate_up_interleaved == 0 || c.gate_up_interleaved == 1);
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_stack_create(const nvfp4_stack_config* cfg, const nvfp4_weight* weights,
                                const uint16_t* x_in, uint16_t* y_out, void* stream,
                                nvfp4_stack** out) {
  if (!out) return NVFP4_ERR_INVALID_ARG;
  *out = nullptr;
  if (!cfg || !weights || !x_in || !y_out || !stream) return NVFP4_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(x_in) % 16 || reinterpret_cast<uintptr_t>(y_out) % 4)
    return NVFP4_ERR_INVALID_ARG;
  if (cfg->M > 8) return NVFP4_ERR_UNSUPPORTED;
  if (!valid_config(*cfg)) return NVFP4_ERR_INVALID_ARG;
  if (cfg->gate_up_interleaved && !nvfp4::silu_plan_ok(cfg->M, cfg->ffn, cfg->hidden))
    return NVFP4_ERR_UNSUPPORTED;
  for (int i = 0; i < cfg->layers * 4; ++i)
    if (!weights[i].codes || !weights[i].scales || !weights[i].gscale) return NVFP4_ERR_INVALID_ARG;
  nvfp4_stack* s = new (std::nothrow) nvfp4_stack;
  if (!s) return NVFP4_ERR_HIP;
  s->cfg = *cfg;
  s->w.assign(weights, weights + (size_t)cfg->layers * 4);
  s->x_in = x_in;
  s->y_out = y_out;
  const nvfp4_stack_config& c = s->cfg;
  const int M = c.M;
  hipStream_t st = static_cast<hipStream_t>(stream);
  nvfp4_status r = NVFP4_OK;
  hipError_t e = hipGetDevice(&s->device);
  const int64_t kmax = std::max({c.hidden, c.q_cols, c.ffn});
  size_t ws = 256;
  ws = std::max(ws, nvfp4_quantize_linear_workspace_bytes(M, c.qkv_n, c.hidden));
  ws = std::max(ws, nvfp4_quantize_linear_workspace_bytes(M, c.hidden, c.q_cols));
  ws = std::max(ws, nvfp4_quantize_linear_workspace_bytes(M, 2 * c.ffn, c.hidden));
  ws = std::max(ws, nvfp4_linear_workspace_bytes(M, c.hidden, c.ffn));
  ws = std::max(ws, nvfp4_quantize_linear_f32_workspace_bytes(M, c.hidden, c.ffn));
  s->ws_bytes = ws;
  s->silu_fused = c.gate_up_interleaved != 0;
  auto alloc = [&](auto** p, size_t bytes) {
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(p), std::max<size_t>(bytes, 256));
  };
  alloc(&s->h, (size_t)M * c.hidden * 2);
  alloc(&s->qkv, (size_t)M * c.qkv_n * 2);
  alloc(&s->o, (size_t)M * c.hidden * 2);
  if (s->silu_fused) {
    alloc(&s->hf, (size_t)M * c.ffn * 4);
    alloc(&s->hamax, NVFP4_AMAX_RECORD_WORDS * 4);
  } else {
    alloc(&s->gu, (size_t)M * 2 * c.ffn * 2);
  }
  alloc(&s->a_codes, (size_t)M * kmax / 2);
  alloc(&s->a_scales, (size_t)M * kmax / 16);
  alloc(&s->a_gscale, 256);
  alloc(&s->ws, ws);
  if (e != hipSuccess) {
    r = hip_err(e);
  } else if ((r = nvfp4_workspace_init(s->ws, ws, st)) == NVFP4_OK) {
    // one eager step (validates every call and initialises the kernels'
    // attributes), then the capture
    r = enqueue_step(s, st);
    if (r == NVFP4_OK && (e = hipStreamSynchronize(st)) != hipSuccess) r = hip_err(e);
    if (r == NVFP4_OK) {
      if ((e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal)) != hipSuccess) {
        r = hip_err(e);
      } else {
        const nvfp4_status rc = enqueue_step(s, st);
        e = hipStreamEndCapture(st, &s->graph);
        if (rc != NVFP4_OK) r = rc;
        else if (e != hipSuccess) r = hip_err(e);
        else if ((e = hipGraphInstantiate(&s->exec, s->graph, nullptr, nullptr, 0)) != hipSuccess)
          r = hip_err(e);
      }
    }
  }
  if (r != NVFP4_OK) {
    free_all(s);
    delete s;
    return r;
  }
  *out = s;
  return NVFP4_OK;
}

nvfp4_status nvfp4_stack_run(nvfp4_stack* s, int steps, void* stream) {
  if (!s || steps < 0) return NVFP4_ERR_INVALID_ARG;
  for (int i = 0; i < steps; ++i) {
    const hipError_t e = hipGraphLaunch(s->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_err(e);
  }
  return NVFP4_OK;
}

nvfp4_status nvfp4_stack_run_eager(nvfp4_stack* s, void* stream) {
  if (!s) return NVFP4_ERR_INVALID_ARG;
  return enqueue_step(s, stream);
}

nvfp4_status nvfp4_stack_destroy(nvfp4_stack* s) {
  if (!s) return NVFP4_ERR_INVALID_ARG;
  free_all(s);
  delete s;
  return NVFP4_OK;
}

}  // extern "C"
