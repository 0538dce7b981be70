// C ABI of the NVFP4 decode-linear library (include/nvfp4.h): argument
// validation on the host before any HIP call, runtime knobs, launch plans,
// and dispatch to the gfx950 kernels.  The runtime knobs play the part of the
// kernel package's configure / status calls in the Python wiring example of
// the "ReSET" GitHub README, section "Run benchmarks" (a threshold on M below
// which the CUDA-core GEMV runs, and a way to read the settings back).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/nvfp4.h"
#include "launch.hpp"
#include "nvfp4_device.hpp"

using nvfp4::GemvPlan;
using nvfp4::round_up;

namespace {

constexpr int kAbiVersion = 1;
constexpr int kLayoutVersion = 1;
constexpr int kMaxM = 8;
constexpr int kMaxDevices = 64;

std::atomic<int64_t> g_opts[NVFP4_OPT_COUNT] = {{0}, {0}, {0}, {1}, {0},
                                                {0}, {0}, {0}, {1}, {0}, {0}};
thread_local int t_last_hip = 0;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

nvfp4_status hip_fail(hipError_t e) {
  t_last_hip = (int)e;
  return NVFP4_ERR_HIP;
}

}  // namespace

namespace nvfp4 {
// for the other host translation units of the library (stack.cpp)
nvfp4_status record_hip_error(hipError_t e) { return hip_fail(e); }
}  // namespace nvfp4
static_assert(NVFP4_AMAX_RECORD_WORDS == nvfp4::kAmaxSlots, "maxima record size");

namespace {

// Current device must be a gfx950; cached per device.
nvfp4_status check_device() {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n == 0) return NVFP4_ERR_NO_DEVICE;
    return hip_fail(e);
  }
  if (dev >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    const hipError_t pe = hipGetDeviceProperties(&prop, dev);
    if (pe != hipSuccess) return hip_fail(pe);
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? NVFP4_OK : NVFP4_ERR_UNSUPPORTED;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_nk(int64_t N, int64_t K) {
  return N >= 1 && K >= 16 && K % 16 == 0 && N <= (int64_t(1) << 30) && K <= (int64_t(1) << 30) &&
         round_up(N, nvfp4::kTileN) * round_up(K, nvfp4::kGroupK) / 2 <= (int64_t(1) << 40);
}

// LDS bytes of one split-kernel workgroup: the decoded activation slice (M
// rows x cps chunks x 64 f16) plus the cross-wave reduction buffer.
int64_t split_lds_bytes(int M, int cpw, int waves) {
  return (int64_t)M * cpw * waves * 128 + (int64_t)waves * M * 128 + 64;
}

bool split_ok(int M, int cpw, int waves) {
  if (waves == 16 && cpw > 8) return false;      // 1024 threads: <= 128 VGPRs per lane
  return split_lds_bytes(M, cpw, waves) <= 65536;
}

constexpr int64_t kLdsBudget = 160 * 1024;
constexpr int64_t kFuseMaxBlocks = 4096;

void finish_workspace(GemvPlan& p, int M) {
  // The arrival counters live in a fixed region at the start of the
  // workspace, so one zero-initialised workspace stays valid across calls of
  // any shape (a counter never lands where another shape left partial sums).
  const int64_t n_pad = (int64_t)p.tiles * nvfp4::kTileN;
  p.ws_partials = p.splits > 1 ? (size_t)round_up((int64_t)p.splits * M * n_pad * 4, 256) : 0;
  p.ws_bytes = p.splits > 1 ? nvfp4::kCounterBytes + p.ws_partials : 0;
}

constexpr int kStreamGrid = 256;   // one streaming workgroup per CU

// K slices per row tile for the streaming kernels: with fewer than 64 row
// tiles, enough (tile, slice) items to occupy more of the 256 workgroups,
// without slices shorter than 8 chunks (512 elements).
int stream_splits(int tiles, int kc) {
  auto eff = [&](int s) {
    const int64_t items = (int64_t)tiles * s;
    const int64_t rounds = (items + kStreamGrid - 1) / kStreamGrid;
    return (double)items / (double)(rounds * kStreamGrid);
  };
  // The split-K tail costs several dependent device-memory round trips, more
  // than the idle CUs cost unless very few row tiles exist.
  if (tiles >= 64 || eff(1) >= 0.85) return 1;
  int best = 1;
  for (int s = 2; s <= 8; ++s) {
    if ((kc + s - 1) / s < 8) break;
    if (eff(s) > eff(best) + 0.02) best = s;
  }
  return best;
}

// Launch plan of the GEMV for (M, N, K) under the current knobs.
//   silu: the gate_up projection with the SiLU * mul epilogue (MFMA, whole
//         row tiles, one K slice)
//   slices: that many K slices (MFMA, whole tiles) on a grid that is a
//         multiple of them, so that every workgroup stays in one slice
// Either returns a plan of kind kGemvSplit when the streaming kernel cannot
// take the shape.
GemvPlan make_plan(int M, int64_t N, int64_t K, bool silu = false, int slices = 0) {
  GemvPlan p = {};
  p.kc = (int)(round_up(K, nvfp4::kGroupK) / nvfp4::kChunkK);
  p.tiles = (int)(round_up(N, nvfp4::kTileN) / nvfp4::kTileN);
  p.nontemporal = g_opts[NVFP4_OPT_NONTEMPORAL].load() ? 1 : 0;
  const int64_t force_kernel = g_opts[NVFP4_OPT_KERNEL].load();
  const int64_t force_cpw = g_opts[NVFP4_OPT_CHUNKS_PER_WAVE].load();
  const int64_t force_split = g_opts[NVFP4_OPT_SPLIT_K].load();
  const int64_t force_waves = g_opts[NVFP4_OPT_WAVES].load();

  // Streaming kernels: one workgroup per CU walks (row tile, K slice) items;
  // they need the whole activation in LDS.  M <= GEMV_MAX_M runs the VALU
  // dot (M <= 3 only), larger M the MFMA dot.
  const int64_t gemv_max_m = g_opts[NVFP4_OPT_GEMV_MAX_M].load();
  const bool auto_kind = force_kernel == 0 && force_cpw == 0;
  const bool special = silu || slices > 0;
  const bool want_mfma =
      special || force_kernel == 3 || (auto_kind && (M > gemv_max_m || M > 3));
  const bool want_valu = !want_mfma && (force_kernel == 1 || auto_kind) && M <= 3;
  if (want_mfma || want_valu) {
    const int max_waves = 8;                               // as compiled
    int want = force_waves > 0 ? std::min<int>((int)force_waves, max_waves)
                               : std::min(max_waves, 8);
    // 16-row half tiles (MFMA only, one K slice): twice the work items, for
    // shapes whose 32-row tiles leave CUs idle.
    const int64_t force_half = g_opts[NVFP4_OPT_HALF_TILES].load();
    const bool h16 = !special && want_mfma && force_split <= 1 &&
                     (force_half == 2 || (force_half == 0 && 2 * p.tiles <= kStreamGrid));
    const int gc = h16 ? 8 : 4;                              // chunks per ring group
    const int s0 = h16 || silu      ? 1
                   : slices > 0     ? slices
                   : force_split > 0 ? (int)force_split
                                     : stream_splits(p.tiles, p.kc);
    const int kcs = (p.kc + s0 - 1) / s0;                 // chunks per slice
    const int64_t force_grid = g_opts[NVFP4_OPT_GRID].load();
    int cpw, waves, cps, splits, grid;
    int64_t items, per_wg;
    // The grid: the fewest rounds of at most 256 workgroups (one per CU), then
    // as few workgroups as keep that number of rounds, so every workgroup
    // streams the same number of items.  A partial last round leaves the
    // memory system to the workgroups still running, which cannot use all
    // of it (1600 row tiles of the 32B gate_up projection: 229 workgroups of
    // 7 items measured 27.8 us at M = 1 and 36.6 us at M = 8, against 29.5
    // and 39.3 us on 192 and 256 workgroups).
    auto shape = [&]() {
      cpw = (int)round_up((kcs + want - 1) / want, gc);
      waves = (kcs + cpw - 1) / cpw;
      cps = cpw * waves;
      splits = (p.kc + cps - 1) / cps;
      items = (int64_t)p.tiles * (h16 ? 2 : 1) * splits;
      if (slices > 0) {
        // gt workgroups per slice, each over tiles b, b + gt, ...
        int64_t rounds = (items + kStreamGrid - 1) / kStreamGrid, gt;
        for (;; ++rounds) {
          gt = ((int64_t)p.tiles + rounds - 1) / rounds;
          if (gt * splits <= kStreamGrid) break;
        }
        grid = (int)(gt * splits);
        per_wg = ((int64_t)p.tiles + gt - 1) / gt;
      } else if (force_grid > 0) {
        grid = (int)std::min<int64_t>(items, force_grid);
        per_wg = (items + grid - 1) / grid;
      } else {
        const int64_t rounds = (items + kStreamGrid - 1) / kStreamGrid;
        grid = (int)((items + rounds - 1) / rounds);
        per_wg = (items + grid - 1) / grid;
      }
    };
    shape();
    // One activation row on the MFMA dot: 4 wavefronts instead of 8 when the
    // items split evenly over 256 workgroups (>= 85% of a whole number of
    // rounds) and each wave would cycle through its whole ring of 3 groups:
    // half the data in flight per CU, twice the stream per wave (8B down
    // 9.3 -> 8.4 us, medians of repeated graph replays).  At 8 rows the dot
    // needs the waves and the CUs (every shape slower).  Kept only where the
    // activation still fits the 4-wave quantizing prologue.
    if (force_waves == 0 && want_mfma && M == 1 && splits == 1 &&
        (int64_t)M * (p.kc * 4) <= nvfp4::qa_max_blocks(M, 4)) {
      const int64_t rounds = (items + kStreamGrid - 1) / kStreamGrid;
      const bool even = items * 100 >= rounds * kStreamGrid * 85;
      if (even && per_wg * (cpw / gc) >= 3) {           // 3: the ring depth at M = 1
        want = 4;
        shape();
      }
    }
    const int64_t act = (int64_t)nvfp4::stream_act_lds(M, p.kc, want_mfma);
    const int64_t slot = (int64_t)waves * M * (h16 ? 16 : 32) * 4;
    const int64_t batch = std::min<int64_t>(per_wg, (kLdsBudget - act) / slot);
    const bool shape_ok = !silu || N % nvfp4::kTileN == 0;
    const bool slices_ok = slices == 0 || (splits > 1 && grid % splits == 0);
    if (waves <= max_waves && batch >= 1 && shape_ok && slices_ok &&
        (splits == 1 || per_wg <= batch * waves * M * 32)) {
      p.kind = want_mfma ? nvfp4::kGemvMfma : nvfp4::kGemvStream;
      p.waves = waves;
      p.depth = 12;
      p.cpw = cpw;
      p.cps = cps;
      p.splits = splits;
      p.batch = (int)batch;
      p.h16 = h16 ? 1 : 0;
      p.grid = grid;        // <= 256: one resident workgroup per CU (the launch reserves LDS)
      finish_workspace(p, M);
      return p;
    }
  }

  // Split kernel: one workgroup per (row tile, K slice).
  p.kind = nvfp4::kGemvSplit;
  if (special) return p;                  // no streaming plan for the fused epilogue / slices
  p.depth = 0;
  int waves = force_waves > 0 ? (int)force_waves : 4;
  int cpw = 4;
  if (force_cpw > 0) {
    cpw = (int)force_cpw;
  } else if (force_split > 0) {
    const int64_t per = (p.kc + force_split - 1) / force_split;          // chunks per slice
    cpw = (int)std::min<int64_t>(16, std::max<int64_t>(4, round_up((per + waves - 1) / waves, 4)));
  } else {
    // Enough workgroups to give every one of the 256 CUs two, with each
    // wavefront streaming as many 1 KiB records as possible (<= 16).
    const int64_t want_wgs = 512;
    const int cands[4] = {16, 12, 8, 4};
    for (int c : cands) {
      const int64_t splits = (p.kc + (int64_t)waves * c - 1) / ((int64_t)waves * c);
      if ((int64_t)p.tiles * splits >= want_wgs) { cpw = c; break; }
    }
  }
  while (cpw > 4 && !split_ok(M, cpw, waves)) cpw -= 4;
  while (waves > 4 && !split_ok(M, cpw, waves)) waves /= 2;
  p.waves = waves;
  p.cpw = cpw;
  p.cps = cpw * p.waves;
  p.splits = (p.kc + p.cps - 1) / p.cps;
  p.grid = p.tiles * p.splits;
  finish_workspace(p, M);
  return p;
}

}  // namespace

namespace nvfp4 {
// for stack.cpp: whether the gate_up GEMV with the SiLU * mul epilogue has a plan
bool silu_plan_ok(int M, int64_t F, int64_t K) {
  return F >= 16 && F % 16 == 0 && make_plan(M, 2 * F, K, true).kind == kGemvMfma;
}
}  // namespace nvfp4

extern "C" {

int nvfp4_abi_version(void) { return kAbiVersion; }
int nvfp4_layout_version(void) { return kLayoutVersion; }
int nvfp4_last_hip_error(void) { return t_last_hip; }

const char* nvfp4_status_string(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARG: return "invalid argument";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported (M > 8, not a gfx950 device, or unknown option)";
    case NVFP4_ERR_NO_DEVICE: return "no HIP device";
    case NVFP4_ERR_WORKSPACE: return "workspace too small";
    case NVFP4_ERR_HIP: return "HIP runtime error (see nvfp4_last_hip_error)";
  }
  return "unknown status";
}

nvfp4_status nvfp4_set_option(int opt, int64_t value) {
  switch (opt) {
    case NVFP4_OPT_GEMV_MAX_M:
      if (value < 0 || value > kMaxM) return NVFP4_ERR_INVALID_ARG;
      break;
    case NVFP4_OPT_SPLIT_K:
      if (value < 0 || value > 4096) return NVFP4_ERR_INVALID_ARG;
      break;
    case NVFP4_OPT_CHUNKS_PER_WAVE:
      if (value < 0 || value > 16 || value % 4) return NVFP4_ERR_INVALID_ARG;
      break;
    case NVFP4_OPT_NONTEMPORAL:
      if (value != 0 && value != 1) return NVFP4_ERR_INVALID_ARG;
      break;
    case NVFP4_OPT_WAVES:
      if (value != 0 && value != 4 && value != 8 && value != 16) return NVFP4_ERR_INVALID_ARG;
      break;
    case NVFP4_OPT_KERNEL:
      if (value < 0 || value > 3) return NVFP4_ERR_INVALID_ARG;
      break;
    case NVFP4_OPT_SPIN_LIMIT:
      if (value < 0 || value > (int64_t(1) << 30)) return NVFP4_ERR_INVALID_ARG;
      break;
    case NVFP4_OPT_GRID:
      if (value < 0 || value > 65536) return NVFP4_ERR_INVALID_ARG;
      break;
    case NVFP4_OPT_FUSE_QUANT:
      if (value != 0 && value != 1) return NVFP4_ERR_INVALID_ARG;
      break;
    case NVFP4_OPT_HALF_TILES:
    case NVFP4_OPT_F32_SLICES:
      if (value < 0 || value > 2) return NVFP4_ERR_INVALID_ARG;
      break;
    default: return NVFP4_ERR_UNSUPPORTED;
  }
  g_opts[opt].store(value);
  return NVFP4_OK;
}

nvfp4_status nvfp4_get_option(int opt, int64_t* value) {
  if (opt < 0 || opt >= NVFP4_OPT_COUNT) return NVFP4_ERR_UNSUPPORTED;
  if (!value) return NVFP4_ERR_INVALID_ARG;
  *value = g_opts[opt].load();
  return NVFP4_OK;
}

nvfp4_status nvfp4_weight_bytes(int64_t N, int64_t K, size_t* codes_bytes, size_t* scales_bytes) {
  if (!codes_bytes || !scales_bytes || !valid_nk(N, K)) return NVFP4_ERR_INVALID_ARG;
  const int64_t np = round_up(N, nvfp4::kTileN), kp = round_up(K, nvfp4::kGroupK);
  *codes_bytes = (size_t)(np * kp / 2);
  *scales_bytes = (size_t)(np * kp / 16);
  return NVFP4_OK;
}

nvfp4_status nvfp4_quantize_weight(const uint16_t* w_bf16, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* w_codes, uint8_t* w_scales, float* w_gscale,
                                   void* stream) {
  if (!w_bf16 || !w_codes || !w_scales || !w_gscale) return NVFP4_ERR_INVALID_ARG;
  if (!valid_nk(N, K) || ldw < K || ldw % 8 != 0) return NVFP4_ERR_INVALID_ARG;
  if (!aligned(w_bf16, 16) || !aligned(w_codes, 16) || !aligned(w_scales, 8) ||
      !aligned(w_gscale, 4))
    return NVFP4_ERR_INVALID_ARG;
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_quantize_weight(w_bf16, N, K, ldw, w_codes, w_scales,
                                                     w_gscale, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_quantize_weight_gate_up(const uint16_t* w_bf16, int64_t F, int64_t K,
                                           int64_t ldw, uint8_t* w_codes, uint8_t* w_scales,
                                           float* w_gscale, void* stream) {
  if (!w_bf16 || !w_codes || !w_scales || !w_gscale) return NVFP4_ERR_INVALID_ARG;
  if (F < 16 || F % 16 != 0 || !valid_nk(2 * F, K) || ldw < K || ldw % 8 != 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!aligned(w_bf16, 16) || !aligned(w_codes, 16) || !aligned(w_scales, 8) ||
      !aligned(w_gscale, 4))
    return NVFP4_ERR_INVALID_ARG;
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_quantize_weight(w_bf16, 2 * F, K, ldw, w_codes, w_scales,
                                                     w_gscale, (hipStream_t)stream, F);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_unpack_weight(const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                                 int64_t K, uint8_t* codes_rowmajor, uint8_t* scales_rowmajor,
                                 void* stream) {
  if (!w_codes || !w_scales || !codes_rowmajor || !scales_rowmajor) return NVFP4_ERR_INVALID_ARG;
  if (!valid_nk(N, K)) return NVFP4_ERR_INVALID_ARG;
  if (!aligned(w_codes, 8) || !aligned(codes_rowmajor, 8)) return NVFP4_ERR_INVALID_ARG;
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_unpack_weight(w_codes, w_scales, N, K, codes_rowmajor,
                                                   scales_rowmajor, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

size_t nvfp4_act_workspace_bytes(int M, int64_t K) {
  if (M < 1 || M > kMaxM || K < 16 || K % 16 != 0 || (int64_t)M * (K >> 4) > nvfp4::kActMaxBlocks)
    return 0;
  return nvfp4::act_plan(M, K).groups > 1 ? nvfp4::kActSyncBytes : 0;
}

nvfp4_status nvfp4_quantize_act(const uint16_t* x_bf16, int M, int64_t K, int64_t ldx,
                                uint8_t* x_codes, uint8_t* x_scales, float* x_gscale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (M > kMaxM) return NVFP4_ERR_UNSUPPORTED;
  if (!x_bf16 || !x_codes || !x_scales || !x_gscale) return NVFP4_ERR_INVALID_ARG;
  if (M < 1 || K < 16 || K % 16 != 0 || (int64_t)M * (K >> 4) > nvfp4::kActMaxBlocks ||
      ldx < K || ldx % 8 != 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(x_codes, 8) || !aligned(x_gscale, 4))
    return NVFP4_ERR_INVALID_ARG;
  const size_t need = nvfp4_act_workspace_bytes(M, K);
  if (need > 0) {
    if (!workspace || !aligned(workspace, 16)) return NVFP4_ERR_INVALID_ARG;
    if (workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
  }
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_quantize_act(
      x_bf16, M, (int)K, ldx, x_codes, x_scales, x_gscale, static_cast<uint32_t*>(workspace),
      (uint32_t)g_opts[NVFP4_OPT_SPIN_LIMIT].load(), (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

size_t nvfp4_quantize_linear_workspace_bytes(int M, int64_t N, int64_t K) {
  if (M < 1 || M > kMaxM || !valid_nk(N, K) ||
      N > (int64_t)nvfp4::kMaxCounterTiles * nvfp4::kTileN ||
      (int64_t)M * (K >> 4) > nvfp4::kActMaxBlocks)
    return 0;
  // At least the sync record: when the call is not fused, its quantizer (the
  // plain one, or the RMS-norm one that needs the record whenever M > 1)
  // runs as its own launch on this workspace.
  size_t need = nvfp4::kActSyncBytes;
  const size_t lin = nvfp4_linear_workspace_bytes(M, N, K);
  const size_t act = nvfp4_act_workspace_bytes(M, K);
  if (lin > need) need = lin;
  if (act > need) need = act;
  return need;
}

namespace {

// Whether the GEMV's prologue quantizes the bf16 activation (every workgroup
// the whole of it) instead of a quantizer launch before the GEMV: up to 4
// blocks per thread, and without the RMS norm and with four or more rows up
// to 8 (the E2M1 encoding runs on the conversion instruction; a second
// launch costs about 5 us at M = 8).  The RMS norm's prologue at 8 blocks
// per thread cost more than its own launch (Qwen3-32B QKV at M = 8 in the
// layer stack: 21.1 us fused, 5.8 + 13.0 us as two launches).
bool fuse_prologue(const GemvPlan& p, int M, int64_t K, bool rms) {
  const int64_t blocks = (int64_t)M * (K >> 4);
  return g_opts[NVFP4_OPT_FUSE_QUANT].load() != 0 && p.kind == nvfp4::kGemvMfma &&
         blocks <= nvfp4::qa_max_blocks(M, p.waves, rms) && blocks <= kFuseMaxBlocks;
}

// nvfp4_quantize_linear (rms = 0), nvfp4_rmsnorm_quantize_linear (rms = 1)
// and, with sg_static set, nvfp4_quantize_linear_static (x_gscale unused)
nvfp4_status quantize_linear_impl(int rms, float eps, float* h_out, const float* sg_static, int M,
                                  int64_t N, int64_t K, const uint16_t* x_bf16, int64_t ldx,
                                  const uint8_t* w_codes, const uint8_t* w_scales,
                                  const float* w_gscale, void* y, int out_dtype, uint8_t* x_codes,
                                  uint8_t* x_scales, float* x_gscale, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (M > kMaxM) return NVFP4_ERR_UNSUPPORTED;
  if (M < 1 || !valid_nk(N, K) || N > (int64_t)nvfp4::kMaxCounterTiles * nvfp4::kTileN ||
      (int64_t)M * (K >> 4) > nvfp4::kActMaxBlocks || ldx < K || ldx % 8 != 0)
    return NVFP4_ERR_INVALID_ARG;
  if (rms && (K > nvfp4::kPrepMaxK || !(eps >= 0.0f) || !std::isfinite(eps)))
    return NVFP4_ERR_INVALID_ARG;
  if (!x_bf16 || !w_codes || !w_scales || !w_gscale || !y || !x_codes || !x_scales ||
      !(sg_static ? sg_static : x_gscale))
    return NVFP4_ERR_INVALID_ARG;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(x_codes, 8) ||
      !aligned(sg_static ? sg_static : x_gscale, 4) ||
      !aligned(w_codes, 16) || !aligned(w_scales, 8) ||
      !aligned(y, out_dtype == NVFP4_OUT_F32 ? 4 : 2) || (h_out && !aligned(h_out, 16)))
    return NVFP4_ERR_INVALID_ARG;
  const GemvPlan p = make_plan(M, N, K);
  const bool fused = fuse_prologue(p, M, K, rms != 0);
  if (!fused) {
    // two launches: the (RMS norm +) activation quantizer, then the linear
    const nvfp4_status st =
        sg_static ? nvfp4_quantize_act_static(x_bf16, M, K, ldx, sg_static, x_codes, x_scales,
                                              stream)
        : rms     ? nvfp4_rmsnorm_quantize_act(x_bf16, M, K, ldx, eps, x_codes, x_scales,
                                               x_gscale, h_out, workspace, workspace_bytes, stream)
                  : nvfp4_quantize_act(x_bf16, M, K, ldx, x_codes, x_scales, x_gscale, workspace,
                                       workspace_bytes, stream);
    if (st != NVFP4_OK) return st;
    return nvfp4_linear(M, N, K, x_codes, x_scales, sg_static ? sg_static : x_gscale, w_codes,
                        w_scales, w_gscale, y, out_dtype, workspace, workspace_bytes, stream);
  }
  if (p.ws_bytes > 0) {
    if (!workspace || !aligned(workspace, 256)) return NVFP4_ERR_INVALID_ARG;
    if (workspace_bytes < p.ws_bytes) return NVFP4_ERR_WORKSPACE;
  }
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_gemv_stream(
      p, M, N, K, x_codes, x_scales, x_gscale, w_codes, w_scales, w_gscale, y, out_dtype,
      workspace, (hipStream_t)stream, x_bf16, ldx, x_codes, x_scales, x_gscale, rms, eps, h_out,
      sg_static);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

}  // namespace

nvfp4_status nvfp4_quantize_act_static(const uint16_t* x_bf16, int M, int64_t K, int64_t ldx,
                                       const float* x_gscale, uint8_t* x_codes, uint8_t* x_scales,
                                       void* stream) {
  if (M > kMaxM) return NVFP4_ERR_UNSUPPORTED;
  if (!x_bf16 || !x_codes || !x_scales || !x_gscale) return NVFP4_ERR_INVALID_ARG;
  if (M < 1 || K < 16 || K % 16 != 0 || (int64_t)M * (K >> 4) > nvfp4::kActMaxBlocks ||
      ldx < K || ldx % 8 != 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(x_codes, 8) || !aligned(x_gscale, 4))
    return NVFP4_ERR_INVALID_ARG;
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_quantize_act(
      x_bf16, M, (int)K, ldx, x_codes, x_scales, nullptr, nullptr, 0, (hipStream_t)stream,
      x_gscale);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_quantize_linear_static(int M, int64_t N, int64_t K, const uint16_t* x_bf16,
                                          int64_t ldx, const float* x_gscale,
                                          const uint8_t* w_codes, const uint8_t* w_scales,
                                          const float* w_gscale, void* y, int out_dtype,
                                          uint8_t* x_codes, uint8_t* x_scales, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (!x_gscale) return M > kMaxM ? NVFP4_ERR_UNSUPPORTED : NVFP4_ERR_INVALID_ARG;
  return quantize_linear_impl(0, 0.0f, nullptr, x_gscale, M, N, K, x_bf16, ldx, w_codes, w_scales,
                              w_gscale, y, out_dtype, x_codes, x_scales, nullptr, workspace,
                              workspace_bytes, stream);
}

nvfp4_status nvfp4_quantize_linear(int M, int64_t N, int64_t K, const uint16_t* x_bf16, int64_t ldx,
                                   const uint8_t* w_codes, const uint8_t* w_scales,
                                   const float* w_gscale, void* y, int out_dtype, uint8_t* x_codes,
                                   uint8_t* x_scales, float* x_gscale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return quantize_linear_impl(0, 0.0f, nullptr, nullptr, M, N, K, x_bf16, ldx, w_codes, w_scales,
                              w_gscale, y, out_dtype, x_codes, x_scales, x_gscale, workspace,
                              workspace_bytes, stream);
}

nvfp4_status nvfp4_rmsnorm_quantize_linear(int M, int64_t N, int64_t K, const uint16_t* x_bf16,
                                           int64_t ldx, float eps, const uint8_t* w_codes,
                                           const uint8_t* w_scales, const float* w_gscale,
                                           void* y, int out_dtype, uint8_t* x_codes,
                                           uint8_t* x_scales, float* x_gscale, float* h_out,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream) {
  return quantize_linear_impl(1, eps, h_out, nullptr, M, N, K, x_bf16, ldx, w_codes, w_scales,
                              w_gscale, y, out_dtype, x_codes, x_scales, x_gscale, workspace,
                              workspace_bytes, stream);
}

namespace {

// Fraction of the 256 CUs' item slots a streaming plan fills.
double plan_eff(const GemvPlan& p) {
  const int64_t items = (int64_t)p.tiles * (p.h16 ? 2 : 1) * p.splits;
  const int64_t per_wg = (items + p.grid - 1) / p.grid;
  return (double)items / (double)(kStreamGrid * per_wg);
}

// The K-slice plan of the binary32 quantize + linear: among 2..16 slices
// whose per-slice blocks fit the prologue, the one that keeps the most CUs
// busy (items / (256 x items per workgroup)), the fewest slices on a tie;
// kind kGemvSplit if none fits.  (Qwen3-32B down at M = 8: 8 slices of 56
// chunks on 256 workgroups; 7 slices would leave 32 CUs idle.)
GemvPlan f32_slice_plan(int M, int64_t N, int64_t K) {
  GemvPlan best = {};
  best.kind = nvfp4::kGemvSplit;
  double best_eff = 0.0;
  for (int sl = 2; sl <= 16; ++sl) {
    const GemvPlan p = make_plan(M, N, K, false, sl);
    if (p.kind != nvfp4::kGemvMfma) continue;
    const int64_t blocks = (int64_t)M * std::min<int64_t>(4 * (int64_t)p.cps, K >> 4);
    if (blocks > nvfp4::qa_max_blocks(M, p.waves, true)) continue;
    const double eff = plan_eff(p);
    if (eff > best_eff + 1e-9) {
      best = p;
      best_eff = eff;
    }
  }
  return best;
}

bool f32_whole_fits(const GemvPlan& p, int M, int64_t K) {
  const int64_t blocks = (int64_t)M * (K >> 4);
  return p.kind == nvfp4::kGemvMfma && blocks <= nvfp4::qa_max_blocks(M, p.waves, true) &&
         blocks <= kFuseMaxBlocks;
}

// Whether nvfp4_quantize_linear_f32 with a maxima record takes the K-slice
// plan ps over the whole-activation plan p (NVFP4_OPT_F32_SLICES).  Off by
// default: every slice is quantized by each of its workgroups and the
// split-K tail costs more than it saves (graph replays: Qwen3-32B down at
// M = 1 17.1 us whole vs 19.9 us in 8 slices; at M = 8 the quantizer with
// the record then the linear 27.8 us vs 31.8 us in 8 slices; Qwen3-8B down
// at M = 8 16.6 vs 17.6 us).
bool f32_take_slices(const GemvPlan& p, const GemvPlan& ps, int M, int64_t K) {
  if (ps.kind != nvfp4::kGemvMfma) return false;
  const int64_t mode = g_opts[NVFP4_OPT_F32_SLICES].load();
  return mode == 2 || (mode == 1 && !f32_whole_fits(p, M, K));
}

nvfp4_status check_ws(const GemvPlan& p, void* workspace, size_t workspace_bytes) {
  if (p.ws_bytes == 0) return NVFP4_OK;
  if (!workspace || !aligned(workspace, 256)) return NVFP4_ERR_INVALID_ARG;
  return workspace_bytes < p.ws_bytes ? NVFP4_ERR_WORKSPACE : NVFP4_OK;
}

}  // namespace

nvfp4_status nvfp4_quantize_act_f32(const float* x_f32, int M, int64_t K, int64_t ldx,
                                    const uint32_t* x_amax, uint8_t* x_codes, uint8_t* x_scales,
                                    float* x_gscale, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (M > kMaxM) return NVFP4_ERR_UNSUPPORTED;
  if (!x_f32 || !x_codes || !x_scales || !x_gscale) return NVFP4_ERR_INVALID_ARG;
  if (M < 1 || K < 16 || K % 16 != 0 || (int64_t)M * (K >> 4) > nvfp4::kActMaxBlocks ||
      ldx < K || ldx % 4 != 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!aligned(x_f32, 16) || !aligned(x_codes, 8) || !aligned(x_gscale, 4) ||
      (x_amax && !aligned(x_amax, 16)))
    return NVFP4_ERR_INVALID_ARG;
  const nvfp4::ActPlan ap = nvfp4::act_plan(M, K);
  if (ap.groups > 1 && !x_amax) {
    if (!workspace || !aligned(workspace, 16)) return NVFP4_ERR_INVALID_ARG;
    if (workspace_bytes < nvfp4::kActSyncBytes) return NVFP4_ERR_WORKSPACE;
  }
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_quantize_act_f32(
      x_f32, M, (int)K, ldx, x_amax, x_codes, x_scales, x_gscale,
      static_cast<uint32_t*>(workspace), (uint32_t)g_opts[NVFP4_OPT_SPIN_LIMIT].load(),
      (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

size_t nvfp4_quantize_linear_f32_workspace_bytes(int M, int64_t N, int64_t K) {
  if (M < 1 || M > kMaxM || !valid_nk(N, K) ||
      N > (int64_t)nvfp4::kMaxCounterTiles * nvfp4::kTileN)
    return 0;
  const GemvPlan p = make_plan(M, N, K);
  size_t b = std::max(nvfp4::kActSyncBytes, p.ws_bytes);
  const GemvPlan ps = f32_slice_plan(M, N, K);
  if (f32_take_slices(p, ps, M, K)) b = std::max(b, ps.ws_bytes);   // it may run
  return b;
}

nvfp4_status nvfp4_quantize_linear_f32(int M, int64_t N, int64_t K, const float* x_f32,
                                       int64_t ldx, const uint32_t* x_amax,
                                       const uint8_t* w_codes, const uint8_t* w_scales,
                                       const float* w_gscale, void* y, int out_dtype,
                                       uint8_t* x_codes, uint8_t* x_scales, float* x_gscale,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  if (M > kMaxM) return NVFP4_ERR_UNSUPPORTED;
  if (M < 1 || !valid_nk(N, K) || N > (int64_t)nvfp4::kMaxCounterTiles * nvfp4::kTileN ||
      (int64_t)M * (K >> 4) > nvfp4::kActMaxBlocks || ldx < K || ldx % 4 != 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!x_f32 || !w_codes || !w_scales || !w_gscale || !y || !x_codes || !x_scales || !x_gscale)
    return NVFP4_ERR_INVALID_ARG;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_INVALID_ARG;
  if (!aligned(x_f32, 16) || !aligned(x_codes, 8) || !aligned(x_gscale, 4) ||
      (x_amax && !aligned(x_amax, 16)) || !aligned(w_codes, 16) || !aligned(w_scales, 8) ||
      !aligned(y, out_dtype == NVFP4_OUT_F32 ? 4 : 2))
    return NVFP4_ERR_INVALID_ARG;
  const bool fuse = g_opts[NVFP4_OPT_FUSE_QUANT].load() != 0;
  GemvPlan p = make_plan(M, N, K);
  int qslice = 0;
  // with the producer's maxima record every workgroup may stay in one K
  // slice and quantize only that slice (the record's maximum covers them all)
  const GemvPlan ps = fuse && x_amax ? f32_slice_plan(M, N, K) : GemvPlan{};
  if (fuse && x_amax && f32_take_slices(p, ps, M, K)) {
    p = ps;
    qslice = 1;
  } else if (!(fuse && f32_whole_fits(p, M, K))) {
    // two launches: the binary32 activation quantizer, then the linear
    const nvfp4_status st = nvfp4_quantize_act_f32(x_f32, M, K, ldx, x_amax, x_codes, x_scales,
                                                   x_gscale, workspace, workspace_bytes, stream);
    if (st != NVFP4_OK) return st;
    return nvfp4_linear(M, N, K, x_codes, x_scales, x_gscale, w_codes, w_scales, w_gscale, y,
                        out_dtype, workspace, workspace_bytes, stream);
  }
  if (nvfp4_status st = check_ws(p, workspace, workspace_bytes); st != NVFP4_OK) return st;
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_gemv_stream(
      p, M, N, K, x_codes, x_scales, x_gscale, w_codes, w_scales, w_gscale, y, out_dtype,
      workspace, (hipStream_t)stream, nullptr, ldx, x_codes, x_scales, x_gscale, 0, 0.0f, nullptr,
      nullptr, x_f32, x_amax, qslice);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_quantize_linear_silu_mul(int M, int64_t F, int64_t K, const uint16_t* x_bf16,
                                            int64_t ldx, int rmsnorm, float eps,
                                            const uint8_t* w_codes, const uint8_t* w_scales,
                                            const float* w_gscale, float* h, int64_t ldh,
                                            uint32_t* h_amax, uint16_t* gu_out, uint8_t* x_codes,
                                            uint8_t* x_scales, float* x_gscale, float* xh_out,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream) {
  if (M > kMaxM) return NVFP4_ERR_UNSUPPORTED;
  const int64_t N = 2 * F;
  if (M < 1 || F < 16 || F % 16 != 0 || !valid_nk(N, K) ||
      (int64_t)M * (K >> 4) > nvfp4::kActMaxBlocks || ldx < K || ldx % 8 != 0 || ldh < F ||
      ldh % 4 != 0)
    return NVFP4_ERR_INVALID_ARG;
  if (rmsnorm != 0 && rmsnorm != 1) return NVFP4_ERR_INVALID_ARG;
  if (rmsnorm && (K > nvfp4::kPrepMaxK || !(eps >= 0.0f) || !std::isfinite(eps)))
    return NVFP4_ERR_INVALID_ARG;
  if (!rmsnorm && xh_out) return NVFP4_ERR_INVALID_ARG;
  if (!x_bf16 || !w_codes || !w_scales || !w_gscale || !h || !h_amax || !x_codes || !x_scales ||
      !x_gscale)
    return NVFP4_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(x_codes, 8) || !aligned(x_gscale, 4) ||
      !aligned(w_codes, 16) || !aligned(w_scales, 8) || !aligned(h, 16) ||
      !aligned(h_amax, 16) || (gu_out && !aligned(gu_out, 2)) || (xh_out && !aligned(xh_out, 16)))
    return NVFP4_ERR_INVALID_ARG;
  const GemvPlan p = make_plan(M, N, K, true);
  if (p.kind != nvfp4::kGemvMfma) return NVFP4_ERR_UNSUPPORTED;
  const bool fused = fuse_prologue(p, M, K, rmsnorm != 0);
  if (!fused) {
    // the (RMS norm +) activation quantizer first; the GEMV then stages its codes
    const nvfp4_status st =
        rmsnorm ? nvfp4_rmsnorm_quantize_act(x_bf16, M, K, ldx, eps, x_codes, x_scales, x_gscale,
                                             xh_out, workspace, workspace_bytes, stream)
                : nvfp4_quantize_act(x_bf16, M, K, ldx, x_codes, x_scales, x_gscale, workspace,
                                     workspace_bytes, stream);
    if (st != NVFP4_OK) return st;
  }
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_gemv_stream(
      p, M, N, K, x_codes, x_scales, x_gscale, w_codes, w_scales, w_gscale, h, 0, workspace,
      (hipStream_t)stream, fused ? x_bf16 : nullptr, ldx, x_codes, x_scales, x_gscale,
      fused ? rmsnorm : 0, eps, fused ? xh_out : nullptr, nullptr, nullptr, nullptr, 0, h_amax,
      ldh, gu_out);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

namespace {

nvfp4_status prep_quantize(int mode, const uint16_t* x, int M, int64_t K, int64_t ld, int64_t ld_min,
                           float eps, uint8_t* codes, uint8_t* scales, float* gscale, float* h_out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (M > kMaxM) return NVFP4_ERR_UNSUPPORTED;
  if (!x || !codes || !scales || !gscale) return NVFP4_ERR_INVALID_ARG;
  if (M < 1 || K < 16 || K % 16 != 0 || K > nvfp4::kPrepMaxK || ld < ld_min || ld % 8 != 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return NVFP4_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(gscale, 4) ||
      (h_out && !aligned(h_out, 16)))
    return NVFP4_ERR_INVALID_ARG;
  if (M > 1) {
    if (!workspace || !aligned(workspace, 16)) return NVFP4_ERR_INVALID_ARG;
    if (workspace_bytes < nvfp4::kActSyncBytes) return NVFP4_ERR_WORKSPACE;
  }
  // One row without a (large enough, aligned) workspace: no sync record, so
  // the one-workgroup-per-row kernel runs; with one, SiLU * mul spreads its
  // blocks over workgroups.
  uint32_t* sync = workspace && aligned(workspace, 16) && workspace_bytes >= nvfp4::kActSyncBytes
                       ? static_cast<uint32_t*>(workspace)
                       : nullptr;
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_prep_quantize(
      mode, x, M, (int)K, ld, eps, codes, scales, gscale, h_out, sync,
      (uint32_t)g_opts[NVFP4_OPT_SPIN_LIMIT].load(), (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

}  // namespace

nvfp4_status nvfp4_rmsnorm_quantize_act(const uint16_t* x_bf16, int M, int64_t K, int64_t ldx,
                                        float eps, uint8_t* x_codes, uint8_t* x_scales,
                                        float* x_gscale, float* h_out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return prep_quantize(0, x_bf16, M, K, ldx, K, eps, x_codes, x_scales, x_gscale, h_out, workspace,
                       workspace_bytes, stream);
}

nvfp4_status nvfp4_silu_mul_quantize_act(const uint16_t* gu_bf16, int M, int64_t K, int64_t ldgu,
                                         uint8_t* x_codes, uint8_t* x_scales, float* x_gscale,
                                         float* h_out, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  return prep_quantize(1, gu_bf16, M, K, ldgu, 2 * K, 0.0f, x_codes, x_scales, x_gscale, h_out,
                       workspace, workspace_bytes, stream);
}

size_t nvfp4_linear_workspace_bytes(int M, int64_t N, int64_t K) {
  if (M < 1 || M > kMaxM || !valid_nk(N, K) ||
      N > (int64_t)nvfp4::kMaxCounterTiles * nvfp4::kTileN)
    return 0;
  return make_plan(M, N, K).ws_bytes;
}

size_t nvfp4_reset_workspace_bytes(int M, int64_t V) {
  if (M < 1 || M > nvfp4::kResetMaxRows || V < 1 || V > nvfp4::kResetMaxV) return 0;
  return nvfp4::kResetCounterBytes +
         (size_t)round_up((int64_t)M * nvfp4::reset_groups_per_row(V) * 16, 256);
}

nvfp4_status nvfp4_reset_temperature(const float* logits, int M, int64_t V, int64_t ldl,
                                     const nvfp4_reset_params* params, float* step_state,
                                     const int32_t* step_end, float* entropy, float* temperature,
                                     float* logits_out, int64_t ldo, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!logits || !params || !step_state || !entropy || !temperature)
    return NVFP4_ERR_INVALID_ARG;
  if (M < 1 || M > nvfp4::kResetMaxRows || V < 1 || V > nvfp4::kResetMaxV || ldl < V ||
      ldl % 4 != 0)
    return NVFP4_ERR_INVALID_ARG;
  const nvfp4_reset_params& q = *params;
  auto pos = [](float v) { return std::isfinite(v) && v > 0.0f; };
  if (!pos(q.t_low) || !pos(q.tau0) || !pos(q.t_base) || !pos(q.t_max))
    return NVFP4_ERR_INVALID_ARG;
  if (!aligned(logits, 16) || !aligned(step_state, 4) || !aligned(entropy, 4) ||
      !aligned(temperature, 4) || (step_end && !aligned(step_end, 4)))
    return NVFP4_ERR_INVALID_ARG;
  if (logits_out && (ldo < V || ldo % 4 != 0 || !aligned(logits_out, 16) ||
                     (logits_out == logits && ldo != ldl)))
    return NVFP4_ERR_INVALID_ARG;
  const size_t need = nvfp4_reset_workspace_bytes(M, V);
  if (!workspace || !aligned(workspace, 16)) return NVFP4_ERR_INVALID_ARG;
  if (workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_reset_temperature(
      logits, M, V, ldl, q.t_low, q.tau0, q.t_base, q.t_max, step_state, step_end, entropy,
      temperature, logits_out, ldo, workspace, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_selftest_e2m1(unsigned long long* result, void* stream) {
  if (!result || !aligned(result, 8)) return NVFP4_ERR_INVALID_ARG;
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_e2m1_selftest(result, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return NVFP4_OK;
  if (!workspace || !aligned(workspace, 4)) return NVFP4_ERR_INVALID_ARG;
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e = nvfp4::launch_fill_zero(workspace, workspace_bytes, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_linear(int M, int64_t N, int64_t K, const uint8_t* x_codes,
                          const uint8_t* x_scales, const float* x_gscale, const uint8_t* w_codes,
                          const uint8_t* w_scales, const float* w_gscale, void* y, int out_dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (M > kMaxM) return NVFP4_ERR_UNSUPPORTED;
  if (M < 1 || !valid_nk(N, K) || N > (int64_t)nvfp4::kMaxCounterTiles * nvfp4::kTileN ||
      K > (int64_t(1) << 28))
    return NVFP4_ERR_INVALID_ARG;
  if (!x_codes || !x_scales || !x_gscale || !w_codes || !w_scales || !w_gscale || !y)
    return NVFP4_ERR_INVALID_ARG;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_INVALID_ARG;
  if (!aligned(x_codes, 8) || !aligned(w_codes, 16) || !aligned(w_scales, 8) ||
      !aligned(y, out_dtype == NVFP4_OUT_F32 ? 4 : 2))
    return NVFP4_ERR_INVALID_ARG;
  const GemvPlan p = make_plan(M, N, K);
  if (p.ws_bytes > 0) {
    if (!workspace || !aligned(workspace, 256)) return NVFP4_ERR_INVALID_ARG;
    if (workspace_bytes < p.ws_bytes) return NVFP4_ERR_WORKSPACE;
  }
  if (nvfp4_status st = check_device(); st != NVFP4_OK) return st;
  const hipError_t e =
      p.kind != nvfp4::kGemvSplit
          ? nvfp4::launch_gemv_stream(p, M, N, K, x_codes, x_scales, x_gscale, w_codes, w_scales,
                                      w_gscale, y, out_dtype, workspace, (hipStream_t)stream)
          : nvfp4::launch_gemv_split(p, M, N, K, x_codes, x_scales, x_gscale, w_codes, w_scales,
                                     w_gscale, y, out_dtype, workspace, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

}  // extern "C"
