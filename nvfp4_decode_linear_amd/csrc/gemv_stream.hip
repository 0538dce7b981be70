// Persistent streaming VALU GEMV for the small-M NVFP4 W4A4 decode linear
// (gfx950): the default kernel whenever the whole K extent of the decoded
// activation fits in LDS.
//
// The operation is the one of "ReSET" GitHub README, "Core components",
// item 2 (nvfp4r): for M <= 8 rows the FP4 weights are streamed once through
// the vector ALUs and every loaded weight serves all M rows.  On gfx950:
//
//  * one workgroup of up to 16 wavefronts per CU walks row tiles blockIdx.x,
//    blockIdx.x + gridDim.x, ...; inside a tile wave w owns the K chunks
//    [w * cpw, (w + 1) * cpw), so a tile needs no reduction outside the
//    workgroup and the kernel needs no workspace;
//  * every wave keeps 3 or 4 groups of 4 weight records (1 KiB each, one
//    64-lane load) in flight and refills a group as soon as it has consumed
//    it; the wave's records of consecutive tiles form one stream, so the
//    loads of the next tile are already in flight while this tile finishes;
//  * the activation is decoded once per workgroup, for the whole K, into LDS
//    as f16 x~ = e2m1(code) * e4m3(scale) (exact); the decode overlaps the
//    first ring loads because its global loads are issued first;
//  * a tile's partial sums meet in LDS (fixed wave order, so the result is
//    the same on every run), are scaled by both tensor scales and written as
//    binary32 or bf16.
#include <type_traits>

#include "gemv_common.hpp"

namespace nvfp4 {

namespace {

using namespace gemv;

constexpr int kStreamXpt = 4;   // activation blocks per thread issued ahead of the ring

// Waves per workgroup the kernel is compiled for: 16 (<= 128 VGPRs) for one
// activation row, 8 (<= 256 VGPRs) for two or three rows, whose register
// footprint does not fit 128 without spilling.  Four or more rows use the
// split kernel (the streaming one would spill).
constexpr int kStreamMaxM = 3;
constexpr int stream_max_waves(int M) { return M == 1 ? 16 : 8; }

// Groups of 4 weight records (4 KiB) each wave keeps in flight.
constexpr int stream_ring_groups(int M) { return M == 3 ? 2 : 3; }

// The MFMA variant keeps 16 result registers per chunk but decodes nothing.
constexpr int mfma_max_waves(int M) { return M <= 3 ? 16 : 8; }
constexpr int mfma_ring_groups(int) { return 3; }

// The grid holds at most one workgroup per CU.  The hardware dispatcher
// packs workgroups onto a CU while its registers and LDS last, so every
// workgroup reserves more than half of the CU's 160 KiB LDS: then no CU can
// hold two and the min(tiles, 256) workgroups spread over distinct CUs.
constexpr size_t kStreamLdsReserve = 80 * 1024 + 1024;

template <int V>
using ic = std::integral_constant<int, V>;

// One workgroup's whole job.  Every wave keeps RG groups of 4 weight records
// in flight.  The numbers of groups the stream starts with and ends with are
// compile-time constants on every path (the paths never merge), so the
// compiler's memory wait counts stay exact: where paths with different
// numbers of outstanding loads merge, it waits for all of them.
template <int M, int RG, bool MF>
__device__ __forceinline__ void stream_body(const GemvArgs& a, uint32_t* lds) {
  const int NW = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const bool nt = a.nontemporal != 0;
  const int kc = a.kc;
  const int row_dw = kc * 32;
  // VALU: x~ as f16 pairs [M][kc * 32 dwords].  MFMA: raw activation codes
  // [M][kc * 4 blocks][2 dwords], then the E4M3 activation scales as floats
  // [kc * 4 blocks][M].  Either is followed by the reduction array
  // [2][NW][M][32] floats.
  uint32_t* xlds = lds;
  float* sa = reinterpret_cast<float*>(lds + M * kc * 8);
  float* red = reinterpret_cast<float*>(MF ? lds + M * kc * 8 + kc * 4 * M : lds + M * row_dw);
  const int kb_row = a.K >> 4;
  const int nblk = M * kc * 4;                // activation 16-blocks, padded K
  const int cpw = a.cpw;                      // chunks per wave per tile, multiple of 4
  const int wc0 = wave * cpw;
  const int wlast = min(wc0 + cpw, kc) - 1;   // last real chunk of this wave
  const int G = gridDim.x;
  const int ntile = (a.tiles - (int)blockIdx.x + G - 1) / G;
  const int ng = ntile * (cpw >> 2);          // groups of 4 records in this wave's stream

  // ---- 1. activation blocks, first batch (issued before any weight load;
  // out-of-range blocks read block 0 and are zeroed, so no load is
  // conditional and the decode below waits only for these loads)
  u32x2 xc[kStreamXpt];
  uint32_t xs[kStreamXpt];
#pragma unroll
  for (int r = 0; r < kStreamXpt; ++r) {
    const int i = threadIdx.x + r * 64 * NW;
    const int m = i / (kc * 4), kb = i - m * (kc * 4);
    const bool ok = i < nblk && kb < kb_row;
    const int64_t cofs = ok ? (int64_t)m * (a.K >> 1) + 8 * kb : 0;
    const int64_t sofs = ok ? (int64_t)m * kb_row + kb : 0;
    xc[r] = *reinterpret_cast<const u32x2*>(a.xc + cofs);
    xs[r] = a.xs[sofs];
    if (!ok) {
      xc[r] = u32x2{0u, 0u};
      xs[r] = 0u;
    }
  }

  // ---- 2. this wave's records form one stream: its cpw chunks of the
  // workgroup's first tile, then of its second tile, ...  Chunks past K
  // (only in the last wave) re-read the wave's last real chunk.
  const uint8_t* wbase = a.wc + 16 * lane;
  const uint8_t* sbase = a.ws + 8 * lane;
  int lt = blockIdx.x, loff = 0;              // load cursor: tile, chunk offset
  u32x4 ring[RG][4];
  u32x2 rsc[RG];
  auto refill = [&](auto Q) __attribute__((always_inline)) {
    constexpr int q = decltype(Q)::value;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t r = (int64_t)lt * kc + min(wc0 + loff + k, wlast);
      if (k == 0) rsc[q] = load_scales(sbase + (r >> 2) * kScaleRecord, nt);
      ring[q][k] = load_codes(wbase + r * kCodeRecord, nt);
    }
    loff += 4;
    if (loff == cpw) {
      loff = 0;
      lt += G;
    }
  };

  // ---- 3. activation into LDS: the first batch from registers, any rest
  // (large M * K only) read now.
  auto prologue = [&]() __attribute__((always_inline)) {
    auto put = [&](int m, int kb, u32x2 c, uint32_t sc) __attribute__((always_inline)) {
      if constexpr (MF) {
        xlds[(m * kc * 4 + kb) * 2] = c.x;
        xlds[(m * kc * 4 + kb) * 2 + 1] = c.y;
        sa[kb * M + m] = e4m3_to_f32(sc);
      } else {
        decode_act_block(c, sc, xlds + m * row_dw + kb * 8);
      }
    };
#pragma unroll
    for (int r = 0; r < kStreamXpt; ++r) {
      const int i = threadIdx.x + r * 64 * NW;
      if (i < nblk) {
        const int m = i / (kc * 4), kb = i - m * (kc * 4);
        put(m, kb, xc[r], xs[r]);
      }
    }
    for (int i = threadIdx.x + kStreamXpt * 64 * NW; i < nblk; i += 64 * NW) {
      const int m = i / (kc * 4), kb = i - m * (kc * 4);
      u32x2 c = {0u, 0u};
      uint32_t sc = 0u;
      if (kb < kb_row) {
        c = *reinterpret_cast<const u32x2*>(a.xc + (int64_t)m * (a.K >> 1) + 8 * kb);
        sc = a.xs[(int64_t)m * kb_row + kb];
      }
      put(m, kb, c, sc);
    }
    __syncthreads();
  };

  const float g = __fmul_rn(a.xg[0], a.wg[0]);
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  // Tile-boundary reduction: K halves (lanes l, l ^ 32), then waves in fixed
  // order through a double-buffered LDS array (so one barrier per tile).
  int ct = blockIdx.x, buf = 0;
  auto finish_tile = [&]() __attribute__((always_inline)) {
    float* rb = red + buf * (NW * M * 32);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      acc[m] += __shfl_xor(acc[m], 32, 64);
      if (h == 0) rb[(wave * M + m) * 32 + lane] = acc[m];
      acc[m] = 0.0f;
    }
    __syncthreads();
    const int n0 = ct * kTileN;
    for (int i = threadIdx.x; i < M * 32; i += 64 * NW) {
      const int m = i >> 5, n = i & 31;
      float v = rb[m * 32 + n];
      for (int q = 1; q < NW; ++q) v += rb[(q * M + m) * 32 + n];
      if (n0 + n < a.N) store_y(a, m, n0 + n, v * g);
    }
    buf ^= 1;
    ct += G;
  };

  // Consume ring group q: chunks coff .. coff + 3 of the current tile.  Branch
  // free (wait counts stay exact): a chunk past K (last wave only) reads a
  // valid activation chunk and gets a zero block scale, so it adds exactly 0.
  // MFMA A operand: lane l holds row r = l % 32 of the 32 x 64 block-diagonal
  // activation tile, K half l / 32.  Row r is activation row ma, block ja of
  // the chunk, chosen so that the 32 x 32 result lands with every lane
  // holding its own weight row n = l % 32 and its own two blocks 2h, 2h + 1
  // (result v = 4i + q of lane l is tile row 8i + 4h + q = (m 2i + q / 2,
  // block 2h + q % 2)).  The lane's 16 A bytes are the block's 8 code bytes,
  // in the low or high half, or zero when the block lies in the other K half
  // (or the row is past M).
  const int ra = lane & 31;
  const int ma = 2 * (ra >> 3) + ((ra & 3) >> 1);
  const int ja = 2 * ((ra >> 2) & 1) + (ra & 1);
  const bool a_on = (h == ((ra >> 2) & 1)) && (ma < M);
  const bool a_lo = a_on && (ra & 1) == 0, a_hi = a_on && (ra & 1) != 0;
  const uint32_t* xa_row = xlds + (ma < M ? ma : 0) * kc * 8 + ja * 2;

  int coff = 0;
  auto consume = [&](auto Q) __attribute__((always_inline)) {
    constexpr int q = decltype(Q)::value;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = wc0 + coff + k;
      uint32_t sb = (k < 2 ? rsc[q].x : rsc[q].y) >> (16 * (k & 1));
      sb = c < kc ? sb : 0u;
      const int cx = min(c, kc - 1);
      if constexpr (MF) {
        const uint32_t* xp = xa_row + cx * 8;
        const uint32_t a0 = xp[0], a1 = xp[1];
        const v8i A = {(int)(a_lo ? a0 : 0u), (int)(a_lo ? a1 : 0u), (int)(a_hi ? a0 : 0u),
                       (int)(a_hi ? a1 : 0u), 0, 0, 0, 0};
        const u32x4 wv = ring[q][k];
        const v8i B = {(int)wv.x, (int)wv.y, (int)wv.z, (int)wv.w, 0, 0, 0, 0};
        const v16f C = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, v16f{}, 4, 4, 0, 127,
                                                                       0, 127);
        const float sw0 = __builtin_amdgcn_cvt_f32_fp8(sb, 0);
        const float sw1 = __builtin_amdgcn_cvt_f32_fp8(sb, 1);
        const float* sap = sa + (4 * cx + 2 * h) * M;          // [block 2h + b][m]
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 2 * (v >> 2) + ((v & 3) >> 1), b = v & 1;
          if constexpr (true) {
            if (m < M) acc[m] = fmaf(C[v], sap[b * M + m] * (b ? sw1 : sw0), acc[m]);
          }
        }
      } else {
        dot_chunk<M>(ring[q][k], sb, xlds + ((cx * 64 + 32 * h) >> 1), row_dw, acc);
      }
    }
    coff += 4;
    if (coff == cpw) {
      finish_tile();
      coff = 0;
    }
  };

  // Short stream (ng < RG groups): load it all, then consume it.
  auto short_stream = [&](auto NG) __attribute__((always_inline)) {
    constexpr int n = decltype(NG)::value;
    static_assert(n >= 1 && n < RG, "a short stream fits the ring");
    refill(ic<0>{});
    if constexpr (n >= 2) refill(ic<(n >= 2 ? 1 : 0)>{});
    if constexpr (n >= 3) refill(ic<(n >= 3 ? 2 : 0)>{});
    prologue();
    consume(ic<0>{});
    if constexpr (n >= 2) consume(ic<(n >= 2 ? 1 : 0)>{});
    if constexpr (n >= 3) consume(ic<(n >= 3 ? 2 : 0)>{});
  };

  // Long stream: prime RG groups, then consume a group and refill its slot
  // with the group RG ahead; the tail consumes R = RG + r remaining groups,
  // refilling only the first r slots.
  auto step = [&](auto Q) __attribute__((always_inline)) {
    consume(Q);
    refill(Q);
  };
  // slot index clamped into the ring for code that is discarded when RG is small
  auto slot = [](auto Q) { return ic<(decltype(Q)::value < RG ? decltype(Q)::value : 0)>{}; };
  auto tail = [&](auto R) __attribute__((always_inline)) {
    constexpr int r = decltype(R)::value;
    static_assert(r < RG, "at most RG - 1 groups left to load");
    if constexpr (r > 0) step(ic<0>{}); else consume(ic<0>{});
    if constexpr (r > 1) step(slot(ic<1>{})); else consume(ic<1>{});
    if constexpr (RG > 2) { if constexpr (r > 2) step(slot(ic<2>{})); else consume(slot(ic<2>{})); }
    if constexpr (RG > 3) { if constexpr (r > 3) step(slot(ic<3>{})); else consume(slot(ic<3>{})); }
    if constexpr (r > 0) consume(ic<0>{});
    if constexpr (r > 1) consume(slot(ic<1>{}));
    if constexpr (r > 2) consume(slot(ic<2>{}));
  };

  static_assert(RG >= 2 && RG <= 4, "ring of 2 to 4 groups");
  if (ng >= RG) {
    refill(ic<0>{});
    refill(ic<1>{});
    if constexpr (RG > 2) refill(ic<2>{});
    if constexpr (RG > 3) refill(ic<3>{});
    prologue();
    int gi = 0;
    for (; gi + 2 * RG <= ng; gi += RG) {
      step(ic<0>{});
      step(ic<1>{});
      if constexpr (RG > 2) step(ic<2>{});
      if constexpr (RG > 3) step(ic<3>{});
    }
    switch (ng - gi - RG) {                   // 0 .. RG - 1 groups still to load
      case 0: tail(ic<0>{}); break;
      case 1: tail(ic<1>{}); break;
      case 2: if constexpr (RG > 2) tail(ic<(RG > 2 ? 2 : 0)>{}); break;
      default: if constexpr (RG > 3) tail(ic<(RG > 3 ? 3 : 0)>{}); break;
    }
  } else {
    switch (ng) {                             // 1 .. RG - 1
      case 1: short_stream(ic<1>{}); break;
      case 2: if constexpr (RG > 2) short_stream(ic<(RG > 2 ? 2 : 1)>{}); break;
      default: if constexpr (RG > 3) short_stream(ic<(RG > 3 ? 3 : 1)>{}); break;
    }
  }
}

// Launch: blockDim.x = 64 * NW (NW <= stream_max_waves(M), every wave owns at least one real
// chunk of each tile); dynamic LDS = x~ [M][kc * 32] dwords followed by the
// reduction array [2][NW][M][32] floats.
template <int M>
__global__ __launch_bounds__(64 * stream_max_waves(M)) void gemv_stream_kernel(GemvArgs a) {
  extern __shared__ uint32_t lds[];
  stream_body<M, stream_ring_groups(M), false>(a, lds);
}

template <int M>
__global__ __launch_bounds__(64 * mfma_max_waves(M)) void gemv_mfma_kernel(GemvArgs a) {
  extern __shared__ uint32_t lds[];
  stream_body<M, mfma_ring_groups(M), true>(a, lds);
}

template <int M, bool MF>
hipError_t launch_m(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  if (p.waves < 1 || p.waves > (MF ? mfma_max_waves(M) : stream_max_waves(M)))
    return hipErrorInvalidValue;
  const size_t need = stream_lds_need(M, p.kc, p.waves, MF);
  const size_t lds = need > kStreamLdsReserve ? need : kStreamLdsReserve;
  const void* fn;
  if constexpr (MF)
    fn = reinterpret_cast<const void*>(&gemv_mfma_kernel<M>);
  else
    fn = reinterpret_cast<const void*>(&gemv_stream_kernel<M>);
  static hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  if constexpr (MF)
    hipLaunchKernelGGL((gemv_mfma_kernel<M>), dim3((unsigned)p.grid), dim3(64 * p.waves), lds, s,
                       a);
  else
    hipLaunchKernelGGL((gemv_stream_kernel<M>), dim3((unsigned)p.grid), dim3(64 * p.waves), lds,
                       s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_stream(const GemvPlan& p, int M, int64_t N, int64_t K, const uint8_t* xc,
                              const uint8_t* xs, const float* xg, const uint8_t* wc,
                              const uint8_t* ws, const float* wg, void* y, int out_bf16,
                              hipStream_t s) {
  GemvArgs a = {};
  a.xc = xc;
  a.xs = xs;
  a.xg = xg;
  a.wc = wc;
  a.ws = ws;
  a.wg = wg;
  a.y = y;
  a.N = (int)N;
  a.n_pad = p.tiles * kTileN;
  a.K = (int)K;
  a.kc = p.kc;
  a.kg = p.kc / 4;
  a.cpw = p.cpw;
  a.splits = 1;
  a.out_bf16 = out_bf16;
  a.nontemporal = p.nontemporal;
  a.tiles = p.tiles;
  if (p.kind == kGemvMfma) {
    switch (M) {
      case 1: return launch_m<1, true>(p, a, s);
      case 2: return launch_m<2, true>(p, a, s);
      case 3: return launch_m<3, true>(p, a, s);
      case 4: return launch_m<4, true>(p, a, s);
      case 5: return launch_m<5, true>(p, a, s);
      case 6: return launch_m<6, true>(p, a, s);
      case 7: return launch_m<7, true>(p, a, s);
      case 8: return launch_m<8, true>(p, a, s);
      default: return hipErrorInvalidValue;
    }
  }
  static_assert(kStreamMaxM == 3, "one case per supported row count");
  switch (M) {
    case 1: return launch_m<1, false>(p, a, s);
    case 2: return launch_m<2, false>(p, a, s);
    case 3: return launch_m<3, false>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4
