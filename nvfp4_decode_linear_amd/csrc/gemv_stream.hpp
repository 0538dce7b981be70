// Persistent streaming GEMV for the small-M NVFP4 W4A4 decode linear (the
// kernel templates; gemv_stream_m<M>.hip instantiate them one row count per
// translation unit, gemv_stream.hip dispatches).
// (gfx950): the default kernels whenever the whole K extent of the
// activation fits in LDS.
//
// The operation is the one of "ReSET" GitHub README, "Core components",
// item 2 (nvfp4r): for M <= 8 rows the FP4 weights are streamed once and
// every loaded weight serves all M rows.  On gfx950:
//
//  * one workgroup of up to 8 wavefronts per CU walks work items blockIdx.x,
//    blockIdx.x + gridDim.x, ...; an item is a 32-row tile and a K slice
//    (normally all of K), whose 4-record groups go to the waves round robin;
//  * every wave keeps 3 groups of 4 weight records (1 KiB each, one 64-lane
//    load) plus their scale record in flight and refills a group as soon as
//    it has consumed it; the wave's groups of consecutive items form one
//    stream, so the next item's loads are in flight while this one finishes;
//  * the dot: either on FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with unit
//    E8M0 scales on a block-diagonal activation operand, giving exact
//    per-16-block partial dot products that the VALU scales by both E4M3
//    block scales), or on the VALU (the activation decoded once into LDS as
//    f16 x~ = e2m1(code) * e4m3(scale), exact, then v_dot2 per block);
//  * an item's partial sums are left per wave in LDS and summed in fixed
//    wave order (the same result on every run) once per batch of items, then
//    scaled by both tensor scales and written as binary32 or bf16; with
//    several K slices they go through the workspace instead, and the last
//    slice of a tile to arrive sums the slices in slice order.
#pragma once

#include <algorithm>
#include <type_traits>

#include "gemv_common.hpp"

namespace nvfp4 {

namespace {

using namespace gemv;

// Quantized activation blocks per thread loaded ahead of the weight loads:
// 4, or 8 at four or more rows (whose shallower ring leaves registers free)
// when 4 do not cover the activation; larger activations are staged whole
// before the weight loads.  The count is a kernel variant so that the loads
// issued are exactly the ones needed.
// The same counts give the bf16 blocks per thread of a prologue that
// quantizes the activation (8 only at four or more rows).
constexpr int kXptSmall = 4, kXptLarge = 8;

// Waves per workgroup the kernel is compiled for: 8 (<= 256 VGPRs).  Even
// one activation row does not fit the 128 VGPRs of 16 waves without
// spilling (26 VGPRs spilled to scratch at M = 1), and the plan runs 8 waves
// anyway.  Four or more rows use the split kernel (the streaming one would
// spill).
constexpr int kStreamMaxM = 3;
constexpr int stream_max_waves(int) { return 8; }

// Groups of 4 weight records (4 KiB) each wave keeps in flight.
constexpr int stream_ring_groups(int M) { return M == 3 ? 2 : 3; }

// The MFMA variant keeps 16 result registers per chunk but decodes nothing;
// its ring has a spare slot (3 groups in flight while it computes; 2 for four
// or more rows), which needs the 256-register budget of 8 waves.  The depth is
// kept low on purpose: the memory system serves the whole grid's requests
// together, so every request waits behind all the data already in flight
// (about 6.5 TB/s drains 10 MB per 1.5 us).  At four or more rows the grid
// runs 8 waves per CU, and 4 groups per wave (38 MB in flight) made every
// exposed wait, the activation's included, about 6 us long; 2 groups (19 MB)
// measured faster on every Qwen3 8B / 32B projection at M = 4 and 8.
constexpr int mfma_max_waves(int) { return 8; }
constexpr int mfma_ring_groups(int M) { return M >= 4 ? 2 : 3; }

// The grid holds at most one workgroup per CU.  The hardware dispatcher
// packs workgroups onto a CU while its registers and LDS last, so every
// workgroup reserves more than half of the CU's 160 KiB LDS: then no CU can
// hold two and the min(tiles, 256) workgroups spread over distinct CUs.
constexpr size_t kStreamLdsReserve = 80 * 1024 + 1024;

template <int V>
using ic = std::integral_constant<int, V>;

// f(ic<0>), f(ic<1>), ..., f(ic<N - 1>), unrolled at compile time
template <int I, int N>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    if constexpr (I < N) {
      f(ic<I>{});
      StaticFor<I + 1, N>::run(f);
    }
  }
};
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  StaticFor<0, N>::run(f);
}

// Row of flat block index i (0 <= i < M * per_row) of an M-row activation:
// i / per_row by M - 1 comparisons (a runtime integer division costs about
// 20 VALU instructions, and the prologue needs several per thread).
template <int M>
__device__ __forceinline__ int row_of(int i, int per_row) {
  int m = 0;
#pragma unroll
  for (int j = 1; j < M; ++j) m += i >= j * per_row ? 1 : 0;
  return m;
}

// Split-K tail of the streaming kernels, after the workgroup's last item:
// wait until its partial sums are stored, count each of its items in at its
// row tile's arrival counter (thread j takes item j, so the atomics overlap),
// and for every tile where this workgroup arrived last, sum the slices in
// slice order (the result does not depend on arrival order), scale, store,
// and put the counter back to zero for the next call.  At most batch * NW *
// M * 32 items per workgroup (the flags reuse the reduction slots).
template <int M>
__device__ __forceinline__ void split_tail(const GemvArgs& a, int nitem, float g, float* red) {
  const int S = a.splits, G = gridDim.x;
  uint32_t* flag = reinterpret_cast<uint32_t*>(red);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int nt = 64 * a.waves;
  for (int j = threadIdx.x; j < nitem; j += nt) {
    const int tile = ((int)blockIdx.x + j * G) / S;
    const uint32_t old =
        __hip_atomic_fetch_add(a.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag[j] = old == (uint32_t)(S - 1);
  }
  __syncthreads();
  // every (item, row, column) of the items this workgroup completes at once
  for (int i = threadIdx.x; i < nitem * M * 32; i += nt) {
    const int j = i / (M * 32), mn = i - j * (M * 32);
    if (!flag[j]) continue;
    const int m = mn >> 5, n = mn & 31;
    const int n0 = ((int)blockIdx.x + j * G) / S * kTileN;
    const float* pp = a.part + (int64_t)m * a.n_pad + n0 + n;
    const int64_t st = (int64_t)M * a.n_pad;
    // the slices' partials in slice order, loaded 8 at a time (all in flight
    // together: a sum over dependent loads would wait for each in turn)
    float v = 0.0f;
    for (int t0 = 0; t0 < S; t0 += 8) {
      float pv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        pv[k] = t0 + k < S ? __hip_atomic_load(pp + (t0 + k) * st, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + k < S) v += pv[k];
    }
    if (n0 + n < a.N) store_y(a, m, n0 + n, v * g);
  }
  for (int j = threadIdx.x; j < nitem; j += nt) {
    if (flag[j]) {
      const int tile = ((int)blockIdx.x + j * G) / S;
      __hip_atomic_store(a.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// One workgroup's whole job.  Every wave keeps RG groups of 4 weight records
// in flight.  The numbers of groups the stream starts with and ends with are
// compile-time constants on every path (the paths never merge), so the
// compiler's memory wait counts stay exact: where paths with different
// numbers of outstanding loads merge, it waits for all of them.
// QA: 0 = the activation arrives quantized; 1 = the prologue quantizes the
// bf16 activation; 2 = it applies the unweighted per-row RMS norm first;
// 3 = it quantizes a binary32 activation (with a.qslice, split K: only this
// workgroup's K slice, the tensor maximum taken from a.amax_in).
// SILU: the gate_up projection (its weight's rows interleaved in groups of
// 16) with SiLU * mul applied in the flush.
template <int M, int RG, int XS, bool MF, bool SPLIT, int QA, bool H16, int XPT = kXptSmall,
          bool SILU = false>
__device__ __forceinline__ void stream_body(const GemvArgs& a, uint32_t* lds) {
  static_assert(!H16 || (MF && !SPLIT), "half tiles: MFMA kernel, one K slice");
  static_assert(!SILU || (MF && !SPLIT && !H16), "SiLU * mul: MFMA kernel, whole tiles, one slice");
  static_assert(QA != 3 || MF, "binary32 activation: MFMA kernel");
  constexpr int GC = H16 ? 8 : 4;             // chunks per ring group
  constexpr int HS = H16 ? 2 : 1;             // items per row tile (16-row halves)
  constexpr int ROWS = kTileN / HS;           // output rows per item
  const int NW = a.waves;                     // = blockDim.x / 64 (not read from the
                                              // dispatch packet: that load would
                                              // delay every other one)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const bool nt = a.nontemporal != 0;
  const int kc = a.kc;
  const int row_dw = kc * 32;
  // MFMA: dwords per activation row of codes, padded by 8 so that the 8
  // rows' A-operand reads of one chunk fall in different LDS banks
  const int xs_row = kc * 8 + 8;
  // VALU: x~ as f16 pairs [M][kc * 32 dwords].  MFMA: raw activation codes
  // [M][kc * 4 blocks][2 dwords] (rows xs_row dwords apart), then the E4M3
  // activation scales as f16
  // (every E4M3 value is an f16 value) [kc * 4 blocks][M], padded to a
  // dword.  Either is followed by the reduction slots [batch][NW][M][ROWS]
  // floats.
  uint32_t* xlds = lds;
  _Float16* sa = reinterpret_cast<_Float16*>(lds + M * xs_row);
  float* red = reinterpret_cast<float*>(MF ? lds + M * xs_row + (kc * 4 * M + 1) / 2
                                           : lds + M * row_dw);
  const int kb_row = a.K >> 4;
  const int nblk = M * kc * 4;                // activation 16-blocks, padded K
  const int cpw = a.cpw;                      // chunks per wave per item, multiple of GC

  const int S = SPLIT ? a.splits : 1;         // K slices per row tile
  const int G = gridDim.x;
  const int nitem = (a.tiles * HS * S - (int)blockIdx.x + G - 1) / G;
  const int ng = nitem * (cpw / GC);          // ring groups in this wave's stream
  // Work item i = (row tile i / S, K slice i % S).  The slice's chunks go
  // to the waves in groups of 4 (one scale record), round robin: this wave
  // owns chunks cb + NW * 4j + k (j < cpw / 4, k < 4, cb = slice * cps + 4 *
  // wave), so at any time the workgroup's waves read adjacent records.  A
  // group past K (last slice only) re-reads the tile's last group, with its
  // scales zeroed.
  // Half tiles (H16): item i is rows 16 (i % 2) .. + 15 of tile i / 2, on
  // the 16x16x128 MFMA; groups are then 8 chunks (two scale records).
  struct Item {
    int tile, slice, half, cb;
  };
  auto item = [&](int i) __attribute__((always_inline)) {
    Item it;
    int th;
    if constexpr (SPLIT) {
      th = i / S;
      it.slice = i - th * S;
    } else {
      th = i;
      it.slice = 0;
    }
    if constexpr (H16) {
      it.tile = th >> 1;
      it.half = th & 1;
    } else {
      it.tile = th;
      it.half = 0;
    }
    it.cb = it.slice * a.cps + GC * wave;
    return it;
  };

  // ---- 1. this wave's records form one stream: its cpw chunks of the
  // workgroup's first item, then of its second item, ...
  const uint8_t* wbase = a.wc + 16 * lane;
  const uint8_t* sbase = a.ws + 8 * lane;
  int li = blockIdx.x, loff = 0;              // load cursor: item, chunk offset
  Item lit = item(li);
  u32x4 ring[RG + XS][4];
  u32x2 rsc[RG + XS];
  u32x2 rsc2[H16 ? RG + XS : 1];              // H16: the group's second scale record
  auto refill = [&](auto Q) __attribute__((always_inline)) {
    constexpr int q = decltype(Q)::value;
    if constexpr (H16) {
      // load k of the group: rows 16 half .. + 15 of chunks cg + 2k, cg + 2k + 1;
      // lane l takes row l % 16 of chunk cg + 2k + l / 32, K half (l / 16) % 2,
      // i.e. in-record lane L of that record (one 16x16x128 MFMA operand)
      const int L = (lane & 15) + 16 * lit.half + 32 * ((lane >> 4) & 1);
      const int cg = lit.cb + loff * NW;
      const int64_t t0 = (int64_t)lit.tile * kc;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = min(cg + 2 * k + (lane >> 5), kc - 1);
        ring[q][k] = load_codes(a.wc + (t0 + c) * kCodeRecord + 16 * L, nt);
      }
      const int64_t g0 = (int64_t)lit.tile * (kc >> 2);
      rsc[q] = load_scales(a.ws + (g0 + min(cg >> 2, (kc >> 2) - 1)) * kScaleRecord + 8 * L, nt);
      rsc2[q] = load_scales(a.ws + (g0 + min((cg >> 2) + 1, (kc >> 2) - 1)) * kScaleRecord + 8 * L,
                            nt);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t r = (int64_t)lit.tile * kc + min(lit.cb + loff * NW + k, kc - 4 + k);
        if (k == 0) rsc[q] = load_scales(sbase + (r >> 2) * kScaleRecord, nt);
        ring[q][k] = load_codes(wbase + r * kCodeRecord, nt);
      }
    }
    loff += GC;
    if (loff == cpw) {
      loff = 0;
      li += G;
      lit = item(li);
    }
  };

  // ---- 2. activation into LDS.  The memory counter that the waits use
  // counts loads in issue order, so a wait for an activation load also waits
  // for every weight load issued before it; all the prologue's loads are
  // therefore issued before the first weight load, in a fixed number (no
  // branch between them and the weight loads), and the waits for them leave
  // the weight loads in flight.  The tensor scales are read at the start,
  // before the weight loads queue up: a scalar load still outstanding holds
  // up every later LDS wait, which shares its counter.  An activation too
  // large for one batch per thread is staged whole before any weight load is
  // issued.
  const float wg_v = a.wg[0];
  const float xg_v = QA ? 0.0f : a.xg[0];
  const float sgs_v = QA && a.sgs ? a.sgs[0] : 0.0f;
  float g = 0.0f;                             // the binary32 product of both tensor scales
  // QA: this thread's activation blocks (bf16 pairs, or binary32 with QA 3)
  uint32_t qv[QA ? XPT : 1][QA == 3 ? 16 : 8];
  u32x2 xc0[QA ? 1 : XPT];                    // else: its first quantized activation blocks
  uint32_t xs0[QA ? 1 : XPT];
  uint32_t rec = 0;                           // QA 3: this thread's share of a.amax_in
  static_assert(QA >= 0 && QA <= 3, "activation prologue mode");
  // the blocks the prologue quantizes: [kb0, kb0 + kbn) of every row (the
  // whole row, or with a.qslice this workgroup's K slice: all its items have
  // slice blockIdx.x % S, the grid being a multiple of S)
  const bool qslice = SPLIT && QA == 3 && a.qslice != 0;
  const int kb0 = qslice ? 4 * ((int)blockIdx.x % S) * a.cps : 0;
  const int kbn = qslice ? min(4 * a.cps, kb_row - kb0) : kb_row;
  auto put = [&](int m, int kb, u32x2 c, uint32_t sc) __attribute__((always_inline)) {
    if constexpr (MF) {
      xlds[m * xs_row + kb * 2] = c.x;
      xlds[m * xs_row + kb * 2 + 1] = c.y;
      sa[kb * M + m] = (_Float16)e4m3_to_f32(sc);
    } else {
      decode_act_block(c, sc, xlds + m * row_dw + kb * 8);
    }
  };
  // QA: the activation quantizer inside the prologue.  Every workgroup reads
  // the whole bf16 activation (at most XPT blocks per thread, all loads in
  // flight together), takes the exact tensor maximum (bf16 magnitudes as
  // integers: workgroup, then wave, then LDS), and quantizes every block with
  // the quantizer's own arithmetic straight into its LDS staging; workgroup 0
  // also writes the canonical codes, scales and tensor scale, bit-identical
  // to the standalone activation quantizer's.
  // (the bf16 loads are issued before the first weight loads, so waiting for
  // them does not wait for the weights)
  // QA == 3: the activation is binary32 (the SiLU * mul output of the
  // gate_up GEMV).  With its producer's record of per-workgroup maxima the
  // tensor maximum comes from the record (the same value), and with slices
  // a workgroup quantizes only the blocks of its own K slice.
  // QA == 2: h = x * (1 / sqrt(mean_k x^2 + eps)) per row in binary32 (the
  // row sums in a fixed order: per thread its blocks in order, then the wave
  // tree, then the waves in order, the same in every workgroup), then the
  // quantizer on h; h is recomputed from the bf16 registers when needed, and
  // workgroup 0 can write it out.
  auto quantize_prologue = [&]() __attribute__((always_inline)) {
    const int T = 64 * NW;
    const int nreal = M * kbn;
    auto& v = qv;
    uint32_t* wred = reinterpret_cast<uint32_t*>(red);
    // the rows' 1 / rms in LDS (a register array indexed by row would be
    // placed in scratch)
    float* rinv = reinterpret_cast<float*>(red) + NW * M;
    auto row_rinv = [&](int m) __attribute__((always_inline)) { return rinv[m]; };
    auto block_h = [&](int r, float rv, float (&hb)[16]) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hb[2 * e] = __fmul_rn(__uint_as_float(v[r][e] << 16), rv);
        hb[2 * e + 1] = __fmul_rn(__uint_as_float(v[r][e] & 0xFFFF0000u), rv);
      }
    };
    if constexpr (QA == 2) {
      float ss[M];
#pragma unroll
      for (int m = 0; m < M; ++m) ss[m] = 0.0f;
#pragma unroll
      for (int r = 0; r < XPT; ++r) {
        if (r > 0 && nreal <= r * T) break;           // uniform: no block r here
        const int i = (int)threadIdx.x + r * T;
        const int mr = i < nreal ? row_of<M>(i, kbn) : M;   // M: no row
        float bs = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x0 = __uint_as_float(v[r][e] << 16);
          const float x1 = __uint_as_float(v[r][e] & 0xFFFF0000u);
          bs = __fadd_rn(bs, __fmul_rn(x0, x0));
          bs = __fadd_rn(bs, __fmul_rn(x1, x1));
        }
#pragma unroll
        for (int m = 0; m < M; ++m) ss[m] = m == mr ? __fadd_rn(ss[m], bs) : ss[m];
      }
      float* wss = reinterpret_cast<float*>(red);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float w = wave_sum_f32(ss[m]);
        if (lane == 0) wss[wave * M + m] = w;
      }
      __syncthreads();
      if ((int)threadIdx.x < M) {
        const int m = threadIdx.x;
        float t = wss[m];
        for (int w = 1; w < NW; ++w) t = __fadd_rn(t, wss[w * M + m]);
        const float ms = __fdiv_rn(t, (float)a.K);
        rinv[m] = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(ms, a.eps)));
      }
      __syncthreads();                                  // wss is reused below
    }
    uint32_t amax = 0;
    uint32_t bmx[XPT];                    // each block's largest magnitude, reused below
#pragma unroll
    for (int r = 0; r < XPT; ++r) {
      if (r > 0 && nreal <= r * T) break;             // uniform: no block r here
      const int i = (int)threadIdx.x + r * T;
      uint32_t b;
      if constexpr (QA == 2) {
        float hb[16];
        block_h(r, row_rinv(i < nreal ? row_of<M>(i, kbn) : 0), hb);
        b = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) b = max(b, __float_as_uint(hb[e]) & 0x7FFFFFFFu);
      } else if constexpr (QA == 3) {
        b = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) b = max(b, v[r][e] & 0x7FFFFFFFu);
      } else {
        b = absmax_bits(v[r]);
      }
      bmx[r] = b;
      amax = max(amax, i < nreal ? b : 0u);
    }
    float sg;
    if (a.sgs) {                                      // uniform: a static tensor scale
      sg = sgs_v;
    } else {
      if (QA == 3 && a.amax_in) amax = rec;           // uniform: the producer's maxima
      amax = wave_max_u32(amax);
      if (lane == 0) wred[wave] = amax;
      __syncthreads();
      amax = 0;
      for (int w = 0; w < NW; ++w) amax = max(amax, wred[w]);
      sg = tensor_scale(QA >= 2 ? __uint_as_float(amax) : bf16_to_f32(amax));
    }
    g = __fmul_rn(sg, wg_v);
    // the canonical codes: workgroup 0, or with slices workgroup s < S (slice s)
    const bool out = qslice ? (int)blockIdx.x < S : blockIdx.x == 0;
#pragma unroll
    for (int r = 0; r < XPT; ++r) {
      const int i = (int)threadIdx.x + r * T;
      if (i < nreal) {
        const int m = row_of<M>(i, kbn), kb = kb0 + i - m * kbn;
        BlockQ q;
        if constexpr (QA == 2) {
          float hb[16];
          block_h(r, row_rinv(m), hb);
          q = quantize_block_f32(hb, __uint_as_float(bmx[r]), sg);
          if (out && a.ho) {
            float4* o = reinterpret_cast<float4*>(a.ho + (int64_t)m * a.K + 16 * kb);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o[e] = make_float4(hb[4 * e], hb[4 * e + 1], hb[4 * e + 2], hb[4 * e + 3]);
          }
        } else if constexpr (QA == 3) {
          float hb[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) hb[e] = __uint_as_float(v[r][e]);
          q = quantize_block_f32(hb, __uint_as_float(bmx[r]), sg);
        } else {
          q = quantize_block_bf16(v[r], bmx[r], sg);
        }
        put(m, kb, u32x2{q.lo, q.hi}, q.scale);
        if (out) {
          *reinterpret_cast<u32x2*>(a.oc + (int64_t)m * (a.K >> 1) + 8 * kb) = u32x2{q.lo, q.hi};
          a.os[(int64_t)m * kb_row + kb] = (uint8_t)q.scale;
        }
      }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && !a.sgs) *a.og = sg;
    const int npad = kc * 4 - kb_row;                 // zero blocks up to the padded K
    for (int i = threadIdx.x; i < M * npad; i += T) {
      const int m = i / npad;
      put(m, kb_row + (i - m * npad), u32x2{0u, 0u}, 0u);
    }
    __syncthreads();
  };
  // QA = 0, an activation larger than the first batch: every block staged
  // before the weight loads are issued (the ring's registers are not live
  // yet), in batches of B blocks per thread with all of a batch's loads in
  // flight together: one batch up to 16 blocks per thread (8192 blocks with
  // 512 threads), else batches of 32.  (Staging after the ring's first
  // weight loads instead measured slower: Qwen3-8B down at M = 8 14.6 ->
  // 16.2 us.)
  const bool stage_first = !QA && nblk > XPT * 64 * NW;
  auto stage_batches = [&](auto BB) __attribute__((always_inline)) {
    constexpr int B = decltype(BB)::value;
    for (int base = threadIdx.x; base < nblk; base += B * 64 * NW) {
      u32x2 c[B];
      uint32_t sc[B];
#pragma unroll
      for (int r = 0; r < B; ++r) {
        const int i = min(base + r * 64 * NW, nblk - 1);
        const int m = row_of<M>(i, kc * 4), kb = i - m * (kc * 4);
        const int kbc = min(kb, kb_row - 1);
        c[r] = *reinterpret_cast<const u32x2*>(a.xc + (int64_t)m * (a.K >> 1) + 8 * kbc);
        sc[r] = a.xs[(int64_t)m * kb_row + kbc];
      }
      // keeps the batch's loads above its (conditional) LDS stores: sunk to
      // their uses they would go out one round trip at a time
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < B; ++r) {
        const int i = base + r * 64 * NW;
        if (i < nblk) {
          const int m = row_of<M>(i, kc * 4), kb = i - m * (kc * 4);
          const bool ok = kb < kb_row;
          put(m, kb, ok ? c[r] : u32x2{0u, 0u}, ok ? sc[r] : 0u);
        }
      }
    }
  };
  auto stage_all = [&]() __attribute__((always_inline)) {
    if (nblk <= 16 * 64 * NW) stage_batches(ic<16>{});
    else stage_batches(ic<32>{});
  };
  auto prologue = [&]() __attribute__((always_inline)) {
    if constexpr (QA) {
      quantize_prologue();
      return;
    }
    g = __fmul_rn(xg_v, wg_v);
    if (!stage_first) {                               // uniform
#pragma unroll
      for (int r = 0; r < XPT; ++r) {
        const int i = threadIdx.x + r * 64 * NW;
        if (i < nblk) {
          const int m = row_of<M>(i, kc * 4), kb = i - m * (kc * 4);
          const bool ok = kb < kb_row;
          put(m, kb, ok ? xc0[r] : u32x2{0u, 0u}, ok ? xs0[r] : 0u);
        }
      }
    }
    __syncthreads();
  };

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  // Item-boundary reduction.  The K halves meet at once (lanes l, l ^ 32);
  // each wave then leaves its partial sum of the item in its own LDS slot
  // [item in batch][wave][M][32] and streams on without waiting for the
  // other waves.  After `batch` items (normally all of the workgroup's), one
  // barrier, then the waves' partials are summed in fixed wave order (the
  // result is the same on every run) and stored: as the output with one K
  // slice, else as the slice's partial sum (device-coherent, combined after
  // the stream), then a barrier before the slots are reused.
  // SILU: the weight's row tiles interleave the gate and up projections in
  // groups of 16 (tile t: rows 0..15 gate columns 16t.., rows 16..31 up of
  // the same columns), so each item holds both factors of its 16 columns.
  // The flush sums both rows the same way, rounds them to bf16 as the
  // projection's bf16 output would be, and stores h = silu(gate) * up
  // (binary32) at column 16t + r.
  int ci = blockIdx.x, jb = 0, done = 0, batch_first = blockIdx.x;
  uint32_t hmax = 0;                          // SILU: this thread's largest |h|
  Item cit = item(ci);
  auto flush = [&](bool last) __attribute__((always_inline)) {
    __syncthreads();
    if constexpr (SILU) {
      constexpr int HALF = kTileN / 2;
      for (int i = threadIdx.x; i < jb * M * HALF; i += 64 * NW) {
        const int j = i / (M * HALF), mr = i - j * (M * HALF);
        const int m = mr / HALF, r = mr - m * HALF;
        const float* sgt = red + j * (NW * M * ROWS) + m * ROWS + r;
        const float* sup = sgt + HALF;
        float vg = sgt[0], vu = sup[0];
        for (int q = 1; q < NW; ++q) {
          vg += sgt[q * M * ROWS];
          vu += sup[q * M * ROWS];
        }
        const Item it = item(batch_first + j * G);
        const int n = it.tile * HALF + r;               // the h column (< F)
        const uint16_t bg = f32_to_bf16_rne(vg * g), bu = f32_to_bf16_rne(vu * g);
        if (a.gu) {                                     // [M][2F]: gate, then up columns
          a.gu[(int64_t)m * a.N + n] = bg;
          a.gu[(int64_t)m * a.N + (a.N >> 1) + n] = bu;
        }
        const float hv = silu_mul(bf16_to_f32(bg), bf16_to_f32(bu));
        reinterpret_cast<float*>(a.y)[(int64_t)m * a.ldh + n] = hv;
        hmax = max(hmax, __float_as_uint(hv) & 0x7FFFFFFFu);
      }
      if (!last) __syncthreads();
      jb = 0;
      return;
    }
    for (int i = threadIdx.x; i < jb * M * ROWS; i += 64 * NW) {
      const int j = i / (M * ROWS), mn = i - j * (M * ROWS);
      const float* sl = red + j * (NW * M * ROWS) + mn;
      float v = sl[0];
      for (int q = 1; q < NW; ++q) v += sl[q * M * ROWS];
      const Item it = item(batch_first + j * G);
      const int m = mn / ROWS, n = it.tile * kTileN + it.half * ROWS + (mn % ROWS);
      if constexpr (SPLIT) {
        __hip_atomic_store(a.part + ((int64_t)it.slice * M + m) * a.n_pad + n, v,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        if (n < a.N) store_y(a, m, n, v * g);
      }
    }
    if (!last) __syncthreads();               // the slots are reused by the next batch
    jb = 0;
  };
  auto finish_tile = [&]() __attribute__((always_inline)) {
    float* sl = red + jb * (NW * M * ROWS) + wave * (M * ROWS);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if constexpr (H16) acc[m] += __shfl_xor(acc[m], 16, 64);     // the 4 K groups of a row
      acc[m] += __shfl_xor(acc[m], 32, 64);
      if (lane < ROWS) sl[m * ROWS + lane] = acc[m];
      acc[m] = 0.0f;
    }
    ++jb;
    ++done;
    ci += G;
    cit = item(ci);
    if (jb == a.batch || done == nitem) {
      flush(done == nitem);
      batch_first = ci;
    }
  };

  // Consume ring group q: chunks cb + NW * coff + 0..3 of the current item.
  // Branch free (wait counts stay exact): a chunk past K reads a valid
  // activation chunk and gets a zero block scale, so it adds exactly 0.
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
  const uint32_t* xa_row = xlds + (ma < M ? ma : 0) * xs_row + ja * 2;

  // H16 A operand (16 x 128, two chunks): lane l holds row r = l % 16, K
  // group l / 16 (32 elements = blocks 2 (l / 16), + 1 of the pair).  Row r
  // is activation row 2 mp + (r / 2) % 2 and block 2 (r / 4) + r % 2 of the
  // pair, so that result v of lane l (row 4 (l / 16) + v) is (row 2 mp + v /
  // 2, block 2 (l / 16) + v % 2): the lane's own weight row and blocks.
  const int kgl = lane >> 4;                  // H16: this lane's K group
  const int r16 = lane & 15;
  const bool a16_on = kgl == (r16 >> 2);
  const int a16_c = (r16 >> 2) >> 1;          // chunk of the row's block within the pair
  const int a16_b = 2 * ((r16 >> 2) & 1) + (r16 & 1);   // its block within that chunk
  const int a16_m = (r16 >> 1) & 1;           // + 2 mp: its activation row

  int coff = 0;
  auto consume16 = [&](auto Q) __attribute__((always_inline)) {
    constexpr int q = decltype(Q)::value;
    const int cg = cit.cb + coff * NW;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = cg + 2 * k + (lane >> 5);           // this lane's chunk
      const int q4 = (2 * k + (lane >> 5)) & 3;         // its place in the scale record
      const u32x2 rec = k < 2 ? rsc[q] : rsc2[q];
      uint32_t sb = (q4 < 2 ? rec.x : rec.y) >> (16 * (q4 & 1));
      sb = c < kc ? sb : 0u;
      const int cx = min(c, kc - 1);
      const int ca = min(cg + 2 * k + a16_c, kc - 1);   // the A row's chunk
      const u32x4 wv = ring[q][k];
      const v8i B = {(int)wv.x, (int)wv.y, (int)wv.z, (int)wv.w, 0, 0, 0, 0};
      const float sw0 = __builtin_amdgcn_cvt_f32_fp8(sb, 0);
      const float sw1 = __builtin_amdgcn_cvt_f32_fp8(sb, 1);
      const _Float16* sap = sa + (4 * cx + 2 * (kgl & 1)) * M;   // [block][m]
#pragma unroll
      for (int mp = 0; mp < (M + 1) / 2; ++mp) {
        const int ma = 2 * mp + a16_m;
        const bool on = a16_on && ma < M;
        const uint32_t* xp = xlds + (ma < M ? ma : 0) * xs_row + (ca * 4 + a16_b) * 2;
        const uint32_t a0 = xp[0], a1 = xp[1];
        const bool lo = on && (r16 & 1) == 0, hi = on && (r16 & 1) != 0;
        const v8i Aop = {(int)(lo ? a0 : 0u), (int)(lo ? a1 : 0u), (int)(hi ? a0 : 0u),
                         (int)(hi ? a1 : 0u), 0, 0, 0, 0};
        const v4f C = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aop, B, v4f{}, 4, 4, 0, 127,
                                                                       0, 127);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 2 * mp + (v >> 1), b = v & 1;
          if (m < M) acc[m] = fmaf(C[v], fmaf((float)sap[b * M + m], b ? sw1 : sw0, 0.0f), acc[m]);
        }
      }
    }
    coff += GC;
    if (coff == cpw) {
      finish_tile();
      coff = 0;
    }
  };
  auto consume = [&](auto Q) __attribute__((always_inline)) {
    if constexpr (H16) {
      consume16(Q);
      return;
    }
    constexpr int q = decltype(Q)::value;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = cit.cb + coff * NW + k;
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
        const _Float16* sap = sa + (4 * cx + 2 * h) * M;       // [block 2h + b][m]
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 2 * (v >> 2) + ((v & 3) >> 1), b = v & 1;
          if constexpr (true) {
            if (m < M) acc[m] = fmaf(C[v], fmaf((float)sap[b * M + m], b ? sw1 : sw0, 0.0f), acc[m]);
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

  // The stream.  Group g of the wave's stream lives in slot g % SL; A = RG
  // groups are loaded ahead.  With a spare slot (SL = A + 1) each step first
  // issues the load of the group A ahead into the slot consumed by the
  // previous step, then consumes its own group, so A groups stay in flight
  // while the wave computes; without one (SL = A) it consumes, then reuses
  // the slot.  The numbers of groups loaded and consumed on every path are
  // compile-time constants, so the memory wait counts stay exact.
  constexpr int A = RG, SL = RG + XS;
  auto step = [&](auto T) __attribute__((always_inline)) {    // position t of SL
    constexpr int t = decltype(T)::value;
    if constexpr (SL > A) {
      refill(ic<(t + A) % SL>{});
      consume(ic<t % SL>{});
    } else {
      consume(ic<t % SL>{});
      refill(ic<t % SL>{});
    }
  };
  // last A + x groups, x of them still to load
  auto tail = [&](auto X) __attribute__((always_inline)) {
    constexpr int x = decltype(X)::value;
    static_for<A + x>([&](auto T) __attribute__((always_inline)) {
      constexpr int t = decltype(T)::value;
      if constexpr (t < x) step(ic<t>{}); else consume(ic<t % SL>{});
    });
  };
  // fewer than A groups in all: load them, then consume them
  auto short_stream = [&](auto NG) __attribute__((always_inline)) {
    constexpr int n = decltype(NG)::value;
    static_for<n>([&](auto T) __attribute__((always_inline)) { refill(T); });
    prologue();
    static_for<n>([&](auto T) __attribute__((always_inline)) { consume(T); });
  };

  static_assert(A >= 2 && A <= 4 && SL <= 5, "ring of 2 to 5 slots");
  // The activation loads: a fixed number per thread (addresses clamped into
  // range, so blocks past the activation reload its last block; such blocks
  // are skipped or zeroed at use), all before the first weight load.
  if constexpr (QA) {
    const int T = 64 * NW;
    const int nreal = M * kbn;
#pragma unroll
    for (int r = 0; r < XPT; ++r) {
      const int i = min((int)threadIdx.x + r * T, nreal - 1);
      const int m = row_of<M>(i, kbn), kb = kb0 + i - m * kbn;
      if constexpr (QA == 3) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.xf + (int64_t)m * a.ldx + 16 * kb);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u32x4 t = src[e];
          qv[r][4 * e] = t.x;
          qv[r][4 * e + 1] = t.y;
          qv[r][4 * e + 2] = t.z;
          qv[r][4 * e + 3] = t.w;
        }
      } else {
        load_block_bf16(a.xb + (int64_t)m * a.ldx + 16 * kb, qv[r]);
      }
    }
    if constexpr (QA == 3) {
      // the maxima record, 4 slots per lane (every wave reads all 256); the
      // same number of loads with no record (then from a valid dummy word)
      const bool hr = a.amax_in != nullptr;
      const uint32_t* rp = hr ? a.amax_in + lane : reinterpret_cast<const uint32_t*>(a.wg);
      uint32_t rv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) rv[k] = rp[hr ? 64 * k : 0];
      rec = hr ? max(max(rv[0], rv[1]), max(rv[2], rv[3])) : 0u;
    }
    __asm__ volatile("" ::: "memory");      // issued before the weight loads, not sunk
  } else {
    if (stage_first) {                                // uniform
      stage_all();
    } else {
#pragma unroll
      for (int r = 0; r < XPT; ++r) {
        const int i = min((int)threadIdx.x + r * 64 * NW, nblk - 1);
        const int m = row_of<M>(i, kc * 4), kb = min(i - m * (kc * 4), kb_row - 1);
        xc0[r] = *reinterpret_cast<const u32x2*>(a.xc + (int64_t)m * (a.K >> 1) + 8 * kb);
        xs0[r] = a.xs[(int64_t)m * kb_row + kb];
      }
      __asm__ volatile("" ::: "memory");    // issued before the weight loads, not sunk
    }
  }
  if (ng >= A) {
    static_for<A>([&](auto T) __attribute__((always_inline)) { refill(T); });
    prologue();
    int gi = 0;
    for (; gi + SL + A <= ng; gi += SL) static_for<SL>(step);
    switch (ng - gi - A) {                    // 0 .. SL - 1 groups still to load
      case 0: tail(ic<0>{}); break;
      case 1: tail(ic<1>{}); break;
      case 2: if constexpr (SL > 2) tail(ic<(SL > 2 ? 2 : 0)>{}); break;
      case 3: if constexpr (SL > 3) tail(ic<(SL > 3 ? 3 : 0)>{}); break;
      default: if constexpr (SL > 4) tail(ic<(SL > 4 ? 4 : 0)>{}); break;
    }
  } else {
    switch (ng) {                             // 1 .. A - 1
      case 1: short_stream(ic<1>{}); break;
      case 2: if constexpr (A > 2) short_stream(ic<(A > 2 ? 2 : 1)>{}); break;
      default: if constexpr (A > 3) short_stream(ic<(A > 3 ? 3 : 1)>{}); break;
    }
  }
  if constexpr (SPLIT) split_tail<M>(a, nitem, g, red);
  if constexpr (SILU) {
    // the record: this workgroup's largest |h| in its slot, zeros past the grid
    uint32_t* wm = reinterpret_cast<uint32_t*>(red);
    const uint32_t w = wave_max_u32(hmax);
    __syncthreads();                          // the last flush has read the slots
    if (lane == 0) wm[wave] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t t = 0;
      for (int q = 0; q < NW; ++q) t = max(t, wm[q]);
      a.amax_out[blockIdx.x] = t;
    }
    if (blockIdx.x == 0)
      for (int i = G + (int)threadIdx.x; i < kAmaxSlots; i += 64 * NW) a.amax_out[i] = 0u;
  }
}

// Launch: blockDim.x = 64 * a.waves (at most stream_max_waves(M) or
// mfma_max_waves(M)); dynamic LDS = the activation followed by the
// reduction slots (stream_lds_need), at least kStreamLdsReserve.
template <int M, bool SPLIT>
__global__ __launch_bounds__(64 * stream_max_waves(M)) void gemv_stream_kernel(GemvArgs a) {
  extern __shared__ uint32_t lds[];
  stream_body<M, stream_ring_groups(M), 0, false, SPLIT, 0, false>(a, lds);
}

template <int M, bool SPLIT, int QA, bool H16, int XPT, bool SILU>
__global__ __launch_bounds__(64 * mfma_max_waves(M)) void gemv_mfma_kernel(GemvArgs a) {
  extern __shared__ uint32_t lds[];
  stream_body<M, mfma_ring_groups(M), 1, true, SPLIT, QA, H16, XPT, SILU>(a, lds);
}

template <int M, bool MF, bool SPLIT, int QA, bool H16, int XPT = kXptSmall, bool SILU = false>
hipError_t launch_ms(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  const size_t need = stream_lds_need(M, p.kc, p.waves, MF, p.batch, H16 ? kTileN / 2 : kTileN);
  const size_t lds = need > kStreamLdsReserve || p.grid > 256 ? need : kStreamLdsReserve;
  const void* fn;
  if constexpr (MF)
    fn = reinterpret_cast<const void*>(&gemv_mfma_kernel<M, SPLIT, QA, H16, XPT, SILU>);
  else
    fn = reinterpret_cast<const void*>(&gemv_stream_kernel<M, SPLIT>);
  static hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  if constexpr (MF)
    hipLaunchKernelGGL((gemv_mfma_kernel<M, SPLIT, QA, H16, XPT, SILU>), dim3((unsigned)p.grid),
                       dim3(64 * p.waves), lds, s, a);
  else
    hipLaunchKernelGGL((gemv_stream_kernel<M, SPLIT>), dim3((unsigned)p.grid),
                       dim3(64 * p.waves), lds, s, a);
  return hipGetLastError();
}

// The MFMA kernels of one (split, half tiles, blocks per thread) shape for
// prologue mode qa (0: quantized, 1: bf16, 2: bf16 + RMS norm, 3: binary32)
// and epilogue (silu: SiLU * mul; whole tiles, one slice, qa <= 2 only).
template <int M, bool SPLIT, bool H16, int XPT>
hipError_t launch_mf(int qa, bool silu, const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  if (silu) {
    if constexpr (!SPLIT && !H16) {
      switch (qa) {
        case 0: return launch_ms<M, true, false, 0, false, XPT, true>(p, a, s);
        case 1: return launch_ms<M, true, false, 1, false, XPT, true>(p, a, s);
        case 2: return launch_ms<M, true, false, 2, false, XPT, true>(p, a, s);
        default: return hipErrorInvalidValue;
      }
    }
    return hipErrorInvalidValue;
  }
  switch (qa) {
    case 0: return launch_ms<M, true, SPLIT, 0, H16, XPT>(p, a, s);
    case 1: return launch_ms<M, true, SPLIT, 1, H16, XPT>(p, a, s);
    case 2: return launch_ms<M, true, SPLIT, 2, H16, XPT>(p, a, s);
    default:   // binary32 blocks take twice the registers: 4 per thread at most
      if constexpr (XPT == kXptSmall) return launch_ms<M, true, SPLIT, 3, H16, XPT>(p, a, s);
      return hipErrorInvalidValue;
  }
}

template <int M, bool MF>
hipError_t launch_m(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  if (p.waves < 1 || p.waves > (MF ? mfma_max_waves(M) : stream_max_waves(M)))
    return hipErrorInvalidValue;
  if constexpr (MF) {
    static_assert(kAmaxSlots == 256, "the record is read as 4 slots per lane");
    const int qa = a.xf ? 3 : a.xb ? (a.rms ? 2 : 1) : 0;
    const bool silu = a.amax_out != nullptr;
    const bool qslice = a.qslice != 0;
    if (p.h16 && (p.splits != 1 || p.cpw % 8)) return hipErrorInvalidValue;
    if (silu && (p.splits != 1 || p.h16 || qa == 3 || a.N % kTileN)) return hipErrorInvalidValue;
    if (qslice && (qa != 3 || p.splits < 2 || p.grid % p.splits || (!a.amax_in && !a.sgs)))
      return hipErrorInvalidValue;
    // blocks the prologue loads per thread: real blocks when it quantizes
    // (of one slice with qslice), blocks of the padded K when it stages a
    // quantized activation
    const int nb = qslice ? M * std::min(4 * p.cps, a.K >> 4)
                   : qa   ? M * (a.K >> 4)
                          : M * p.kc * 4;
    const int cap_s = kXptSmall * 64 * p.waves, cap_l = kXptLarge * 64 * p.waves;
    if (qa && nb > qa_max_blocks(M, p.waves, qa == 3)) return hipErrorInvalidValue;
    // a quantized activation past the large batch is staged whole first
    const bool large = M >= 4 && qa != 3 && nb > cap_s && !(qa == 0 && nb > cap_l);
    if constexpr (M >= 4) {
      if (large) {
        if (p.h16) return launch_mf<M, false, true, kXptLarge>(qa, silu, p, a, s);
        return p.splits > 1 ? launch_mf<M, true, false, kXptLarge>(qa, silu, p, a, s)
                            : launch_mf<M, false, false, kXptLarge>(qa, silu, p, a, s);
      }
    }
    if (p.h16) return launch_mf<M, false, true, kXptSmall>(qa, silu, p, a, s);
    return p.splits > 1 ? launch_mf<M, true, false, kXptSmall>(qa, silu, p, a, s)
                        : launch_mf<M, false, false, kXptSmall>(qa, silu, p, a, s);
  }
  if (a.xb || a.xf || a.amax_out) return hipErrorInvalidValue;   // the VALU dot: quantized input
  return p.splits > 1 ? launch_ms<M, MF, true, 0, false>(p, a, s)
                      : launch_ms<M, MF, false, 0, false>(p, a, s);
}

}  // namespace

// The launcher of the streaming kernels for M rows (mf: MFMA dot, else the
// VALU dot, M <= 3), defined in gemv_stream_m<M>.hip.
template <int M>
hipError_t launch_stream_rows(const GemvPlan& p, const GemvArgs& a, hipStream_t s, bool mf);

}  // namespace nvfp4
