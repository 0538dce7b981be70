// VALU GEMV / skinny GEMM for the small-M NVFP4 W4A4 decode linear (gfx950).
//
// The operation is the one of "ReSET" GitHub README, "Core components",
// item 2 (nvfp4r): at M <= 8 a matrix-core tile would be mostly empty, so
// the FP4 weights are streamed through the vector ALUs once and every loaded
// weight serves all M activation rows.  This is the gfx950 design of that
// idea, not a translation of the Blackwell kernel:
//
//  * weights come from the device-tiled layout (include/nvfp4.h), so each
//    64-lane load is one contiguous 1 KiB record (32 rows x 64 K) streamed
//    with non-temporal loads; lane l owns row l % 32 and K half l / 32;
//  * a workgroup handles one 32-row tile and one K slice.  Its prologue
//    decodes the slice of the M quantized activation rows into LDS as f16
//    x~ = e2m1(code) * e4m3(scale) (exact: at most 6 significant bits,
//    magnitudes in [2^-10, 2688]), which every wavefront then reads by
//    broadcast dword reads (the 32 lanes of one K half share an address);
//  * FP4 weights decode in registers with the gfx950 packed FP4 -> f16
//    conversion (scale operand 1.0), and v_dot2_f32_f16 sums each 16-block
//    exactly in binary32 (products <= 8 significant bits, one block's
//    products share one scale, so no partial sum rounds);
//  * each block partial p is folded in with one fma by the weight's E4M3
//    block scale: acc += p * S_w;
//  * the two K halves of a row meet with one cross-lane swap, the waves of a
//    workgroup through LDS, and the K slices (split-K) through a workspace
//    that the last-arriving workgroup of a tile sums in slice order (so the
//    result does not depend on arrival order), then scales by both tensor
//    scales and writes binary32 or bf16.
#include "gemv_common.hpp"

namespace nvfp4 {

namespace {

using namespace gemv;

// One workgroup = one 32-row tile x one K slice of CPW * NW chunks; wave w
// streams chunks [w * CPW, (w + 1) * CPW) of the slice.  Order of work:
//   1. issue this thread's activation-block loads (L2 hits),
//   2. issue every weight-record load of the wave (CPW x 1 KiB per wave, so
//      one HBM round trip covers the whole slice),
//   3. decode the activation slice into LDS once the (earlier) activation
//      loads land, barrier,
//   4. dot each chunk as its record arrives.
template <int M, int CPW, int NW>
__global__ __launch_bounds__(64 * NW) void gemv_split_kernel(GemvArgs a) {
  constexpr int CPS = CPW * NW;                      // chunks per slice
  constexpr int XBLK = M * CPS * 4;                  // activation 16-blocks per slice
  constexpr int XPT = (XBLK + 64 * NW - 1) / (64 * NW);
  constexpr int ROW_DW = CPS * 32;                   // LDS dwords per activation row
  extern __shared__ uint32_t xlds[];                 // [M][CPS * 64] f16
  __shared__ float red[NW][M][32];
  __shared__ int last_flag;

  const int tile = blockIdx.x / a.splits;
  const int s = blockIdx.x - tile * a.splits;
  const int c0 = s * CPS;
  const int cend = min(c0 + CPS, a.kc);
  const int kb_row = a.K >> 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const bool nt = a.nontemporal != 0;

  // ---- 1. activation blocks of this thread
  u32x2 xc[XPT];
  uint32_t xs[XPT];
#pragma unroll
  for (int r = 0; r < XPT; ++r) {
    const int i = threadIdx.x + r * 64 * NW;
    const int m = i / (CPS * 4), jb = i - m * (CPS * 4);
    const int kb = c0 * 4 + jb;
    xc[r] = u32x2{0u, 0u};
    xs[r] = 0u;
    if (i < XBLK && kb < kb_row) {
      xc[r] = *reinterpret_cast<const u32x2*>(a.xc + (int64_t)m * (a.K >> 1) + 8 * kb);
      xs[r] = a.xs[(int64_t)m * kb_row + kb];
    }
  }

  // ---- 2. weight records of this wave (indices clamped into the slice so a
  // wave past the end of a ragged slice re-reads valid records it then skips)
  const int wc0 = c0 + wave * CPW;
  const int last = cend - 1;
  const uint8_t* wrec = a.wc + (int64_t)tile * a.kc * kCodeRecord + 16 * lane;
  const uint8_t* srec = a.ws + (int64_t)tile * a.kg * kScaleRecord + 8 * lane;
  u32x4 w[CPW];
  u32x2 sc[CPW / 4];
#pragma unroll
  for (int i = 0; i < CPW; ++i)
    w[i] = load_codes(wrec + (int64_t)min(wc0 + i, last) * kCodeRecord, nt);
#pragma unroll
  for (int g = 0; g < CPW / 4; ++g)
    sc[g] = load_scales(srec + (int64_t)(min(wc0 + 4 * g, last) >> 2) * kScaleRecord, nt);

  // ---- 3. x~ = e2m1(code) * e4m3(scale) as f16 into LDS (zeros past K)
#pragma unroll
  for (int r = 0; r < XPT; ++r) {
    const int i = threadIdx.x + r * 64 * NW;
    if (i < XBLK) {
      const int m = i / (CPS * 4), jb = i - m * (CPS * 4);
      decode_act_block(xc[r], xs[r], xlds + m * ROW_DW + jb * 8);
    }
  }
  __syncthreads();

  // ---- 4. dot: per 16-block an exact f16 dot2 sum, then one fma by S_w
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    if (wc0 + i < cend) {
      const uint32_t sb = (((i & 3) < 2) ? sc[i >> 2].x : sc[i >> 2].y) >> (16 * (i & 1));
      dot_chunk<M>(w[i], sb, xlds + (((wave * CPW + i) * 64 + 32 * h) >> 1), ROW_DW, acc);
    }
  }

  // ---- reduce: K halves (lanes l, l^32), then waves (LDS, fixed order)
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] += __shfl_xor(acc[m], 32, 64);
  if (h == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) red[wave][m][lane] = acc[m];
  }
  __syncthreads();

  const float g = __fmul_rn(a.xg[0], a.wg[0]);
  const int n0 = tile * kTileN;
  for (int i = threadIdx.x; i < M * 32; i += 64 * NW) {
    const int m = i >> 5, n = i & 31;
    float v = red[0][m][n];
#pragma unroll
    for (int q = 1; q < NW; ++q) v += red[q][m][n];
    if (a.splits == 1) {
      if (n0 + n < a.N) store_y(a, m, n0 + n, v * g);
    } else {
      // device-coherent store (no L2 write-back of unrelated lines needed)
      __hip_atomic_store(a.part + ((int64_t)s * M + m) * a.n_pad + n0 + n, v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (a.splits == 1) return;

  // ---- split-K tail.  Partials and the tile's arrival counter are
  // device-scope atomics; each workgroup waits for its partial stores to
  // complete before it counts itself in.  The last to arrive sums the slices
  // in slice order (so the result does not depend on arrival order) and
  // resets the counter for the next call.
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.cnt + tile, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (old == (uint32_t)(a.splits - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  for (int i = threadIdx.x; i < M * 32; i += 64 * NW) {
    const int m = i >> 5, n = i & 31;
    float v = 0.0f;
    for (int t = 0; t < a.splits; ++t)
      v += __hip_atomic_load(a.part + ((int64_t)t * M + m) * a.n_pad + n0 + n, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    if (n0 + n < a.N) store_y(a, m, n0 + n, v * g);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int M, int CPW, int NW>
hipError_t launch_mcw(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  const size_t lds = (size_t)M * CPW * NW * 64 * sizeof(uint16_t);
  hipLaunchKernelGGL((gemv_split_kernel<M, CPW, NW>), dim3((unsigned)(p.tiles * p.splits)),
                     dim3(64 * NW), lds, s, a);
  return hipGetLastError();
}

template <int M, int CPW>
hipError_t launch_mc(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  switch (p.waves) {
    case 4: return launch_mcw<M, CPW, 4>(p, a, s);
    case 8: return launch_mcw<M, CPW, 8>(p, a, s);
    case 16:
      if constexpr (CPW <= 8) return launch_mcw<M, CPW, 16>(p, a, s);
      else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int M>
hipError_t launch_m(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  switch (p.cpw) {
    case 4: return launch_mc<M, 4>(p, a, s);
    case 8: return launch_mc<M, 8>(p, a, s);
    case 12: return launch_mc<M, 12>(p, a, s);
    case 16: return launch_mc<M, 16>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t dispatch_m(int M, const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  switch (M) {
    case 1: return launch_m<1>(p, a, s);
    case 2: return launch_m<2>(p, a, s);
    case 3: return launch_m<3>(p, a, s);
    case 4: return launch_m<4>(p, a, s);
    case 5: return launch_m<5>(p, a, s);
    case 6: return launch_m<6>(p, a, s);
    case 7: return launch_m<7>(p, a, s);
    case 8: return launch_m<8>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv_split(const GemvPlan& p, int M, int64_t N, int64_t K, const uint8_t* xc,
                            const uint8_t* xs, const float* xg, const uint8_t* wc,
                            const uint8_t* ws, const float* wg, void* y, int out_bf16,
                            void* workspace, hipStream_t s) {
  GemvArgs a;
  a.xc = xc;
  a.xs = xs;
  a.xg = xg;
  a.wc = wc;
  a.ws = ws;
  a.wg = wg;
  a.y = y;
  a.cnt = reinterpret_cast<uint32_t*>(workspace);
  a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + kCounterBytes);
  a.N = (int)N;
  a.n_pad = p.tiles * kTileN;
  a.K = (int)K;
  a.kc = p.kc;
  a.kg = p.kc / 4;
  a.cps = p.cps;
  a.cpw = p.cpw;
  a.splits = p.splits;
  a.out_bf16 = out_bf16;
  a.nontemporal = p.nontemporal;
  return dispatch_m(M, p, a, s);
}

}  // namespace nvfp4
