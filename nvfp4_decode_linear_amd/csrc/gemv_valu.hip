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
//    broadcast;
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
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct GemvArgs {
  const uint8_t* xc;
  const uint8_t* xs;
  const float* xg;
  const uint8_t* wc;
  const uint8_t* ws;
  const float* wg;
  void* y;
  float* part;
  uint32_t* cnt;
  int N;
  int n_pad;
  int K;
  int kc;
  int kg;
  int cps;
  int cpw;
  int splits;
  int out_bf16;
};

template <bool NT>
__device__ inline u32x4 load_codes(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

template <bool NT>
__device__ inline u32x2 load_scales(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  else return *reinterpret_cast<const u32x2*>(p);
}

__device__ inline uint32_t f16x2_bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline f16x2 bits_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// 8 E2M1 codes (one dword) -> 4 dwords of f16 pairs, in element order.
__device__ inline void decode8(uint32_t w, uint32_t (&o)[4]) {
  o[0] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
  o[1] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
  o[2] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
  o[3] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
}

struct Group {
  u32x4 w[4];
  u32x2 s;
};

template <int M, int NW, bool NT>
__global__ __launch_bounds__(64 * NW) void gemv_valu_kernel(GemvArgs a) {
  extern __shared__ uint32_t xlds[];                // [M][cps * 32] f16 pairs
  __shared__ float red[NW][M][32];
  __shared__ int last_flag;

  const int tile = blockIdx.x / a.splits;
  const int s = blockIdx.x - tile * a.splits;
  const int c0 = s * a.cps;
  const int cend = min(c0 + a.cps, a.kc);
  const int kb_row = a.K >> 4;
  const int row_dw = a.cps * 32;                    // dwords per activation row in LDS

  // ---- prologue: x~ for this K slice into LDS (zeros past K)
  for (int i = threadIdx.x; i < M * a.cps * 4; i += 64 * NW) {
    const int m = i / (a.cps * 4), jb = i - m * (a.cps * 4);
    const int kb = c0 * 4 + jb;
    u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = {0u, 0u, 0u, 0u};
    if (kb < kb_row) {
      const u32x2 cw = *reinterpret_cast<const u32x2*>(a.xc + (int64_t)m * (a.K >> 1) + 8 * kb);
      const _Float16 sa = (_Float16)e4m3_to_f32(a.xs[(int64_t)m * kb_row + kb]);
      const f16x2 sa2 = {sa, sa};
      uint32_t d0[4], d1[4];
      decode8(cw.x, d0);
      decode8(cw.y, d1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o0[q] = f16x2_bits(bits_f16x2(d0[q]) * sa2);
        o1[q] = f16x2_bits(bits_f16x2(d1[q]) * sa2);
      }
    }
    u32x4* dst = reinterpret_cast<u32x4*>(xlds + m * row_dw + jb * 8);
    dst[0] = o0;
    dst[1] = o1;
  }
  __syncthreads();

  // ---- main loop: stream this wavefront's chunks of the tile
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int wc0 = c0 + wave * a.cpw;
  const int wcend = min(wc0 + a.cpw, cend);
  const uint8_t* wrec = a.wc + (int64_t)tile * a.kc * kCodeRecord + 16 * lane;
  const uint8_t* srec = a.ws + (int64_t)tile * a.kg * kScaleRecord + 8 * lane;

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  auto load_group = [&](int c) {
    Group g;
#pragma unroll
    for (int q = 0; q < 4; ++q) g.w[q] = load_codes<NT>(wrec + (int64_t)(c + q) * kCodeRecord);
    g.s = load_scales<NT>(srec + (int64_t)(c >> 2) * kScaleRecord);
    return g;
  };

  auto compute_group = [&](const Group& g, int c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t sb = (q < 2 ? g.s.x : g.s.y) >> (16 * (q & 1));
      const float sw[2] = {__builtin_amdgcn_cvt_f32_fp8(sb, 0), __builtin_amdgcn_cvt_f32_fp8(sb, 1)};
      const int xbase = ((c + q - c0) * 64 + 32 * h) >> 1;     // dword offset in a row
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint32_t wa[4], wb[4];
        decode8(g.w[q][2 * b], wa);
        decode8(g.w[q][2 * b + 1], wb);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4* xp = reinterpret_cast<const u32x4*>(xlds + m * row_dw + xbase + 8 * b);
          const u32x4 x0 = xp[0], x1 = xp[1];
          float p = 0.0f;
#pragma unroll
          for (int d = 0; d < 4; ++d)
            p = __builtin_amdgcn_fdot2(bits_f16x2(wa[d]), bits_f16x2(x0[d]), p, false);
#pragma unroll
          for (int d = 0; d < 4; ++d)
            p = __builtin_amdgcn_fdot2(bits_f16x2(wb[d]), bits_f16x2(x1[d]), p, false);
          acc[m] = fmaf(p, sw[b], acc[m]);
        }
      }
    }
  };

  if (wc0 < wcend) {
    Group cur = load_group(wc0);
    for (int c = wc0; c < wcend; c += 4) {
      Group nxt;
      const bool more = c + 4 < wcend;
      if (more) nxt = load_group(c + 4);
      compute_group(cur, c);
      if (more) cur = nxt;
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
    for (int w = 1; w < NW; ++w) v += red[w][m][n];
    if (a.splits == 1) {
      if (n0 + n < a.N) {
        const float yv = v * g;
        if (a.out_bf16)
          reinterpret_cast<uint16_t*>(a.y)[(int64_t)m * a.N + n0 + n] = f32_to_bf16_rne(yv);
        else
          reinterpret_cast<float*>(a.y)[(int64_t)m * a.N + n0 + n] = yv;
      }
    } else {
      a.part[((int64_t)s * M + m) * a.n_pad + n0 + n] = v;
    }
  }
  if (a.splits == 1) return;

  // ---- split-K tail: the last workgroup of this tile sums the slices in
  // slice order and resets the tile's counter for the next call.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(a.cnt + tile, 1u);
    last_flag = (old == (uint32_t)(a.splits - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  for (int i = threadIdx.x; i < M * 32; i += 64 * NW) {
    const int m = i >> 5, n = i & 31;
    float v = 0.0f;
    for (int t = 0; t < a.splits; ++t)
      v += __builtin_nontemporal_load(a.part + ((int64_t)t * M + m) * a.n_pad + n0 + n);
    if (n0 + n < a.N) {
      const float yv = v * g;
      if (a.out_bf16)
        reinterpret_cast<uint16_t*>(a.y)[(int64_t)m * a.N + n0 + n] = f32_to_bf16_rne(yv);
      else
        reinterpret_cast<float*>(a.y)[(int64_t)m * a.N + n0 + n] = yv;
    }
  }
  if (threadIdx.x == 0) a.cnt[tile] = 0u;
}

template <int M, int NW, bool NT>
hipError_t launch_m(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  const size_t lds = (size_t)M * p.cps * 64 * sizeof(uint16_t);
  hipLaunchKernelGGL((gemv_valu_kernel<M, NW, NT>), dim3((unsigned)(p.tiles * p.splits)),
                     dim3(64 * NW), lds, s, a);
  return hipGetLastError();
}

template <int NW, bool NT>
hipError_t dispatch_m(int M, const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  switch (M) {
    case 1: return launch_m<1, NW, NT>(p, a, s);
    case 2: return launch_m<2, NW, NT>(p, a, s);
    case 3: return launch_m<3, NW, NT>(p, a, s);
    case 4: return launch_m<4, NW, NT>(p, a, s);
    case 5: return launch_m<5, NW, NT>(p, a, s);
    case 6: return launch_m<6, NW, NT>(p, a, s);
    case 7: return launch_m<7, NW, NT>(p, a, s);
    case 8: return launch_m<8, NW, NT>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv_valu(const GemvPlan& p, int M, int64_t N, int64_t K, const uint8_t* xc,
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
  a.part = reinterpret_cast<float*>(workspace);
  a.cnt = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(workspace) + p.ws_partials);
  a.N = (int)N;
  a.n_pad = p.tiles * kTileN;
  a.K = (int)K;
  a.kc = p.kc;
  a.kg = p.kc / 4;
  a.cps = p.cps;
  a.cpw = p.cpw;
  a.splits = p.splits;
  a.out_bf16 = out_bf16;
  if (p.waves != 4) return hipErrorInvalidValue;
  return p.nontemporal ? dispatch_m<4, true>(M, p, a, s) : dispatch_m<4, false>(M, p, a, s);
}

}  // namespace nvfp4
