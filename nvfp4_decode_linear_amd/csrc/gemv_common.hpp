// Pieces shared by the two VALU GEMV kernels of the small-M NVFP4 W4A4
// decode linear (gfx950): arguments, weight-record loads, packed FP4 decode,
// the per-chunk dot, and the output store.
#pragma once

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace gemv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

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
  int nontemporal;
  int tiles;
  int batch;     // streaming kernels: items reduced together (LDS slots)
  int waves;     // streaming kernels: wavefronts per workgroup
  // activation quantized inside the GEMV (nvfp4_quantize_linear): the bf16
  // input [M][ldx] and the canonical NVFP4 outputs workgroup 0 writes
  const uint16_t* xb;
  int64_t ldx;
  uint8_t* oc;
  uint8_t* os;
  float* og;
  int rms;       // nonzero: RMS-normalise each row (epsilon eps) before quantizing
  float eps;
  float* ho;     // optional binary32 h [M][K] (workgroup 0)
  const float* sgs;  // a caller-supplied (static) activation tensor scale: the
                     // prologue then takes no tensor maximum and writes no og
  // binary32 activation [M][ldx] quantized in the prologue (instead of xb)
  const float* xf;
  // the tensor maximum of xf as a record of per-workgroup maxima
  // [kAmaxSlots] (|x| bit patterns; their maximum is the tensor's), or null
  const uint32_t* amax_in;
  int qslice;    // split K with amax_in: each workgroup quantizes only its K slice
  // SiLU * mul epilogue (gate_up projection, rows [0, F) gate, [F, 2F) up):
  // y is h [M][ldh] binary32, gu (optional) the bf16 gate_up output [M][N],
  // amax_out the record of this launch's per-workgroup maxima of |h|
  uint32_t* amax_out;
  int64_t ldh;
  uint16_t* gu;
};

__device__ inline u32x4 load_codes(const uint8_t* p, bool nt) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  return nt ? __builtin_nontemporal_load(q) : *q;
}

__device__ inline u32x2 load_scales(const uint8_t* p, bool nt) {
  const u32x2* q = reinterpret_cast<const u32x2*>(p);
  return nt ? __builtin_nontemporal_load(q) : *q;
}

__device__ inline uint32_t f16x2_bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline f16x2 bits_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// 8 E2M1 codes (one dword) -> 4 dwords of f16 pairs, in element order.
__device__ __forceinline__ void decode8(uint32_t w, uint32_t (&o)[4]) {
  o[0] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
  o[1] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
  o[2] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
  o[3] = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
}

__device__ __forceinline__ void store_y(const GemvArgs& a, int m, int n, float v) {
  if (a.out_bf16)
    reinterpret_cast<uint16_t*>(a.y)[(int64_t)m * a.N + n] = f32_to_bf16_rne(v);
  else
    reinterpret_cast<float*>(a.y)[(int64_t)m * a.N + n] = v;
}

// One 64-element chunk of one row tile (this lane: row l % 32, K half
// l / 32, i.e. 32 codes = two 16-blocks) against the M activation rows.
// Each block's 16 products are summed exactly by v_dot2_f32_f16 (x~ has at
// most 6 significant bits, the codes 2, the block shares one activation
// scale), then folded in with one fma by the weight's E4M3 block scale.
//   w   16 code bytes of the record (two blocks, element order)
//   sb  the two E4M3 scale bytes of those blocks (low 16 bits)
//   xh  LDS dwords of activation row 0 at this chunk and K half; row m at
//       xh + m * row_dw (f16 pairs of x~ = e2m1(code) * e4m3(scale))
template <int M>
__device__ __forceinline__ void dot_chunk(const u32x4& w, uint32_t sb, const uint32_t* xh, int row_dw,
                                 float (&acc)[M]) {
  const float sw0 = __builtin_amdgcn_cvt_f32_fp8(sb, 0);
  const float sw1 = __builtin_amdgcn_cvt_f32_fp8(sb, 1);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    uint32_t wa[4], wb[4];
    decode8(w[2 * b], wa);
    decode8(w[2 * b + 1], wb);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      // Dword reads (paired into ds_read2_b32): on gfx950 the 64- and
      // 128-bit LDS reads of this pattern run several times slower.
      const uint32_t* xp = xh + m * row_dw + 8 * b;
      const u32x4 x0 = {xp[0], xp[1], xp[2], xp[3]};
      const u32x4 x1 = {xp[4], xp[5], xp[6], xp[7]};
      float p = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        p = __builtin_amdgcn_fdot2(bits_f16x2(wa[d]), bits_f16x2(x0[d]), p, false);
#pragma unroll
      for (int d = 0; d < 4; ++d)
        p = __builtin_amdgcn_fdot2(bits_f16x2(wb[d]), bits_f16x2(x1[d]), p, false);
      acc[m] = fmaf(p, b ? sw1 : sw0, acc[m]);
    }
  }
}

// x~ for one activation 16-block: 8 code bytes and the E4M3 scale byte ->
// 16 f16 values (8 dwords) written to LDS at dst.
__device__ __forceinline__ void decode_act_block(u32x2 codes, uint32_t scale, uint32_t* dst) {
  const _Float16 sa = (_Float16)e4m3_to_f32(scale);
  const f16x2 sa2 = {sa, sa};
  uint32_t d0[4], d1[4];
  decode8(codes.x, d0);
  decode8(codes.y, d1);
  u32x4 o0, o1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o0[q] = f16x2_bits(bits_f16x2(d0[q]) * sa2);
    o1[q] = f16x2_bits(bits_f16x2(d1[q]) * sa2);
  }
  reinterpret_cast<u32x4*>(dst)[0] = o0;
  reinterpret_cast<u32x4*>(dst)[1] = o1;
}

}  // namespace gemv
}  // namespace nvfp4
