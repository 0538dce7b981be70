// Device-side helpers shared by the NVFP4 kernels (gfx950 only).
//
// Format: NVFP4 as used by the small-M W4A4 decode linear of "ReSET:
// Accurate Latency-Critical NVFP4 Reasoning via Step-Aware Temperature
// Scaling" (GitHub README, "Core components", item 2): E2M1 elements (OCP MX
// v1.0, 5.3.3), one E4M3 "FN" scale (OCP OFP8 v1.0) per 16 elements along K,
// one binary32 scale per tensor.  The quantizer arithmetic below must stay
// bit-identical to the IEEE reading documented in include/nvfp4.h: every
// step is one correctly rounded binary32 operation (explicit __fdiv_rn /
// __fmul_rn, the translation unit is built with -ffp-contract=off and keeps
// binary32 denormals).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Tiled weight layout (layout version 1; see include/nvfp4.h).
constexpr int kTileN = 32;          // rows per tile
constexpr int kChunkK = 64;         // elements per 1 KiB code record row-pair
constexpr int kGroupK = 256;        // elements per 512 B scale record
constexpr int kCodeRecord = 1024;   // bytes
constexpr int kScaleRecord = 512;   // bytes
constexpr int kWave = 64;

// 6 * 448: largest E2M1 magnitude times largest E4M3 scale.
constexpr float kAmaxToScale = 2688.0f;

// ---------------------------------------------------------------- codecs

// E4M3 byte (0x00..0x7E) -> binary32, exact.
__host__ __device__ inline float e4m3_to_f32(uint32_t b) {
  const uint32_t e = b >> 3, m = b & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9, exact
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Non-negative finite binary32 -> E4M3 byte: nearest, ties to even mantissa,
// saturating at 448 (0x7E).
__device__ inline uint32_t f32_to_e4m3_rne_sat(float sigma) {
  sigma = fminf(sigma, 448.0f);
  if (sigma < 0.015625f) {                       // below 2^-6: grid m * 2^-9
    // sigma * 512 is exact; rint rounds half to even.  8 -> 0x08 (2^-6).
    return (uint32_t)__builtin_rintf(__fmul_rn(sigma, 512.0f));
  }
  uint32_t u = __float_as_uint(sigma);
  u += 0x7FFFFu + ((u >> 20) & 1u);              // keep 3 mantissa bits, RNE
  return (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
}

// binary32 -> E2M1 code: nearest magnitude of {0,.5,1,1.5,2,3,4,6}, ties to
// the even code, saturating at 6; sign bit from the sign of y.
__device__ inline uint32_t f32_to_e2m1_rne_sat(float y) {
  const float a = fabsf(y);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(y) >> 28) & 8u);
}

// Two binary32 values -> two E2M1 codes in one byte (y0 in the low nibble),
// by gfx950's v_cvt_scalef32_pk_fp4_f32 with a unit scale (so the instruction
// itself does no scaling arithmetic).  It computes exactly
// f32_to_e2m1_rne_sat of each value: nearest, ties to the even code,
// saturating at 6, the code's sign bit the input's sign bit (also for -0 and
// for binary32 denormals).  The two were compared on the device over every
// finite binary32 pattern, each paired with its negation, with no difference.
__device__ inline uint32_t e2m1x2(float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0) & 0xFFu;
}

// The same two codes written into byte SEL of `old`, its other bytes kept
// (also checked on the device over every finite pattern).
template <int SEL>
__device__ inline uint32_t e2m1x2_into(uint32_t old, float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y0, y1, 1.0f, SEL);
}

// 16 values y(0..15) -> the block's two code dwords (element 2i in the low
// nibble of byte i), one conversion per pair written straight into place.
template <class Y>
__device__ __forceinline__ void pack_e2m1_block(const Y& y, uint32_t& lo, uint32_t& hi) {
  lo = e2m1x2_into<0>(0u, y(0), y(1));
  lo = e2m1x2_into<1>(lo, y(2), y(3));
  lo = e2m1x2_into<2>(lo, y(4), y(5));
  lo = e2m1x2_into<3>(lo, y(6), y(7));
  hi = e2m1x2_into<0>(0u, y(8), y(9));
  hi = e2m1x2_into<1>(hi, y(10), y(11));
  hi = e2m1x2_into<2>(hi, y(12), y(13));
  hi = e2m1x2_into<3>(hi, y(14), y(15));
}

// One block of 16 bf16 values (32 bytes, 16-byte aligned) as 8 packed pairs.
__device__ inline void load_block_bf16(const uint16_t* p, uint32_t (&v)[8]) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
  const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p + 8);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Largest |x| of a bf16 block as a bf16 magnitude pattern (these order like
// integers, so the maximum is exact).
__device__ inline uint32_t absmax_bits(const uint32_t (&v)[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = v[i] & 0x7FFF7FFFu;
    m = max(m, max(a & 0xFFFFu, a >> 16));
  }
  return m;
}

// Tensor scale from the tensor amax: amax / 2688, replaced by 1 when 0.
__device__ inline float tensor_scale(float amax) {
  float sg = __fdiv_rn(amax, kAmaxToScale);
  return sg == 0.0f ? 1.0f : sg;
}

struct BlockQ {
  uint32_t scale;     // E4M3 byte
  uint32_t lo, hi;    // 16 packed E2M1 codes (element 2i in the low nibble)
};

// Quantize one 16-element block of bf16 values (8 packed pairs) given the
// tensor scale: sigma = a / (sg*6); scale = E4M3(sigma); T = S*sg;
// r = 1/T (0 if T == 0); code_i = E2M1(x_i * r).
// The block's largest magnitude (absmax_bits(v), a bf16 pattern) may be
// passed in when the caller already has it.
__device__ inline BlockQ quantize_block_bf16(const uint32_t (&v)[8], uint32_t amax_bits, float sg) {
  const float a = __uint_as_float(amax_bits << 16);
  const float d = __fmul_rn(sg, 6.0f);
  const uint32_t sb = f32_to_e4m3_rne_sat(__fdiv_rn(a, d));
  const float T = __fmul_rn(e4m3_to_f32(sb), sg);
  const float r = (T == 0.0f) ? 0.0f : __fdiv_rn(1.0f, T);
  BlockQ q;
  q.scale = sb;
  // element e: bf16 pair e / 2, low half for even e
  pack_e2m1_block(
      [&](int e) __attribute__((always_inline)) {
        const uint32_t b = v[e >> 1];
        return __fmul_rn(__uint_as_float((e & 1) ? (b & 0xFFFF0000u) : (b << 16)), r);
      },
      q.lo, q.hi);
  return q;
}

__device__ inline BlockQ quantize_block_bf16(const uint32_t (&v)[8], float sg) {
  return quantize_block_bf16(v, absmax_bits(v), sg);
}

// Same for a block given as 16 binary32 values (fused stack kernels); a is
// the block's largest magnitude.
__device__ inline BlockQ quantize_block_f32(const float (&x)[16], float a, float sg) {
  const float d = __fmul_rn(sg, 6.0f);
  const uint32_t sb = f32_to_e4m3_rne_sat(__fdiv_rn(a, d));
  const float T = __fmul_rn(e4m3_to_f32(sb), sg);
  const float r = (T == 0.0f) ? 0.0f : __fdiv_rn(1.0f, T);
  BlockQ q;
  q.scale = sb;
  pack_e2m1_block([&](int e) __attribute__((always_inline)) { return __fmul_rn(x[e], r); },
                  q.lo, q.hi);
  return q;
}

__device__ inline BlockQ quantize_block_f32(const float (&x)[16], float sg) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(x[i]));
  return quantize_block_f32(x, a, sg);
}

// ---------------------------------------------------------- reductions

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

__device__ inline float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// binary32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// silu(g) * u = g / (1 + e^-g) * u in binary32: a correctly rounded add,
// divide and multiply around the device exponential.  The one definition of
// the element operation between the gate_up and down projections, used by
// the standalone SiLU quantizers and by the gate_up GEMV's fused epilogue.
__device__ inline float silu_mul(float g, float u) {
  const float sig = __fdiv_rn(g, __fadd_rn(1.0f, expf(-g)));
  return __fmul_rn(sig, u);
}

}  // namespace nvfp4
