// NVFP4 quantization kernels for gfx950: activation quantizer (every decode
// step), weight quantizer into the device-tiled layout (once per model
// load), the inverse tiling, and a zero-fill.
//
// The quantizer reading (tensor amax -> tensor scale; per 16-block E4M3
// scale; per element E2M1 code, all binary32, round to nearest even) is the
// one documented in include/nvfp4.h.  W4A4 = both operands of the decode
// linear are NVFP4: "ReSET" GitHub README, "Core components", item 2; the
// weights are converted offline: README, "Quantize a model to NVFP4".
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ activations
//
// The tensor amax is a reduction over every element of the M x K activation
// (bf16 magnitudes compared as integers, exact) and must be known before any
// block can be scaled.  Each thread owns BPT blocks of 16 (block b0, b0 +
// stride, ...), loads them all up front (clamped addresses, so no load is
// conditional and all are in flight together) and keeps them in registers
// through the reduction.  With more than one workgroup the workgroup maxima
// meet in a 16-byte sync record of the caller's workspace:
//   word 0: running amax (atomic max), word 1: arrivals, word 2: departures.
// Thread 0 of each workgroup adds its maximum, arrives, and polls the
// arrivals until all workgroups have arrived; the last workgroup to depart
// puts all three words back to zero, so the record is zero between calls
// (graph replays included).  The poll is bounded: a workgroup that gives up
// (the grid is not co-resident, or the spin limit is forced low) computes
// the amax itself from the whole tensor, which gives the same value.
constexpr int kActThreads = 256;
constexpr int kActMaxGroups = 256;
constexpr uint32_t kActDefaultSpin = 1u << 20;

__device__ inline uint32_t block_reduce_max(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t all = 0;
#pragma unroll
  for (int w = 0; w < kActThreads / kWave; ++w) all = max(all, red[w]);
  __syncthreads();                              // red is reused
  return all;
}

__device__ inline void store_block(uint8_t* codes, uint8_t* scales, int K, int m, int j,
                                   const BlockQ& q) {
  u32x2 c;
  c.x = q.lo;
  c.y = q.hi;
  *reinterpret_cast<u32x2*>(codes + (int64_t)m * (K >> 1) + 8 * j) = c;
  scales[(int64_t)m * (K >> 4) + j] = (uint8_t)q.scale;
}

// amax of the whole tensor by one workgroup (the fallback path)
__device__ uint32_t tensor_amax_bits(const uint16_t* x, int M, int K, int64_t ldx, uint32_t* red) {
  const int nbr = K >> 4, nb = M * nbr;
  uint32_t amax = 0;
  for (int b = threadIdx.x; b < nb; b += kActThreads) {
    const int m = b / nbr, j = b - m * nbr;
    uint32_t v[8];
    load_block_bf16(x + (int64_t)m * ldx + 16 * j, v);
    amax = max(amax, absmax_bits(v));
  }
  return block_reduce_max(amax, red);
}

constexpr uint32_t kGaveUp = 0xFFFFFFFFu;

// Tensor maximum over the workgroups of the grid: each passes the maximum of
// its part (a non-negative binary32 or bf16 magnitude pattern; these order
// like integers) and gets back the maximum over all of them, or kGaveUp if
// it stopped polling (then it must compute the maximum alone).  Called by all
// threads of every workgroup; thread 0 talks to the sync record.
__device__ uint32_t combine_amax(uint32_t amax, uint32_t* sync, uint32_t spin_limit,
                                 uint32_t* shared_slot) {
  if (threadIdx.x == 0) {
    const uint32_t G = gridDim.x;
    __hip_atomic_fetch_max(sync, amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __hip_atomic_fetch_add(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t all = kGaveUp;
    for (uint32_t i = 0;; ++i) {
      const uint32_t c = __hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (c >= G) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        all = __hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      if (i + 1 >= spin_limit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    *shared_slot = all;
    // depart (the amax load above has returned: its value is in `all`)
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint32_t d =
        __hip_atomic_fetch_add(sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == G - 1) {                             // every workgroup has read: reset
      __hip_atomic_store(sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  return *shared_slot;
}

// sg_static: a caller-supplied tensor scale (a calibrated, static activation
// scale); then no tensor maximum is taken, every workgroup quantizes its own
// blocks alone, and gscale is not written.
template <int BPT>
__global__ __launch_bounds__(kActThreads) void act_quant_kernel(
    const uint16_t* __restrict__ x, int M, int K, int64_t ldx, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gscale, uint32_t* sync,
    uint32_t spin_limit, const float* __restrict__ sg_static) {
  __shared__ uint32_t red[kActThreads / kWave];
  __shared__ uint32_t shared_amax;
  const int nbr = K >> 4;
  const int nb = M * nbr;
  const int stride = gridDim.x * kActThreads;
  const int b0 = blockIdx.x * kActThreads + threadIdx.x;
  uint32_t v[BPT][8];
#pragma unroll
  for (int r = 0; r < BPT; ++r) {
    const int b = min(b0 + r * stride, nb - 1);
    const int m = b / nbr, j = b - m * nbr;
    load_block_bf16(x + (int64_t)m * ldx + 16 * j, v[r]);
  }
  float sg;
  if (sg_static) {                              // uniform: no tensor maximum
    sg = *sg_static;
  } else {
    uint32_t amax = 0;
#pragma unroll
    for (int r = 0; r < BPT; ++r) amax = max(amax, absmax_bits(v[r]));
    amax = block_reduce_max(amax, red);
    if (gridDim.x > 1) {
      amax = combine_amax(amax, sync, spin_limit, &shared_amax);
      if (amax == kGaveUp) amax = tensor_amax_bits(x, M, K, ldx, red);
    }
    sg = tensor_scale(bf16_to_f32(amax));
    if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = sg;
  }
#pragma unroll
  for (int r = 0; r < BPT; ++r) {
    const int b = b0 + r * stride;
    if (b < nb) {
      const int m = b / nbr, j = b - m * nbr;
      store_block(codes, scales, K, m, j, quantize_block_bf16(v[r], sg));
    }
  }
}

// The same quantizer on a binary32 activation (the SiLU * mul output that
// the gate_up GEMV writes).  amax_in: that producer's record of per-workgroup
// maxima (kAmaxSlots |x| bit patterns, zero past its grid); then the tensor
// maximum is the record's largest entry and no workgroup waits for another.
// Without it the maxima are combined as above (a workgroup that gives up
// takes the maximum of the whole tensor alone).
__device__ inline void load_block_f32(const float* p, float (&h)[16]) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const u32x4 t = q[e];
    h[4 * e] = __uint_as_float(t.x);
    h[4 * e + 1] = __uint_as_float(t.y);
    h[4 * e + 2] = __uint_as_float(t.z);
    h[4 * e + 3] = __uint_as_float(t.w);
  }
}

__device__ inline uint32_t absmax_bits_f32(const float (&h)[16]) {
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) m = max(m, __float_as_uint(h[e]) & 0x7FFFFFFFu);
  return m;
}

template <int BPT>
__global__ __launch_bounds__(kActThreads) void act_quant_f32_kernel(
    const float* __restrict__ x, int M, int K, int64_t ldx, const uint32_t* __restrict__ amax_in,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gscale,
    uint32_t* sync, uint32_t spin_limit) {
  __shared__ uint32_t red[kActThreads / kWave];
  __shared__ uint32_t shared_amax;
  const int nbr = K >> 4;
  const int nb = M * nbr;
  const int stride = gridDim.x * kActThreads;
  const int b0 = blockIdx.x * kActThreads + threadIdx.x;
  float v[BPT][16];
  uint32_t bm[BPT];
#pragma unroll
  for (int r = 0; r < BPT; ++r) {
    const int b = min(b0 + r * stride, nb - 1);
    const int m = b / nbr, j = b - m * nbr;
    load_block_f32(x + (int64_t)m * ldx + 16 * j, v[r]);
  }
  uint32_t amax = 0;
#pragma unroll
  for (int r = 0; r < BPT; ++r) {
    bm[r] = absmax_bits_f32(v[r]);
    amax = max(amax, bm[r]);
  }
  if (amax_in) {                                // uniform: the producer's maxima
    amax = threadIdx.x < kAmaxSlots ? amax_in[threadIdx.x] : 0u;
    amax = block_reduce_max(amax, red);
  } else {
    amax = block_reduce_max(amax, red);
    if (gridDim.x > 1) {
      amax = combine_amax(amax, sync, spin_limit, &shared_amax);
      if (amax == kGaveUp) {                    // the whole tensor, this workgroup alone
        uint32_t a2 = 0;
        for (int b = threadIdx.x; b < nb; b += kActThreads) {
          const int m = b / nbr, j = b - m * nbr;
          float hh[16];
          load_block_f32(x + (int64_t)m * ldx + 16 * j, hh);
          a2 = max(a2, absmax_bits_f32(hh));
        }
        amax = block_reduce_max(a2, red);
      }
    }
  }
  const float sg = tensor_scale(__uint_as_float(amax));
  if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = sg;
#pragma unroll
  for (int r = 0; r < BPT; ++r) {
    const int b = b0 + r * stride;
    if (b < nb) {
      const int m = b / nbr, j = b - m * nbr;
      store_block(codes, scales, K, m, j, quantize_block_f32(v[r], __uint_as_float(bm[r]), sg));
    }
  }
}

// ------------------------------------------------- fused stack quantizers
//
// The activation quantizer applied to a binary32 h computed in the same
// kernel from the previous linear's bf16 output (the layer stack between its
// linears): h = x / sqrt(mean(x^2) + eps) per row (unweighted RMS norm), or
// h = silu(g) * u with g, u the two halves of a gate_up row.  One workgroup
// of 1024 threads per row; thread t owns blocks t, t + 1024, ... of the row
// and keeps their h in registers through the tensor-amax combine.  h may be
// written out (binary32) for checking.
constexpr int kPrepThreads = 1024;
enum PrepMode { kPrepRms = 0, kPrepSilu = 1 };

__device__ inline void load16_bf16_f32(const uint16_t* p, float (&h)[16]) {
  uint32_t v[8];
  load_block_bf16(p, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[2 * i] = __uint_as_float(v[i] << 16);
    h[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

// sum over the workgroup in a fixed order (the same on every run and in
// every workgroup that computes it)
__device__ inline float block_sum_f32(float v, float* red) {
  v = wave_sum_f32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float all = red[0];
#pragma unroll
  for (int w = 1; w < kPrepThreads / kWave; ++w) all += red[w];
  __syncthreads();
  return all;
}

// h = silu(g) * u for block j of a row (gate g = row[0, K), up u = row[K, 2K))
__device__ inline void silu_mul_block(const uint16_t* row, int K, int j, float (&h)[16]) {
  float u[16];
  load16_bf16_f32(row + 16 * j, h);
  load16_bf16_f32(row + K + 16 * j, u);
#pragma unroll
  for (int i = 0; i < 16; ++i) h[i] = silu_mul(h[i], u[i]);
}

// h of this thread's blocks of row `row` (blocks past the row are zero)
template <int MODE, int BPT>
__device__ inline void prep_row(const uint16_t* row, int K, float eps, float (&h)[BPT][16],
                                float* red) {
  const int nbr = K >> 4;
#pragma unroll
  for (int r = 0; r < BPT; ++r) {
    const int j = min((int)threadIdx.x + r * kPrepThreads, nbr - 1);
    if constexpr (MODE == kPrepSilu) {
      silu_mul_block(row, K, j, h[r]);
    } else {
      load16_bf16_f32(row + 16 * j, h[r]);
    }
    if ((int)threadIdx.x + r * kPrepThreads >= nbr) {
#pragma unroll
      for (int i = 0; i < 16; ++i) h[r][i] = 0.0f;
    }
  }
  if constexpr (MODE == kPrepRms) {
    float ss = 0.0f;
#pragma unroll
    for (int r = 0; r < BPT; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = __fadd_rn(ss, __fmul_rn(h[r][i], h[r][i]));
    const float ms = __fdiv_rn(block_sum_f32(ss, red), (float)K);
    const float rinv = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(ms, eps)));
#pragma unroll
    for (int r = 0; r < BPT; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) h[r][i] = __fmul_rn(h[r][i], rinv);
  }
}

template <int BPT>
__device__ inline uint32_t amax_bits_f32(const float (&h)[BPT][16]) {
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < BPT; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(h[r][i]) & 0x7FFFFFFFu);
  return m;
}

template <int MODE, int BPT>
__global__ __launch_bounds__(kPrepThreads) void prep_quant_kernel(
    const uint16_t* __restrict__ x, int K, int64_t ldx, float eps, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gscale, float* __restrict__ h_out,
    uint32_t* sync, uint32_t spin_limit) {
  __shared__ float red[kPrepThreads / kWave];
  __shared__ uint32_t shared_amax;
  const int m = blockIdx.x;
  const int nbr = K >> 4;
  float h[BPT][16];
  prep_row<MODE, BPT>(x + (int64_t)m * ldx, K, eps, h, red);
  if (h_out) {
#pragma unroll
    for (int r = 0; r < BPT; ++r) {
      const int j = (int)threadIdx.x + r * kPrepThreads;
      if (j < nbr) {
        float4* o = reinterpret_cast<float4*>(h_out + (int64_t)m * K + 16 * j);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = make_float4(h[r][4 * q], h[r][4 * q + 1], h[r][4 * q + 2], h[r][4 * q + 3]);
      }
    }
  }
  uint32_t amax = wave_max_u32(amax_bits_f32<BPT>(h));
  if ((threadIdx.x & 63) == 0) reinterpret_cast<uint32_t*>(red)[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = 0;
#pragma unroll
  for (int w = 0; w < kPrepThreads / kWave; ++w)
    amax = max(amax, reinterpret_cast<uint32_t*>(red)[w]);
  __syncthreads();
  if (gridDim.x > 1) {
    amax = combine_amax(amax, sync, spin_limit, &shared_amax);
    if (amax == kGaveUp) {                        // every row's h, this workgroup alone
      amax = 0;
      for (int mm = 0; mm < (int)gridDim.x; ++mm) {
        float hh[BPT][16];
        prep_row<MODE, BPT>(x + (int64_t)mm * ldx, K, eps, hh, red);
        amax = max(amax, amax_bits_f32<BPT>(hh));
      }
      amax = wave_max_u32(amax);
      if ((threadIdx.x & 63) == 0) reinterpret_cast<uint32_t*>(red)[threadIdx.x >> 6] = amax;
      __syncthreads();
      amax = 0;
#pragma unroll
      for (int w = 0; w < kPrepThreads / kWave; ++w)
        amax = max(amax, reinterpret_cast<uint32_t*>(red)[w]);
    }
  }
  const float sg = tensor_scale(__uint_as_float(amax));
  if (m == 0 && threadIdx.x == 0) *gscale = sg;
#pragma unroll
  for (int r = 0; r < BPT; ++r) {
    const int j = (int)threadIdx.x + r * kPrepThreads;
    if (j < nbr) store_block(codes, scales, K, m, j, quantize_block_f32(h[r], sg));
  }
}

// SiLU * mul + quantization spread over workgroups of kActThreads threads:
// thread t of workgroup w owns flat block i = w * kActThreads + t of the M x
// K/16 blocks (row i / (K/16)), one block each, so the exp / divide work of a
// row is shared by many CUs instead of one.  The tensor maximum is combined
// across the grid as in act_quant_kernel (bounded poll; a workgroup that
// gives up recomputes every block's h itself).  h and the codes are those of
// prep_quant_kernel<kPrepSilu, *>: the same per-element operations and the
// same exact maximum.
__global__ __launch_bounds__(kActThreads) void silu_quant_spread_kernel(
    const uint16_t* __restrict__ x, int M, int K, int64_t ldx, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gscale, float* __restrict__ h_out,
    uint32_t* sync, uint32_t spin_limit) {
  __shared__ uint32_t red[kActThreads / kWave];
  __shared__ uint32_t shared_amax;
  const int nbr = K >> 4, nall = M * nbr;
  const int i = (int)blockIdx.x * kActThreads + (int)threadIdx.x;
  const int ic = min(i, nall - 1);
  const int m = ic / nbr, j = ic - m * nbr;
  float h[16];
  silu_mul_block(x + (int64_t)m * ldx, K, j, h);
  uint32_t bmax = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) bmax = max(bmax, __float_as_uint(h[e]) & 0x7FFFFFFFu);
  if (h_out && i < nall) {
    float4* o = reinterpret_cast<float4*>(h_out + (int64_t)m * K + 16 * j);
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
  }
  uint32_t amax = block_reduce_max(i < nall ? bmax : 0u, red);
  if (gridDim.x > 1) {
    amax = combine_amax(amax, sync, spin_limit, &shared_amax);
    if (amax == kGaveUp) {                        // every block's h, this workgroup alone
      uint32_t a2 = 0;
      for (int b = threadIdx.x; b < nall; b += kActThreads) {
        const int mm = b / nbr, jj = b - mm * nbr;
        float hh[16];
        silu_mul_block(x + (int64_t)mm * ldx, K, jj, hh);
#pragma unroll
        for (int e = 0; e < 16; ++e) a2 = max(a2, __float_as_uint(hh[e]) & 0x7FFFFFFFu);
      }
      amax = block_reduce_max(a2, red);
    }
  }
  const float sg = tensor_scale(__uint_as_float(amax));
  if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = sg;
  if (i < nall) store_block(codes, scales, K, m, j, quantize_block_f32(h, __uint_as_float(bmax), sg));
}

// ---------------------------------------------------------------- weights

__global__ void wq_init_kernel(uint32_t* slot) { *slot = 0u; }

// Tensor amax of the bf16 weight; the slot holds the binary32 bits of the
// running maximum (non-negative floats order like their bit patterns).
__global__ __launch_bounds__(256) void wq_amax_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                      int64_t K, int64_t ldw, uint32_t* slot) {
  const int64_t vpr = K >> 3;
  const int64_t total = N * vpr;
  uint32_t amax = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / vpr, v = i - r * vpr;
    const u32x4 q = *reinterpret_cast<const u32x4*>(w + r * ldw + 8 * v);
    const uint32_t t[4] = {q.x & 0x7FFF7FFFu, q.y & 0x7FFF7FFFu, q.z & 0x7FFF7FFFu,
                           q.w & 0x7FFF7FFFu};
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = max(amax, max(t[k] & 0xFFFFu, t[k] >> 16));
  }
  amax = wave_max_u32(amax);
  if ((threadIdx.x & 63) == 0 && amax != 0u) atomicMax(slot, amax << 16);
}

// One thread per (row tile, K chunk, lane): quantizes the two 16-blocks the
// lane owns in the tiled layout and writes its 16 code bytes and 2 scale
// bytes.  Padding rows and columns are written as zeros.  gate_up_f > 0: the
// interleaved gate_up order (tiled row 32t + r <- source row 16t + r for r <
// 16, F + 16t + r - 16 for r >= 16).
__global__ __launch_bounds__(256) void wq_blocks_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                        int64_t K, int64_t ldw, int kc, int kg,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales,
                                                        const uint32_t* __restrict__ slot,
                                                        int64_t gate_up_f) {
  const float sg = tensor_scale(__uint_as_float(*slot));
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rec = gid >> 6;
  const int l = (int)(gid & 63);
  const int64_t t = rec / kc;
  const int c = (int)(rec - t * kc);
  const int64_t n = t * kTileN + (l & 31);
  const int64_t k0 = (int64_t)c * kChunkK + 32 * (l >> 5);
  u32x4 out = {0u, 0u, 0u, 0u};
  uint32_t sc = 0;
  const int r = l & 31;
  const int64_t src = gate_up_f > 0 ? (r < 16 ? 16 * t + r : gate_up_f + 16 * t + (r - 16)) : n;
  if (n < N) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t kb = k0 + 16 * b;
      if (kb < K) {
        uint32_t v[8];
        load_block_bf16(w + src * ldw + kb, v);
        const BlockQ q = quantize_block_bf16(v, sg);
        out[2 * b] = q.lo;
        out[2 * b + 1] = q.hi;
        sc |= q.scale << (8 * b);
      }
    }
  }
  *reinterpret_cast<u32x4*>(codes + rec * kCodeRecord + 16 * l) = out;
  const int g = c >> 2, q = c & 3;
  *reinterpret_cast<uint16_t*>(scales + (t * kg + g) * kScaleRecord + 8 * l + 2 * q) =
      (uint16_t)sc;
}

__global__ void wq_finalize_kernel(uint32_t* slot) {
  const float sg = tensor_scale(__uint_as_float(*slot));
  *reinterpret_cast<float*>(slot) = sg;
}

// Tiled -> canonical, one thread per (row, 16-block).
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int64_t N,
                                                     int64_t K, int kc, int kg,
                                                     uint8_t* __restrict__ codes_rm,
                                                     uint8_t* __restrict__ scales_rm) {
  const int64_t nbr = K >> 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= N * nbr) return;
  const int64_t n = gid / nbr, j = gid - n * nbr;
  const int64_t t = n / kTileN;
  const int r = (int)(n - t * kTileN);
  const int64_t k = 16 * j;
  const int64_t c = k / kChunkK;
  const int h = (int)((k % kChunkK) / 32), b = (int)((k % 32) / 16);
  const int l = r + 32 * h;
  const u32x2 v =
      *reinterpret_cast<const u32x2*>(codes + (t * kc + c) * kCodeRecord + 16 * l + 8 * b);
  *reinterpret_cast<u32x2*>(codes_rm + n * (K >> 1) + 8 * j) = v;
  const int64_t g = k / kGroupK;
  const int q = (int)((k % kGroupK) / kChunkK);
  scales_rm[n * nbr + j] = scales[(t * kg + g) * kScaleRecord + 8 * l + 2 * q + b];
}

// Every finite binary32 pattern (exponent field below 255), each paired with
// its negation: the instruction encoder e2m1x2 against the rounding rule
// f32_to_e2m1_rne_sat.  out[0] += mismatching patterns, out[1] += patterns
// checked.  Thread t covers patterns [t * per, (t + 1) * per).
__global__ __launch_bounds__(256) void e2m1_selftest_kernel(unsigned long long* out,
                                                            uint64_t per) {
  const uint64_t beg = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * per;
  unsigned long long bad = 0, seen = 0;
  for (uint64_t k = 0; k < per; ++k) {
    const uint64_t idx = beg + k;
    if (idx >> 32) break;
    const uint32_t u = (uint32_t)idx;
    if ((u & 0x7F800000u) == 0x7F800000u) continue;
    const float y = __uint_as_float(u), z = __uint_as_float(u ^ 0x80000000u);
    const uint32_t ref = f32_to_e2m1_rne_sat(y) | (f32_to_e2m1_rne_sat(z) << 4);
    bad += e2m1x2(y, z) != ref;
    // the byte-select forms write the same byte into position 1, 2 or 3 of
    // the old dword and keep its other bytes
    const uint32_t old = 0xA5C3E10Fu ^ u;
    bad += e2m1x2_into<1>(old, y, z) != ((old & ~0x0000FF00u) | (ref << 8));
    bad += e2m1x2_into<2>(old, y, z) != ((old & ~0x00FF0000u) | (ref << 16));
    bad += e2m1x2_into<3>(old, y, z) != ((old & ~0xFF000000u) | (ref << 24));
    ++seen;
  }
  atomicAdd(out, bad);
  atomicAdd(out + 1, seen);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

}  // namespace

ActPlan act_plan(int M, int64_t K) {
  const int64_t nb = (int64_t)M * (K >> 4);
  ActPlan p;
  if (nb <= 4 * kActThreads) {                  // one workgroup, up to 4 blocks per thread
    p.groups = 1;
    p.bpt = (int)((nb + kActThreads - 1) / kActThreads);
  } else {
    p.groups = (int)std::min<int64_t>((nb + kActThreads - 1) / kActThreads, kActMaxGroups);
    p.bpt = (int)((nb + (int64_t)p.groups * kActThreads - 1) / ((int64_t)p.groups * kActThreads));
  }
  if (p.bpt == 3) p.bpt = 4;
  return p;
}

hipError_t launch_quantize_act(const uint16_t* x, int M, int K, int64_t ldx, uint8_t* codes,
                               uint8_t* scales, float* gscale, uint32_t* sync, uint32_t spin_limit,
                               hipStream_t s, const float* sg_static) {
  const ActPlan p = act_plan(M, K);
  const uint32_t spin = spin_limit ? spin_limit : kActDefaultSpin;
  switch (p.bpt) {
    case 1:
      hipLaunchKernelGGL(act_quant_kernel<1>, dim3(p.groups), dim3(kActThreads), 0, s, x, M, K,
                         ldx, codes, scales, gscale, sync, spin, sg_static);
      break;
    case 2:
      hipLaunchKernelGGL(act_quant_kernel<2>, dim3(p.groups), dim3(kActThreads), 0, s, x, M, K,
                         ldx, codes, scales, gscale, sync, spin, sg_static);
      break;
    case 4:
      hipLaunchKernelGGL(act_quant_kernel<4>, dim3(p.groups), dim3(kActThreads), 0, s, x, M, K,
                         ldx, codes, scales, gscale, sync, spin, sg_static);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_act_f32(const float* x, int M, int K, int64_t ldx,
                                   const uint32_t* amax_in, uint8_t* codes, uint8_t* scales,
                                   float* gscale, uint32_t* sync, uint32_t spin_limit,
                                   hipStream_t s) {
  static_assert(kAmaxSlots <= kActThreads, "one record slot per thread");
  const ActPlan p = act_plan(M, K);
  const uint32_t spin = spin_limit ? spin_limit : kActDefaultSpin;
#define NVFP4_ACT_F32(BPT)                                                                     \
  hipLaunchKernelGGL(act_quant_f32_kernel<BPT>, dim3(p.groups), dim3(kActThreads), 0, s, x, M, \
                     K, ldx, amax_in, codes, scales, gscale, sync, spin)
  switch (p.bpt) {
    case 1: NVFP4_ACT_F32(1); break;
    case 2: NVFP4_ACT_F32(2); break;
    case 4: NVFP4_ACT_F32(4); break;
    default: return hipErrorInvalidValue;
  }
#undef NVFP4_ACT_F32
  return hipGetLastError();
}

int prep_bpt(int64_t K) { return (K >> 4) <= kPrepThreads ? 1 : 2; }

hipError_t launch_prep_quantize(int mode, const uint16_t* x, int M, int K, int64_t ldx, float eps,
                                uint8_t* codes, uint8_t* scales, float* gscale, float* h_out,
                                uint32_t* sync, uint32_t spin_limit, hipStream_t s) {
  const uint32_t spin = spin_limit ? spin_limit : kActDefaultSpin;
  const dim3 g(M), b(kPrepThreads);
#define NVFP4_PREP(MODE, BPT)                                                                  \
  hipLaunchKernelGGL((prep_quant_kernel<MODE, BPT>), g, b, 0, s, x, K, ldx, eps, codes, scales, \
                     gscale, h_out, sync, spin)
  const int bpt = prep_bpt(K);
  if (mode == kPrepSilu && sync) {
    const int groups = (M * (K >> 4) + kActThreads - 1) / kActThreads;   // <= 64
    hipLaunchKernelGGL(silu_quant_spread_kernel, dim3(groups), dim3(kActThreads), 0, s, x, M, K,
                       ldx, codes, scales, gscale, h_out, sync, spin);
    return hipGetLastError();
  }
  if (mode == kPrepRms) {
    if (bpt == 1) NVFP4_PREP(kPrepRms, 1);
    else NVFP4_PREP(kPrepRms, 2);
  } else {
    if (bpt == 1) NVFP4_PREP(kPrepSilu, 1);
    else NVFP4_PREP(kPrepSilu, 2);
  }
#undef NVFP4_PREP
  return hipGetLastError();
}

hipError_t launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* codes, uint8_t* scales, float* gscale, hipStream_t s,
                                  int64_t gate_up_f) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(gscale);
  const int64_t n_pad = round_up(N, kTileN), k_pad = round_up(K, kGroupK);
  const int kc = (int)(k_pad / kChunkK), kg = (int)(k_pad / kGroupK);
  hipLaunchKernelGGL(wq_init_kernel, dim3(1), dim3(1), 0, s, slot);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t vecs = N * (K >> 3);
  const int64_t amax_blocks = std::min<int64_t>((vecs + 255) / 256, 4096);
  hipLaunchKernelGGL(wq_amax_kernel, dim3((unsigned)amax_blocks), dim3(256), 0, s, w, N, K, ldw,
                     slot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t threads = (n_pad / kTileN) * kc * kWave;
  hipLaunchKernelGGL(wq_blocks_kernel, dim3((unsigned)(threads / 256)), dim3(256), 0, s, w, N, K,
                     ldw, kc, kg, codes, scales, slot, gate_up_f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(wq_finalize_kernel, dim3(1), dim3(1), 0, s, slot);
  return hipGetLastError();
}

hipError_t launch_unpack_weight(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                                uint8_t* codes_rm, uint8_t* scales_rm, hipStream_t s) {
  const int64_t k_pad = round_up(K, kGroupK);
  const int kc = (int)(k_pad / kChunkK), kg = (int)(k_pad / kGroupK);
  const int64_t total = N * (K >> 4);
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, codes,
                     scales, N, K, kc, kg, codes_rm, scales_rm);
  return hipGetLastError();
}

hipError_t launch_e2m1_selftest(unsigned long long* out, hipStream_t s) {
  hipError_t e = launch_fill_zero(out, 16, s);
  if (e != hipSuccess) return e;
  const unsigned blocks = 8192, threads = 256;           // 2^21 threads x 2048 = 2^32
  hipLaunchKernelGGL(e2m1_selftest_kernel, dim3(blocks), dim3(threads), 0, s, out,
                     (uint64_t)1 << 11);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((words + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace nvfp4
