// ReSET's step-aware decoding temperature on gfx950: the token entropy of
// every logits row, the running entropy of the current reasoning step, the
// temperature chosen from both, and the logits divided by it.  The method is
// the logits processor of the "ReSET" GitHub README, section "Core
// components", item 1 (the step-level uncertainty estimated online, the
// temperature adapted from token- and step-level entropy); its
// hyper-parameters t_low and tau0 are the ones the README's "Run benchmarks"
// command passes.  The rule that maps the entropies to a temperature is not
// given there; the one computed here is stated in include/nvfp4.h.
//
// Kernel 1, one row per grid row, C workgroups per row: each workgroup holds
// its share of the row in registers, takes its maximum m_c, then S_c = sum
// e^(z - m_c) and T_c = sum e^(z - m_c) (z - m_c) (masked -inf logits add
// nothing), reduces in a fixed order (per thread, wave tree, waves in
// order), stores (m_c, S_c, T_c) with device-coherent stores and counts in at
// the row's counter.  The last workgroup of the row to arrive combines the C
// partials in workgroup order (so the result is the same on every run):
//   m = max m_c, S = sum S_c e^(m_c - m), T = sum (T_c + (m_c - m) S_c) e^(m_c - m),
//   H = log S - T / S,
// updates the row's step statistics, writes H and the temperature, and puts
// the counter back to zero.  Kernel 2 divides every logit by its row's
// temperature (one correctly rounded division each).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kEntThreads = 256;
constexpr int kEntVec = 4;                          // floats per load
constexpr int kEntRounds = 4;                       // loads per thread
constexpr int kEntPerGroup = kEntThreads * kEntVec * kEntRounds;   // 4096 logits

struct EntArgs {
  const float* z;
  int64_t ldz;
  int64_t V;
  int C;                 // workgroups per row
  float* part;           // [M][C][4] (m, S, T, unused)
  uint32_t* cnt;         // [M]
  float* state;          // [M][2] running sum, count
  const int32_t* step_end;
  float* h_out;
  float* t_out;
  float t_low, tau0, t_base, t_max;
};

__device__ inline float wave_reduce_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline float wave_reduce_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Rows of up to kEntMaxGroups groups (kResetMaxV = 2^20 logits).
constexpr int kEntMaxGroups = 256;
static_assert((int64_t)kEntMaxGroups * kEntPerGroup == kResetMaxV, "vocabulary limit");

__global__ __launch_bounds__(kEntThreads) void entropy_partial_kernel(EntArgs a) {
  __shared__ float red[3][kEntThreads / 64];
  __shared__ float cpart[3 * kEntMaxGroups];
  __shared__ int last;
  const int c = blockIdx.x, row = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* zr = a.z + (int64_t)row * a.ldz;
  const int64_t c0 = (int64_t)c * kEntPerGroup;
  // this thread's logits: rounds r of 4 consecutive columns, -inf past V
  float v[kEntRounds][kEntVec];
#pragma unroll
  for (int r = 0; r < kEntRounds; ++r) {
    const int64_t col = c0 + ((int64_t)r * kEntThreads + threadIdx.x) * kEntVec;
    if (col + kEntVec <= a.V) {
      const float4 q = *reinterpret_cast<const float4*>(zr + col);
      v[r][0] = q.x; v[r][1] = q.y; v[r][2] = q.z; v[r][3] = q.w;
    } else {
#pragma unroll
      for (int e = 0; e < kEntVec; ++e) v[r][e] = col + e < a.V ? zr[col + e] : -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < kEntRounds; ++r)
#pragma unroll
    for (int e = 0; e < kEntVec; ++e) mx = fmaxf(mx, v[r][e]);
  mx = wave_reduce_max(mx);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  mx = red[0][0];
#pragma unroll
  for (int w = 1; w < kEntThreads / 64; ++w) mx = fmaxf(mx, red[0][w]);
  float s = 0.0f, t = 0.0f;
  if (mx != -INFINITY) {                            // uniform: a workgroup past V has no logits
#pragma unroll
    for (int r = 0; r < kEntRounds; ++r)
#pragma unroll
      for (int e = 0; e < kEntVec; ++e) {
        const float d = v[r][e] - mx;
        const float ex = expf(d);
        s += ex;
        t += ex > 0.0f ? ex * d : 0.0f;             // masked logits (-inf) add nothing
      }
  }
  s = wave_reduce_sum(s);
  t = wave_reduce_sum(t);
  __syncthreads();                                  // red[0] has been read
  if (lane == 0) { red[1][wave] = s; red[2][wave] = t; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float S = red[1][0], T = red[2][0];
    for (int w = 1; w < kEntThreads / 64; ++w) { S += red[1][w]; T += red[2][w]; }
    float* p = a.part + ((int64_t)row * a.C + c) * 4;
    __hip_atomic_store(p, mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 1, S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 2, T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint32_t old =
        __hip_atomic_fetch_add(a.cnt + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == (uint32_t)(a.C - 1);
  }
  __syncthreads();
  if (!last) return;                              // uniform: the workgroup's own flag
  // the last workgroup of the row: every thread loads partials (all loads in
  // flight together; one dependent load after another would cost a round
  // trip each), then thread 0 combines them in workgroup order
  const float* p = a.part + (int64_t)row * a.C * 4;
  for (int k = threadIdx.x; k < 3 * a.C; k += kEntThreads) {
    const int g = k / 3, f = k - 3 * g;
    cpart[k] = __hip_atomic_load(p + 4 * g + f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  float M = -INFINITY;
  for (int k = 0; k < a.C; ++k) M = fmaxf(M, cpart[3 * k]);
  float S = 0.0f, T = 0.0f;
  for (int k = 0; k < a.C; ++k) {
    const float mk = cpart[3 * k];
    if (mk == -INFINITY) continue;                 // a workgroup with no logits
    const float sk = cpart[3 * k + 1];
    const float tk = cpart[3 * k + 2];
    const float sh = mk - M;
    const float f = expf(sh);
    S += sk * f;
    T += (tk + sh * sk) * f;
  }
  const float H = logf(S) - T / S;
  float* st = a.state + 2 * row;
  float ssum = st[0], scount = st[1];
  if (a.step_end && a.step_end[row] != 0) { ssum = 0.0f; scount = 0.0f; }
  ssum += H;
  scount += 1.0f;
  const float hstep = ssum / scount;
  const float temp = H < a.tau0 ? a.t_low : fminf(a.t_max, a.t_base * fmaxf(1.0f, hstep / a.tau0));
  st[0] = ssum;
  st[1] = scount;
  a.h_out[row] = H;
  a.t_out[row] = temp;
  __hip_atomic_store(a.cnt + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kScaleThreads = 256;

// out[row][col] = z[row][col] / t[row] (out may be z itself)
__global__ __launch_bounds__(kScaleThreads) void scale_rows_kernel(const float* z, int64_t ldz,
                                                                   int64_t V, const float* t,
                                                                   float* out, int64_t ldo) {
  const int row = blockIdx.y;
  const float tr = t[row];
  const float* zr = z + (int64_t)row * ldz;
  float* orow = out + (int64_t)row * ldo;
  for (int64_t col = ((int64_t)blockIdx.x * kScaleThreads + threadIdx.x) * 4; col < V;
       col += (int64_t)gridDim.x * kScaleThreads * 4) {
    if (col + 4 <= V) {
      float4 q = *reinterpret_cast<const float4*>(zr + col);
      q.x = __fdiv_rn(q.x, tr); q.y = __fdiv_rn(q.y, tr);
      q.z = __fdiv_rn(q.z, tr); q.w = __fdiv_rn(q.w, tr);
      *reinterpret_cast<float4*>(orow + col) = q;
    } else {
      for (int64_t e = col; e < V; ++e) orow[e] = __fdiv_rn(zr[e], tr);
    }
  }
}

}  // namespace

int reset_groups_per_row(int64_t V) { return (int)((V + kEntPerGroup - 1) / kEntPerGroup); }

hipError_t launch_reset_temperature(const float* z, int M, int64_t V, int64_t ldz, float t_low,
                                    float tau0, float t_base, float t_max, float* state,
                                    const int32_t* step_end, float* h_out, float* t_out,
                                    float* z_out, int64_t ldo, void* workspace, hipStream_t s) {
  EntArgs a;
  a.z = z;
  a.ldz = ldz;
  a.V = V;
  a.C = reset_groups_per_row(V);
  a.cnt = static_cast<uint32_t*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kResetCounterBytes);
  a.state = state;
  a.step_end = step_end;
  a.h_out = h_out;
  a.t_out = t_out;
  a.t_low = t_low;
  a.tau0 = tau0;
  a.t_base = t_base;
  a.t_max = t_max;
  if (a.C > kEntMaxGroups) return hipErrorInvalidValue;
  hipLaunchKernelGGL(entropy_partial_kernel, dim3((unsigned)a.C, (unsigned)M), dim3(kEntThreads),
                     0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !z_out) return e;
  const int64_t per_row = (V + kScaleThreads * 4 - 1) / (kScaleThreads * 4);
  const unsigned gx = (unsigned)(per_row < 64 ? per_row : 64);
  hipLaunchKernelGGL(scale_rows_kernel, dim3(gx, (unsigned)M), dim3(kScaleThreads), 0, s, z, ldz, V,
                     t_out, z_out, ldo);
  return hipGetLastError();
}

}  // namespace nvfp4
