// fa_probe.hip -- matrix-core throughput probe for gfx950 (MI355X): how many dense bf16 FLOP/s the
// v_mfma_f32_32x32x16_bf16 pipes of this GPU sustain, and at which shader clock, so that the attention
// kernels' rate can be quoted against the peak this particular GPU reaches as well as the data-sheet peak.
//
// Every wave issues independent MFMAs back to back from register operands (no memory traffic in the timed
// loop): 8 A fragments and 2 B fragments of pseudo-random bf16 values of unit magnitude (the matrix cores draw
// more power, and the chip clocks lower, on random operands than on constant ones), 4 accumulators. Two waves
// per SIMD keep the pipe fed while one waits on a dependent accumulator. Each workgroup records its shader
// cycles (s_memtime) and its 100 MHz real-time ticks (s_memrealtime); their ratio is the shader clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;   // 4 waves
constexpr int kMfmaPerIter = 8;      // MFMAs per wave per loop iteration

__device__ __forceinline__ float unit_random(uint32_t x) {
  // integer hash (multiply-xorshift) to a value in [-1, 1)
  x *= 0x9e3779b1u;
  x ^= x >> 15;
  x *= 0x85ebca77u;
  x ^= x >> 13;
  return (float)(x & 0xffffu) * (1.f / 32768.f) - 1.f;
}

__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_probe_kernel(
    float* __restrict__ sink, unsigned long long* __restrict__ clk, int iters) {
  const int tid = threadIdx.x;
  const uint32_t seed = (uint32_t)(blockIdx.x * kProbeThreads + tid) * 64u;
  bf16x8 a[8], b[2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) a[i][e] = (__bf16)unit_random(seed + 8 * i + e);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) b[i][e] = (__bf16)unit_random(seed + 7919u + 8 * i + e);
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = (f32x16){};

  const unsigned long long t0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kMfmaPerIter; ++i)
      acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i >> 2], acc[i & 3], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * kProbeThreads + tid] = s;  // keeps the products live
  if (tid == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

int fa_probe_mfma_bf16(float* sink, unsigned long long* clk, int n_wg, int iters, hipStream_t stream) {
  if (!sink || !clk) return 1;
  if (n_wg < 1 || n_wg > (1 << 20) || iters < 1) return 2;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)n_wg), dim3(kProbeThreads), 0, stream, sink, clk, iters);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

double fa_probe_flop_per_wg_iter(void) {
  // 4 waves x 8 MFMAs x (2 * 32 * 32 * 16) FLOP
  return (double)(kProbeThreads / 64) * kMfmaPerIter * 2.0 * 32 * 32 * 16;
}

int fa_probe_threads(void) { return kProbeThreads; }

}  // extern "C"
