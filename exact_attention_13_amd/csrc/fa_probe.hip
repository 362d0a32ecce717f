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

// Issue-mix probe: 8-wave workgroups (waves w and w + 4 share a SIMD), one per CU when launched 256 wide. Per loop
// iteration a wave issues, by mode:
//   0: 8 MFMAs (8 independent accumulators)
//   1: 8 MFMAs and 8 exp2
//   2: 8 MFMAs, 8 exp2 and 24 FMAs (the softmax's ratio of exponentials and other vector work to products)
//   3: waves 0-3 the 8 MFMAs of mode 0, waves 4-7 the 8 exp2 and 24 FMAs of mode 2 (one role per wave of a SIMD)
//   4: 8 exp2 and 24 FMAs
// The exp2 and FMA chains are independent of the products; each wave records its shader cycles over the loop.
constexpr int kMixThreads = 512;

// One wave's loop: per iteration 8 products (MF), 8 exp2 (EX) and 24 FMAs (FM), each set compiled in or out.
template <bool MF, bool EX, bool FM>
__device__ __forceinline__ void mix_loop(f32x16 (&acc)[8], float (&x)[8], bf16x8 a, bf16x8 b, int iters) {
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (MF) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
      if constexpr (EX) x[i] = __builtin_amdgcn_exp2f(-x[i]);
      if constexpr (FM) {
        x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
        x[i] = __builtin_fmaf(x[i], 0.998f, 0.002f);
        x[i] = __builtin_fmaf(x[i], 0.997f, 0.003f);
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kMixThreads) void issue_mix_kernel(float* __restrict__ sink,
                                                                unsigned long long* __restrict__ cyc, int iters) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: a role is a whole loop
  const uint32_t seed = (uint32_t)(blockIdx.x * kMixThreads + tid) * 64u;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)unit_random(seed + e);
    b[e] = (__bf16)unit_random(seed + 31u + e);
  }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = (f32x16){};
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.25f * unit_random(seed + 97u + i);
  __syncthreads();
  const unsigned long long t0 = __builtin_readcyclecounter();
  if constexpr (MODE == 0) mix_loop<true, false, false>(acc, x, a, b, iters);
  if constexpr (MODE == 1) mix_loop<true, true, false>(acc, x, a, b, iters);
  if constexpr (MODE == 2) mix_loop<true, true, true>(acc, x, a, b, iters);
  if constexpr (MODE == 3) {
    if (wave < 4) {
      mix_loop<true, false, false>(acc, x, a, b, iters);
    } else {
      mix_loop<false, true, true>(acc, x, a, b, iters);
    }
  }
  if constexpr (MODE == 4) mix_loop<false, true, true>(acc, x, a, b, iters);
  const unsigned long long t1 = __builtin_readcyclecounter();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i] + acc[i][0] + acc[i][15];
  sink[blockIdx.x * kMixThreads + tid] = s;
  if ((tid & 63) == 0) cyc[blockIdx.x * (kMixThreads / 64) + wave] = t1 - t0;
}

// Atomic-add probe: the rate of fp32 atomic adds (global_atomic_add_f32, no return) into device memory, in 64 KiB
// tiles of 16384 floats, the size of a 128 x 128 fp32 block. 8-wave workgroups; per round a workgroup adds 1.0 to
// every float of one tile, each lane 32 floats 512 apart (coalesced). The tile a workgroup takes in round r:
//   0: (7 wg + r) mod T                          distinct tiles in a round, each reached from any XCD
//   1: (wg mod 8) + 8 ((wg / 8 + r) mod (T/8))   tile t only from workgroups wg = t (mod 8), which the dispatcher
//                                                places on one XCD (workgroups go round-robin over the 8 XCDs)
//   2: (wg / 32 + r) mod T                       32 consecutive workgroups (every XCD) on the same tile at once
//   3: as 0, plain stores of 1.0 instead of atomic adds (the write rate to compare with)
constexpr int kAtomThreads = 512;
constexpr int kAtomTileFloats = 16384;

template <int MODE>
__global__ __launch_bounds__(kAtomThreads) void atomic_add_probe_kernel(float* __restrict__ buf, int tiles,
                                                                        int rounds) {
  const int wg = blockIdx.x, tid = threadIdx.x;
  for (int r = 0; r < rounds; ++r) {
    int tile;
    if constexpr (MODE == 1) {
      tile = (wg & 7) + 8 * ((wg / 8 + r) % (tiles / 8));
    } else if constexpr (MODE == 2) {
      tile = (wg / 32 + r) % tiles;
    } else {
      tile = (int)(((long long)wg * 7 + r) % tiles);
    }
    float* p = buf + (size_t)tile * kAtomTileFloats + tid;
#pragma unroll
    for (int i = 0; i < kAtomTileFloats / kAtomThreads; ++i) {
      if constexpr (MODE == 3) {
        p[i * kAtomThreads] = 1.0f;
      } else {
        unsafeAtomicAdd(p + i * kAtomThreads, 1.0f);  // hardware fp32 add on device memory
      }
    }
  }
}

}  // namespace

extern "C" {

int fa_probe_issue_mix(int mode, float* sink, unsigned long long* cyc, int n_wg, int iters, hipStream_t stream) {
  if (!sink || !cyc) return 1;
  if (mode < 0 || mode > 4 || n_wg < 1 || n_wg > (1 << 20) || iters < 1) return 2;
  const dim3 grid((unsigned)n_wg), block(kMixThreads);
  switch (mode) {
    case 0: hipLaunchKernelGGL(issue_mix_kernel<0>, grid, block, 0, stream, sink, cyc, iters); break;
    case 1: hipLaunchKernelGGL(issue_mix_kernel<1>, grid, block, 0, stream, sink, cyc, iters); break;
    case 2: hipLaunchKernelGGL(issue_mix_kernel<2>, grid, block, 0, stream, sink, cyc, iters); break;
    case 3: hipLaunchKernelGGL(issue_mix_kernel<3>, grid, block, 0, stream, sink, cyc, iters); break;
    default: hipLaunchKernelGGL(issue_mix_kernel<4>, grid, block, 0, stream, sink, cyc, iters); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int fa_probe_issue_mix_threads(void) { return kMixThreads; }

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

int fa_probe_atomic_add(int mode, float* buf, int tiles, int n_wg, int rounds, hipStream_t stream) {
  if (!buf) return 1;
  if (mode < 0 || mode > 3 || tiles < 8 || tiles % 8 != 0 || tiles > (1 << 16) || n_wg < 1 || n_wg > (1 << 20) ||
      rounds < 1)
    return 2;
  const dim3 grid((unsigned)n_wg), block(kAtomThreads);
  switch (mode) {
    case 0: hipLaunchKernelGGL(atomic_add_probe_kernel<0>, grid, block, 0, stream, buf, tiles, rounds); break;
    case 1: hipLaunchKernelGGL(atomic_add_probe_kernel<1>, grid, block, 0, stream, buf, tiles, rounds); break;
    case 2: hipLaunchKernelGGL(atomic_add_probe_kernel<2>, grid, block, 0, stream, buf, tiles, rounds); break;
    default: hipLaunchKernelGGL(atomic_add_probe_kernel<3>, grid, block, 0, stream, buf, tiles, rounds); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int fa_probe_atomic_tile_floats(void) { return kAtomTileFloats; }

}  // extern "C"
