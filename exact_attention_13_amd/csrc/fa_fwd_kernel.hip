// fa_fwd_kernel.hip -- exact fused attention forward for gfx950 (MI355X, CDNA4).
//
// Computes o = softmax(scale * q k^T [causal]) v and lse = ln sum exp(scale * q k^T) tile by tile with a
// running row maximum m and running row sum l (unite.ai page "Flash Attention: revolutionizing transformer
// efficiency": "Flash Attention Algorithm", "The Math Behind Flash Attention" items 1-2, "Implementation
// Details"), so the N x N score matrix never leaves registers. The FlashAttention-2 changes listed on the
// systems-analysis.info page "FlashAttention-2 (VI)" (section "Kiến trúc kỹ thuật và nguyên lý hoạt động",
// items 1-3) are kept: the 1/l division happens once per row at the end, workgroups are spread over blocks
// of query rows as well as over batch x heads, and inside a workgroup each wave owns its own query rows
// (no cross-wave reduction, K/V tiles shared read-only through LDS).
//
// gfx950 mapping (one workgroup = 4 waves = 128 query rows; one wave = 32 query rows):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (fp32 accumulate). With S transposed, lane l of a wave holds
//     scores of query row (l % 32) only, so the row max needs one exchange between lanes l and l ^ 32
//     (v_permlane32_swap) and the row sum needs none until the end.
//   * The S^T accumulator is, after conversion to bf16, exactly the B operand of O^T = V^T P^T on the same
//     MFMA shape. The K rows are fed to the first product in an order that swaps bits 2 and 3 of the row
//     index, which makes the 8 keys a lane holds for the second product contiguous.
//   * The V^T operand is read from row-major V in LDS with ds_read_b64_tr_b16 (transposing LDS read).
//   * O^T accumulates per lane for one query row, so the rescale by alpha = exp2(m_old - m_new) is a
//     per-lane scalar multiply.
//   * exp2 with log2(e) folded into the scale: p = exp2(s * c - m * c), c = scale * log2(e), one FMA.
//   * K/V tiles of 64 keys are double-buffered in LDS: the global loads for tile j+1 are issued before the
//     MFMAs of tile j and written to the other buffer after them; one barrier per tile.
//   * Causal: a workgroup visits only key tiles that meet its rows, a wave skips tiles entirely above its
//     rows, and the mask is applied only on tiles that cross the diagonal or the sequence end.
//   * The linear workgroup id is remapped so that (when B*H is a multiple of 8) every query block of a head
//     runs on the same XCD (workgroups are dealt to the 8 XCDs round-robin) and shares that XCD's L2, and
//     causal work starts with the longest query blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBc = 64;                     // keys per K/V tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_permlane32_swap exchanges the upper 32 lanes of its first operand with the lower 32 lanes of its second.
// Fed x twice, every lane ends up holding {x[l], x[l ^ 32]} across the two results, in an order that depends
// on the half; max and sum of the two are therefore the pair reductions for every lane.
__device__ __forceinline__ float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup -> (head bh, query block qb). Workgroups are dispatched to XCDs round-robin by linear id.
__device__ __forceinline__ void map_workgroup(int lin, int nq, int bh_count, bool causal, int& bh, int& qb) {
  if ((bh_count & 7) == 0) {
    const int xcd = lin & 7, t = lin >> 3, per = bh_count >> 3;  // heads per XCD
    if (causal) {
      qb = nq - 1 - t / per;
      bh = xcd + 8 * (t % per);
    } else {
      bh = xcd + 8 * (t / nq);
      qb = t % nq;
    }
  } else {
    if (causal) {
      qb = nq - 1 - lin / bh_count;
      bh = lin % bh_count;
    } else {
      bh = lin / nq;
      qb = lin % nq;
    }
  }
}

// ------------------------------------------------------------------------------------------------------------
// bf16 kernel
// ------------------------------------------------------------------------------------------------------------
template <int D>
struct Bf16Cfg {
  static constexpr int kStrideK = D + 8;   // LDS row stride of K in elements (+16 B: 16-B reads of 16 rows hit
                                           // distinct banks)
  static constexpr int kStrideV = D + 16;  // LDS row stride of V (+32 B: the transposing reads of 4 rows x
                                           // 32 B hit distinct banks)
  static constexpr int kTileK = kBc * kStrideK;
  static constexpr int kTileV = kBc * kStrideV;
  static constexpr int kLdsBytes = 2 * (kTileK + kTileV) * 2;
  static constexpr int kChunksPerRow = D / 8;                         // 16-byte chunks per row
  static constexpr int kChunks = kBc * kChunksPerRow / kThreads;      // per thread per tensor per tile
  static constexpr int kDB = D / 16;                                  // K-steps of the first product
  static constexpr int kCB = D / 32;                                  // 32-column blocks of the output
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int N, int BH, float scale) {
  using C = Bf16Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  lds_char* smem = (lds_char*)smem_raw;
  lds_char* ks_base = smem;                                 // 2 buffers of K [kBc][kStrideK]
  lds_char* vs_base = smem + 2 * C::kTileK * 2;             // 2 buffers of V [kBc][kStrideV]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;

  const int nq = gridDim.x;
  int bh, qb;
  map_workgroup(blockIdx.x + nq * blockIdx.y, nq, BH, CAUSAL, bh, qb);

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const __bf16* qh = q + head_off;
  const __bf16* kh = k + head_off;
  const __bf16* vh = v + head_off;

  const int q_lo = qb * kBr;
  const int q_last = min(q_lo + kBr, N) - 1;                 // last real query row of the workgroup
  const int n_tiles = CAUSAL ? (q_last / kBc + 1) : (N + kBc - 1) / kBc;
  const int q0w = q_lo + wave * kRowsPerWave;                 // first query row of this wave
  const int my_q = q0w + l32;                                 // query row of this lane

  // ---- Q fragments: lane holds q[my_q][16*kb + 8*h .. +7] (B operand of S^T = K Q^T)
  bf16x8 qf[C::kDB];
#pragma unroll
  for (int kb = 0; kb < C::kDB; ++kb) {
    if (my_q < N) {
      qf[kb] = *(const bf16x8*)(qh + (size_t)my_q * D + 16 * kb + 8 * h);
    } else {
      qf[kb] = (bf16x8){};
    }
  }

  // ---- K/V tile staging: each thread moves kChunks 16-byte chunks of K and of V per tile
  u32x4 kreg[C::kChunks], vreg[C::kChunks];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int p = 0; p < C::kChunks; ++p) {
      const int c = tid + kThreads * p;
      const int row = c / C::kChunksPerRow, col = (c % C::kChunksPerRow) * 8;
      const int key = j * kBc + row;
      if (key < N) {
        kreg[p] = *(const u32x4*)(kh + (size_t)key * D + col);
        vreg[p] = *(const u32x4*)(vh + (size_t)key * D + col);
      } else {
        kreg[p] = (u32x4){0u, 0u, 0u, 0u};
        vreg[p] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
    lds_char* ks = ks_base + buf * C::kTileK * 2;
    lds_char* vs = vs_base + buf * C::kTileV * 2;
#pragma unroll
    for (int p = 0; p < C::kChunks; ++p) {
      const int c = tid + kThreads * p;
      const int row = c / C::kChunksPerRow, col = (c % C::kChunksPerRow) * 8;
      *(__attribute__((address_space(3))) u32x4*)(ks + (row * C::kStrideK + col) * 2) = kreg[p];
      *(__attribute__((address_space(3))) u32x4*)(vs + (row * C::kStrideV + col) * 2) = vreg[p];
    }
  };

  // K row this lane feeds to the first product: bits 2 and 3 of l32 swapped.
  const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  // Byte offsets (within a buffer) of this lane's K fragment reads and transposing V reads.
  const int k_off = (krow * C::kStrideK + 8 * h) * 2;
  const int v_off = ((8 * h + (lane & 15) / 4) * C::kStrideV + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  const float c2 = scale * kLog2e;
  float m_run = -INFINITY;  // running max of raw scores q.k for row my_q
  float l_run = 0.f;        // this lane's share of the running sum (keys it holds)
  f32x16 oacc[C::kCB];
#pragma unroll
  for (int cb = 0; cb < C::kCB; ++cb) oacc[cb] = (f32x16){};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const bool more = (j + 1) < n_tiles;
    if (more) load_tile(j + 1);

    const int kv0 = j * kBc;
    const bool active = (q0w < N) && (!CAUSAL || kv0 <= q0w + kRowsPerWave - 1);
    if (active) {
      const lds_char* ks = ks_base + buf * C::kTileK * 2;
      const lds_char* vs = vs_base + buf * C::kTileV * 2;

      // ---- S^T = K Q^T for keys kv0 .. kv0+63 (two 32-key blocks)
      f32x16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[b] = (f32x16){};
#pragma unroll
        for (int kb = 0; kb < C::kDB; ++kb) {
          const bf16x8 kf =
              *(const __attribute__((address_space(3))) bf16x8*)(ks + k_off + (32 * b * C::kStrideK + 16 * kb) * 2);
          s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kb], s[b], 0, 0, 0);
        }
      }
      // s[b][r] is the score of query my_q and key kv0 + 32b + 16(r/8) + 8h + r%8.

      // ---- mask (only tiles that cross the diagonal or the end of the sequence)
      const bool need_mask = (kv0 + kBc > N) || (CAUSAL && kv0 + kBc - 1 > q0w);
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * b + 16 * (r >> 3) + 8 * h + (r & 7);
            const bool vis = (key < N) && (!CAUSAL || key <= my_q);
            s[b][r] = vis ? s[b][r] : -INFINITY;
          }
      }

      // ---- online softmax statistics
      float mx = s[0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
      mx = pair_max32(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // a row with no visible key so far
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      const float nb = -m_use * c2;
      float rowsum = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x16 p;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c2, nb));
          rowsum += p[r];
        }
        pf[2 * b] = __builtin_convertvector(p.lo, bf16x8);
        pf[2 * b + 1] = __builtin_convertvector(p.hi, bf16x8);
      }
      l_run = l_run * alpha + rowsum;
      m_run = m_new;
#pragma unroll
      for (int cb = 0; cb < C::kCB; ++cb) oacc[cb] *= alpha;

      // ---- O^T += V^T P^T: 4 K-steps of 16 keys; lane slot 8h+e <-> key kv0 + 16m + 8h + e
#pragma unroll
      for (int cb = 0; cb < C::kCB; ++cb) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const lds_char* va = vs + v_off + ((16 * m) * C::kStrideV + 32 * cb) * 2;
          const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(va));
          const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(va + 4 * C::kStrideV * 2));
          const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[m], oacc[cb], 0, 0, 0);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: o = acc / l once per row, lse = m*scale + ln l
  const float l_tot = pair_sum32(l_run);
  if (my_q < N) {
    const float inv = 1.f / l_tot;
    __bf16* orow = o + head_off + (size_t)my_q * D;
#pragma unroll
    for (int cb = 0; cb < C::kCB; ++cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // oacc[cb][4g + i] is column 32cb + 8g + 4h + i of row my_q
        f32x4 x = {oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv, oacc[cb][4 * g + 2] * inv,
                   oacc[cb][4 * g + 3] * inv};
        *(bf16x4*)(orow + 32 * cb + 8 * g + 4 * h) = __builtin_convertvector(x, bf16x4);
      }
    }
    if (h == 0) {
      const float m_fin = (m_run == -INFINITY) ? 0.f : m_run;
      lse[(size_t)bh * N + my_q] = (m_fin * c2 + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------------------------------------------------
// fp32 kernel: same decomposition on v_mfma_f32_32x32x2f32 (one fp32 per lane per operand), single-buffered
// ------------------------------------------------------------------------------------------------------------
template <int D>
struct F32Cfg {
  static constexpr int kStrideK = D + 1;  // odd stride: the column reads of 32 rows spread over the banks
  static constexpr int kStrideV = D + 4;
  static constexpr int kLdsBytes = kBc * (kStrideK + kStrideV) * 4;
  static constexpr int kChunksPerRow = D / 4;                    // 16-byte chunks per row
  static constexpr int kChunks = kBc * kChunksPerRow / kThreads;
  static constexpr int kCB = D / 32;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_fwd_f32_kernel(const float* __restrict__ q,
                                                              const float* __restrict__ k,
                                                              const float* __restrict__ v, float* __restrict__ o,
                                                              float* __restrict__ lse, int N, int BH, float scale) {
  using C = F32Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  __attribute__((address_space(3))) float* ks = (__attribute__((address_space(3))) float*)smem_raw;
  __attribute__((address_space(3))) float* vs = ks + kBc * C::kStrideK;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int nq = gridDim.x;
  int bh, qb;
  map_workgroup(blockIdx.x + nq * blockIdx.y, nq, BH, CAUSAL, bh, qb);

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const int q_lo = qb * kBr;
  const int q_last = min(q_lo + kBr, N) - 1;
  const int n_tiles = CAUSAL ? (q_last / kBc + 1) : (N + kBc - 1) / kBc;
  const int q0w = q_lo + wave * kRowsPerWave;
  const int my_q = q0w + l32;

  // Q fragments: lane holds q[my_q][2*kb + h]
  float qf[D / 2];
#pragma unroll
  for (int kb = 0; kb < D / 2; ++kb) qf[kb] = (my_q < N) ? q[head_off + (size_t)my_q * D + 2 * kb + h] : 0.f;

  const float c2 = scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[C::kCB];
#pragma unroll
  for (int cb = 0; cb < C::kCB; ++cb) oacc[cb] = (f32x16){};

  for (int j = 0; j < n_tiles; ++j) {
    const int kv0 = j * kBc;
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int p = 0; p < C::kChunks; ++p) {
      const int c = tid + kThreads * p;
      const int row = c / C::kChunksPerRow, col = (c % C::kChunksPerRow) * 4;
      const int key = kv0 + row;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key < N) {
        kx = *(const f32x4*)(k + head_off + (size_t)key * D + col);
        vx = *(const f32x4*)(v + head_off + (size_t)key * D + col);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ks[row * C::kStrideK + col + e] = kx[e];
      *(__attribute__((address_space(3))) f32x4*)(vs + row * C::kStrideV + col) = vx;
    }
    __syncthreads();

    const bool active = (q0w < N) && (!CAUSAL || kv0 <= q0w + kRowsPerWave - 1);
    if (!active) continue;

    // S^T = K Q^T: s[b][r] is the score of query my_q and key kv0 + 32b + 8(r/4) + 4h + r%4
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = (f32x16){};
#pragma unroll
      for (int kb = 0; kb < D / 2; ++kb)
        s[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[(32 * b + l32) * C::kStrideK + 2 * kb + h], qf[kb], s[b], 0,
                                                   0, 0);
    }
    const bool need_mask = (kv0 + kBc > N) || (CAUSAL && kv0 + kBc - 1 > q0w);
    if (need_mask) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool vis = (key < N) && (!CAUSAL || key <= my_q);
          s[b][r] = vis ? s[b][r] : -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
    mx = pair_max32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
    const float nb = -m_use * c2;
    float rowsum = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[b][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c2, nb));
        rowsum += s[b][r];
      }
    l_run = l_run * alpha + rowsum;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < C::kCB; ++cb) oacc[cb] *= alpha;
    // O^T += V^T P^T, one key pair per MFMA: lane slot h <-> key kv0 + 32b + 8(r/4) + 4h + r%4
#pragma unroll
    for (int cb = 0; cb < C::kCB; ++cb)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key_local = 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key_local * C::kStrideV + 32 * cb + l32], s[b][r],
                                                         oacc[cb], 0, 0, 0);
        }
  }

  const float l_tot = pair_sum32(l_run);
  if (my_q < N) {
    const float inv = 1.f / l_tot;
    float* orow = o + head_off + (size_t)my_q * D;
#pragma unroll
    for (int cb = 0; cb < C::kCB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv, oacc[cb][4 * g + 2] * inv,
                   oacc[cb][4 * g + 3] * inv};
        *(f32x4*)(orow + 32 * cb + 8 * g + 4 * h) = x;
      }
    if (h == 0) {
      const float m_fin = (m_run == -INFINITY) ? 0.f : m_run;
      lse[(size_t)bh * N + my_q] = (m_fin * c2 + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------------------------------------------------
// launchers (arguments already validated by the C ABI layer)
// ------------------------------------------------------------------------------------------------------------
template <int D, bool CAUSAL>
static hipError_t launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                              float scale, hipStream_t stream) {
  constexpr int lds = Bf16Cfg<D>::kLdsBytes;
  auto kern = fa_fwd_bf16_kernel<D, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + kBr - 1) / kBr), (unsigned)BH);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, (const __bf16*)q, (const __bf16*)k,
                     (const __bf16*)v, (__bf16*)o, lse, N, BH, scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N,
                             float scale, hipStream_t stream) {
  constexpr int lds = F32Cfg<D>::kLdsBytes;
  auto kern = fa_fwd_f32_kernel<D, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + kBr - 1) / kBr), (unsigned)BH);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, q, k, v, o, lse, N, BH, scale);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                           bool causal, float scale, hipStream_t stream) {
  if (d == 64) return causal ? launch_bf16<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                             : launch_bf16<64, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch_bf16<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_bf16<128, false>(q, k, v, o, lse, BH, N, scale, stream);
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N, int d,
                          bool causal, float scale, hipStream_t stream) {
  if (d == 64) return causal ? launch_f32<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                             : launch_f32<64, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch_f32<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_f32<128, false>(q, k, v, o, lse, BH, N, scale, stream);
}

int query_rows_per_workgroup() { return kBr; }

}  // namespace fa
