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

#include <type_traits>

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
  // LDS row strides in elements. K: +16 B, so the 16-byte fragment reads of 16 different rows in one LDS
  // pass land on distinct banks. V: +64 B, so the transposing reads of 4 consecutive rows x 64 B in one pass
  // land on distinct banks (with +32 B every second row overlapped and each read took two passes).
  static constexpr int kStrideK = D + 8;
  static constexpr int kStrideV = D + 32;
  static constexpr int kTileK = kBc * kStrideK;                 // elements per K buffer
  static constexpr int kTileV = kBc * kStrideV;
  static constexpr int kLdsBytes = 2 * (kTileK + kTileV) * 2;   // two buffers of each
  static constexpr int kChunksPerRow = D / 8;                   // 16-byte chunks per row
  static constexpr int kChunks = kBc * kChunksPerRow / kThreads;  // per thread, per tensor, per tile
  static constexpr int kDB = D / 16;                            // K-steps of the first product
  static constexpr int kCB = D / 32;                            // 32-column blocks of the output
};

// A raw buffer descriptor over [base, base + bytes): loads at offsets >= bytes return zero. gfx9-family
// descriptor flags word. Only the per-lane offset is range-checked, so a tile's start goes into the base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

template <int V>
using Int = std::integral_constant<int, V>;

// Lazy rescaling: the exponent reference m_ref only moves when some row's new maximum exceeds it by more
// than this (log2 units), so unnormalised weights stay <= 2^8 and the O rescale is skipped on most tiles.
// Any reference gives the same softmax; lse and 1/l use the final reference.
constexpr float kRescaleLog2 = 8.f;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int N, int BH, float scale) {
  using C = Bf16Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  lds_char* const smem = (lds_char*)smem_raw;
  // layout: K buffer 0 | K buffer 1 | V buffer 0 | V buffer 1

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

  // ---- K/V tile staging through registers: kChunks 16-byte chunks of K and of V per thread per tile.
  // The per-thread byte offset inside a tile never changes; the tile start is in the descriptor.
  int goff[C::kChunks];   // byte offset of chunk p inside a tile in device memory
  int soff_k[C::kChunks]; // byte offset of chunk p inside K buffer 0 in LDS
  int soff_v[C::kChunks]; // byte offset of chunk p inside V buffer 0 in LDS
#pragma unroll
  for (int p = 0; p < C::kChunks; ++p) {
    const int c = tid + kThreads * p;
    const int row = c / C::kChunksPerRow, col = (c % C::kChunksPerRow) * 8;
    goff[p] = (row * D + col) * 2;
    soff_k[p] = (row * C::kStrideK + col) * 2;
    soff_v[p] = 2 * C::kTileK * 2 + (row * C::kStrideV + col) * 2;
  }
  u32x4 kreg[C::kChunks], vreg[C::kChunks];
  auto load_tile = [&](int j) {
    const int bytes = min(N - j * kBc, kBc) * D * 2;          // rows past N read as zero
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kh + (size_t)j * kBc * D, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vh + (size_t)j * kBc * D, bytes);
#pragma unroll
    for (int p = 0; p < C::kChunks; ++p) {
      kreg[p] = __builtin_amdgcn_raw_buffer_load_b128(kr, goff[p], 0, 0);
      vreg[p] = __builtin_amdgcn_raw_buffer_load_b128(vr, goff[p], 0, 0);
    }
  };
  auto store_tile = [&](auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
#pragma unroll
    for (int p = 0; p < C::kChunks; ++p) {
      *(__attribute__((address_space(3))) u32x4*)(smem + soff_k[p] + BUF * C::kTileK * 2) = kreg[p];
      *(__attribute__((address_space(3))) u32x4*)(smem + soff_v[p] + BUF * C::kTileV * 2) = vreg[p];
    }
  };

  // K row this lane feeds to the first product: bits 2 and 3 of l32 swapped.
  const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  // This lane's K fragment reads and transposing V reads (buffer 0).
  const lds_char* const k_rd = smem + (krow * C::kStrideK + 8 * h) * 2;
  const lds_char* const v_rd =
      smem + 2 * C::kTileK * 2 +
      ((8 * h + (lane & 15) / 4) * C::kStrideV + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  const float c2 = scale * kLog2e;
  float m_ref = -INFINITY;  // exponent reference (raw-score units) for row my_q
  float l_run = 0.f;        // this lane's share of the running sum (the keys it holds)
  f32x16 oacc[C::kCB];
#pragma unroll
  for (int cb = 0; cb < C::kCB; ++cb) oacc[cb] = (f32x16){};

  auto compute_tile = [&](int j, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int kv0 = j * kBc;
    const lds_char* ks = k_rd + BUF * C::kTileK * 2;
    const lds_char* vs = v_rd + BUF * C::kTileV * 2;

    // ---- S^T = K Q^T for keys kv0 .. kv0+63 (two 32-key blocks)
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = (f32x16){};
#pragma unroll
      for (int kb = 0; kb < C::kDB; ++kb) {
        const bf16x8 kf =
            *(const __attribute__((address_space(3))) bf16x8*)(ks + (32 * b * C::kStrideK + 16 * kb) * 2);
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
    mx = pair_max32(mx);  // row max over this tile's 64 keys
    const bool grow = (m_ref == -INFINITY) || ((mx - m_ref) * c2 > kRescaleLog2);
    if (__any(grow)) {
      const float m_new = fmaxf(m_ref, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // no visible key yet: any finite reference
      const float alpha = __builtin_amdgcn_exp2f((m_ref - m_use) * c2);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < C::kCB; ++cb) oacc[cb] *= alpha;
      m_ref = m_use;
    }
    const float nb = -m_ref * c2;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8 pf[4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x16 p;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c2, nb));
        rs[r & 3] += p[r];
      }
      pf[2 * b] = __builtin_convertvector(p.lo, bf16x8);
      pf[2 * b + 1] = __builtin_convertvector(p.hi, bf16x8);
    }
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);

    // ---- O^T += V^T P^T: 4 K-steps of 16 keys; lane slot 8h+e <-> key kv0 + 16m + 8h + e
#pragma unroll
    for (int cb = 0; cb < C::kCB; ++cb) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const lds_char* va = vs + ((16 * m) * C::kStrideV + 32 * cb) * 2;
        const bf16x4 v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(va));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(va + 4 * C::kStrideV * 2));
        const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[m], oacc[cb], 0, 0, 0);
      }
    }
  };

  // One tile: prefetch tile j+1 into registers, compute tile j from LDS buffer BUF, then write tile j+1 into
  // the other buffer; one barrier per tile. Waves whose rows lie entirely above tile j (causal) only help
  // with the copy.
  auto step = [&](int j, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const bool more = (j + 1) < n_tiles;
    if (more) load_tile(j + 1);
    const bool active = (q0w < N) && (!CAUSAL || j * kBc <= q0w + kRowsPerWave - 1);
    if (active) compute_tile(j, bufc);
    if (more) store_tile(Int<BUF ^ 1>{});
    __syncthreads();
  };

  load_tile(0);
  store_tile(Int<0>{});
  __syncthreads();
  for (int j = 0; j < n_tiles; j += 2) {
    step(j, Int<0>{});
    if (j + 1 < n_tiles) step(j + 1, Int<1>{});
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
    if (h == 0) lse[(size_t)bh * N + my_q] = (m_ref * c2 + __builtin_amdgcn_logf(l_tot)) * kLn2;
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
