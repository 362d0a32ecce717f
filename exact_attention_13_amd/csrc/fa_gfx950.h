// fa_gfx950.h -- device helpers shared by the attention kernels for gfx950 (MI355X, CDNA4): vector types,
// lane-pair reductions, raw buffer descriptors, LDS-DMA tile copies and the copy-wait barrier.
#ifndef FA_MI355X_FA_GFX950_H
#define FA_MI355X_FA_GFX950_H
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// v_permlane32_swap exchanges the upper 32 lanes of its first operand with the lower 32 lanes of its second.
// Fed x twice, every lane ends up holding {x[l], x[l ^ 32]} across the two results, in an order that depends
// The maximum of the row-max reductions: IEEE 754-2019 maximum (v_maximum3_f32 on gfx950), which propagates a
// NaN where fmaxf would skip it and needs no quieting instructions before each chain (fmaxf costs two).
__device__ __forceinline__ float row_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// on the half; max and sum of the two are therefore the pair reductions for every lane.
__device__ __forceinline__ float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return row_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A raw buffer descriptor over [base, base + bytes): loads at offsets >= bytes return zero (also when the
// destination is LDS). gfx9-family descriptor flags word. Only the per-lane offset is range-checked, so a tile's
// start goes into the base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// One LDS-DMA copy: each lane moves 16 bytes from the descriptor's range at byte offset `off` to
// lds_base + 16 * lane (lds_base must be the same for the whole wave). Kept in a plain (non-template) function:
// written directly inside the kernel template, the builtin made the host compilation pass drop the kernel's
// launch stub without a diagnostic.
__device__ __forceinline__ void lds_copy16_inline(__amdgpu_buffer_rsrc_t r, lds_char* lds_base, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, off, 0, 0, 0);
}

// Workgroup -> (head bh, query block qb). Workgroups are dispatched to XCDs round-robin by linear id. When B*H
// is a multiple of 8, XCD x takes the key/value heads x, x+8, x+16, ... (each with its `group` query heads) when
// their count is a multiple of 8, else the query heads x, x+8, ...: a group's query heads share an L2, and heads
// of every batch run on every XCD (per-batch work differs under key padding).
__device__ __forceinline__ void map_workgroup(int lin, int nq, int bh_count, int group, bool causal, int& bh,
                                              int& qb) {
  if ((bh_count & 7) == 0) {
    const int xcd = lin & 7, t = lin >> 3, per = bh_count >> 3;  // heads per XCD
    int jh;                                                      // this XCD's jh-th head
    if (causal) {
      qb = nq - 1 - t / per;
      jh = t % per;
    } else {
      jh = t / nq;
      qb = t % nq;
    }
    bh = ((bh_count / group) & 7) == 0 ? (xcd + 8 * (jh / group)) * group + jh % group : xcd + 8 * jh;
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

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}
__device__ __forceinline__ int wave_max_i32(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

// Packed batches of at most 64 sequences: the work items (sequence b, block kb) of one head in decreasing order of
// their cost, nb_b - kb when `causal` (block kb of a causal kernel numbered from its most expensive end) and nb_b
// otherwise, ties by b, then kb, so that the longest items start first and the short ones fill in behind them. nb
// is this lane's sequence's block count (lane b holds sequence b; 0 past the last sequence). Returns false when
// `rank` is past the last item; all lanes get the same result.
__device__ bool longest_first_item(int rank, int nb, bool causal, int& b_out, int& kb_out) {
  const int lane = threadIdx.x & 63;
  const int total = wave_sum_i32(nb);  // one item per key block
  if (rank >= total) return false;
  // items with more than W visited tiles
  auto above = [&](int W) { return wave_sum_i32(causal ? max(0, nb - W) : (nb > W ? nb : 0)); };
  int lo = 1, hi = max(wave_max_i32(nb), 1);  // above(hi) = 0 <= rank < total = above(0)
  while (lo < hi) {  // the smallest W >= 1 with above(W) <= rank: the work of item `rank`
    const int mid = (lo + hi) / 2;
    if (above(mid) <= rank) hi = mid; else lo = mid + 1;
  }
  const int W = lo, j = rank - above(W);  // position inside that work level
  // causal: each sequence with nb >= W holds one item of work W (kb = nb - W); otherwise each sequence with nb == W
  // holds W of them
  const bool in_level = causal ? (nb >= W) : (nb == W);
  const uint64_t mask = __ballot(in_level);
  const int s = causal ? j : j / W;  // which sequence of the level, in index order
  const int before = __popcll(mask & ((1ull << lane) - 1ull));
  const uint64_t pick = __ballot(in_level && before == s);
  const int b = __builtin_ctzll(pick);
  const int nb_b = __shfl(nb, b);
  b_out = b;
  kb_out = causal ? nb_b - W : j % W;
  return true;
}

// Packed batches: workgroup `lin` -> (item rank, query head hq). Consecutive groups of 8 workgroups land on the 8
// XCDs; with H a multiple of 8, XCD x takes the key/value heads x, x+8, ... with all their query heads (when H/group
// is a multiple of 8), else the query heads x, x+8, ..., as map_workgroup does for B*H heads.
__device__ __forceinline__ void map_packed(int lin, int H, int group, int& rank, int& hq) {
  if ((H & 7) == 0) {
    const int xcd = lin & 7, t = lin >> 3, per = H >> 3;
    const int slot = t % per;
    rank = t / per;
    hq = ((H / group) & 7) == 0 ? (xcd + 8 * (slot / group)) * group + slot % group : xcd + 8 * slot;
  } else {
    rank = lin / H;
    hq = lin % H;
  }
}

// The block counts (rows per block `rows`) of the sequences of a packed batch, lane b holding sequence b's; offsets
// clamped to [0, T_total], lengths to N.
__device__ __forceinline__ int packed_blocks(const int* cu_seqlens, int nbatch, int T_total, int N, int rows) {
  const int lane = threadIdx.x & 63;
  if (lane >= nbatch) return 0;
  const int lo = min(max(cu_seqlens[lane], 0), T_total);
  const int hi = min(max(cu_seqlens[lane + 1], lo), T_total);
  return (min(hi - lo, N) + rows - 1) / rows;
}

template <int V>
using Int = std::integral_constant<int, V>;

// Wait until at most N vector-memory operations of this wave are outstanding (the LDS-DMA copies), then join
// the workgroup. The barrier is written as a statement with a memory clobber: the compiler may not move memory
// accesses across it, and no fence is emitted (a release fence would wait for every copy in flight, including
// the ones meant to overlap the next tile).
template <int N>
__device__ __forceinline__ void wait_copies_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  // s_waitcnt fields (gfx9): vmcnt[3:0] and [15:14], expcnt[6:4] = 7 (no wait), lgkmcnt[11:8] = 0 (LDS reads done)
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  asm volatile("s_barrier" ::: "memory");
}

}  // namespace fa
#endif
