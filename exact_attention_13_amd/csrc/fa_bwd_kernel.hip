// fa_bwd_kernel.hip -- gradients of the exact attention forward for gfx950 (MI355X, CDNA4).
//
// The pages name a faster backward pass and the recomputation of the attention matrix from stored statistics
// instead of storing it (unite.ai page "Flash Attention: revolutionizing transformer efficiency": the key ideas
// after "Enter Flash Attention", item 2; "FlashAttention-2", item 2). With the forward's lse and an upstream
// gradient dO of o, per query row i and visible key j:
//     p_ij = exp(scale q_i.k_j - lse_i),  D_i = dO_i . o_i,  dS_ij = p_ij (dO_i . v_j - D_i)
//     dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i p_ij dO_i
// (dk, dv summed over the query heads of a key/value group). Two kernels, neither with atomics, so every call
// gives the same bits:
//   * fa_bwd_dq_kernel: one workgroup per block of 256 query rows (8 waves x 32 rows), K/V tiles of 64 keys
//     streamed through LDS exactly like the forward. S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_32x32x16_bf16
//     put one query row in each lane, so p = exp2(s*c - lse*log2e) and dS^T = p (dP^T - D) need only the lane's
//     own lse and D (the dP^T accumulators start at -D, so the products leave dP^T - D); dQ^T += K^T dS^T takes
//     dS^T from registers as the B operand and K^T by transposing LDS reads
//     (ds_read_b64_tr_b16). It also computes D_i from the o and dO rows it loads anyway and writes (-D_i,
//     lse_i*log2e) to the workspace.
//   * fa_bwd_dkdv_kernel: one workgroup per block of 128 keys of one key/value head, 8 waves: each block of 32
//     keys belongs to a pair of waves on one SIMD, one accumulating dV (from S and p), the other dK (from dP and
//     dS), so each holds half the accumulators and two waves share every SIMD. Query tiles of 128 rows (q, dO
//     and the workspace values) of every query head of the group stream through LDS. S = Q K^T and dP = dO V^T
//     put one key in each lane (K or V rows stay in registers as the B operand); dV^T += dO^T P and
//     dK^T += Q^T dS take P and dS from registers as B operands and dO^T, Q^T by transposing LDS reads; p
//     passes from the first wave of the pair to the second through LDS.
// The workspace holds -D_i and lse_i*log2e as two planes per head, [B*H][2][Npad] float, Npad = N rounded up to
// 128; rows N .. Npad-1 hold 0 and lse2 = +inf, which makes p (and dS) of those rows exactly 0 in the dk/dv
// kernel. With the planes apart, each wave of the dk/dv kernel reads from LDS only the plane it uses (the p wave
// lse2, the dS wave -D), half the bytes of reading interleaved pairs; -D goes straight into the dS wave's dP
// accumulators as their starting value, so the MFMAs leave dP - D with no subtraction.
// Key padding (the forward's per-batch count Nk of valid keys, triton-transformer README usage example "ex. BERT"):
// the dq kernel visits only the key tiles below Nk and masks keys >= Nk like the sequence end; the dk/dv kernel
// masks them, loads no k or v row past Nk and writes zero gradients for them. With Nk = 0 no tile is visited
// (o = 0, lse = -inf there), so every gradient of the batch is 0.
// Packed variable-length batches (VARLEN, the layout of the packed forward: q, o, dO, dq [T, H, d], k, v, dk, dv
// [T, Hkv, d], lse [H, T], sequence b = tokens cu[b] .. cu[b+1]-1, offsets clamped to [0, T]): rows of a head are
// H*d (Hkv*d) elements apart, every copy range ends with the sequence's last row, and workgroups whose query or
// key block lies past their sequence return at once, so no row of another sequence is read or written. The
// workspace keeps its layout, with N = max_seqlen as the per-head stride.
// S and dP are computed in both kernels (7 matrix products instead of the 5 of a single pass with atomic dq
// updates): the price of determinism.
//
// LDS tiles are read both row-wise (16 bytes per lane, A operands) and transposed (8 bytes per lane, 4
// rows x 64 bytes per 32 lanes). One XOR swizzle of the 16-byte chunks serves both without bank conflicts:
// chunk c of row r is stored at c ^ (4 (t % (CPR/4)) + (t / (CPR/4)) % 4), t = r / RPG (CPR = d/8 chunks per row,
// RPG = 16/CPR rows per 256 bytes).
#include "fa_gfx950.h"
#include "fa_launch.h"

namespace fa {

constexpr int kBwdRows = 32;                   // rows per wave: query rows (dq) or keys (dk, dv)
constexpr int kBwdBlock = 4 * kBwdRows;        // keys per dk/dv workgroup (4 wave pairs); workspace row granule
constexpr int kDqWaves = 8;                    // dq kernel: waves per workgroup
constexpr int kDqBlock = kDqWaves * kBwdRows;  // dq kernel: query rows per workgroup
constexpr int kBwdTile = 64;                   // keys per LDS tile (dq)
constexpr int kWsTileBytes = 1024;             // LDS slot for one tile of workspace values: 128 -D, then 128 lse2

// Workspace rows per head: N rounded up to 128, a whole number of the dk/dv kernel's 128-row query tiles. The dq
// grid covers them all (padding rows included) and skips its own rows past them.
__host__ __device__ constexpr int ws_rows(int N) { return (N + kBwdBlock - 1) / kBwdBlock * kBwdBlock; }

template <int D, int ROWS = kBwdTile>
struct BwdTile {
  static constexpr int RB = 2 * D;      // bytes per row
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int RPG = 16 / CPR;  // rows per 256 bytes
  static constexpr int Q4 = CPR / 4;
  static constexpr int kBytes = ROWS * RB;
  static constexpr int kInsts = kBytes / 1024;  // wave-instructions to copy one tile
  __device__ static constexpr int swz(int r) { return 4 * ((r / RPG) % Q4) + ((r / RPG) / Q4) % 4; }
  // byte offset of bf16 element (r, col) of the tile
  __device__ static constexpr int at(int r, int col) { return r * RB + ((col / 8) ^ swz(r)) * 16 + (col % 8) * 2; }
};

__device__ __forceinline__ int swap_bits23(int l) { return (l & ~12) | ((l & 4) << 1) | ((l & 8) >> 1); }

// 8 consecutive rows (8h .. 8h+7 of a 16-row step) of one 32-column block, transposed: two ds_read_b64_tr_b16.
__device__ __forceinline__ bf16x8 read_tr8(const lds_char* p0, const lds_char* p1) {
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p0));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p1));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Issue order for a block of n LDS-read-fed MFMAs (scheduling groups: 0x100 = LDS read, 0x008 = MFMA): 4 reads,
// then one MFMA per further read, so each operand is read about four MFMAs before it is used.
template <int n>
__device__ __forceinline__ void schedule_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < n - 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

__device__ __forceinline__ float dot8(bf16x8 a, bf16x8 b) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)a[e], (float)b[e], s);
  return s;
}

// ------------------------------------------------------------------------------------------------------------
// dq (and the workspace values -D_i, lse_i*log2e)
// ------------------------------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(64 * kDqWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dq_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ o, const float* __restrict__ lse, const __bf16* __restrict__ dout,
    __bf16* __restrict__ dq, float* __restrict__ ws, int N, int BH, float scale, int group, int H,
    const int* __restrict__ kv_len, const int* __restrict__ cu_seqlens, int T_total) {
  using T = BwdTile<D>;
  constexpr int NW = kDqWaves, kDB = D / 16, kCB = D / 32, kCopies = T::kInsts / NW;
  static_assert(T::kInsts % NW == 0, "tile copy must split evenly over the waves");
  // 2 K stages, then 2 V stages (64 KiB at d = 128). Static rather than dynamic, so that its address is known when
  // instructions are selected and the stage offsets fold into the reads' immediate offsets.
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * T::kBytes];
  lds_char* const kst = (lds_char*)smem_raw;  // 2 K stages
  lds_char* const vst = kst + 2 * T::kBytes;  // 2 V stages

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nq = gridDim.x;
  int bh, qb;
  if (VARLEN && BH / H <= 64) {
    // packed batches: (sequence, query block) items in longest-first order (causal: the last blocks, which visit
    // the most key tiles, first)
    const int nb = packed_blocks(cu_seqlens, BH / H, T_total, N, kDqBlock);
    int rank, hq, b, kb;
    map_packed(blockIdx.x + nq * blockIdx.y, H, group, rank, hq);
    if (!longest_first_item(rank, nb, CAUSAL, b, kb)) return;  // the whole workgroup: no item left
    bh = __builtin_amdgcn_readfirstlane(b * H + hq);
    qb = __builtin_amdgcn_readfirstlane(CAUSAL ? __shfl(nb, b) - 1 - kb : kb);
  } else {
    map_workgroup(blockIdx.x + nq * blockIdx.y, nq, BH, group, CAUSAL, bh, qb);
  }
  int start = 0, Ns = N;  // this head's sequence: its first token and length
  if constexpr (VARLEN) {
    const int lo = min(max(cu_seqlens[bh / H], 0), T_total);
    const int hi = min(max(cu_seqlens[bh / H + 1], lo), T_total);
    start = __builtin_amdgcn_readfirstlane(lo);
    Ns = __builtin_amdgcn_readfirstlane(min(hi - lo, N));  // no longer than max_seqlen (= N)
  }
  const int q_lo = qb * kDqBlock;
  if (VARLEN && q_lo >= Ns) return;  // the whole workgroup: no row of this block (nor its padding) exists
  const int hq = bh % H, Hkv = H / group;
  const int qpitch = VARLEN ? H * D : D;   // elements between consecutive rows of q, o, dO and dq
  const int kpitch = VARLEN ? Hkv * D : D;  // ... of k and v
  const int kpitch_b = 2 * kpitch;
  const size_t head_off = VARLEN ? ((size_t)start * H + hq) * D : (size_t)bh * (size_t)N * D;
  const size_t kv_off = VARLEN ? ((size_t)start * Hkv + hq / group) * D : (size_t)(bh / group) * (size_t)N * D;
  const size_t lse_off = VARLEN ? (size_t)hq * T_total + start : (size_t)bh * N;
  const __bf16* kh = k + kv_off;
  const __bf16* vh = v + kv_off;
  const int Nk = kv_len ? __builtin_amdgcn_readfirstlane(min(max(kv_len[bh / H], 0), N)) : Ns;

  const int q_last = min(q_lo + kDqBlock, Ns) - 1;
  const int key_tiles = (Nk + kBwdTile - 1) / kBwdTile;
  const int n_tiles = CAUSAL ? min(q_last / kBwdTile + 1, key_tiles) : key_tiles;
  const int q0w = q_lo + wave * kBwdRows;
  const int my_q = q0w + l32;
  const int wave_tiles =
      (q0w >= Ns) ? 0 : (CAUSAL ? min(n_tiles, (q0w + kBwdRows - 1) / kBwdTile + 1) : n_tiles);

  // This lane's query row: q and dO fragments (B operands of S^T = K Q^T and dP^T = V dO^T), and D_i = dO_i . o_i
  bf16x8 qf[kDB], df[kDB];
  float dpart = 0.f;
#pragma unroll
  for (int kb = 0; kb < kDB; ++kb) {
    if (my_q < Ns) {
      const size_t e = head_off + (size_t)my_q * qpitch + 16 * kb + 8 * h;
      qf[kb] = *(const bf16x8*)(q + e);
      df[kb] = *(const bf16x8*)(dout + e);
      dpart += dot8(df[kb], *(const bf16x8*)(o + e));
    } else {
      qf[kb] = (bf16x8){};
      df[kb] = (bf16x8){};
    }
  }
  const float Di = pair_sum32(dpart);
  // rows past the sequence: lse2 = +inf makes every p of the row exactly 0 (D is 0 there: dO was not loaded)
  const float lse2 = (my_q < Ns) ? lse[lse_off + my_q] * kLog2e : INFINITY;
  const int npad = ws_rows(N);
  if (my_q < npad && h == 0) {
    float* w = ws + (size_t)bh * 2 * npad + my_q;
    w[0] = -Di;  // stored negated: the dk/dv kernel starts its dP accumulators at -D
    w[npad] = lse2;
  }

  // LDS-DMA: copy instruction p of this wave writes chunk positions (wave + NW p)*64 + lane of the tile
  int dma[kCopies];
#pragma unroll
  for (int p = 0; p < kCopies; ++p) {
    const int pos = (wave + NW * p) * 64 + lane;
    const int row = pos / T::CPR, phys = pos % T::CPR;
    dma[p] = row * kpitch_b + (phys ^ T::swz(row)) * 16;
  }
  auto copy_tile = [&](const __bf16* src, lds_char* dst, int j) __attribute__((always_inline)) {
    const int row0 = j * kBwdTile;
    // rows past Nk arrive as zeros: the range ends with the last valid row (only tiles below Nk are copied, so
    // Nk >= 1 here); scalar byte count and base keep the descriptor in scalar registers (readfirstlane between
    // the min and the max keeps the pair from fusing into v_med3_i32, a vector instruction)
    const int rows = max(0, __builtin_amdgcn_readfirstlane(min(Nk - row0, kBwdTile)));
    const int bytes = rows > 0 ? (rows - 1) * kpitch_b + T::RB : 0;
    const int row_base = __builtin_amdgcn_readfirstlane(min(row0, Nk - 1));
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)row_base * kpitch, bytes);
#pragma unroll
    for (int p = 0; p < kCopies; ++p) lds_copy16_inline(r, dst + (wave + NW * p) * 1024, dma[p]);
  };

  // Row reads of K and V (A operands): row 32b + swap_bits23(l32), columns 16kb + 8h .. +7. The swizzle depends
  // on the row only modulo 16 here, so one offset per kb serves both 32-key blocks.
  const int krow = swap_bits23(l32);
  int row_off[kDB];
#pragma unroll
  for (int kb = 0; kb < kDB; ++kb) row_off[kb] = T::at(krow, 16 * kb + 8 * h);
  // Transposing reads of K (A operand of dQ^T = K^T dS^T): rows 16m + 8h + 4 half + (lane&15)/4, columns
  // 32cb + 16((lane>>4)&1) + 4(lane&3); the swizzle does not depend on m.
  int tr_off[kCB][2];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int half = 0; half < 2; ++half)
      tr_off[cb][half] =
          T::at(8 * h + 4 * half + (lane & 15) / 4, 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  const float c2 = scale * kLog2e;
  f32x16 acc[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) acc[cb] = (f32x16){};
  f32x16 negD;  // -D_i in every value: the starting value of the dP^T accumulators (the lane's row is i)
#pragma unroll
  for (int r = 0; r < 16; ++r) negD[r] = -Di;

  // One 64-key tile from the stage at byte `at`. Value r of block b is key j*64 + 32b + 16(r/8) + 8h + r%8.
  auto compute = [&](int j, int at) __attribute__((always_inline)) {
    const lds_char* ks = kst + at;
    const lds_char* vs = vst + at;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = (f32x16){};
      dp[b] = negD;  // the products then leave dP^T - D, with no subtraction per value
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kb = 0; kb < kDB; ++kb) {
        const bf16x8 kf = *(const __attribute__((address_space(3))) bf16x8*)(ks + 32 * b * T::RB + row_off[kb]);
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kb], s[b], 0, 0, 0);
        const bf16x8 vf = *(const __attribute__((address_space(3))) bf16x8*)(vs + 32 * b * T::RB + row_off[kb]);
        dp[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[kb], dp[b], 0, 0, 0);
      }
    schedule_reads_ahead<4 * kDB>();
    const int kv0 = j * kBwdTile;
    if ((kv0 + kBwdTile > Nk) || (CAUSAL && kv0 + kBwdTile - 1 > q0w)) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * b + 16 * (r >> 3) + 8 * h + (r & 7);
          const bool vis = (key < Nk) && (!CAUSAL || key <= my_q);
          s[b][r] = vis ? s[b][r] : -INFINITY;
        }
    }
    // dQ^T += K^T dS^T one 16-key step at a time; the K^T fragments of step m+1 are read during step m
    auto read_kt = [&](int m, bf16x8(&kt)[kCB]) __attribute__((always_inline)) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
        kt[cb] = read_tr8(ks + 16 * m * T::RB + tr_off[cb][0], ks + 16 * m * T::RB + tr_off[cb][1]);
    };
    bf16x8 kta[kCB], ktb[kCB];
    read_kt(0, kta);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      bf16x8(&cur)[kCB] = (m & 1) ? ktb : kta;
      bf16x8(&nxt)[kCB] = (m & 1) ? kta : ktb;
      const f32x8 x = (m & 1) ? s[m >> 1].hi : s[m >> 1].lo;
      const f32x8 y = (m & 1) ? dp[m >> 1].hi : dp[m >> 1].lo;
      f32x8 ds;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c2, -lse2));
        ds[e] = p * y[e];
      }
      const bf16x8 dsb = __builtin_convertvector(ds, bf16x8);
      if (m < 3) read_kt(m + 1, nxt);
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[cb], dsb, acc[cb], 0, 0, 0);
    }
  };

  // Two-stage ring: copy tile j+1 while tile j is computed; one barrier per tile. The tiles this wave computes
  // (j < wave_tiles) run in a loop of their own, two per iteration with the stage fixed at compile time and no
  // condition around the computation (a conditional there made the compiler copy the accumulators at every
  // join); the remaining tiles of the workgroup only copy and join the barriers.
  auto issue = [&](int j, int S) __attribute__((always_inline)) {
    if (j + 1 < n_tiles) {
      copy_tile(kh, kst + (S ^ 1) * T::kBytes, j + 1);
      copy_tile(vh, vst + (S ^ 1) * T::kBytes, j + 1);
    }
  };
  if (n_tiles > 0) {
    copy_tile(kh, kst, 0);
    copy_tile(vh, vst, 0);
    wait_copies_and_barrier<0>();
  }
  int j = 0;
  for (; j + 1 < wave_tiles; j += 2) {
    issue(j, 0);
    compute(j, 0);
    wait_copies_and_barrier<0>();
    issue(j + 1, 1);
    compute(j + 1, T::kBytes);
    wait_copies_and_barrier<0>();
  }
  if (j < wave_tiles) {
    issue(j, 0);
    compute(j, 0);
    wait_copies_and_barrier<0>();
    ++j;
  }
  for (; j < n_tiles; ++j) {
    issue(j, j & 1);
    wait_copies_and_barrier<0>();
  }

  // dq_i = scale * acc; acc[cb][4g + i] is column 32cb + 8g + 4h + i of row my_q
  if (my_q < Ns) {
    __bf16* row = dq + head_off + (size_t)my_q * qpitch;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = {acc[cb][4 * g] * scale, acc[cb][4 * g + 1] * scale, acc[cb][4 * g + 2] * scale,
                         acc[cb][4 * g + 3] * scale};
        *(bf16x4*)(row + 32 * cb + 8 * g + 4 * h) = __builtin_convertvector(x, bf16x4);
      }
  }
}

// ------------------------------------------------------------------------------------------------------------
// dk, dv
// ------------------------------------------------------------------------------------------------------------
// Join the workgroup once this wave's LDS accesses are done (vector-memory copies may stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0), vmcnt and expcnt no wait
  asm volatile("s_barrier" ::: "memory");
}

constexpr int kDkdvWaves = 8;   // 4 pairs of waves; the two waves of a pair share a SIMD and a block of 32 keys
constexpr int kDkdvTile = 128;  // query rows per LDS tile: four 32-row sub-blocks
constexpr int kPSlotBytes = 2 * 64 * 16;  // p of one 32 x 32 sub-block, bf16, as the two 16-row steps of 64 lanes

// Waves w and w+4 run on the same SIMD and own the same 32 keys: the p wave (w < 4) computes S = Q K^T, p and
// dV^T += dO^T P; the dS wave computes dP = dO V^T, then (after the sub-block's barrier) dS = p (dP - D) from the
// p the other wave left in LDS, and dK^T += Q^T dS. Each holds half the accumulators, so two waves share a SIMD.
// A key block's work is a list of iterations, one per (query head of the group, query tile), head by head. With
// nsplit > 1, the grid's y extent is BHkv * nsplit: workgroup part z of a key block takes iterations
// n*z/nsplit .. n*(z+1)/nsplit - 1 of the n and writes its dk and dv in fp32 to part ([2][nsplit][BHkv][N][D]:
// dk, then dv) for fa_bwd_reduce_kernel. The parts of one key block are handed out together, so the
// longest-first order of causal blocks holds over all of them.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(64 * kDkdvWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dkdv_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ ws, __bf16* __restrict__ dk,
    __bf16* __restrict__ dv, int N, int BHkv, float scale, int group, int Hkv, const int* __restrict__ kv_len,
    const int* __restrict__ cu_seqlens, int T_total, float* __restrict__ part, int nsplit) {
  using T = BwdTile<D, kDkdvTile>;
  constexpr int NW = kDkdvWaves, kDB = D / 16, kCB = D / 32, kCopies = T::kInsts / NW;
  constexpr int kSub = kDkdvTile / kBwdRows;  // 32-row sub-blocks per query tile
  static_assert(T::kInsts % NW == 0, "tile copy must split evenly over the waves");
  // 146 KiB at d = 128; static, as in the dq kernel, so that stage offsets fold into the reads
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * (2 * T::kBytes + kWsTileBytes) + 8 * kPSlotBytes];
  lds_char* const qst = (lds_char*)smem_raw;       // 2 q stages
  lds_char* const dst = qst + 2 * T::kBytes;       // 2 dO stages
  lds_char* const wst = dst + 2 * T::kBytes;       // 2 workspace stages
  lds_char* const pst = wst + 2 * kWsTileBytes;    // 2 p slots per pair

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pw = wave < 4;
  const int pair = wave & 3;
  const int nk = gridDim.x;
  int bkv, kblk, zs;
  const int nbatch = BHkv / Hkv;
  if (VARLEN && nbatch <= 64) {
    // packed batches: consecutive workgroups are the Hkv heads (times the nsplit parts) of one (sequence, key
    // block) item (so a head stays on one XCD when Hkv is a multiple of 8), items in longest-first order
    const int nb = packed_blocks(cu_seqlens, nbatch, T_total, N, kBwdBlock);
    const int lin = blockIdx.x + nk * blockIdx.y;
    int b, kb;
    if (!longest_first_item(lin / (Hkv * nsplit), nb, CAUSAL, b, kb)) return;  // the whole workgroup: no item left
    const int u = lin % (Hkv * nsplit);
    bkv = __builtin_amdgcn_readfirstlane(b * Hkv + u % Hkv);
    zs = __builtin_amdgcn_readfirstlane(u / Hkv);
    kblk = __builtin_amdgcn_readfirstlane(kb);
  } else {
    int t, u;
    map_workgroup(blockIdx.x + nk * blockIdx.y, nk, BHkv * nsplit, 1, CAUSAL, u, t);
    bkv = u % BHkv;
    zs = u / BHkv;
    // causal: the first key blocks see the most query rows; map_workgroup hands out the last index first
    kblk = CAUSAL ? nk - 1 - t : t;
  }
  int start = 0, Ns = N;  // this head's sequence: its first token and length
  if constexpr (VARLEN) {
    const int lo = min(max(cu_seqlens[bkv / Hkv], 0), T_total);
    const int hi = min(max(cu_seqlens[bkv / Hkv + 1], lo), T_total);
    start = __builtin_amdgcn_readfirstlane(lo);
    Ns = __builtin_amdgcn_readfirstlane(min(hi - lo, N));  // no longer than max_seqlen (= N)
  }
  const int k0 = kblk * kBwdBlock;
  if (VARLEN && k0 >= Ns) return;  // the whole workgroup: its keys lie past this sequence
  const int H = Hkv * group;
  const int qpitch = VARLEN ? H * D : D;   // elements between consecutive rows of q and dO
  const int kpitch = VARLEN ? Hkv * D : D;  // ... of k, v, dk and dv
  const int qpitch_b = 2 * qpitch;
  const size_t kv_off = VARLEN ? ((size_t)start * Hkv + bkv % Hkv) * D : (size_t)bkv * (size_t)N * D;
  const int bh0 = bkv * group;  // first query head (of B*H) of this key/value head's group
  const int Nk = kv_len ? __builtin_amdgcn_readfirstlane(min(max(kv_len[bkv / Hkv], 0), N)) : Ns;

  const int kw0 = k0 + pair * kBwdRows;
  const int my_k = kw0 + l32;

  // This lane's key: k fragments (p wave, B operand of S = Q K^T) or v fragments (dS wave, of dP = dO V^T); keys
  // past Nk read as zeros (their contents may be anything), so dP and dS stay finite and exactly 0 there
  bf16x8 kvf[kDB];
  const __bf16* kvsrc = pw ? k : v;
#pragma unroll
  for (int kb = 0; kb < kDB; ++kb)
    kvf[kb] = (my_k < Nk) ? *(const bf16x8*)(kvsrc + kv_off + (size_t)my_k * kpitch + 16 * kb + 8 * h) : (bf16x8){};

  int dma[kCopies];
#pragma unroll
  for (int p = 0; p < kCopies; ++p) {
    const int pos = (wave + NW * p) * 64 + lane;
    const int row = pos / T::CPR, phys = pos % T::CPR;
    dma[p] = row * qpitch_b + (phys ^ T::swz(row)) * 16;
  }
  // Query tiles t0 .. nqt-1 of each of the group's query heads. Key blocks and query tiles are both 128 rows,
  // so under causal masking the first tile (t0 = this key block) is the only one that crosses the diagonal.
  const int nqt = (Ns + kDkdvTile - 1) / kDkdvTile;
  const int t0 = CAUSAL ? kblk : 0;
  const int per_head = nqt - t0;
  const int n_all = (k0 < Nk) ? group * per_head : 0;  // a block of padded keys only writes zeros
  const int it_lo = (int)((long long)n_all * zs / nsplit), it_hi = (int)((long long)n_all * (zs + 1) / nsplit);
  const int npad = ws_rows(N);
  auto copy_iter = [&](int it, int S) __attribute__((always_inline)) {
    const int hq = bh0 + it / per_head;
    const int row0 = (t0 + it % per_head) * kDkdvTile;
    // first element of row 0 of query head hq
    const size_t base = VARLEN ? ((size_t)start * H + hq % H) * D : (size_t)hq * N * D;
    const int rows = max(0, __builtin_amdgcn_readfirstlane(min(Ns - row0, kDkdvTile)));  // scalar, no v_med3_i32
    const int row_base = __builtin_amdgcn_readfirstlane(min(row0, Ns - 1));
    const int bytes = rows > 0 ? (rows - 1) * qpitch_b + T::RB : 0;  // ends with the sequence's last row
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + base + (size_t)row_base * qpitch, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dout + base + (size_t)row_base * qpitch, bytes);
#pragma unroll
    for (int p = 0; p < kCopies; ++p) {
      lds_copy16_inline(rq, qst + S * T::kBytes + (wave + NW * p) * 1024, dma[p]);
      lds_copy16_inline(rd, dst + S * T::kBytes + (wave + NW * p) * 1024, dma[p]);
    }
    if (wave == 0) {  // the tile's 128 D values, then its 128 lse2 values (always inside the padded workspace)
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(ws + 2 * (size_t)hq * npad + row0, (npad + kDkdvTile) * 4);
      lds_copy16_inline(rw, wst + S * kWsTileBytes, (lane & 31) * 16 + (lane >> 5) * npad * 4);
    }
  };

  // Row reads (A operands of S = Q K^T and dP = dO V^T): row 32sb + swap_bits23(l32), columns 16kb + 8h .. +7
  const int qrow = swap_bits23(l32);
  int row_off[kDB];
#pragma unroll
  for (int kb = 0; kb < kDB; ++kb) row_off[kb] = T::at(qrow, 16 * kb + 8 * h);
  // Transposing reads (A operands of dV^T = dO^T P and dK^T = Q^T dS)
  int tr_off[kCB][2];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int half = 0; half < 2; ++half)
      tr_off[cb][half] =
          T::at(8 * h + 4 * half + (lane & 15) / 4, 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  const float c2 = scale * kLog2e;
  f32x16 acc[kCB];  // dV^T (p wave) or dK^T (dS wave) of this pair's keys
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) acc[cb] = (f32x16){};

  // Sub-block sb of the query tile in stage S. In S and dP, lane = key my_k and value r is query row
  // 16(r/8) + 8h + r%8 of the sub-block (q and dO rows fed in swap_bits23 order); p travels from the p wave to
  // the dS wave through the pair's LDS slot (sb % 2) in exactly that register layout. The role is a compile-time
  // parameter: each role runs a loop of its own (with the same barriers), so the accumulators are not merged
  // across role branches inside the loop.
  // The operands a sub-block needs first, read one sub-block ahead: the A fragments of its first product (q rows
  // for the p wave, dO rows for the dS wave) and four f32x4 of the workspace (lse2 of its rows for the p wave,
  // -D for the dS wave; value group g <-> rows 32sb + 8h + {0..3, 4..7, 16..19, 20..23}[g]).
  auto read_pre = [&](int S, int sb, auto role_c, bf16x8 (&a)[kDB], f32x4 (&w)[4]) __attribute__((always_inline)) {
    constexpr bool pw = decltype(role_c)::value;
    const lds_char* rows_src = (pw ? qst : dst) + S * T::kBytes;
#pragma unroll
    for (int kb = 0; kb < kDB; ++kb)
      a[kb] = *(const __attribute__((address_space(3))) bf16x8*)(rows_src + 32 * sb * T::RB + row_off[kb]);
    const __attribute__((address_space(3))) f32x4* wp =
        (const __attribute__((address_space(3))) f32x4*)(wst + S * kWsTileBytes + (pw ? 512 : 0) +
                                                         (32 * sb + 8 * h) * 4);
    w[0] = wp[0];
    w[1] = wp[1];
    w[2] = wp[4];
    w[3] = wp[5];
  };
  auto sub_block = [&](int it, int S, int sb, auto role_c, const bf16x8 (&a)[kDB], const f32x4 (&w)[4],
                       bf16x8 (&a_nx)[kDB], f32x4 (&w_nx)[4]) __attribute__((always_inline)) {
    constexpr bool pw = decltype(role_c)::value;
    const lds_char* qs = qst + S * T::kBytes;
    const lds_char* os = dst + S * T::kBytes;
    lds_char* ps = pst + ((sb & 1) * 4 + pair) * kPSlotBytes;
    const int row0 = (t0 + it % per_head) * kDkdvTile;
    f32x16 x = (f32x16){};
    if constexpr (!pw)
      x = (f32x16){w[0][0], w[0][1], w[0][2], w[0][3], w[1][0], w[1][1], w[1][2], w[1][3],
                   w[2][0], w[2][1], w[2][2], w[2][3], w[3][0], w[3][1], w[3][2], w[3][3]};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < kDB; ++kb) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], kvf[kb], x, 0, 0, 0);
    if (sb + 1 < kSub) read_pre(S, sb + 1, role_c, a_nx, w_nx);
    __builtin_amdgcn_sched_barrier(0);
    const lds_char* tr_src = pw ? os : qs;    // dO^T for dV^T, q^T for dK^T
    if constexpr (pw) {
      const int qlo = row0 + 32 * sb;
      if ((qlo + kBwdRows > Ns) || (kw0 + kBwdRows > Nk) || (CAUSAL && qlo < kw0 + kBwdRows - 1)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qlo + 16 * (r >> 3) + 8 * h + (r & 7);
          const bool vis = (qi < Ns) && (my_k < Nk) && (!CAUSAL || my_k <= qi);
          x[r] = vis ? x[r] : -INFINITY;
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f32x8 pv;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pv[4 * u + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * m + 4 * u + e], c2, -w[2 * m + u][e]));
        const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
        *(__attribute__((address_space(3))) bf16x8*)(ps + (m * 64 + lane) * 16) = pb;
        const int rbase = (32 * sb + 16 * m) * T::RB;
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          const bf16x8 at_ = read_tr8(tr_src + rbase + tr_off[cb][0], tr_src + rbase + tr_off[cb][1]);
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at_, pb, acc[cb], 0, 0, 0);
        }
      }
      lds_barrier();  // p of this sub-block is in the slot
    } else {
      lds_barrier();  // wait for p of this sub-block
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 pb = *(const __attribute__((address_space(3))) bf16x8*)(ps + (m * 64 + lane) * 16);
        f32x8 dsv;
#pragma unroll
        for (int e = 0; e < 8; ++e) dsv[e] = (float)pb[e] * x[8 * m + e];
        const bf16x8 dsb = __builtin_convertvector(dsv, bf16x8);
        const int rbase = (32 * sb + 16 * m) * T::RB;
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          const bf16x8 at_ = read_tr8(tr_src + rbase + tr_off[cb][0], tr_src + rbase + tr_off[cb][1]);
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at_, dsb, acc[cb], 0, 0, 0);
        }
      }
    }
  };

  // Stage ring: the copy of tile it+1 goes into the other stage after the first sub-block of tile it; every wave
  // finished reading that stage (tile it-1) before the barrier that ended tile it-1, and the barrier that ends
  // tile it also waits for the copies. The last tile copies itself again (harmless, in bounds), so the copy is
  // unconditional.
  if (it_hi > it_lo) {
    copy_iter(it_lo, 0);
    wait_copies_and_barrier<0>();
  }
  auto run = [&](auto role_c) __attribute__((always_inline)) {
    static_assert(kSub % 2 == 0, "sub-blocks alternate between two operand sets");
    for (int it = it_lo; it < it_hi; ++it) {
      const int S = (it - it_lo) & 1;
      bf16x8 a0[kDB], a1[kDB];
      f32x4 w0[4], w1[4];
      read_pre(S, 0, role_c, a0, w0);
#pragma unroll
      for (int sb = 0; sb < kSub; sb += 2) {
        sub_block(it, S, sb, role_c, a0, w0, a1, w1);
        if (sb == 0) copy_iter(min(it + 1, it_hi - 1), S ^ 1);
        sub_block(it, S, sb + 1, role_c, a1, w1, a0, w0);
      }
      wait_copies_and_barrier<0>();
    }
  };
  if (pw) {
    run(std::true_type{});
  } else {
    run(std::false_type{});
  }

  // dk_j = scale * dK^T, dv_j = dV^T; [cb][4g + i] is column 32cb + 8g + 4h + i of key row my_k (0 past Nk)
  if (my_k < Ns) {
    const float f = (my_k < Nk) ? (pw ? 1.f : scale) : 0.f;
    if (nsplit == 1) {
      __bf16* row = (pw ? dv : dk) + kv_off + (size_t)my_k * kpitch;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 a = {acc[cb][4 * g] * f, acc[cb][4 * g + 1] * f, acc[cb][4 * g + 2] * f,
                           acc[cb][4 * g + 3] * f};
          *(bf16x4*)(row + 32 * cb + 8 * g + 4 * h) = __builtin_convertvector(a, bf16x4);
        }
    } else {
      float* row = part + ((((size_t)(pw ? 1 : 0) * nsplit + zs) * BHkv + bkv) * N + my_k) * D;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(row + 32 * cb + 8 * g + 4 * h) = (f32x4){acc[cb][4 * g] * f, acc[cb][4 * g + 1] * f,
                                                             acc[cb][4 * g + 2] * f, acc[cb][4 * g + 3] * f};
    }
  }
}

// Sums the nsplit partial dk and dv of a head-split dk/dv launch in split order and writes them in bf16: one thread
// per 8 columns of one key row of one key/value head (rows past a packed sequence's end are not written, as in the
// unsplit kernel).
template <int D, bool VARLEN>
__global__ __launch_bounds__(256) void fa_bwd_reduce_kernel(const float* __restrict__ part, int nsplit,
                                                           __bf16* __restrict__ dk, __bf16* __restrict__ dv, int N,
                                                           int BHkv, int Hkv, const int* __restrict__ cu_seqlens,
                                                           int T_total) {
  constexpr int kTpr = D / 8;  // threads per row
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t rows = (size_t)BHkv * N;
  if (t >= rows * kTpr) return;
  const size_t r = t / kTpr;
  const int c0 = (int)(t % kTpr) * 8;
  const int bkv = (int)(r / N), i = (int)(r % N);
  size_t out;
  if constexpr (VARLEN) {
    const int lo = min(max(cu_seqlens[bkv / Hkv], 0), T_total);
    const int hi = min(max(cu_seqlens[bkv / Hkv + 1], lo), T_total);
    if (i >= min(hi - lo, N)) return;
    out = ((size_t)(lo + i) * Hkv + bkv % Hkv) * D + c0;
  } else {
    out = r * D + c0;
  }
  const size_t stride = rows * D;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const float* src = part + (size_t)which * nsplit * stride + r * D + c0;
    f32x4 a = *(const f32x4*)src, b = *(const f32x4*)(src + 4);
    for (int sp = 1; sp < nsplit; ++sp) {
      a += *(const f32x4*)(src + sp * stride);
      b += *(const f32x4*)(src + sp * stride + 4);
    }
    __bf16* dst = (which ? dv : dk) + out;
    *(bf16x4*)dst = __builtin_convertvector(a, bf16x4);
    *(bf16x4*)(dst + 4) = __builtin_convertvector(b, bf16x4);
  }
}

// ------------------------------------------------------------------------------------------------------------
// launcher (arguments already validated by the C ABI layer)
// ------------------------------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN = false>
static hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, float* ws, int B, int H, int Hkv,
                             int N, float scale, const int* kv_len, hipStream_t stream,
                             const int* cu_seqlens = nullptr, int T_total = 0) {
  const int group = H / Hkv;
  auto ka = fa_bwd_dq_kernel<D, CAUSAL, VARLEN>;  // both kernels allocate their LDS statically
  auto kb = fa_bwd_dkdv_kernel<D, CAUSAL, VARLEN>;
  const unsigned nblk = (unsigned)((N + kBwdBlock - 1) / kBwdBlock);
  const unsigned nblk_dq = (unsigned)((N + kDqBlock - 1) / kDqBlock);
  hipLaunchKernelGGL(ka, dim3(nblk_dq, (unsigned)(B * H)), dim3(64 * kDqWaves), 0, stream, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, (const __bf16*)o, lse, (const __bf16*)dout, (__bf16*)dq, ws,
                     N, B * H, scale, group, H, kv_len, cu_seqlens, T_total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nsplit = bwd_head_split(B, H, Hkv, N);
  float* part = nsplit > 1 ? (float*)((char*)ws + bwd_planes_bytes(B, H, N)) : nullptr;
  hipLaunchKernelGGL(kb, dim3(nblk, (unsigned)(B * Hkv * nsplit)), dim3(64 * kDkdvWaves), 0, stream,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, (const float*)ws,
                     (__bf16*)dk, (__bf16*)dv, N, B * Hkv, scale, group, Hkv, kv_len, cu_seqlens, T_total, part,
                     nsplit);
  if (nsplit == 1) return hipGetLastError();
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t threads = (size_t)B * Hkv * N * (D / 8);
  hipLaunchKernelGGL((fa_bwd_reduce_kernel<D, VARLEN>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     (const float*)part, nsplit, (__bf16*)dk, (__bf16*)dv, N, B * Hkv, Hkv, cu_seqlens, T_total);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* ws, int B, int H, int Hkv, int N,
                           int d, bool causal, float scale, const int* kv_len, hipStream_t stream) {
#define FA_BWD(D, C) launch_bwd<D, C>(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, Hkv, N, scale, kv_len, stream)
  if (d == 64) return causal ? FA_BWD(64, true) : FA_BWD(64, false);
  return causal ? FA_BWD(128, true) : FA_BWD(128, false);
#undef FA_BWD
}

hipError_t launch_bwd_varlen_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv, float* ws, const int* cu_seqlens,
                                  int B, int H, int Hkv, int T_total, int max_seqlen, int d, bool causal, float scale,
                                  hipStream_t stream) {
#define FA_BWD(D, C)                                                                                         \
  launch_bwd<D, C, true>(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, Hkv, max_seqlen, scale, nullptr, stream, \
                         cu_seqlens, T_total)
  if (d == 64) return causal ? FA_BWD(64, true) : FA_BWD(64, false);
  return causal ? FA_BWD(128, true) : FA_BWD(128, false);
#undef FA_BWD
}

}  // namespace fa
