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
// gfx950 mapping of the bf16 kernel (one workgroup = 8 or 4 waves; one wave = 32 query rows):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (fp32 accumulate). With S transposed, lane l of a wave holds
//     scores of query row (l % 32) only, so the row max needs one exchange between lanes l and l ^ 32
//     (v_permlane32_swap) and the row sum needs none until the end.
//   * The S^T accumulator is, after conversion to bf16, exactly the B operand of O^T = V^T P^T on the same
//     MFMA shape. The K rows are fed to the first product in an order that swaps bits 2 and 3 of the row
//     index, which makes the 8 keys a lane holds for each 16-key step of the second product contiguous.
//   * The V^T operand is read from row-major V in LDS with ds_read_b64_tr_b16 (transposing LDS read).
//   * O^T accumulates per lane for one query row, so the rescale by alpha = exp2(m_old - m_new) is a
//     per-lane scalar multiply, done only when some row maximum grew by more than 2^8.
//   * exp2 with log2(e) folded into the scale: p = exp2(s * c - m * c), c = scale * log2(e), one FMA.
//   * The row sum l adds the bf16-rounded weights (the values the MFMA multiplies V by), two per
//     v_dot2c_f32_bf16, so o is the exact weighted average under those weights.
//   * The second product runs one 16-key step at a time, so the exponentials of step m+1 and the V reads of
//     step m+1 overlap the MFMAs of step m; K fragment reads are issued about four MFMAs ahead.
//   * K/V tiles (128 keys for 8-wave workgroups, 64 for 4-wave ones) go device memory -> LDS by LDS-DMA
//     (buffer_load ... lds) through a 2-stage ring: tile j+1 is copied while tile j is computed; one barrier per
//     tile. The LDS layouts are XOR-swizzled so that the K fragment reads, the transposing V reads and the DMA
//     writes are all free of bank conflicts.
//   * Few query rows (the split shape, SPL = 2): each group of 32 rows gets two waves, which take the two 64-key
//     halves of every 128-key tile with partial (m, l, O) of their own; at the end the second hands its partial
//     to the first through LDS and the first merges them (the block-merge rule of the unite.ai page, "The Math
//     Behind Flash Attention" item 2, in its corrected reading) and writes o and lse. Every SIMD then holds two
//     waves even when the rows alone would give it one.
//   * Causal: a workgroup visits only key tiles that meet its rows, a wave skips tiles entirely above its
//     rows, and the mask is applied only on tiles that cross the diagonal or the sequence end.
//   * The linear workgroup id is remapped so that (when B*H is a multiple of 8) every query block of a head
//     runs on the same XCD (workgroups are dealt to the 8 XCDs round-robin) and shares that XCD's L2, and
//     causal work starts with the longest query blocks. XCDs take key/value heads round-robin, so the query
//     heads that share a key/value head (grouped-query attention) also share an L2.
//   * Grouped/multi-query attention (the unite.ai page, section "FlashAttention-2", item 3): query head bh
//     reads key/value head bh / group, group = H / Hkv consecutive query heads per key/value head.
//   * Key padding (a per-batch count Nk of valid keys, triton-transformer README usage example "ex. BERT"):
//     tiles past Nk are not visited and keys >= Nk are masked like the sequence end; a row with no visible key
//     gets o = 0 and lse = -inf.
//   * Packed variable-length batches (VARLEN): q, o [T, H, d] and k, v [T, Hkv, d] hold B sequences back to back,
//     sequence b being tokens cu[b] .. cu[b+1]-1; each is its own attention problem. Rows of one head are then
//     H*d (or Hkv*d) elements apart instead of d; the copies and loads take that pitch, and a tile's copy range
//     ends with the sequence's last row, so rows past it arrive as zeros exactly as past N. Query blocks past
//     the sequence's end return at once. lse is [H, T].
// The fp32 kernel keeps the same decomposition on v_mfma_f32_32x32x2f32 with a simple single-buffered loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_gfx950.h"
#include "fa_launch.h"

namespace fa {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBc = 64;                     // keys per K/V tile

// ------------------------------------------------------------------------------------------------------------
// bf16 kernel
// ------------------------------------------------------------------------------------------------------------
// LDS layouts are unpadded and XOR-swizzled at 16-byte-chunk granularity. A tile is 64 rows x D bf16 (row of
// RB = 2D bytes, CPR = D/8 chunks); chunk c of row r is stored at chunk position c ^ swz(r). LDS has 64 4-byte
// banks, i.e. 16 bank groups of 16 bytes, so a bank group is (r % RPG) * CPR + position with RPG = 16 / CPR rows per
// 256 bytes.
//  * K is read 16 bytes per lane, 16 lanes per LDS pass, 16 different rows at one chunk:
//    swz_k(r) = (r / RPG) % CPR puts those 16 reads in 16 different bank groups.
//  * V is read by ds_read_b64_tr_b16, 32 lanes per pass, 4 consecutive rows x 4 consecutive chunks:
//    swz_v(r) = 4 * ((r / RPG) % (CPR / 4)) spreads the 4 rows over different groups of 4 chunks.
//  * Tiles are written by LDS-DMA (buffer_load ... lds): one wave-instruction writes 64 consecutive chunks, lane i
//    chunk i, so each lane fetches from device memory the chunk whose swizzled position is its own.
template <int D>
struct Tile {
  static constexpr int RB = 2 * D;        // bytes per row
  static constexpr int CPR = D / 8;       // 16-byte chunks per row
  static constexpr int RPG = 16 / CPR;    // rows per 256 bytes
  static constexpr int kBytes = kBc * RB; // one K or V tile
  static constexpr int kInsts = kBytes / 1024;  // wave-instructions to copy one tile
  __device__ static constexpr int swz_k(int r) { return (r / RPG) % CPR; }
  __device__ static constexpr int swz_v(int r) { return 4 * ((r / RPG) % (CPR / 4)); }
};

// Lazy rescaling: the exponent reference m_ref only moves when some row's new maximum exceeds it by more
// than this (log2 units), so unnormalised weights stay <= 2^8 and the O rescale is skipped on most tiles.
// Any reference gives the same softmax; lse and 1/l use the final reference.
constexpr float kRescaleLog2 = 8.f;

// bf16 kernel: NW waves x 32 query rows per workgroup, K/V tiles of KT x 64 keys (each 64-key part is one
// swizzled Tile in LDS), ST-stage ring holding K and V of the same tile; every wave runs S_j, softmax,
// O += P_j V_j.
template <int D, bool CAUSAL, int NW, int ST, int KT, bool VARLEN, int SPL = 1>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int N, int BH, float scale, int H, int group,
    const int* __restrict__ kv_len, const int* __restrict__ cu_seqlens, int T_total) {
  using T = Tile<D>;
  constexpr int kGroups = NW / SPL;              // row groups (SPL waves share a group's rows, splitting the keys)
  constexpr int kBrW = kGroups * kRowsPerWave;   // query rows per workgroup
  constexpr int kWKT = KT / SPL;                 // 64-key parts of each tile that one wave computes
  constexpr int kDB = D / 16;                    // K-steps of the first product
  constexpr int kCB = D / 32;                    // 32-column blocks of the output
  constexpr int kCopies = T::kInsts / NW;        // copy instructions per wave per tensor per 64-key part
  constexpr int kBcT = KT * kBc;                 // keys per tile
  constexpr int kStage = KT * T::kBytes;         // bytes of one tensor's tile in LDS
  constexpr int kWaitKeep = 2 * KT * kCopies;    // copy instructions per wave per tile (K and V)
  static_assert(T::kInsts % NW == 0, "tile copy must split evenly over the waves");
  static_assert(ST == 2 || ST == 3, "pipeline depth");
  static_assert(KT == 1 || KT == 2, "tile width");
  static_assert((SPL == 1 || SPL == 2) && KT % SPL == 0 && NW % SPL == 0, "key split");
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  lds_char* const smem = (lds_char*)smem_raw;
  lds_char* const kst = smem;                    // ST K stages
  lds_char* const vst = smem + ST * kStage;      // ST V stages

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;

  const int nq = gridDim.x;
  int bh, qb;
  if (VARLEN && BH / H <= 64) {
    // packed batches: (sequence, query block) items in longest-first order (causal: the last blocks, which visit
    // the most key tiles, first)
    const int nb = packed_blocks(cu_seqlens, BH / H, T_total, N, kBrW);
    int rank, hq_, b, kb;
    map_packed(blockIdx.x + nq * blockIdx.y, H, group, rank, hq_);
    if (!longest_first_item(rank, nb, CAUSAL, b, kb)) return;  // the whole workgroup: no item left
    bh = __builtin_amdgcn_readfirstlane(b * H + hq_);
    qb = __builtin_amdgcn_readfirstlane(CAUSAL ? __shfl(nb, b) - 1 - kb : kb);
  } else {
    map_workgroup(blockIdx.x + nq * blockIdx.y, nq, BH, group, CAUSAL, bh, qb);
    if constexpr (CAUSAL && NW == 4 && SPL == 2) {
      // The 64-row causal shape runs its whole grid at once, two workgroups per CU; a CU receives the workgroups
      // at dispatch positions L and L + total/2. The second half of the longest-first order is reversed, so those
      // two take complementary query blocks (qb and nq-1-qb) and every CU gets about the same work.
      if (qb < nq / 2) qb = nq / 2 - 1 - qb;
    }
  }

  // Packed sequences: this head's sequence starts at token `start` and has Ns tokens (offsets clamped to
  // [0, T_total], so a malformed offset array cannot send an access outside the tensors); otherwise Ns = N.
  int start = 0, Ns = N;
  if constexpr (VARLEN) {
    const int lo = min(max(cu_seqlens[bh / H], 0), T_total);
    const int hi = min(max(cu_seqlens[bh / H + 1], lo), T_total);
    start = __builtin_amdgcn_readfirstlane(lo);
    Ns = __builtin_amdgcn_readfirstlane(min(hi - lo, N));  // no longer than max_seqlen (= N)
  }
  const int q_lo = qb * kBrW;
  if (VARLEN && q_lo >= Ns) return;  // the whole workgroup: its query block lies past this sequence
  const int hq = bh % H;
  const int qpitch = VARLEN ? H * D : D;              // elements between consecutive rows of q and o
  const int kpitch = VARLEN ? (H / group) * D : D;    // ... of k and v
  const int kpitch_b = 2 * kpitch;
  const size_t head_off = VARLEN ? ((size_t)start * H + hq) * D : (size_t)bh * (size_t)N * D;
  const size_t kv_off = VARLEN ? ((size_t)start * (H / group) + hq / group) * D
                               : (size_t)(bh / group) * (size_t)N * D;  // key/value head of this query head
  const size_t lse_off = VARLEN ? (size_t)hq * T_total + start : (size_t)bh * N;
  const __bf16* qh = q + head_off;
  const __bf16* kh = k + kv_off;
  const __bf16* vh = v + kv_off;
  // valid keys of this batch (key-padding mask), clamped to [0, N]
  const int Nk = kv_len ? __builtin_amdgcn_readfirstlane(min(max(kv_len[bh / H], 0), N)) : Ns;

  const int q_last = min(q_lo + kBrW, Ns) - 1;             // last real query row of the workgroup
  const int key_tiles = (Nk + kBcT - 1) / kBcT;             // tiles holding valid keys
  const int n_tiles = CAUSAL ? min(q_last / kBcT + 1, key_tiles) : key_tiles;
  const int kpart = wave / kGroups;                         // which part of each tile's keys this wave takes
  const int kofs = kpart * kWKT * kBc;                         // ... as an offset of keys into the tile
  const int q0w = q_lo + (wave % kGroups) * kRowsPerWave;   // first query row of this wave
  const int my_q = q0w + l32;                               // query row of this lane
  // Tiles j < wave_tiles hold at least one key visible to this wave's rows.
  const int wave_tiles =
      (q0w >= Ns) ? 0
                  : (CAUSAL ? (q0w + kRowsPerWave - 1 < kofs ? 0
                                                             : min(n_tiles, (q0w + kRowsPerWave - 1 - kofs) / kBcT + 1))
                            : n_tiles);

  // ---- Q fragments: lane holds q[my_q][16*kb + 8*h .. +7] (B operand of S^T = K Q^T)
  bf16x8 qf[kDB];
#pragma unroll
  for (int kb = 0; kb < kDB; ++kb) {
    if (my_q < Ns) {
      qf[kb] = *(const bf16x8*)(qh + (size_t)my_q * qpitch + 16 * kb + 8 * h);
    } else {
      qf[kb] = (bf16x8){};
    }
  }

  // ---- tile copies (LDS-DMA). Copy instruction p of this wave writes chunk positions g*64 .. g*64+63 of the
  // tile, g = wave + NW*p; this lane writes position g*64 + lane and fetches the chunk stored there.
  int dma_k[kCopies], dma_v[kCopies];  // byte offsets inside the tile in device memory
#pragma unroll
  for (int p = 0; p < kCopies; ++p) {
    const int pos = (wave + NW * p) * 64 + lane;
    const int row = pos / T::CPR, phys = pos % T::CPR;
    dma_k[p] = row * kpitch_b + (phys ^ T::swz_k(row)) * 16;
    dma_v[p] = row * kpitch_b + (phys ^ T::swz_v(row)) * 16;
  }
  // Copy tile j of K (or V) into the stage starting `at` bytes into the K (or V) ring.
  auto copy_part = [&](const __bf16* src, lds_char* ring, int j, int at, const int(&dma)[kCopies])
      __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const int row0 = j * kBcT + t * kBc;
      // rows past Nk arrive as zeros: the range ends with the last valid row (rows are kpitch_b >= RB bytes
      // apart). The descriptor must stay in scalar registers (else every copy is wrapped in a loop over distinct
      // descriptors): readfirstlane between the min and the max keeps the pair from fusing into v_med3_i32, a
      // vector instruction, so the whole computation is scalar.
      const int rows = max(0, __builtin_amdgcn_readfirstlane(min(Nk - row0, kBc)));
      const int bytes = rows > 0 ? (rows - 1) * kpitch_b + T::RB : 0;
      const int row_base = __builtin_amdgcn_readfirstlane(min(row0, Nk - 1));
      const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)row_base * kpitch, bytes);
#pragma unroll
      for (int p = 0; p < kCopies; ++p)
        lds_copy16_inline(r, ring + at + t * T::kBytes + (wave + NW * p) * 1024, dma[p]);
    }
  };
  auto copy_k = [&](int j, int at) __attribute__((always_inline)) { copy_part(kh, kst, j, at, dma_k); };
  auto copy_v = [&](int j, int at) __attribute__((always_inline)) { copy_part(vh, vst, j, at, dma_v); };

  // ---- this lane's LDS read offsets (stage 0)
  // K: row 32b + krow (krow = l32 with bits 2 and 3 swapped, see the header), chunk 2kb + h. swz_k depends only
  // on the row modulo 32 here, so one offset per kb serves both 32-key blocks.
  const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  int k_off[kDB];
#pragma unroll
  for (int kb = 0; kb < kDB; ++kb) k_off[kb] = krow * T::RB + ((2 * kb + h) ^ T::swz_k(krow)) * 16;
  // V (transposing read): rows 16m + 8h + 4*half + (lane&15)/4, columns 32cb + 16*((lane>>4)&1) + 4*(lane&3).
  // swz_v depends on the row only through (lane&15)/4 here, so one offset per cb serves every m and half.
  const int vrow = 8 * h + (lane & 15) / 4;
  int v_off[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int col = 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    v_off[cb] = vrow * T::RB + ((col / 8) ^ T::swz_v(vrow)) * 16 + (col % 8) * 2;
  }
  // Read addresses: an LDS instruction's immediate offset reaches 64 KiB and the V ring lies above that. One
  // base register per fragment column (the ring's start plus this lane's offset, opaque to the compiler, which
  // otherwise re-forms the sum for every read) lets every read of every stage and step carry the rest in its
  // immediate: no address arithmetic in the loop.
  int v_base[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    v_base[cb] = (int)(size_t)(vst + kpart * kWKT * T::kBytes + v_off[cb]);
    asm volatile("" : "+v"(v_base[cb]));
  }
  int k_base[kDB];
#pragma unroll
  for (int kb = 0; kb < kDB; ++kb) {
    k_base[kb] = (int)(size_t)(kst + kpart * kWKT * T::kBytes + k_off[kb]);
    asm volatile("" : "+v"(k_base[kb]));
  }

  const float c2 = scale * kLog2e;
  float m_ref = -INFINITY;  // exponent reference (raw-score units) for row my_q
  float l_run = 0.f;        // this lane's share of the running sum (the keys it holds)
  // A tile whose row maximum exceeds m_grow = m_ref + kRescaleLog2 / c2 moves the reference; nb = -m_ref * c2 is
  // the exponent offset of the weights. Until a key of the row has been seen (m_ref = -inf) every finite maximum
  // exceeds m_grow, and nb = 0 leaves the weights of a fully masked tile at exactly 0.
  const float grow_gap = kRescaleLog2 / c2;
  float m_grow = -INFINITY, nb = 0.f;
  f32x16 oacc[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) oacc[cb] = (f32x16){};

  // S^T = K_j Q^T from the K stage at byte `kat` (2KT blocks of 32 keys; block b = rows 32(b%2).. of part b/2).
  // s[b][r] is the score of query my_q and key j*64KT + 32b + 16(r/8) + 8h + r%8.
  auto qk = [&](f32x16(&s)[2 * kWKT], int kat) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < 2 * kWKT; ++b) {
      s[b] = (f32x16){};
#pragma unroll
      for (int kb = 0; kb < kDB; ++kb) {
        const bf16x8 kf = *(const __attribute__((address_space(3))) bf16x8*)(
            (lds_char*)(size_t)k_base[kb] + (kat + (b >> 1) * T::kBytes + 32 * (b & 1) * T::RB));
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kb], s[b], 0, 0, 0);
      }
    }
    // Issue order for the block above (scheduling groups: 0x100 = LDS read, 0x008 = MFMA): 4 fragment reads,
    // then one MFMA per further read, so each K fragment is read ~4 MFMAs before it is used.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * kWKT * kDB - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // Mask (only tiles that cross the diagonal or the end of the valid keys), row max and (rarely) the move of
  // the exponent reference, for tile j held in s.
  auto stats = [&](f32x16(&s)[2 * kWKT], int j) __attribute__((always_inline)) {
    const int kv0 = j * kBcT + kofs;  // first key of this wave's part of tile j
    if ((kv0 + kWKT * kBc > Nk) || (CAUSAL && kv0 + kWKT * kBc - 1 > q0w)) {
      // key kv0 + 8h + o (o = 32b + 16(r/8) + r%8) is visible iff key < Nk and (causal) key <= my_q, i.e. iff
      // o <= lim: one compare against a constant per score
      const int lim = (CAUSAL ? min(Nk - 1, my_q) : Nk - 1) - kv0 - 8 * h;
#pragma unroll
      for (int b = 0; b < 2 * kWKT; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = (32 * b + 16 * (r >> 3) + (r & 7) <= lim) ? s[b][r] : -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < 2 * kWKT; ++b)
#pragma unroll
      for (int r = (b == 0); r < 16; ++r) mx = row_max(mx, s[b][r]);
    mx = pair_max32(mx);  // row max over this tile's keys
    const bool grow = mx > m_grow;
    if (__any(grow)) {
      const float m_new = fmaxf(m_ref, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // no visible key yet: any finite reference
      const float alpha = __builtin_amdgcn_exp2f((m_ref - m_use) * c2);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) oacc[cb] *= alpha;
      m_ref = m_use;
      m_grow = m_ref + grow_gap;
      nb = -m_ref * c2;
    }
  };

  // P = exp2(s*c2 - m_ref*c2) and O^T += V^T P^T from the V stage at byte `vat`, one 16-key step m at a time:
  // the 8 exponentials of step m+1 can run on the vector ALU while the MFMAs of step m run, and the V fragments
  // of step m+1 are read during step m. Lane slot 8h+e of step m <-> key j*64KT + 16m + 8h + e.
  auto softmax_pv = [&](f32x16(&s)[2 * kWKT], int vat) __attribute__((always_inline)) {
    float rs[2] = {0.f, 0.f};
    auto read_v = [&](int m, bf16x8(&vf)[kCB]) __attribute__((always_inline)) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const lds_char* va = (lds_char*)(size_t)v_base[cb] + (vat + (m >> 2) * T::kBytes + 16 * (m & 3) * T::RB);
        const bf16x4 v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(va));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(va + 4 * T::RB));
        vf[cb] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    bf16x8 vfa[kCB], vfb[kCB];
    read_v(0, vfa);
#pragma unroll
    for (int m = 0; m < 4 * kWKT; ++m) {
      bf16x8(&vcur)[kCB] = (m & 1) ? vfb : vfa;
      bf16x8(&vnxt)[kCB] = (m & 1) ? vfa : vfb;
      f32x8 x = (m & 1) ? s[m >> 1].hi : s[m >> 1].lo;
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c2, nb));
      const bf16x8 pf = __builtin_convertvector(p, bf16x8);
      // Row sum of the rounded weights (the ones the MFMA multiplies V by), two per v_dot2c_f32_bf16.
      rs[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 0, 1), kOnes2, rs[0], false);
      rs[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 2, 3), kOnes2, rs[1], false);
      rs[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 4, 5), kOnes2, rs[0], false);
      rs[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 6, 7), kOnes2, rs[1], false);
      if (m < 4 * kWKT - 1) read_v(m + 1, vnxt);
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur[cb], pf, oacc[cb], 0, 0, 0);
    }
    l_run += rs[0] + rs[1];
  };

  f32x16 s[2 * kWKT];
  {
    // One tile: start copying tile j+ST-1 into the stage tile j-1 used (every wave finished it before the last
    // barrier), compute tile j, wait for this wave's copies of tile j+1, barrier.
    auto step = [&](int j, auto stc) __attribute__((always_inline)) {
      constexpr int S = decltype(stc)::value;
      const bool issue = j + ST - 1 < n_tiles;
      if (issue) {
        copy_k(j + ST - 1, ((S + ST - 1) % ST) * kStage);
        copy_v(j + ST - 1, ((S + ST - 1) % ST) * kStage);
      }
      if (j < wave_tiles) {
        qk(s, S * kStage);
        stats(s, j);
        softmax_pv(s, S * kStage);
      }
      if (ST == 3 && issue) {
        wait_copies_and_barrier<kWaitKeep>();  // tile j+2's copies may stay in flight
      } else {
        wait_copies_and_barrier<0>();
      }
    };
    // prologue: tiles 0 .. ST-2 into stages 0 .. ST-2 (none when the batch has no valid key; n_tiles is the
    // same for the whole workgroup)
    if (n_tiles > 0) {
      copy_k(0, 0);
      copy_v(0, 0);
      if (ST == 3 && n_tiles > 1) {
        copy_k(1, kStage);
        copy_v(1, kStage);
        wait_copies_and_barrier<kWaitKeep>();
      } else {
        wait_copies_and_barrier<0>();
      }
    }
    for (int j = 0; j < n_tiles; j += ST) {
      step(j, Int<0>{});
      if (j + 1 < n_tiles) step(j + 1, Int<1>{});
      if constexpr (ST == 3) {
        if (j + 2 < n_tiles) step(j + 2, Int<2>{});
      }
    }
  }

  // ---- epilogue: o = acc / l once per row, lse = m*scale + ln l. l >= 1 whenever a key is visible (the weight
  // of the maximum is >= 1); l == 0 only for a row without visible keys: o = 0, lse = -inf.
  float l_tot = pair_sum32(l_run);
  if constexpr (SPL == 2) {
    // The two waves of a row group hold partial (m, l, O) over the two halves of every tile's keys; the second
    // hands its partial to the first through LDS (the ring is free: every wave passed the last tile's barrier),
    // which merges them with the block-merge rule. A partial without visible keys (l = 0) has no maximum.
    constexpr int kSlot = 64 * 16 * 4 * kCB + 2 * 64 * 4;  // O (4 kCB f32x4 per lane), then m and l per lane
    lds_char* const slot = smem + (wave % kGroups) * kSlot;
    if (kpart == 1) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(__attribute__((address_space(3))) f32x4*)(slot + ((cb * 4 + g) * 64 + lane) * 16) =
              (f32x4){oacc[cb][4 * g], oacc[cb][4 * g + 1], oacc[cb][4 * g + 2], oacc[cb][4 * g + 3]};
      *(__attribute__((address_space(3))) float*)(slot + 16 * 64 * 4 * kCB + lane * 4) = m_ref;
      *(__attribute__((address_space(3))) float*)(slot + 16 * 64 * 4 * kCB + 256 + lane * 4) = l_tot;
    }
    wait_copies_and_barrier<0>();
    if (kpart == 1) return;  // the first wave of the group writes the row group's o and lse
    const float m1 = *(const __attribute__((address_space(3))) float*)(slot + 16 * 64 * 4 * kCB + lane * 4);
    const float l1 = *(const __attribute__((address_space(3))) float*)(slot + 16 * 64 * 4 * kCB + 256 + lane * 4);
    const float m0e = l_tot > 0.f ? m_ref : -INFINITY, m1e = l1 > 0.f ? m1 : -INFINITY;
    const float mm = fmaxf(m0e, m1e);
    const float m_use = (mm == -INFINITY) ? 0.f : mm;
    const float a0 = __builtin_amdgcn_exp2f((m0e - m_use) * c2), a1 = __builtin_amdgcn_exp2f((m1e - m_use) * c2);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 w = *(const __attribute__((address_space(3))) f32x4*)(slot + ((cb * 4 + g) * 64 + lane) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[cb][4 * g + e] = oacc[cb][4 * g + e] * a0 + w[e] * a1;
      }
    l_tot = l_tot * a0 + l1 * a1;
    m_ref = m_use;
  }
  if (my_q < Ns) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* orow = o + head_off + (size_t)my_q * qpitch;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // oacc[cb][4g + i] is column 32cb + 8g + 4h + i of row my_q
        f32x4 x = {oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv, oacc[cb][4 * g + 2] * inv,
                   oacc[cb][4 * g + 3] * inv};
        *(bf16x4*)(orow + 32 * cb + 8 * g + 4 * h) = __builtin_convertvector(x, bf16x4);
      }
    }
    if (h == 0)
      lse[lse_off + my_q] = l_tot > 0.f ? (m_ref * c2 + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
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
  map_workgroup(blockIdx.x + nq * blockIdx.y, nq, BH, 1, CAUSAL, bh, qb);

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
template <int D, bool CAUSAL, int NW, int ST, int KT, bool VARLEN = false, int SPL = 1>
static hipError_t launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                              float scale, int H, int group, const int* kv_len, hipStream_t stream,
                              const int* cu_seqlens = nullptr, int T_total = 0) {
  constexpr int lds = 2 * ST * KT * Tile<D>::kBytes;
  constexpr int rows = NW / SPL * kRowsPerWave;
  auto kern = fa_fwd_bf16_kernel<D, CAUSAL, NW, ST, KT, VARLEN, SPL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + rows - 1) / rows), (unsigned)BH);
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), lds, stream, (const __bf16*)q, (const __bf16*)k,
                     (const __bf16*)v, (__bf16*)o, lse, N, BH, scale, H, group, kv_len, cu_seqlens, T_total);
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

// Workgroup shape, from the number of query rows to spread over the 256 CUs of an MI355X:
//  * wide: 8 waves x 32 rows (256 rows, 128-key tiles, one workgroup per CU) when the grid has at least two such
//    workgroups per CU;
//  * narrow: 4 waves x 32 rows (128 rows, 64-key tiles, two workgroups per CU) when it has at least two of those
//    per CU;
//  * split: otherwise (too few rows to give every SIMD two waves of 32 rows): 8 waves x 128 rows, the two waves
//    of each 32-row group taking the two 64-key halves of every 128-key tile and merging their partial (m, l, O)
//    at the end. Short sequences of few heads (and long ones of very few) get two waves per SIMD this way.
//  * split64 (causal, d = 64, not for packed batches): the split shape on 64 rows and 4 waves, when its grid fits
//    on the chip at two workgroups per CU (at most 512): every 64-row block is resident at once and each CU pairs a
//    long causal block with a short one (see the mapping in the kernel). Same arithmetic per row as the split
//    shape, so the same bits.
// Wide, narrow and split differ in where the exponent reference may move and in the order of the sums, so their
// outputs can differ in the last bit; each is deterministic, and the packed entry point chooses among them the same
// way from max_seqlen.
constexpr long long kTwoPerCu = 512;
enum class Shape { kWide = 0, kNarrow = 1, kSplit = 2, kSplit64 = 3 };
static Shape fwd_shape(int N, int BH, int d, bool causal, bool packed) {
  if ((long long)((N + 255) / 256) * BH >= kTwoPerCu) return Shape::kWide;
  if ((long long)((N + 127) / 128) * BH >= kTwoPerCu) return Shape::kNarrow;
  if (causal && d == 64 && !packed && (long long)((N + 63) / 64) * BH <= kTwoPerCu) return Shape::kSplit64;
  return Shape::kSplit;
}
// (NW, KT, SPL) of each shape; the ring always has 2 stages.
#define FA_WIDE 8, 2, 1
#define FA_NARROW 4, 1, 1
#define FA_SPLIT 8, 2, 2
#define FA_SPLIT64 4, 2, 2

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                           int N, int d, bool causal, float scale, const int* kv_len, hipStream_t stream) {
  const int BH = B * H, group = H / Hkv;
#define FA_LAUNCH(D, C, NW, KT, SPL) \
  launch_bf16<D, C, NW, 2, KT, false, SPL>(q, k, v, o, lse, BH, N, scale, H, group, kv_len, stream)
#define FA_D2(NW, KT, SPL)                                                                       \
  (d == 64 ? (causal ? FA_LAUNCH(64, true, NW, KT, SPL) : FA_LAUNCH(64, false, NW, KT, SPL)) \
           : (causal ? FA_LAUNCH(128, true, NW, KT, SPL) : FA_LAUNCH(128, false, NW, KT, SPL)))
#define FA_D(...) FA_D2(__VA_ARGS__)
  switch (fwd_shape(N, BH, d, causal, false)) {
    case Shape::kWide: return FA_D(FA_WIDE);
    case Shape::kNarrow: return FA_D(FA_NARROW);
    case Shape::kSplit64: return launch_bf16<64, true, 4, 2, 2, false, 2>(q, k, v, o, lse, BH, N, scale, H, group,
                                                                         kv_len, stream);
    default: return FA_D(FA_SPLIT);
  }
#undef FA_D
#undef FA_D2
#undef FA_LAUNCH
}

hipError_t launch_fwd_varlen_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                  const int* cu_seqlens, int B, int H, int Hkv, int T_total, int max_seqlen, int d,
                                  bool causal, float scale, hipStream_t stream) {
  const int BH = B * H, group = H / Hkv, N = max_seqlen;
#define FA_LAUNCH(D, C, NW, KT, SPL)                                                                                 \
  launch_bf16<D, C, NW, 2, KT, true, SPL>(q, k, v, o, lse, BH, N, scale, H, group, nullptr, stream, cu_seqlens, \
                                          T_total)
#define FA_D2(NW, KT, SPL)                                                                       \
  (d == 64 ? (causal ? FA_LAUNCH(64, true, NW, KT, SPL) : FA_LAUNCH(64, false, NW, KT, SPL)) \
           : (causal ? FA_LAUNCH(128, true, NW, KT, SPL) : FA_LAUNCH(128, false, NW, KT, SPL)))
#define FA_D(...) FA_D2(__VA_ARGS__)
  switch (fwd_shape(N, BH, d, causal, true)) {
    case Shape::kWide: return FA_D(FA_WIDE);
    case Shape::kNarrow: return FA_D(FA_NARROW);
    default: return FA_D(FA_SPLIT);
  }
#undef FA_D
#undef FA_D2
#undef FA_LAUNCH
}

// The name of the instance the two launchers above pick, as the kernel's template arguments spell it.
const char* fwd_instance_bf16(int BH, int N, int d, bool causal, bool packed) {
#define FA_NAME2(D, C, V, NW, KT, SPL) "fa_fwd_bf16_kernel<" #D ", " #C ", " #NW ", 2, " #KT ", " #V ", " #SPL ">"
#define FA_NAME(D, C, V, ...) FA_NAME2(D, C, V, __VA_ARGS__)
#define FA_NAMES(S)                                                                              \
  {{{FA_NAME(64, false, false, S), FA_NAME(64, false, true, S)},                                 \
    {FA_NAME(64, true, false, S), FA_NAME(64, true, true, S)}},                                  \
   {{FA_NAME(128, false, false, S), FA_NAME(128, false, true, S)},                               \
    {FA_NAME(128, true, false, S), FA_NAME(128, true, true, S)}}}
  static const char* const names[3][2][2][2] = {FA_NAMES(FA_WIDE), FA_NAMES(FA_NARROW), FA_NAMES(FA_SPLIT)};
  const Shape shape = fwd_shape(N, BH, d, causal, packed);
  if (shape == Shape::kSplit64) return FA_NAME(64, true, false, FA_SPLIT64);
#undef FA_NAMES
#undef FA_NAME
#undef FA_NAME2
  return names[(int)shape][d == 128][causal][packed];
}
#undef FA_WIDE
#undef FA_NARROW
#undef FA_SPLIT
#undef FA_SPLIT64

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N, int d,
                          bool causal, float scale, hipStream_t stream) {
  if (d == 64) return causal ? launch_f32<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                             : launch_f32<64, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch_f32<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_f32<128, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace fa
