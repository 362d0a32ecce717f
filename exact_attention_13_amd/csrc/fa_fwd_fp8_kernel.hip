// fa_fwd_fp8_kernel.hip -- exact attention forward of per-tensor-scaled fp8 (float8_e4m3fn) inputs, gfx950.
//
// FP8 is listed among the FlashAttention-3 techniques on the unite.ai page "Flash Attention: revolutionizing
// transformer efficiency" (section "FlashAttention-3", items 2-3). The real inputs are q8 * s_q, k8 * s_k and
// v8 * s_v (one fp32 scale per tensor); the algorithm is the bf16 kernel's (tiles of keys through LDS, running
// maximum and sum, 1/l once at the end) on the fp8 matrix instruction v_mfma_f32_32x32x64_f8f6f4 (K = 64, twice
// the bf16 rate):
//   * S^T = K Q^T per 32-key block: A = 32 K rows (32 bytes of d per lane), B = the lane's query row (Q in
//     registers). The scales fold into the exponent constant: p = exp2(s * c - m * c), c = scale s_q s_k log2 e.
//   * The instruction contracts lane half h, byte e of A with lane half h, byte e of B, so which d (or key) a
//     byte slot holds is free as long as both operands agree. K rows are fed so that in block b of a 64-key part
//     value r of lane half h is key 32h + 16b + r: the 32 p values of a lane half are the 32 consecutive keys
//     32h .. 32h+31, exactly what the V^T operand of O^T += V^T P^T holds for that half.
//   * V arrives transposed ([B, H, d, N]) so that V^T rows (one d column, consecutive keys) are contiguous: the
//     A operand of O^T += V^T P^T is two 16-byte LDS reads per lane, and P^T is the B operand straight from
//     registers (p rounded to e4m3 with v_cvt_pk_fp8_f32).
//   * The row sum l adds the rounded weights the product used, so o is a weighted average under them: one more
//     O^T-shaped instruction per 64 keys with an all-ones A operand gives sum_j p_j for every query lane.
//   * o = acc * s_v / l in bf16, lse in natural log as the bf16 kernel. Lazy rescaling keeps p at most 2^8 (up to
//     the rounding of the threshold m_ref + 8 / c), well inside e4m3's range (448).
//   * 8-wave workgroups take a tile's weights against the current reference first and form the row maximum only
//     when some row's weights sum to 2^8 or more, the only case in which the reference could have to move (the
//     tile loop below); the softmax work per key is then exponential, FMA and conversion.
#include <type_traits>

#include "fa_gfx950.h"
#include "fa_launch.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8Rows = 32;  // query rows per wave
constexpr int kF8Part = 64;  // keys per LDS part (one K part and one V^T part)
constexpr float kF8Rescale = 8.f;
constexpr float kF8SumLimit = 256.f;  // 2^kF8Rescale

// K part: 64 rows of d bytes; V^T part: d rows of 64 bytes. 16-byte chunks are XOR-swizzled so that each 16-byte
// read (16 lanes, 16 rows, one chunk) hits 16 different bank groups. A lane's 32-byte fragment is two chunks c, c+1
// (c even), read separately: the swizzle may store them in either order.
template <int D>
struct F8Tile {
  static constexpr int KRB = D;          // bytes per K row
  static constexpr int KCPR = D / 16;    // chunks per K row
  static constexpr int KRPG = 16 / KCPR; // K rows per 256 bytes
  static constexpr int VRB = kF8Part;    // bytes per V^T row
  static constexpr int kBytes = kF8Part * D;  // one K part or one V^T part
  static constexpr int kInsts = kBytes / 1024;
  // K rows read together are {16b' + t, 32 + 16b' + t}: distinct (t / KRPG) and bit 5 of the row
  __device__ static constexpr int swz_k(int r) {
    return ((r / KRPG) & (KCPR / 2 - 1)) | (((r >> 5) & 1) * (KCPR / 2));
  }
  // V^T rows read together are 16 consecutive d columns, 4 per 256 bytes
  __device__ static constexpr int swz_v(int r) { return (r >> 2) & 3; }
};

// A 32-byte fragment from two 16-byte chunks; the second chunk sits at the first one's offset ^ 16 (rows start on
// 32-byte boundaries and the pair differs only in the lowest chunk bit).
__device__ __forceinline__ i32x8 lds_read32(const lds_char* base, int off) {
  const u32x4 a = *(const __attribute__((address_space(3))) u32x4*)(base + off);
  const u32x4 b = *(const __attribute__((address_space(3))) u32x4*)(base + (off ^ 16));
  return (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // fp8 e4m3 for both operands (format fields 0), no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, bool CAUSAL, int NW, int KT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ vt,
    __bf16* __restrict__ o, float* __restrict__ lse, int N, int BH, float c2, float v_scale) {
  using T = F8Tile<D>;
  constexpr int kKS = D / 64;      // 64-wide d steps of S^T
  constexpr int kCB = D / 32;      // 32-column blocks of O^T
  constexpr int kTileInsts = KT * T::kInsts;  // copy instructions per tensor per tile
  constexpr int kCopies = kTileInsts / NW;
  constexpr int kBcT = KT * kF8Part;
  constexpr int kStage = KT * T::kBytes;
  static_assert(kTileInsts % NW == 0, "tile copy must split evenly over the waves");
  // 2 K stages, then 2 V^T stages (at most 64 KiB). Static rather than dynamic: its address is then known when
  // instructions are selected, so the stage and part offsets fold into the reads' immediate offsets instead of
  // costing a vector add per fragment address and tile.
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * kStage];
  lds_char* const kst = (lds_char*)smem_raw;  // 2 K stages
  lds_char* const vst = kst + 2 * kStage;     // 2 V^T stages

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nq = gridDim.x;
  int bh, qb;
  map_workgroup(blockIdx.x + nq * blockIdx.y, nq, BH, 1, CAUSAL, bh, qb);
  const size_t head_off = (size_t)bh * (size_t)N * D;  // q, k, o (and v^T: d rows of N)
  const uint8_t* kh = k + head_off;
  const uint8_t* vh = vt + head_off;

  const int q_lo = qb * (NW * kF8Rows);
  const int q_last = min(q_lo + NW * kF8Rows, N) - 1;
  const int n_tiles = CAUSAL ? (q_last / kBcT + 1) : (N + kBcT - 1) / kBcT;
  const int q0w = q_lo + wave * kF8Rows;
  const int my_q = q0w + l32;
  const int wave_tiles = (q0w >= N) ? 0 : (CAUSAL ? min(n_tiles, (q0w + kF8Rows - 1) / kBcT + 1) : n_tiles);

  // Q fragments: d bytes 64ks + 32h .. +31 of row my_q (B operand of S^T = K Q^T)
  i32x8 qf[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    if (my_q < N) {
      const u32x4* p = (const u32x4*)(q + head_off + (size_t)my_q * D + 64 * ks + 32 * h);
      const u32x4 a = p[0], b = p[1];
      qf[ks] = (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    } else {
      qf[ks] = (i32x8){};
    }
  }

  // LDS-DMA: copy instruction g = wave + NW p of a tile writes chunk positions (g % kInsts)*64 .. +63 of part
  // g / kInsts. K part: position pos -> row pos / KCPR; V^T part: row pos / 4 (64-byte rows).
  int dk_off[kCopies], dv_off[kCopies], part[kCopies];
#pragma unroll
  for (int p = 0; p < kCopies; ++p) {
    const int g = wave + NW * p;
    part[p] = g / T::kInsts;  // wave-uniform
    const int pos = (g % T::kInsts) * 64 + lane;
    const int kr = pos / T::KCPR, kc = pos % T::KCPR;
    dk_off[p] = kr * T::KRB + (kc ^ T::swz_k(kr)) * 16;
    const int vr = pos / 4, vc = pos % 4;
    dv_off[p] = vr * N + (vc ^ T::swz_v(vr)) * 16;  // byte offset in v^T from the part's first key
  }
  auto copy_tile = [&](int j, int at) __attribute__((always_inline)) {
    __amdgpu_buffer_rsrc_t rk[KT], rv[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const int key0 = j * kBcT + t * kF8Part;
      // K: rows past N arrive as zeros. V^T: d rows of N bytes from key0; columns past N read the next row's
      // keys (weighted by p = 0) and the range ends with the last row's valid keys.
      const int kbytes = __builtin_amdgcn_readfirstlane(max(0, min(N - key0, kF8Part)) * T::KRB);
      const int kbase = __builtin_amdgcn_readfirstlane(min(key0, N - 1));
      const int vbytes = __builtin_amdgcn_readfirstlane(max(0, (D - 1) * N + min(N - key0, kF8Part)));
      rk[t] = make_rsrc(kh + (size_t)kbase * D, kbytes);
      rv[t] = make_rsrc(vh + kbase, vbytes);
    }
#pragma unroll
    for (int p = 0; p < kCopies; ++p) {
      const int g = wave + NW * p;
      const bool second = (KT == 2) && part[p] == 1;
      lds_copy16_inline(second ? rk[KT - 1] : rk[0], kst + at + g * 1024, dk_off[p]);
      lds_copy16_inline(second ? rv[KT - 1] : rv[0], vst + at + g * 1024, dv_off[p]);
    }
  };

  // K row of A-lane row i in block b' of a part: 32((i>>2)&1) + 16b' + 4(i>>3) + (i&3), so that value r of
  // lane half h is key 32h + 16b' + r. Its bytes 64ks + 32h .. +31 are chunks 4ks + 2h and 4ks + 2h + 1.
  int k_off[2][kKS];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int kr = 32 * ((l32 >> 2) & 1) + 16 * b + 4 * (l32 >> 3) + (l32 & 3);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) k_off[b][ks] = kr * T::KRB + ((4 * ks + 2 * h) ^ T::swz_k(kr)) * 16;
  }
  // V^T row (d column) 32cb + l32, keys 32h .. +31 = chunks 2h, 2h + 1
  int v_off[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int vr = 32 * cb + l32;
    v_off[cb] = vr * T::VRB + ((2 * h) ^ T::swz_v(vr)) * 16;
  }

  float m_ref = -INFINITY;
  // A tile whose row maximum exceeds m_grow = m_ref + kF8Rescale / c2 moves the reference. Every row sees key 0 in
  // its first tile, so the first maximum is finite and always exceeds the starting m_grow = -inf.
  const float grow_gap = kF8Rescale / c2;
  float m_grow = -INFINITY;
  float nb = 0.f;  // -m_ref * c2, the exponent offset of every weight (set with the first reference)
  f32x16 oacc[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) oacc[cb] = (f32x16){};
  // 8-wave workgroups test each tile's row sums of the weights before forming the row maximum (below); the tile's
  // sum is then read by the vector ALU and added to l_run. 4-wave workgroups chain the sums on the matrix core in
  // lacc (every value: the sum of the rounded weights of this lane's query row) and never wait for them.
  constexpr bool kSumCheck = NW == 8;
  float l_run = 0.f;
  f32x16 lacc = (f32x16){};
  // e4m3 1.0 in every byte, made opaque so that it stays in VGPRs instead of being rebuilt from SGPRs every tile
  i32x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int w = 0x38383838;
    asm volatile("" : "+v"(w));
    ones[i] = w;
  }

  auto step = [&](int j, int S, auto first_c) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_c)::value;  // tile 0 (j == 0)
    const bool issue = j + 1 < n_tiles;
    if (issue) copy_tile(j + 1, (S ^ 1) * kStage);
    if (j < wave_tiles) {
      const lds_char* ks_ = kst + S * kStage;
      const lds_char* vs_ = vst + S * kStage;
      // S^T blocks: part t, block b': value r of lane half h is key j*kBcT + 64t + 32h + 16b' + r; masked scores
      // are -inf.
      auto products = [&](f32x16(&s)[2 * KT], bool again) __attribute__((always_inline)) {
        // A second formation of the same scores reads its fragments through offsets the compiler cannot see
        // through; it would otherwise reuse the first one's scores and hold them in registers across the tile.
        int ko[2][kKS];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks) {
            ko[b][ks] = k_off[b][ks];
            if (again) asm volatile("" : "+v"(ko[b][ks]));
          }
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            f32x16 acc = (f32x16){};
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks) {
              const i32x8 kf = lds_read32(ks_ + t * T::kBytes, ko[b][ks]);
              acc = mfma_f8(kf, qf[ks], acc);
            }
            s[2 * t + b] = acc;
          }
        {
          // Issue order (scheduling groups: 0x100 LDS read, 0x008 MFMA): the fragments of four products first,
          // then each product followed by the reads of the fragment four products ahead.
          constexpr int kN = 2 * KT * kKS;
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * (kN < 4 ? kN : 4), 0);
#pragma unroll
          for (int i = 0; i + 4 < kN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, kN < 4 ? kN : 4, 0);
        }
        const int kv0 = j * kBcT;
        if ((kv0 + kBcT > N) || (CAUSAL && kv0 + kBcT - 1 > q0w)) {
          // key kv0 + 32h + o (o = 64t + 16b + r) is visible iff key < N and (causal) key <= my_q, i.e. iff
          // o <= lim
          const int lim = (CAUSAL ? min(N - 1, my_q) : N - 1) - kv0 - 32 * h;
#pragma unroll
          for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                s[2 * t + b][r] = (64 * t + 16 * b + r <= lim) ? s[2 * t + b][r] : -INFINITY;
        }
      };
      // Row maximum of the tile; when some row's maximum exceeds m_grow, every row's reference moves to its
      // maximum (O and l rescaled). Returns whether it moved.
      auto move_reference = [&](const f32x16(&s)[2 * KT]) __attribute__((always_inline)) -> bool {
        float mx = s[0][0];
#pragma unroll
        for (int i = 0; i < 2 * KT; ++i)
#pragma unroll
          for (int r = (i == 0); r < 16; ++r) mx = row_max(mx, s[i][r]);
        mx = pair_max32(mx);
        const bool grow = mx > m_grow;
        if (!__any(grow)) return false;
        const float m_new = fmaxf(m_ref, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_ref - m_use) * c2);
        if constexpr (kSumCheck) {
          l_run *= alpha;
        } else {
          lacc *= alpha;
        }
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) oacc[cb] *= alpha;
        m_ref = m_use;
        m_grow = m_ref + grow_gap;
        nb = -m_ref * c2;
        return true;
      };
      // Weights of the tile's parts against the current reference (lane half h holds keys 32h + e, e = 16b' + r,
      // as bytes e of the B operand) and their row sum on the matrix core (an all-ones A operand): every value of
      // `ts` is the sum for this lane's query row.
      i32x8 pf[KT];
      f32x16 ts;
      auto weights = [&](const f32x16(&s)[2 * KT]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const f32x16& sv = s[2 * t + (w >> 2)];
            const int r0 = 4 * (w & 3);
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0], c2, nb));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0 + 1], c2, nb));
            const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0 + 2], c2, nb));
            const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0 + 3], c2, nb));
            // the first conversion writes the low half of the word, the second the high half; the word starts
            // as p0's bits (any value would do), so no register has to be cleared first
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(p0), false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
            pf[t][w] = word;
          }
        ts = mfma_f8(ones, pf[0], kSumCheck ? (f32x16){} : lacc);
#pragma unroll
        for (int t = 1; t < KT; ++t) ts = mfma_f8(ones, pf[t], ts);
      };
      // The row maximum matters only when the reference may have to move, i.e. when some weight would reach 2^8
      // (kF8Rescale). Tile 0 sets every row's first reference (each row of the wave sees key 0), so it forms the
      // maximum first. In 8-wave workgroups later tiles take the weights against the current reference first: if
      // every row's rounded weights sum to less than 2^8 (a NaN or saturated weight fails the test), no weight
      // reached 2^8, no row maximum exceeded m_grow (up to the rounding of the exponent argument) and the weights
      // stand. Otherwise the scores are formed again (K is still in LDS), the maximum decides the move as on tile
      // 0, and the weights are taken again. (4-wave workgroups, one wave per SIMD, would wait for the sum with no
      // other wave to fill the matrix core: they form the maximum on every tile.)
      f32x16 s[2 * KT];
      products(s, false);
      if constexpr (kFirst || !kSumCheck) {
        move_reference(s);
        weights(s);
      } else {
        weights(s);
        if (!__all(ts[0] < kF8SumLimit)) {
          products(s, true);
          move_reference(s);
          weights(s);
        }
      }
      if constexpr (kSumCheck) {
        l_run += ts[0];
      } else {
        lacc = ts;
      }
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          const i32x8 vf = lds_read32(vs_ + t * T::kBytes, v_off[cb]);
          oacc[cb] = mfma_f8(vf, pf[t], oacc[cb]);
        }
    }
    wait_copies_and_barrier<0>();
  };
  if (n_tiles > 0) {
    copy_tile(0, 0);
    wait_copies_and_barrier<0>();
  }
  // tile 0 on its own (it sets the first reference), then the stages alternate
  if (n_tiles > 0) step(0, 0, std::true_type{});
  for (int j = 1; j < n_tiles; j += 2) {
    step(j, 1, std::false_type{});
    if (j + 1 < n_tiles) step(j + 1, 0, std::false_type{});
  }

  // o = acc * s_v / l, lse = m*c/log2e + ln l (c holds scale * s_q * s_k * log2 e)
  const float l_tot = kSumCheck ? l_run : lacc[0];
  if (my_q < N) {
    const float f = v_scale / l_tot;
    __bf16* orow = o + head_off + (size_t)my_q * D;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = {oacc[cb][4 * g] * f, oacc[cb][4 * g + 1] * f, oacc[cb][4 * g + 2] * f,
                         oacc[cb][4 * g + 3] * f};
        *(bf16x4*)(orow + 32 * cb + 8 * g + 4 * h) = __builtin_convertvector(x, bf16x4);
      }
    if (h == 0) lse[(size_t)bh * N + my_q] = (m_ref * c2 + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL, int NW, int KT>
static hipError_t launch_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, int BH, int N,
                             float c2, float v_scale, hipStream_t stream) {
  auto kern = fa_fwd_fp8_kernel<D, CAUSAL, NW, KT>;
  const dim3 grid((unsigned)((N + NW * kF8Rows - 1) / (NW * kF8Rows)), (unsigned)BH);
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), 0, stream, (const uint8_t*)q, (const uint8_t*)k,
                     (const uint8_t*)vt, (__bf16*)o, lse, N, BH, c2, v_scale);
  return hipGetLastError();
}

// Same workgroup-shape rule as the bf16 kernel: 8 waves and 128-key tiles when the grid has two such workgroups
// per CU, else 4 waves and 64-key tiles.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, int BH, int N, int d,
                          bool causal, float scale, float q_scale, float k_scale, float v_scale,
                          hipStream_t stream) {
  const float c2 = scale * q_scale * k_scale * kLog2e;
  const bool wide = (long long)((N + 255) / 256) * BH >= 512;
#define FA_F8(D, C, NW, KT) launch_fp8<D, C, NW, KT>(q, k, vt, o, lse, BH, N, c2, v_scale, stream)
  if (wide) {
    if (d == 64) return causal ? FA_F8(64, true, 8, 2) : FA_F8(64, false, 8, 2);
    return causal ? FA_F8(128, true, 8, 2) : FA_F8(128, false, 8, 2);
  }
  if (d == 64) return causal ? FA_F8(64, true, 4, 1) : FA_F8(64, false, 4, 1);
  return causal ? FA_F8(128, true, 4, 1) : FA_F8(128, false, 4, 1);
#undef FA_F8
}

}  // namespace fa
