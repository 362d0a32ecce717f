/* fa_probe.h -- C ABI of libfa_probe.so, a measurement aid shipped beside libfa.so (not part of the attention
 * path): a dense bf16 matrix-core throughput probe for gfx950 (MI355X).
 *
 * It runs v_mfma_f32_32x32x16_bf16 back to back on register operands of pseudo-random unit-magnitude bf16
 * values (no memory traffic in the timed loop), two waves per SIMD, and records each workgroup's shader cycles
 * and 100 MHz real-time ticks. The caller times the launch (HIP events on `stream`) and derives
 *   FLOP/s        = n_wg * iters * fa_probe_flop_per_wg_iter() / elapsed seconds
 *   shader clock  = sum(cycles) / sum(ticks) * 100 MHz
 * which quote the attention kernels against the rate the matrix cores of this GPU sustain at the clock its power
 * limit allows, next to the data-sheet peak (2516.6 TFLOP/s at 2.4 GHz).
 */
#ifndef FA_MI355X_FA_PROBE_H
#define FA_MI355X_FA_PROBE_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue the probe on `stream`.
 *   sink  : device float[n_wg * fa_probe_threads()] (written; keeps the products live)
 *   clk   : device unsigned long long[2 * n_wg] (written: cycles, then real-time ticks, per workgroup)
 *   n_wg  : workgroups, 1 .. 2^20 (use several per compute unit: 2048 fills MI355X's 256 CUs 8 times over)
 *   iters : loop iterations per wave, >= 1 (8 MFMAs each)
 * Returns 0 once enqueued; 1 if a pointer is NULL, 2 if n_wg or iters is out of range, 3 if the launch failed.
 * The library allocates nothing and keeps no state. */
int fa_probe_mfma_bf16(float* sink, unsigned long long* clk, int n_wg, int iters, hipStream_t stream);

/* FLOPs one workgroup performs per loop iteration (4 waves x 8 MFMAs x 32768). */
double fa_probe_flop_per_wg_iter(void);

/* Threads per workgroup of the probe (the sink holds one float per thread). */
int fa_probe_threads(void);

/* Issue-mix probe: can the matrix cores run while the vector ALU computes exponentials? 8-wave workgroups
 * (waves w and w+4 share a SIMD; launch 256 of them for one per CU); per loop iteration each wave issues
 *   mode 0: 8 MFMAs;  1: 8 MFMAs + 8 exp2;  2: 8 MFMAs + 8 exp2 + 24 FMAs (all in the same wave);
 *   mode 3: waves 0-3 8 MFMAs, waves 4-7 8 exp2 + 24 FMAs (one role per wave of a SIMD);  4: 8 exp2 + 24 FMAs,
 * the vector chains independent of the products.
 *   sink : device float[n_wg * fa_probe_issue_mix_threads()] (written; keeps the results live)
 *   cyc  : device unsigned long long[8 * n_wg] (written: shader cycles over the loop, per wave)
 *   n_wg : workgroups, 1 .. 2^20;  iters : loop iterations, >= 1
 * Returns 0 once enqueued; 1 if a pointer is NULL, 2 if mode, n_wg or iters is out of range, 3 if the launch
 * failed. Cycles per iteration = cyc / iters. */
int fa_probe_issue_mix(int mode, float* sink, unsigned long long* cyc, int n_wg, int iters, hipStream_t stream);

/* Threads per workgroup of the issue-mix probe. */
int fa_probe_issue_mix_threads(void);

/* Atomic-add probe: how fast fp32 atomic adds into device memory run, for a kernel that would sum 128 x 128 fp32
 * partial blocks from many workgroups into one buffer. 512-thread workgroups; per round each adds 1.0 to every
 * float of one 64 KiB tile (fa_probe_atomic_tile_floats() floats), coalesced, without return. The tile of
 * workgroup wg in round r, by mode:
 *   0: (7 wg + r) mod tiles, any XCD;  1: only workgroups wg = t (mod 8) touch tile t (one XCD per tile, the
 *   dispatcher placing workgroups round-robin over the 8 XCDs);  2: 32 consecutive workgroups on one tile at once;
 *   3: as 0 with plain stores of 1.0 (the write rate to compare with).
 *   buf    : device float[tiles * fa_probe_atomic_tile_floats()], caller-allocated; modes 0-2 add to it (clear it
 *            first to check the sum: n_wg * rounds * fa_probe_atomic_tile_floats() per launch), mode 3 sets it to 1
 *   tiles  : 8 .. 65536, a multiple of 8;  n_wg : workgroups, 1 .. 2^20;  rounds : tiles per workgroup, >= 1
 * Returns 0 once enqueued; 1 if buf is NULL, 2 if an argument is out of range, 3 if the launch failed.
 * Bytes per launch = n_wg * rounds * 4 * fa_probe_atomic_tile_floats(). */
int fa_probe_atomic_add(int mode, float* buf, int tiles, int n_wg, int rounds, hipStream_t stream);

/* Floats per tile of the atomic-add probe (16384). */
int fa_probe_atomic_tile_floats(void);

#ifdef __cplusplus
}
#endif
#endif
