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

#ifdef __cplusplus
}
#endif
#endif
