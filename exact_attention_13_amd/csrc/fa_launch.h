// fa_launch.h -- internal interface between the C ABI layer and the kernels (not installed, not public).
#ifndef FA_MI355X_FA_LAUNCH_H
#define FA_MI355X_FA_LAUNCH_H
#include <hip/hip_runtime_api.h>

namespace fa {
// Enqueue one attention-forward kernel. Arguments must already be valid (d is 64 or 128, BH >= 1, N >= 1,
// pointers device-resident and aligned); returns the launch status.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                           bool causal, float scale, hipStream_t stream);
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N, int d,
                          bool causal, float scale, hipStream_t stream);
}  // namespace fa
#endif
