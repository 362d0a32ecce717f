// fa_launch.h -- internal interface between the C ABI layer and the kernels (not installed, not public).
#ifndef FA_MI355X_FA_LAUNCH_H
#define FA_MI355X_FA_LAUNCH_H
#include <hip/hip_runtime_api.h>

namespace fa {
// Enqueue one attention-forward kernel. Arguments must already be valid (d is 64 or 128, B, H, N >= 1, Hkv >= 1
// dividing H, pointers device-resident and aligned); returns the launch status. k and v have Hkv heads; kv_len
// is NULL or B device int32 counts of valid keys (clamped to [0, N] by the kernel).
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                           int N, int d, bool causal, float scale, const int* kv_len, hipStream_t stream);
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N, int d,
                          bool causal, float scale, hipStream_t stream);
}  // namespace fa
#endif
