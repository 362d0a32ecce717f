// launch_stubs.cpp -- host-only stand-ins for the kernel launchers of fa_launch.h, for the sanitizer build of the
// C ABI (fa_api.hip compiled with g++ -fsanitize=address,undefined and no GPU code). Each records the call and
// its sizes and returns hipSuccess; nothing touches a device.
#include <stdint.h>

#include "fa_launch.h"

namespace fa {
int g_calls = 0;      // launcher calls since the last reset
int g_last[8] = {0};  // sizes of the last call: B*H (or BH), N (or total), d, causal, Hkv, max_seqlen

static hipError_t record(int a, int b, int c, int d, int e = 0, int f = 0) {
  ++g_calls;
  g_last[0] = a; g_last[1] = b; g_last[2] = c; g_last[3] = d; g_last[4] = e; g_last[5] = f;
  return hipSuccess;
}

hipError_t launch_fwd_bf16(const void*, const void*, const void*, void*, float*, int B, int H, int Hkv, int N, int d,
                           bool causal, float, const int*, hipStream_t) {
  return record(B * H, N, d, causal, Hkv);
}
hipError_t launch_fwd_varlen_bf16(const void*, const void*, const void*, void*, float*, const int*, int B, int H,
                                  int Hkv, int T_total, int max_seqlen, int d, bool causal, float, hipStream_t) {
  return record(B * H, T_total, d, causal, Hkv, max_seqlen);
}
hipError_t launch_fwd_fp8(const void*, const void*, const void*, void*, float*, int BH, int N, int d, bool causal,
                          float, float, float, float, hipStream_t) {
  return record(BH, N, d, causal);
}
hipError_t launch_fwd_f32(const float*, const float*, const float*, float*, float*, int BH, int N, int d, bool causal,
                          float, hipStream_t) {
  return record(BH, N, d, causal);
}
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const float*, const void*, void*,
                           void*, void*, float*, int B, int H, int Hkv, int N, int d, bool causal, float, const int*,
                           hipStream_t) {
  return record(B * H, N, d, causal, Hkv);
}
hipError_t launch_bwd_varlen_bf16(const void*, const void*, const void*, const void*, const float*, const void*,
                                  void*, void*, void*, float*, const int*, int B, int H, int Hkv, int T_total,
                                  int max_seqlen, int d, bool causal, float, hipStream_t) {
  return record(B * H, T_total, d, causal, Hkv, max_seqlen);
}
const char* fwd_instance_bf16(int, int, int, bool, bool) { return "stub"; }
}  // namespace fa

namespace fa {
// stand-in for the scratch buffer's device address (never dereferenced on the host)
hipError_t scratch_address(hipStream_t, void** out) {
  *out = (void*)(uintptr_t)(uint64_t(0x3f) << 56);
  return hipSuccess;
}
}  // namespace fa
