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
// Packed variable-length batches: q, o [T, H, d], k, v [T, Hkv, d], lse [H, T]; sequence b is tokens
// cu_seqlens[b] .. cu_seqlens[b+1]-1 (device int32, B+1 entries), none longer than max_seqlen >= 1.
hipError_t launch_fwd_varlen_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                  const int* cu_seqlens, int B, int H, int Hkv, int T_total, int max_seqlen, int d,
                                  bool causal, float scale, hipStream_t stream);
// fp8 (float8_e4m3fn) q, k [B*H, N, d] and v^T [B*H, d, N] with per-tensor scales; bf16 o. N % 16 == 0.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, int BH, int N, int d,
                          bool causal, float scale, float q_scale, float k_scale, float v_scale, hipStream_t stream);
// Name of the bf16 forward kernel instance launch_fwd_bf16 (packed false) or launch_fwd_varlen_bf16 (packed true,
// N = max_seqlen) enqueues for B*H = BH heads of N rows and head dim d (64 or 128).
const char* fwd_instance_bf16(int BH, int N, int d, bool causal, bool packed);
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N, int d,
                          bool causal, float scale, hipStream_t stream);
// Enqueue the two gradient kernels (dq and the workspace values, then dk and dv). Arguments must already be valid
// (d is 64 or 128, B, H, N >= 1, Hkv >= 1 dividing H, pointers device-resident and aligned, ws of
// bwd_workspace_bytes(B, H, Hkv, N, d) bytes); kv_len as launch_fwd_bf16 (the forward's lengths); returns the launch
// status.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* ws, int B, int H, int Hkv, int N,
                           int d, bool causal, float scale, const int* kv_len, hipStream_t stream);
// The gradient kernels on packed variable-length batches (layout of launch_fwd_varlen_bf16; dq as q, dk and dv
// as k); ws of bwd_workspace_bytes(B, H, Hkv, max_seqlen, d) bytes.
hipError_t launch_bwd_varlen_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv, float* ws, const int* cu_seqlens,
                                  int B, int H, int Hkv, int T_total, int max_seqlen, int d, bool causal, float scale,
                                  hipStream_t stream);
// The dk/dv kernel runs one workgroup per (128-key block, key/value head) and visits every (query head of the
// head's group, 128-row query tile) in turn. When that grid would give fewer than two workgroups per CU (256 CUs),
// each block's visits are divided over `split` workgroups: the fewest that reach 512 workgroups, at most one per
// visit of the longest block and at most 64. Each writes fp32 partial dk and dv, and a reduction kernel sums
// them in split order.
inline int bwd_head_split(int B, int H, int Hkv, int N) {
  const long long tiles = (N + 127) / 128, wgs = tiles * B * Hkv;
  if (wgs >= 512) return 1;
  long long s = (512 + wgs - 1) / wgs;
  if (s > (long long)(H / Hkv) * tiles) s = (long long)(H / Hkv) * tiles;
  return (int)(s < 64 ? s : 64);
}
// Workspace of the gradient kernels: -D_i and lse_i*log2e planes, [B*H][2][N rounded up to 128] float; then,
// with a head split s > 1, the partial dk and dv, [2][s][B*Hkv][N][d] float.
inline size_t bwd_planes_bytes(int B, int H, int N) {
  return (size_t)B * (size_t)H * (size_t)((N + 127) / 128 * 128) * 2 * sizeof(float);
}
// The library's own device scratch buffer (fa_scratch.hip): the gradient workspace of fa_bwd_noalloc, for callers
// that cannot allocate. One copy per device, kept until the process ends.
constexpr size_t kScratchBytes = size_t(64) << 20;
// Device address of the scratch buffer on the device `stream` belongs to (the current device for the null stream),
// looked up once per device with that device current.
hipError_t scratch_address(hipStream_t stream, void** out);
inline size_t bwd_workspace_bytes(int B, int H, int Hkv, int N, int d) {
  const int s = bwd_head_split(B, H, Hkv, N);
  const size_t parts = s > 1 ? 2 * (size_t)s * B * Hkv * (size_t)N * d * sizeof(float) : 0;
  return bwd_planes_bytes(B, H, N) + parts;
}
}  // namespace fa
#endif
