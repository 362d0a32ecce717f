// fa_api.hip -- the C ABI declared in include/fa.h: host-side validation, then one kernel launch.
//
// Every check except the launch status runs before any HIP call, so argument errors are reported the same
// way with or without a GPU present.
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr int kVersion = 10700;  // 1.7.0
constexpr long long kMaxHeads = 65535;   // B*H is the grid's y extent
constexpr long long kMaxN = 1LL << 30;
// The gradient kernels read the workspace's two planes of one head through a 32-bit byte range and offset
// (2 x 4 bytes per row), so their sequence length stays well below 2^29.
constexpr long long kMaxNBwd = 1LL << 28;

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

// Shared argument checks. elt = bytes per q/k/v/o element; k and v have Hkv heads; kv_len (B ints) is checked
// only when `with_len` is set.
int validate(const void* q, const void* k, const void* v, const void* o, const float* lse, const int* kv_len,
             bool with_len, int B, int H, int Hkv, int N, int d, int causal, float scale, size_t elt, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0 || Hkv < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  if (Hkv == 0 || H % Hkv != 0) return FA_ERR_SHAPE;
  if ((long long)B * H > kMaxHeads || N > kMaxN) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse || (with_len && !kv_len)) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;
  if (with_len && ((uintptr_t)kv_len & 3)) return FA_ERR_ALIGN;
  const size_t rows = (size_t)B * (size_t)H * (size_t)N;
  const size_t tb = rows * (size_t)d * elt;                                  // bytes of q or o
  const size_t kb = (size_t)B * (size_t)Hkv * (size_t)N * (size_t)d * elt;  // bytes of k or v
  const size_t lb = rows * sizeof(float);
  if (overlaps(o, tb, q, tb) || overlaps(o, tb, k, kb) || overlaps(o, tb, v, kb)) return FA_ERR_ALIAS;
  if (overlaps(lse, lb, q, tb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) || overlaps(lse, lb, o, tb))
    return FA_ERR_ALIAS;
  if (with_len) {
    const size_t nb = (size_t)B * sizeof(int);
    if (overlaps(o, tb, kv_len, nb) || overlaps(lse, lb, kv_len, nb)) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

int run_bf16(const void* q, const void* k, const void* v, void* o, float* lse, const int* kv_len, bool with_len,
             int B, int H, int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  bool empty = false;
  const int rc = validate(q, k, v, o, lse, kv_len, with_len, B, H, Hkv, N, d, causal, scale, 2, &empty);
  if (rc != FA_OK || empty) return rc;
  const hipError_t e = fa::launch_fwd_bf16(q, k, v, o, lse, B, H, Hkv, N, d, causal != 0, scale,
                                           with_len ? kv_len : nullptr, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Checks of the gradient call: the forward's shape rules, then the nine tensors and the workspace.
int validate_bwd(const void* const* in, int n_in, void* const* out, int n_out, const float* lse, const float* ws,
                 bool with_ws, int B, int H, int Hkv, int N, int d, int causal, float scale, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0 || Hkv < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  if (Hkv == 0 || H % Hkv != 0) return FA_ERR_SHAPE;
  if ((long long)B * H > kMaxHeads || N > kMaxNBwd) return FA_ERR_SHAPE;
  for (int i = 0; i < n_in; ++i)
    if (!in[i]) return FA_ERR_NULL;
  for (int i = 0; i < n_out; ++i)
    if (!out[i]) return FA_ERR_NULL;
  if (!lse || (with_ws && !ws)) return FA_ERR_NULL;
  for (int i = 0; i < n_in; ++i)
    if ((uintptr_t)in[i] & 15) return FA_ERR_ALIGN;
  for (int i = 0; i < n_out; ++i)
    if ((uintptr_t)out[i] & 15) return FA_ERR_ALIGN;
  if (((uintptr_t)lse & 3) || (with_ws && ((uintptr_t)ws & 15))) return FA_ERR_ALIGN;
  return FA_OK;
}

// with_ws false: the workspace is the library's scratch buffer (fa_bwd_noalloc), looked up after every check.
int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
            void* dk, void* dv, float* workspace, bool with_ws, const int* kv_len, bool with_len, int B, int H,
            int H_kv, int N, int d, int causal, float scale, hipStream_t stream) {
  const void* in[] = {q, k, v, o, dout};
  void* out[] = {dq, dk, dv};
  bool empty = false;
  int rc = validate_bwd(in, 5, out, 3, lse, workspace, with_ws, B, H, H_kv, N, d, causal, scale, &empty);
  if (rc != FA_OK || empty) return rc;
  if (with_len && !kv_len) return FA_ERR_NULL;
  if (with_len && ((uintptr_t)kv_len & 3)) return FA_ERR_ALIGN;
  // byte ranges: q, o, dout, dq are [B,H,N,d]; k, v, dk, dv are [B,H_kv,N,d]; lse [B,H,N]; kv_len [B]; the
  // workspace
  const size_t tq = (size_t)B * H * N * d * 2, tk = (size_t)B * H_kv * N * d * 2, tl = (size_t)B * H * N * 4;
  const size_t tw = fa::bwd_workspace_bytes(B, H, H_kv, N, d);
  if (!with_ws && tw > fa::kScratchBytes) return FA_ERR_SCRATCH;
  const void* rin[] = {q, k, v, o, dout, lse, kv_len};
  const size_t nin[] = {tq, tk, tk, tq, tq, tl, with_len ? (size_t)B * sizeof(int) : 0};
  void* rout[] = {dq, dk, dv, workspace};
  const size_t nout[] = {tq, tk, tk, with_ws ? tw : 0};  // the scratch buffer is the library's own memory
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(rout[i], nout[i], rin[j], nin[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(rout[i], nout[i], rout[j], nout[j])) return FA_ERR_ALIAS;
  }
  if (!with_ws) {
    void* p = nullptr;
    if (fa::scratch_address(stream, &p) != hipSuccess) return FA_ERR_HIP;
    workspace = (float*)p;
  }
  const hipError_t e = fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, H_kv, N, d,
                                           causal != 0, scale, with_len ? kv_len : nullptr, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int run_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens, int B,
               int H, int Hkv, int total, int max_seqlen, int d, int causal, float scale, hipStream_t stream) {
  if (B < 0 || H < 0 || Hkv < 0 || total < 0 || max_seqlen < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || total == 0) return FA_OK;  // no token: nothing to compute
  if (max_seqlen == 0 || max_seqlen > total) return FA_ERR_SHAPE;
  if (Hkv == 0 || H % Hkv != 0) return FA_ERR_SHAPE;
  if ((long long)B * H > kMaxHeads || total > kMaxN) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3) return FA_ERR_ALIGN;
  const size_t tq = (size_t)total * H * d * 2, tk = (size_t)total * Hkv * d * 2, tl = (size_t)total * H * 4;
  const size_t tc = (size_t)(B + 1) * sizeof(int);
  const void* in[] = {q, k, v, cu_seqlens};
  const size_t nin[] = {tq, tk, tk, tc};
  for (int j = 0; j < 4; ++j)
    if (overlaps(o, tq, in[j], nin[j]) || overlaps(lse, tl, in[j], nin[j])) return FA_ERR_ALIAS;
  if (overlaps(o, tq, lse, tl)) return FA_ERR_ALIAS;
  const hipError_t e = fa::launch_fwd_varlen_bf16(q, k, v, o, lse, cu_seqlens, B, H, Hkv, total, max_seqlen, d,
                                                  causal != 0, scale, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int run_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, float* workspace, const int* cu_seqlens, int B, int H, int Hkv,
                   int total, int max_seqlen, int d, int causal, float scale, hipStream_t stream) {
  if (B < 0 || H < 0 || Hkv < 0 || total < 0 || max_seqlen < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || total == 0) return FA_OK;
  if (max_seqlen == 0 || max_seqlen > total) return FA_ERR_SHAPE;
  if (Hkv == 0 || H % Hkv != 0) return FA_ERR_SHAPE;
  if ((long long)B * H > kMaxHeads || total > kMaxN || max_seqlen > kMaxNBwd) return FA_ERR_SHAPE;
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv, workspace};
  for (const void* x : ptrs) {
    if (!x) return FA_ERR_NULL;
    if ((uintptr_t)x & 15) return FA_ERR_ALIGN;
  }
  if (!lse || !cu_seqlens) return FA_ERR_NULL;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3) return FA_ERR_ALIGN;
  const size_t tq = (size_t)total * H * d * 2, tk = (size_t)total * Hkv * d * 2, tl = (size_t)total * H * 4;
  const size_t tw = fa::bwd_workspace_bytes(B, H, Hkv, max_seqlen, d), tc = (size_t)(B + 1) * sizeof(int);
  const void* rin[] = {q, k, v, o, dout, lse, cu_seqlens};
  const size_t nin[] = {tq, tk, tk, tq, tq, tl, tc};
  void* rout[] = {dq, dk, dv, workspace};
  const size_t nout[] = {tq, tk, tk, tw};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(rout[i], nout[i], rin[j], nin[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(rout[i], nout[i], rout[j], nout[j])) return FA_ERR_ALIAS;
  }
  const hipError_t e = fa::launch_bwd_varlen_bf16(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens, B, H,
                                                  Hkv, total, max_seqlen, d, causal != 0, scale, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, int causal,
           float scale, hipStream_t stream) {
  return run_bf16(q, k, v, o, lse, nullptr, false, B, H, H, N, d, causal, scale, stream);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N, int d,
               int causal, float scale, hipStream_t stream) {
  return run_bf16(q, k, v, o, lse, nullptr, false, B, H, H_kv, N, d, causal, scale, stream);
}

int fa_fwd_kpad(const void* q, const void* k, const void* v, void* o, float* lse, const int* kv_len, int B, int H,
                int H_kv, int N, int d, int causal, float scale, hipStream_t stream) {
  return run_bf16(q, k, v, o, lse, kv_len, true, B, H, H_kv, N, d, causal, scale, stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens, int B,
                  int H, int H_kv, int total, int max_seqlen, int d, int causal, float scale, hipStream_t stream) {
  return run_varlen(q, k, v, o, lse, cu_seqlens, B, H, H_kv, total, max_seqlen, d, causal, scale, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, float* workspace, int B, int H, int H_kv, int N, int d, int causal, float scale,
           hipStream_t stream) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, true, nullptr, false, B, H, H_kv, N, d, causal, scale,
                 stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, int causal, float scale,
                   hipStream_t stream) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, false, nullptr, false, B, H, H_kv, N, d, causal, scale,
                 stream);
}

int fa_bwd_kpad(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, float* workspace, const int* kv_len, int B, int H, int H_kv, int N, int d,
                int causal, float scale, hipStream_t stream) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, true, kv_len, true, B, H, H_kv, N, d, causal, scale,
                 stream);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* workspace, const int* cu_seqlens, int B, int H, int H_kv,
                  int total, int max_seqlen, int d, int causal, float scale, hipStream_t stream) {
  return run_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens, B, H, H_kv, total, max_seqlen, d,
                        causal, scale, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || H_kv <= 0 || H % H_kv != 0 || (d != 64 && d != 128)) return 0;
  if ((long long)B * H > kMaxHeads || N > kMaxNBwd) return 0;  // sizes the gradient calls reject
  return fa::bwd_workspace_bytes(B, H, H_kv, N, d);
}

int fa_fwd_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, float q_scale, float k_scale,
               float v_scale, int B, int H, int N, int d, int causal, float scale, hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
  for (float s : {q_scale, k_scale, v_scale})
    if (!(s > 0.f) || !isfinite(s)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  // v^T rows of N bytes start on 16-byte boundaries; byte offsets inside one head's v^T stay below 2^31
  if ((long long)B * H > kMaxHeads || N % 16 != 0 || N > (1 << 24)) return FA_ERR_SHAPE;
  if (!q || !k || !vt || !o || !lse) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)vt | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;
  const size_t elems = (size_t)B * H * N * d;
  const size_t ob = 2 * elems, lb = (size_t)B * H * N * 4;
  if (overlaps(o, ob, q, elems) || overlaps(o, ob, k, elems) || overlaps(o, ob, vt, elems)) return FA_ERR_ALIAS;
  if (overlaps(lse, lb, q, elems) || overlaps(lse, lb, k, elems) || overlaps(lse, lb, vt, elems) ||
      overlaps(lse, lb, o, ob))
    return FA_ERR_ALIAS;
  const hipError_t e = fa::launch_fwd_fp8(q, k, vt, o, lse, B * H, N, d, causal != 0, scale, q_scale, k_scale,
                                          v_scale, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, hipStream_t stream) {
  bool empty = false;
  const int rc = validate(q, k, v, o, lse, nullptr, false, B, H, H, N, d, causal, scale, 4, &empty);
  if (rc != FA_OK || empty) return rc;
  const hipError_t e = fa::launch_fwd_f32(q, k, v, o, lse, B * H, N, d, causal != 0, scale, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_fwd_instance(int B, int H, int N, int d, int causal, int packed) {
  if (B < 1 || H < 1 || N < 1 || (long long)B * H > kMaxHeads || N > kMaxN) return nullptr;
  if ((d != 64 && d != 128) || (causal != 0 && causal != 1) || (packed != 0 && packed != 1)) return nullptr;
  return fa::fwd_instance_bf16(B * H, N, d, causal != 0, packed != 0);
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a tensor, lse, kv_len, cu_seqlens or workspace pointer is NULL";
    case FA_ERR_SHAPE:
      return "bad shape: B, H, N must be >= 0, B*H <= 65535, N <= 2^30, H_kv >= 1 dividing H "
             "(fp8: N a multiple of 16, at most 2^24; packed: 1 <= max_seqlen <= total <= 2^30; gradient calls: "
             "N and max_seqlen at most 2^28)";
    case FA_ERR_HEADDIM: return "unsupported head dimension: d must be 64 or 128";
    case FA_ERR_ALIGN:
      return "misaligned pointer: tensors and the workspace need 16-byte alignment, lse, kv_len and cu_seqlens "
             "4-byte";
    case FA_ERR_ARG: return "bad argument: scales must be finite and > 0, causal must be 0 or 1";
    case FA_ERR_ALIAS: return "an output (o, lse, dq, dk, dv, workspace) overlaps an input or another output";
    case FA_ERR_HIP: return "the HIP runtime reported an error when launching the kernel";
    case FA_ERR_SCRATCH:
      return "fa_bwd_noalloc: the gradient workspace of this problem exceeds the library's 64 MiB scratch buffer "
             "(use fa_bwd with a caller-allocated workspace)";
    default: return "unknown error code";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
