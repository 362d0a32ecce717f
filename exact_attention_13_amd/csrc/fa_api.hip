// fa_api.hip -- the C ABI declared in include/fa.h: host-side validation, then one kernel launch.
//
// Every check except the launch status runs before any HIP call, so argument errors are reported the same
// way with or without a GPU present.
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr int kVersion = 10100;  // 1.1.0
constexpr long long kMaxHeads = 65535;   // B*H is the grid's y extent
constexpr long long kMaxN = 1LL << 30;

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

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, hipStream_t stream) {
  bool empty = false;
  const int rc = validate(q, k, v, o, lse, nullptr, false, B, H, H, N, d, causal, scale, 4, &empty);
  if (rc != FA_OK || empty) return rc;
  const hipError_t e = fa::launch_fwd_f32(q, k, v, o, lse, B * H, N, d, causal != 0, scale, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a q/k/v/o/lse/kv_len pointer is NULL";
    case FA_ERR_SHAPE: return "bad shape: B, H, N must be >= 0, B*H <= 65535, N <= 2^30, H_kv >= 1 dividing H";
    case FA_ERR_HEADDIM: return "unsupported head dimension: d must be 64 or 128";
    case FA_ERR_ALIGN: return "misaligned pointer: q, k, v, o need 16-byte alignment, lse and kv_len 4-byte";
    case FA_ERR_ARG: return "bad argument: scale must be finite and > 0, causal must be 0 or 1";
    case FA_ERR_ALIAS: return "o or lse overlaps an input (q, k, v, kv_len), or o overlaps lse";
    case FA_ERR_HIP: return "the HIP runtime reported an error when launching the kernel";
    default: return "unknown error code";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
