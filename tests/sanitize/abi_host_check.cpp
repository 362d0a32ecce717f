// abi_host_check.cpp -- drives the C ABI's host-side validation (fa_api.hip, built with g++ and
// -fsanitize=address,undefined against launch_stubs.cpp) through every entry point: valid calls that reach a
// launcher, every error code, the largest sizes the ABI accepts and sizes just past them. Fake device addresses
// are never dereferenced. Prints one line per failed check and exits with the number of failures (0: all passed);
// the sanitizers abort the process on the first memory error or undefined behaviour.
#include <stdint.h>
#include <stdio.h>

#include "fa.h"

namespace fa {
extern int g_calls;
extern int g_last[8];
}  // namespace fa

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      ++failures;                                                          \
      printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);             \
    }                                                                      \
  } while (0)

// fake device addresses: 16-byte aligned, 2^56 bytes apart, so that no tensor of any accepted size overlaps another
static void* at(int slot) { return (void*)(uintptr_t)((uint64_t)(slot + 1) << 56); }
static float* atf(int slot) { return (float*)at(slot); }
static int* ati(int slot) { return (int*)at(slot); }

static int fwd(int B, int H, int N, int d, int causal, float scale) {
  return fa_fwd(at(0), at(1), at(2), at(3), atf(4), B, H, N, d, causal, scale, nullptr);
}

int main() {
  const float sc = 0.125f;
  // ---- valid calls reach the launcher with the caller's sizes
  fa::g_calls = 0;
  CHECK(fwd(2, 16, 4096, 128, 0, sc) == FA_OK);
  CHECK(fa::g_calls == 1 && fa::g_last[0] == 32 && fa::g_last[1] == 4096 && fa::g_last[2] == 128);
  CHECK(fa_fwd_gqa(at(0), at(1), at(2), at(3), atf(4), 1, 32, 8, 1000, 64, 1, sc, nullptr) == FA_OK);
  CHECK(fa::g_calls == 2 && fa::g_last[3] == 1 && fa::g_last[4] == 8);
  CHECK(fa_fwd_kpad(at(0), at(1), at(2), at(3), atf(4), ati(5), 3, 4, 2, 77, 128, 0, sc, nullptr) == FA_OK);
  CHECK(fa_fwd_varlen(at(0), at(1), at(2), at(3), atf(4), ati(5), 3, 8, 8, 1000, 600, 64, 1, sc, nullptr) == FA_OK);
  CHECK(fa::g_last[1] == 1000 && fa::g_last[5] == 600);
  CHECK(fa_fwd_f32(atf(0), atf(1), atf(2), atf(3), atf(4), 1, 1, 128, 64, 0, sc, nullptr) == FA_OK);
  CHECK(fa_fwd_fp8(at(0), at(1), at(2), at(3), atf(4), 1.f, 1.f, 1.f, 1, 2, 4096, 128, 1, sc, nullptr) == FA_OK);
  CHECK(fa_bwd(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), atf(9), 2, 8, 2, 1000, 128, 1, sc,
               nullptr) == FA_OK);
  CHECK(fa_bwd_kpad(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), atf(9), ati(10), 2, 8, 8, 100,
                    64, 0, sc, nullptr) == FA_OK);
  CHECK(fa_bwd_varlen(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), atf(9), ati(10), 2, 4, 1, 500,
                      300, 128, 1, sc, nullptr) == FA_OK);
  CHECK(fa_bwd_noalloc(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), 2, 16, 16, 4096, 128, 0, sc,
                       nullptr) == FA_OK);
  CHECK(fa::g_last[0] == 32 && fa::g_last[1] == 4096);
  const int calls = fa::g_calls;
  CHECK(calls == 10);

  // ---- the largest accepted sizes, and one past them
  CHECK(fwd(65535, 1, 1 << 30, 128, 1, sc) == FA_OK);
  CHECK(fwd(65536, 1, 64, 64, 0, sc) == FA_ERR_SHAPE);
  CHECK(fwd(1, 1, (1 << 30) + 1, 64, 0, sc) == FA_ERR_SHAPE);
  CHECK(fwd(0x7fffffff, 0x7fffffff, 64, 64, 0, sc) == FA_ERR_SHAPE);
  CHECK(fa_bwd(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), atf(9), 1, 1, 1, (1 << 28) + 1, 64, 0,
               sc, nullptr) == FA_ERR_SHAPE);
  CHECK(fa_fwd_fp8(at(0), at(1), at(2), at(3), atf(4), 1.f, 1.f, 1.f, 1, 1, 100, 64, 0, sc, nullptr) ==
        FA_ERR_SHAPE);  // N not a multiple of 16
  CHECK(fa_bwd_workspace_bytes(65535, 1, 1, 1 << 28, 128) > 0);
  CHECK(fa_bwd_workspace_bytes(1, 1, 1, 1 << 28, 128) > 0);
  CHECK(fa_bwd_workspace_bytes(65536, 1, 1, 64, 64) == 0);          // sizes the gradient calls reject
  CHECK(fa_bwd_workspace_bytes(1, 1, 1, (1 << 28) + 1, 64) == 0);
  CHECK(fa_bwd_workspace_bytes(0x7fffffff, 0x7fffffff, 1, 0x7fffffff, 128) == 0);
  CHECK(fa_bwd_workspace_bytes(-1, 1, 1, 64, 64) == 0);

  // ---- every error code of the plain forward
  CHECK(fa_fwd(nullptr, at(1), at(2), at(3), atf(4), 1, 1, 64, 64, 0, sc, nullptr) == FA_ERR_NULL);
  CHECK(fa_fwd(at(0), at(1), at(2), at(3), nullptr, 1, 1, 64, 64, 0, sc, nullptr) == FA_ERR_NULL);
  CHECK(fwd(-1, 1, 64, 64, 0, sc) == FA_ERR_SHAPE);
  CHECK(fwd(1, 1, 64, 96, 0, sc) == FA_ERR_HEADDIM);
  CHECK(fa_fwd((char*)at(0) + 8, at(1), at(2), at(3), atf(4), 1, 1, 64, 64, 0, sc, nullptr) == FA_ERR_ALIGN);
  CHECK(fa_fwd(at(0), at(1), at(2), at(3), (float*)((char*)at(4) + 2), 1, 1, 64, 64, 0, sc, nullptr) ==
        FA_ERR_ALIGN);
  CHECK(fwd(1, 1, 64, 64, 2, sc) == FA_ERR_ARG);
  CHECK(fwd(1, 1, 64, 64, 0, 0.f) == FA_ERR_ARG);
  CHECK(fwd(1, 1, 64, 64, 0, -1.f) == FA_ERR_ARG);
  CHECK(fwd(1, 1, 64, 64, 0, 1.f / 0.f) == FA_ERR_ARG);
  CHECK(fwd(1, 1, 64, 64, 0, 0.f / 0.f) == FA_ERR_ARG);
  CHECK(fa_fwd(at(0), at(1), at(2), (char*)at(0) + 4096, atf(4), 1, 1, 64, 64, 0, sc, nullptr) == FA_ERR_ALIAS);
  CHECK(fa_fwd(at(0), at(1), at(2), at(3), (float*)((char*)at(3) + 64), 1, 1, 64, 64, 0, sc, nullptr) ==
        FA_ERR_ALIAS);
  CHECK(fwd(0, 4, 64, 64, 0, sc) == FA_OK && fwd(4, 0, 64, 64, 0, sc) == FA_OK && fwd(4, 4, 0, 64, 0, sc) == FA_OK);
  CHECK(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 64, 64, 0, sc, nullptr) == FA_OK);
  // grouped heads, key padding, packed batches
  CHECK(fa_fwd_gqa(at(0), at(1), at(2), at(3), atf(4), 1, 8, 3, 64, 64, 0, sc, nullptr) == FA_ERR_SHAPE);
  CHECK(fa_fwd_gqa(at(0), at(1), at(2), at(3), atf(4), 1, 8, 0, 64, 64, 0, sc, nullptr) == FA_ERR_SHAPE);
  CHECK(fa_fwd_kpad(at(0), at(1), at(2), at(3), atf(4), nullptr, 1, 8, 8, 64, 64, 0, sc, nullptr) == FA_ERR_NULL);
  CHECK(fa_fwd_kpad(at(0), at(1), at(2), at(3), atf(4), (int*)((char*)at(5) + 2), 1, 8, 8, 64, 64, 0, sc, nullptr) ==
        FA_ERR_ALIGN);
  CHECK(fa_fwd_kpad(at(0), at(1), at(2), at(3), atf(4), (int*)at(3), 1, 8, 8, 64, 64, 0, sc, nullptr) ==
        FA_ERR_ALIAS);
  CHECK(fa_fwd_varlen(at(0), at(1), at(2), at(3), atf(4), ati(5), 3, 8, 8, 1000, 1001, 64, 1, sc, nullptr) ==
        FA_ERR_SHAPE);
  CHECK(fa_fwd_varlen(at(0), at(1), at(2), at(3), atf(4), ati(5), 3, 8, 8, 1000, 0, 64, 1, sc, nullptr) ==
        FA_ERR_SHAPE);
  CHECK(fa_fwd_varlen(at(0), at(1), at(2), at(3), atf(4), nullptr, 3, 8, 8, 1000, 10, 64, 1, sc, nullptr) ==
        FA_ERR_NULL);
  CHECK(fa_fwd_varlen(at(0), at(1), at(2), at(3), atf(4), ati(5), 3, 8, 8, 0, 0, 64, 1, sc, nullptr) == FA_OK);
  // gradients: every output must be apart from every input and from each other
  CHECK(fa_bwd(at(0), at(1), at(2), at(3), atf(4), at(5), at(0), at(7), at(8), atf(9), 1, 4, 4, 64, 64, 0, sc,
               nullptr) == FA_ERR_ALIAS);
  CHECK(fa_bwd(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(6), at(8), atf(9), 1, 4, 4, 64, 64, 0, sc,
               nullptr) == FA_ERR_ALIAS);
  CHECK(fa_bwd(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), nullptr, 1, 4, 4, 64, 64, 0, sc,
               nullptr) == FA_ERR_NULL);
  CHECK(fa_bwd(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), (float*)((char*)at(9) + 4), 1, 4, 4,
               64, 64, 0, sc, nullptr) == FA_ERR_ALIGN);
  CHECK(fa_bwd_kpad(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), atf(9), nullptr, 1, 4, 4, 64, 64,
                    0, sc, nullptr) == FA_ERR_NULL);
  CHECK(fa_bwd_varlen(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), atf(9), ati(10), 2, 4, 1, 500,
                      (1 << 28) + 1, 128, 1, sc, nullptr) == FA_ERR_SHAPE);
  CHECK(fa_fwd_fp8(at(0), at(1), at(2), at(3), atf(4), 0.f, 1.f, 1.f, 1, 2, 64, 128, 1, sc, nullptr) == FA_ERR_ARG);
  // the no-allocation gradient call: the scratch limit, then the checks of fa_bwd
  CHECK(fa_bwd_noalloc(at(0), at(1), at(2), at(3), atf(4), at(5), at(6), at(7), at(8), 1, 32, 1, 16384, 128, 1, sc,
                       nullptr) == FA_ERR_SCRATCH);
  CHECK(fa_bwd_noalloc(at(0), at(1), at(2), at(3), atf(4), at(5), nullptr, at(7), at(8), 1, 4, 4, 64, 64, 0, sc,
                       nullptr) == FA_ERR_NULL);
  CHECK(fa_bwd_noalloc(at(0), at(1), at(2), at(3), atf(4), at(5), at(1), at(7), at(8), 1, 4, 4, 64, 64, 0, sc,
                       nullptr) == FA_ERR_ALIAS);
  CHECK(fa_bwd_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 4, 64,
                       64, 0, sc, nullptr) == FA_OK);
  // no rejected call reached a launcher
  CHECK(fa::g_calls == calls + 1);  // + the largest accepted forward above

  // ---- strings
  for (int c = -1; c <= 8; ++c) CHECK(fa_strerror(c) != nullptr && fa_strerror(c)[0] != '\0');
  CHECK(fa_version() > 0);
  CHECK(fa_fwd_instance(1, 1, 64, 64, 0, 0) != nullptr && fa_fwd_instance(0, 1, 64, 64, 0, 0) == nullptr);

  printf("abi_host_check: %d failed\n", failures);
  return failures;
}
