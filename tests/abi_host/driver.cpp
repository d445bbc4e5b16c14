// Drives every C entry point of fa355.h and fa355_unfused.h through valid and
// invalid arguments against the stand-in launchers of stubs.cpp. Built with
// -fsanitize=address,undefined by tests/test_abi.py; prints "ABI OK" and
// exits 0 when every check holds, else names the first failed check.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/fa355.h"
#include "../../include/fa355_unfused.h"
#include "stubs.h"

static int g_fail = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      g_fail = 1;                                                \
    }                                                            \
  } while (0)

// Aligned dummy addresses: never dereferenced (the launchers are stubs).
static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static const uintptr_t A = 0x100000, W = 0x200000;

static bool saw(const char* which, int BH, int N, int d, float scale, bool causal) {
  return g_last.which && strcmp(g_last.which, which) == 0 && g_last.BH == BH && g_last.N == N &&
         g_last.d == d && g_last.scale == scale && g_last.causal == causal;
}

int main() {
  void* s = P(0x1230);   // a stream handle, passed through untouched
  float* lse = static_cast<float*>(P(A));

  // ---- fa_fwd
  CHECK(fa_fwd(P(A), P(A), P(A), P(A), lse, 2, 3, 100, 128, 0.5f, 1, s) == FA_OK);
  CHECK(saw("fwd", 6, 100, 128, 0.5f, true) && g_last.stream == s);
  CHECK(fa_fwd(nullptr, P(A), P(A), P(A), lse, 1, 1, 16, 64, 1.f, 0, s) == FA_ERR_NULL);
  CHECK(fa_fwd(P(A), P(A), P(A), P(A), lse, 1, 1, 0, 64, 1.f, 0, s) == FA_ERR_SHAPE);
  CHECK(fa_fwd(P(A), P(A), P(A), P(A), lse, 1024, 1024, 1024, 64, 1.f, 0, s) == FA_ERR_SHAPE);
  CHECK(fa_fwd(P(A), P(A), P(A), P(A), lse, 1, 1, 16, 96, 1.f, 0, s) == FA_ERR_HEADDIM);
  CHECK(fa_fwd(P(A), P(A), P(A), P(A), lse, 1, 1, 16, 64, NAN, 0, s) == FA_ERR_SCALE);
  CHECK(fa_fwd(P(A), P(A + 8), P(A), P(A), lse, 1, 1, 16, 64, 1.f, 0, s) == FA_ERR_ALIGN);
  CHECK(fa_fwd_persistent(P(A), P(A), P(A), P(A), lse, 4, 8, 300, 64, -0.5f, 0, s) == FA_OK);
  CHECK(saw("fwd_persistent", 32, 300, 64, -0.5f, false));
  CHECK(fa_fwd_persistent(P(A), P(A), P(A), nullptr, lse, 1, 1, 16, 64, 1.f, 0, s) == FA_ERR_NULL);
  CHECK(fa_fwd_persistent(P(A), P(A), P(A), P(A), lse, 1, 1, 16, 80, 1.f, 0, s) == FA_ERR_HEADDIM);
  CHECK(fa_fwd_persistent(P(A), P(A), P(A), P(A), lse, 1, 1, 16, 64, INFINITY, 0, s) ==
        FA_ERR_SCALE);
  CHECK(fa_fwd_persistent(P(A), P(A), P(A + 4), P(A), lse, 1, 1, 16, 64, 1.f, 0, s) ==
        FA_ERR_ALIGN);
  CHECK(fa_fwd_kernel_name(1, 1, 16, 64, 0) != nullptr);
  CHECK(fa_fwd_kernel_name(1, 1, 16, 65, 0) == nullptr);
  const int calls_after_fwd = g_last.calls;   // fa_fwd and fa_fwd_persistent

  // ---- fa_bwd (+ workspace), fa_bwd_noalloc, fa_bwd_kernel_name
  const size_t ws = fa_bwd_workspace_bytes(2, 16, 2048, 128);
  CHECK(ws == (size_t)2 * 16 * 2048 * 4);
  CHECK(fa_bwd_workspace_bytes(1, 1, 1, 64) == 256);
  CHECK(fa_bwd_workspace_bytes(0, 1, 1, 64) == 0);
  CHECK(fa_bwd(P(A), P(A), P(A), P(A), P(A), lse, P(A), P(A), P(A), P(W), ws, 2, 16, 2048, 128,
               0.25f, 1, s) == FA_OK);
  CHECK(saw("bwd", 32, 2048, 128, 0.25f, true) && g_last.ws == P(W));
  CHECK(fa_bwd(P(A), P(A), P(A), P(A), P(A), lse, P(A), P(A), P(A), P(W), ws - 1, 2, 16, 2048,
               128, 0.25f, 1, s) == FA_ERR_WORKSPACE);
  CHECK(fa_bwd(P(A), P(A), P(A), P(A), P(A), lse, P(A), P(A), P(A), nullptr, ws, 2, 16, 2048,
               128, 0.25f, 1, s) == FA_ERR_WORKSPACE);
  CHECK(fa_bwd(P(A), P(A), P(A), P(A), nullptr, lse, P(A), P(A), P(A), P(W), ws, 2, 16, 2048,
               128, 0.25f, 1, s) == FA_ERR_NULL);
  CHECK(fa_bwd(P(A), P(A), P(A), P(A), P(A), lse, P(A), P(A), P(A), P(W + 4), ws, 2, 16, 2048,
               128, 0.25f, 1, s) == FA_ERR_ALIGN);
  CHECK(fa_bwd_noalloc(P(A), P(A), P(A), P(A), P(A), lse, P(A), P(A), P(A), 1, 1024, 4096, 64,
                       0.125f, 0, s) == FA_OK);
  CHECK(saw("bwd", 1024, 4096, 64, 0.125f, false) && g_last.ws == P(kScratchAddr));
  CHECK(fa_bwd_noalloc(P(A), P(A), P(A), P(A), P(A), lse, P(A), P(A), P(A), 1, 1024, 4097, 64,
                       0.125f, 0, s) == FA_ERR_TOO_LARGE);
  CHECK(fa_bwd_noalloc(P(A), P(A), P(A), P(A), P(A), lse, P(A), P(A), nullptr, 1, 1, 16, 64,
                       0.125f, 0, s) == FA_ERR_NULL);
  CHECK(fa_bwd_kernel_name(1, 1, 16, 64, 1) != nullptr);
  CHECK(fa_bwd_kernel_name(1, 1, 16, 48, 1) == nullptr);

  // ---- fa_fa1_fwd, fa_decode_fwd, fa_unfused_fwd
  const size_t w1 = fa_fa1_workspace_bytes(1, 2, 300, 64);
  CHECK(w1 >= (size_t)2 * 300 * 66 * 4);
  CHECK(fa_fa1_fwd(P(A), P(A), P(A), P(A), lse, P(W), w1, 1, 2, 300, 64, 0.1f, 1, s) == FA_OK);
  CHECK(saw("fa1", 2, 300, 64, 0.1f, true) && g_last.ws == P(W));
  CHECK(fa_fa1_fwd(P(A), P(A), P(A), P(A), lse, P(W), w1 - 1, 1, 2, 300, 64, 0.1f, 1, s) ==
        FA_ERR_WORKSPACE);
  const size_t wd = fa_decode_workspace_bytes(2, 4, 8, 1000, 128);
  CHECK(wd > 0);
  CHECK(fa_decode_fwd(P(A), P(A), P(A), P(A), lse, P(W), wd, 2, 4, 8, 1000, 128, 0.2f, 1, s) ==
        FA_OK);
  CHECK(saw("decode", 8, 1000, 128, 0.2f, true) && g_last.Nq == 8);
  CHECK(fa_decode_fwd(P(A), P(A), P(A), P(A), lse, P(W), wd, 2, 4, 33, 1000, 128, 0.2f, 0, s) ==
        FA_ERR_SHAPE);
  CHECK(fa_decode_fwd(P(A), P(A), P(A), P(A), lse, P(W), wd, 2, 4, 8, 4, 128, 0.2f, 1, s) ==
        FA_ERR_SHAPE);
  const size_t wu = fa_unfused_workspace_bytes(1, 2, 300, 128);
  CHECK(wu == (size_t)2 * 300 * 300 * 4 + 128);   // rounded up to 256 bytes
  CHECK(fa_unfused_fwd(P(A), P(A), P(A), P(A), lse, P(W), wu, 1, 2, 300, 128, 0.3f, 0, s) ==
        FA_OK);
  CHECK(saw("unfused", 2, 300, 128, 0.3f, false));
  CHECK(fa_unfused_fwd(P(A), P(A), P(A), P(A), lse, P(W), wu - 1, 1, 2, 300, 128, 0.3f, 0, s) ==
        FA_ERR_WORKSPACE);
  CHECK(fa_unfused_fwd(P(A), P(A), P(A), P(A), lse, P(W), wu, 1, 2, 300, 128, INFINITY, 0, s) ==
        FA_ERR_SCALE);

  // ---- every invalid call above launched nothing
  CHECK(calls_after_fwd == 2);
  CHECK(g_last.calls == 7);

  // ---- fa_strerror covers every code
  for (int c = 0; c <= 9; ++c) CHECK(strcmp(fa_strerror(c), "unknown fa355 error code") != 0);
  CHECK(strcmp(fa_strerror(10), "unknown fa355 error code") == 0);
  CHECK(strcmp(fa_strerror(-1), "unknown fa355 error code") == 0);

  if (g_fail) return 1;
  printf("ABI OK\n");
  return 0;
}
