// Host-only stand-ins for the kernel launchers behind the C ABI, so that the
// entry points' validation code (fa_api.cpp, fa_unfused_api.cpp) can be built
// with g++ and the address / undefined-behaviour sanitizers and run on a
// machine without a GPU. Each launcher records its arguments instead of
// launching anything; no memory behind a pointer is ever touched.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stubs.h"

LastCall g_last;

static void record(const char* which, int BH, int N, int d, float scale, bool causal,
                   const void* ws, hipStream_t stream) {
  g_last.which = which;
  g_last.BH = BH;
  g_last.N = N;
  g_last.d = d;
  g_last.scale = scale;
  g_last.causal = causal;
  g_last.ws = ws;
  g_last.stream = stream;
  g_last.calls += 1;
}

namespace fa {

hipError_t fwd_dispatch(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*,
                        int BH, int N, int d, float scale, bool causal, hipStream_t stream) {
  record("fwd", BH, N, d, scale, causal, nullptr, stream);
  return hipSuccess;
}
hipError_t fwd_persistent_dispatch(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*,
                                   float*, int BH, int N, int d, float scale, bool causal,
                                   hipStream_t stream) {
  record("fwd_persistent", BH, N, d, scale, causal, nullptr, stream);
  return hipSuccess;
}
bool fwd_uses_two_group_kernel(int, int N, int d, bool) { return d == 128 && N >= 8192; }
bool fwd_uses_split_kernel(int, int, int) { return false; }
bool fwd_uses_split_groups(int, int, int) { return false; }
bool fwd_uses_paired_split(int, int, int, bool) { return false; }
bool bwd_dq_uses_split(int BH, int N, bool) { return (int64_t)BH * ((N + 127) / 128) <= 256; }

hipError_t bwd_dispatch(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                        const uint16_t*, const float*, uint16_t*, uint16_t*, uint16_t*,
                        float* dvec, int BH, int N, int d, float scale, bool causal,
                        hipStream_t stream) {
  record("bwd", BH, N, d, scale, causal, dvec, stream);
  return hipSuccess;
}

size_t bwd_noalloc_max_rows() { return size_t(1) << 22; }
hipError_t bwd_noalloc_scratch(float** out) {
  *out = reinterpret_cast<float*>(kScratchAddr);
  return hipSuccess;
}

size_t fa1_workspace_floats(int BH, int N, int d) { return (size_t)BH * N * (d + 2); }
hipError_t fa1_fwd_dispatch(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*,
                            float* ws, int BH, int N, int d, float scale, bool causal,
                            hipStream_t stream) {
  record("fa1", BH, N, d, scale, causal, ws, stream);
  return hipSuccess;
}

int decode_splits(int, int Nk, int* chunk) {
  *chunk = 256;
  return (Nk + 255) / 256;
}
hipError_t decode_dispatch(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*,
                           float* ws, int BH, int Nq, int Nk, int d, float scale, bool causal,
                           hipStream_t stream) {
  record("decode", BH, Nk, d, scale, causal, ws, stream);
  g_last.Nq = Nq;
  return hipSuccess;
}

hipError_t unfused_fwd_dispatch(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*,
                                float*, float* ws, int BH, int N, int d, float scale, bool causal,
                                hipStream_t stream, bool* blas_failed) {
  record("unfused", BH, N, d, scale, causal, ws, stream);
  *blas_failed = false;
  return hipSuccess;
}

}  // namespace fa
