// C ABI of libfa355_unfused.so, the unfused attention comparator: argument
// validation and dispatch to its kernels. A library of its own so that the
// fused library (libfa355.so) does not depend on rocBLAS.
//
// Every check runs before the first HIP or rocBLAS call, so an invalid call
// returns an error code without launching anything.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fa355_unfused.h"
#include "fa_validate.h"

namespace fa {
hipError_t unfused_fwd_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                uint16_t* o, float* lse, float* ws, int BH, int N, int d,
                                float scale, bool causal, hipStream_t stream, bool* blas_failed);
}  // namespace fa

using fa::aligned16;
using fa::check_shape;
using fa::round256;

extern "C" {

size_t fa_unfused_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  return round256((size_t)B * H * N * (size_t)N * sizeof(float));
}

int fa_unfused_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                   float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != FA_OK) return rc;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const size_t need = fa_unfused_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, lse, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  bool blas_failed = false;
  hipError_t e = fa::unfused_fwd_dispatch(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
      static_cast<float*>(workspace), B * H, N, d, scale, causal != 0,
      static_cast<hipStream_t>(stream), &blas_failed);
  if (blas_failed) return FA_ERR_BLAS;
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}


}  // extern "C"
