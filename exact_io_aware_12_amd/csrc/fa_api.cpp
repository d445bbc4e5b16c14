// C ABI of libfa355.so: argument validation and dispatch to the HIP kernels.
//
// Every check runs before the first HIP call, so an invalid call returns an
// error code without launching anything (and works on a machine with no GPU).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fa355.h"
#include "fa_validate.h"

namespace fa {
hipError_t fwd_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* o, float* lse, int BH, int N, int d, float scale,
                        bool causal, hipStream_t stream);
hipError_t fwd_persistent_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* o, float* lse, int BH, int N, int d, float scale,
                                   bool causal, hipStream_t stream);
bool fwd_uses_two_group_kernel(int BH, int N, int d, bool causal);
bool fwd_uses_split_kernel(int BH, int N, int d);
bool fwd_uses_split_groups(int BH, int N, int d);
bool fwd_uses_paired_split(int BH, int N, int d, bool causal);
bool bwd_dq_uses_split(int BH, int N, bool causal);
hipError_t bwd_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* o, const uint16_t* dout, const float* lse,
                        uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dvec, int BH, int N,
                        int d, float scale, bool causal, hipStream_t stream);
size_t bwd_noalloc_max_rows();
hipError_t bwd_noalloc_scratch(float** out);
size_t fa1_workspace_floats(int BH, int N, int d);
hipError_t fa1_fwd_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* o, float* lse, float* ws, int BH, int N, int d,
                            float scale, bool causal, hipStream_t stream);
int decode_splits(int BH, int Nk, int* chunk);
hipError_t decode_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, float* ws, int BH, int Nq, int Nk, int d, float scale,
                           bool causal, hipStream_t stream);
}  // namespace fa

using fa::aligned16;
using fa::check_shape;
using fa::kMaxElems;
using fa::round256;

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int N, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != FA_OK) return rc;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  hipError_t e = fa::fwd_dispatch(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, B * H, N, d, scale,
      causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int N, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != FA_OK) return rc;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  hipError_t e = fa::fwd_persistent_dispatch(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, B * H, N, d, scale,
      causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_fwd_kernel_name(int B, int H, int N, int d, int causal) {
  if (check_shape(B, H, N, d) != FA_OK) return nullptr;
  if (fa::fwd_uses_paired_split(B * H, N, d, causal != 0))
    return "fa_fwd_pp_kernel (keys split between the groups, two query tiles per workgroup)";
  if (fa::fwd_uses_split_kernel(B * H, N, d)) return "fa_fwd_pp_kernel (keys split between the groups)";
  if (fa::fwd_uses_split_groups(B * H, N, d)) return "fa_fwd_kernel (keys split between two groups)";
  return fa::fwd_uses_two_group_kernel(B * H, N, d, causal != 0) ? "fa_fwd_pp_kernel"
                                                                 : "fa_fwd_kernel";
}

const char* fa_bwd_kernel_name(int B, int H, int N, int d, int causal) {
  if (check_shape(B, H, N, d) != FA_OK) return nullptr;
  return fa::bwd_dq_uses_split(B * H, N, causal != 0)
             ? "fa_bwd_dq_kernel (keys split between two groups) + fa_bwd_dkdv_kernel"
             : "fa_bwd_dq_kernel + fa_bwd_dkdv_kernel";
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  const size_t rows = (size_t)B * H * N;
  return round256(rows * sizeof(float));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
           void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != FA_OK) return rc;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const size_t need = fa_bwd_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  float* dvec = static_cast<float*>(workspace);
  hipError_t e = fa::bwd_dispatch(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o),
      static_cast<const uint16_t*>(dout), lse, static_cast<uint16_t*>(dq),
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), dvec, B * H, N, d, scale,
      causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                   int H, int N, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != FA_OK) return rc;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if ((size_t)B * H * N > fa::bwd_noalloc_max_rows()) return FA_ERR_TOO_LARGE;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  float* dvec = nullptr;
  if (fa::bwd_noalloc_scratch(&dvec) != hipSuccess) return FA_ERR_HIP;
  hipError_t e = fa::bwd_dispatch(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o),
      static_cast<const uint16_t*>(dout), lse, static_cast<uint16_t*>(dq),
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), dvec, B * H, N, d, scale,
      causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fa1_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  return round256(fa::fa1_workspace_floats(B * H, N, d) * sizeof(float));
}

int fa_fa1_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
               void* workspace, size_t workspace_bytes, int B, int H, int N, int d, float scale,
               int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int rc = check_shape(B, H, N, d);
  if (rc != FA_OK) return rc;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const size_t need = fa_fa1_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, lse, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  hipError_t e = fa::fa1_fwd_dispatch(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
      static_cast<float*>(workspace), B * H, N, d, scale, causal != 0,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

static int check_decode(int B, int H, int Nq, int Nk, int d, int causal) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (Nq > 32 || (causal && Nq > Nk)) return FA_ERR_SHAPE;
  if ((int64_t)B * H * Nk * d > kMaxElems) return FA_ERR_SHAPE;
  return FA_OK;
}

size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (check_decode(B, H, Nq, Nk, d, 0) != FA_OK) return 0;
  int chunk = 0;
  const size_t ns = (size_t)fa::decode_splits(B * H, Nk, &chunk);
  const size_t rows = (size_t)B * H * ns * Nq;
  return round256(rows * d * sizeof(float)) + round256(rows * sizeof(float));
}

int fa_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d,
                  float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int rc = check_decode(B, H, Nq, Nk, d, causal);
  if (rc != FA_OK) return rc;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const size_t need = fa_decode_workspace_bytes(B, H, Nq, Nk, d);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, lse, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  hipError_t e = fa::decode_dispatch(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
      static_cast<float*>(workspace), B * H, Nq, Nk, d, scale, causal != 0,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape: B, H and N must be >= 1 and B*H*N*d < 2^31";
    case FA_ERR_HEADDIM: return "unsupported head dimension: d must be 64 or 128";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_ALIGN: return "every pointer must be 16-byte aligned";
    case FA_ERR_WORKSPACE: return "workspace is NULL or too small";
    case FA_ERR_HIP: return "the HIP runtime reported a launch error";
    case FA_ERR_BLAS: return "rocBLAS reported an error (unfused comparator only)";
    case FA_ERR_TOO_LARGE:
      return "B*H*N exceeds the 4194304 rows of fa_bwd_noalloc's static scratch";
    default: return "unknown fa355 error code";
  }
}

}  // extern "C"
