/*
 * fa355_unfused.h -- C ABI of libfa355_unfused.so: unfused ("standard")
 * attention on AMD Instinct MI355X (gfx950), kept as a measured comparator of
 * the fused library (fa355.h, libfa355.so). It is a library of its own because
 * it calls rocBLAS for its two plain GEMMs; the fused library does not.
 *
 * Conventions (tensor layout, head dimensions, scale, causal mask, alignment,
 * stream, error codes) are those of fa355.h.
 *
 * Ownership: the caller allocates every buffer, including the workspace. On
 * its first call on a device the library creates one rocBLAS handle for that
 * device (rocBLAS allocates its own scratch memory then) and keeps it until
 * the process ends. Calls are serialized inside the library (the handle's
 * stream is set per call).
 */
#ifndef FA355_UNFUSED_H_
#define FA355_UNFUSED_H_

#include "fa355.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Unfused ("standard") attention: the same O and LSE as fa_fwd, computed by
 * the three-step decomposition that the fused pass avoids, kept as a
 * measured comparator. Method: the interview answer's "standard attention"
 * steps and "FlashAttention and Triton" (chapter 19), section 19.2:
 *   1. S = scale * Q K^T is written to memory (fp32, library GEMM);
 *   2. a row-wise softmax pass (section 19.11: one workgroup per row, row
 *      max, exp, row sum) reads S, applies the causal mask and writes P
 *      (bf16) and the LSE;
 *   3. O = P V (library GEMM, fp32 accumulate, bf16 out).
 *   q, k, v, o, lse  : as for fa_fwd
 *   workspace        : device memory of workspace_bytes bytes, at least
 *                      fa_unfused_workspace_bytes(B,H,N,d): holds S as fp32
 *                      [B,H,N,N], then P as bf16 over the first half of each
 *                      S row; contents on return are unspecified.
 * Returns FA_ERR_BLAS when rocBLAS fails.
 */
FA355_API size_t fa_unfused_workspace_bytes(int B, int H, int N, int d);
FA355_API int fa_unfused_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
           float scale, int causal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA355_UNFUSED_H_ */
