/*
 * fa355.h -- C ABI of the fused exact attention library for AMD Instinct
 * MI355X (gfx950): libfa355.so.
 *
 * The operation is exact softmax attention per (batch, head):
 *     S = scale * Q K^T            (N x N, never written to memory)
 *     P = softmax(S) row by row    (N x N, never written to memory)
 *     O = P V
 * as defined in "FlashAttention core principles" (lesson 1), section 1, and
 * "FlashAttention and Triton" (chapter 19), section 19.1. The forward pass
 * streams K/V tiles and keeps a running row max and row sum (lesson 1,
 * sections 3-4; chapter 19, section 19.5); it saves one logsumexp per row.
 * The backward pass recomputes S and P tile by tile from that statistic
 * (lesson 1, section 5; the interview answer's "3. Recomputation" block).
 *
 * Common conventions
 *   - Tensors Q, K, V, O, dO, dQ, dK, dV are bf16 (IEEE-754 binary32 with the
 *     low 16 bits dropped, round-to-nearest-even), laid out [B, H, N, d]
 *     contiguous (d fastest), in device memory of the current HIP device.
 *   - LSE is fp32 [B, H, N]: the natural-log logsumexp of the row's scaled,
 *     masked scores, i.e. m + ln(sum_j exp(s_j - m)).
 *   - d (head dimension) must be 64 or 128. N >= 1 is any length (the last
 *     tile may be partial). B, H >= 1. B*H*N*d must fit in 2^31 - 1 elements.
 *   - scale multiplies Q K^T; any finite value, including 0, is accepted.
 *   - causal != 0: query i attends key j iff j <= i (queries and keys share
 *     the same positions 0..N-1).
 *   - Every pointer must be 16-byte aligned. Outputs must not alias inputs.
 *   - stream is a hipStream_t (NULL = the legacy default stream). Calls only
 *     enqueue work and return; results are visible after the stream is
 *     synchronised. Kernel faults surface at that synchronisation.
 *   - Ownership: the caller allocates and frees every buffer, including the
 *     workspaces. fa_fwd and fa_bwd keep no state between calls, allocate no
 *     memory and are safe to call from several host threads. The unfused
 *     comparator lives in its own library (fa355_unfused.h,
 *     libfa355_unfused.so) so that this one does not depend on rocBLAS.
 *   - Errors: 0 (FA_OK) on success, else one of the FA_ERR_* codes below.
 *     Arguments are validated before any HIP call, so an invalid call launches
 *     nothing and touches no memory. No C++ exception crosses this ABI.
 */
#ifndef FA355_H_
#define FA355_H_

#include <stddef.h>

#if defined(__GNUC__)
#define FA355_API __attribute__((visibility("default")))
#else
#define FA355_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL                        */
  FA_ERR_SHAPE = 2,     /* B, H or N < 1, or B*H*N*d overflows               */
  FA_ERR_HEADDIM = 3,   /* d is not 64 or 128                                */
  FA_ERR_SCALE = 4,     /* scale is NaN or infinite                          */
  FA_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned                  */
  FA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than required           */
  FA_ERR_HIP = 7,       /* the HIP runtime reported a launch error           */
  FA_ERR_BLAS = 8,      /* rocBLAS reported an error (libfa355_unfused only) */
  FA_ERR_TOO_LARGE = 9  /* B*H*N above FA_BWD_NOALLOC_MAX_ROWS               */
};

/* Largest B*H*N that fa_bwd_noalloc accepts (its static scratch: 16 MiB). */
#define FA_BWD_NOALLOC_MAX_ROWS 4194304

/*
 * Forward pass: O = softmax(scale * Q K^T [causal mask]) V and the per-row
 * LSE (lesson 1, section 4 pseudocode and section 5's saved statistics).
 *   q, k, v : in,  bf16 [B,H,N,d]
 *   o       : out, bf16 [B,H,N,d]
 *   lse     : out, fp32 [B,H,N]
 */
FA355_API int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * Name of the kernel fa_fwd launches for this shape:
 *   "fa_fwd_kernel": 128-row query tiles, two independent 4-wave workgroups
 *     per CU;
 *   "fa_fwd_pp_kernel": long d = 128 sequences, 256-row workgroups whose two
 *     4-wave groups alternate MFMA and VALU clusters;
 *   "fa_fwd_pp_kernel (keys split between the groups)": d = 128, N >= 1024
 *     and at most 256 query tiles of 128 rows; both groups own the same 128
 *     rows, take alternate key tiles and merge their partial results;
 *   "fa_fwd_pp_kernel (keys split between the groups, two query tiles per
 *     workgroup)": causal, d = 128, N >= 4096 and 257-512 query tiles of 128
 *     rows; the same split, each workgroup taking a heavy and a light tile;
 *   "fa_fwd_kernel (keys split between two groups)": d = 64 with the same
 *     grid limits; 8-wave workgroups of two 4-wave groups on the same rows.
 * All compute the same values up to the order of fp32 sums. NULL when the
 * shape is invalid. The string is static; no GPU is touched.
 */
FA355_API const char* fa_fwd_kernel_name(int B, int H, int N, int d, int causal);

/*
 * Size in bytes of the workspace fa_bwd needs for this shape: the fp32
 * [B,H,N] row statistic D_i = sum_c dO_ic O_ic, rounded up to 256 bytes.
 * Returns 0 when the shape is invalid.
 */
FA355_API size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass of fa_fwd (lesson 1, section 5): recomputes S and P per tile
 * from Q, K and the saved LSE, and returns the gradients of sum(O * dO):
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D) * scale with
 *   D_i = sum_j P_ij dP_ij = dO_i . O_i (the row sum over the whole row),
 *   dQ = dS K,  dK = dS^T Q.
 *   q, k, v, o, dout : in, bf16 [B,H,N,d]  (o and lse as returned by fa_fwd
 *                      for the same q, k, v, scale and causal)
 *   lse              : in, fp32 [B,H,N]
 *   dq, dk, dv       : out, bf16 [B,H,N,d]
 *   workspace        : scratch device memory of workspace_bytes bytes, at
 *                      least fa_bwd_workspace_bytes(B,H,N,d); its contents on
 *                      entry are ignored and on return are unspecified.
 * dK and dV are accumulated over query tiles by one workgroup per key tile,
 * dQ over key tiles by one workgroup per query tile (S and dP are computed
 * in both; a workgroup's two wave groups, when it has two, add their partial
 * sums in a fixed order), so all three gradients are deterministic.
 */
FA355_API int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
           float scale, int causal, void* stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments, kernels and results as fa_bwd
 * (bit-identical outputs); the row statistic D lives in a static device
 * array of the library instead of the caller's workspace.
 *   - B*H*N must be at most FA_BWD_NOALLOC_MAX_ROWS, else FA_ERR_TOO_LARGE
 *     (checked before any HIP call).
 *   - Allocates nothing: no hipMalloc/hipFree and no allocating library call.
 *     The array (16 MiB) exists on every device the library is loaded on
 *     until the process ends; its address is looked up once per device on
 *     the first call there (a HIP error then gives FA_ERR_HIP).
 *   - Every call on one device uses that device's one array: calls that
 *     overlap in time on one device (two streams, two host threads) race and
 *     give undefined gradients. Serialize them (one stream, or events).
 */
FA355_API int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * Names of the two kernels fa_bwd launches for this shape, in launch order:
 *   "fa_bwd_dq_kernel (keys split between two groups) + fa_bwd_dkdv_kernel"
 *     when the dQ grid is small (causal: at most 512 query tiles of 128 rows;
 *     non-causal: at most 256): two 4-wave groups per query tile take
 *     alternate key tiles and add their partial dQ in a fixed order;
 *   "fa_bwd_dq_kernel + fa_bwd_dkdv_kernel" otherwise.
 * Both compute the same values up to the order of fp32 sums. NULL when the
 * shape is invalid. The string is static; no GPU is touched.
 */
FA355_API const char* fa_bwd_kernel_name(int B, int H, int N, int d, int causal);

/*
 * Decode attention: Nq (1..32) query rows against an Nk-row key/value cache
 * per (batch, head) -- the KV-cache use named in the interview answer's bonus
 * points -- with the same exact softmax as fa_fwd. The keys are split over
 * many workgroups; each keeps the online-softmax statistics of lesson 1,
 * sections 3-4 over its split, and a second kernel merges the partial
 * results: LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 *   q, o      : bf16 [B,H,Nq,d] (in, out)
 *   k, v      : bf16 [B,H,Nk,d] (in)
 *   lse       : out, fp32 [B,H,Nq]
 *   causal    : the queries are the last Nq positions: query i may attend
 *               keys 0 .. Nk-Nq+i (requires Nq <= Nk)
 *   workspace : device memory of at least fa_decode_workspace_bytes(...)
 *               bytes for the per-split partial O (fp32) and LSE; contents on
 *               entry ignored, on return unspecified.
 * B*H*Nk*d must fit in 2^31 - 1 elements. Other conventions as for fa_fwd.
 */
FA355_API size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);
FA355_API int fa_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d,
           float scale, int causal, void* stream);

/*
 * The same O and LSE as fa_fwd computed in the other loop order, kept as a
 * measured comparator: the outer loop runs over key/value tiles and the inner
 * loop over query tiles (the interview answer's bonus points; "FlashAttention
 * and Triton", section 19.7 on the move from the first to the second
 * version). One workgroup handles one (batch, head); between key tiles each
 * query tile's unnormalised output and its running max and sum live in the
 * workspace, read and rewritten once per (key tile, query tile) pair with the
 * online-softmax rescaling of lesson 1, section 3.
 *   q, k, v, o, lse : as for fa_fwd
 *   workspace       : device memory of at least fa_fa1_workspace_bytes(...)
 *                     bytes (fp32 running state of every query row); contents
 *                     on entry ignored, on return unspecified.
 */
FA355_API size_t fa_fa1_workspace_bytes(int B, int H, int N, int d);
FA355_API int fa_fa1_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
           float scale, int causal, void* stream);

/*
 * The same O and LSE as fa_fwd on a persistent grid, kept as a measured
 * scheduling comparator (the interview answer's bonus points: persistent
 * workgroups and load balancing of the causal tiles). It runs the 128-row
 * forward kernel of fa_fwd, but with at most two resident workgroups per CU
 * (512), each looping over query tiles in a static heaviest-first "snake"
 * order within its XCD's heads; fa_fwd instead launches one workgroup per
 * query tile and lets the hardware dispatcher balance them. Same arguments,
 * conventions and errors as fa_fwd; allocates nothing. Results equal fa_fwd's
 * wherever fa_fwd runs the same kernel ("fa_fwd_kernel" from
 * fa_fwd_kernel_name), and otherwise up to the order of fp32 sums.
 */
FA355_API int fa_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/* A static, human-readable description of an FA_* code. */
FA355_API const char* fa_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H_ */
