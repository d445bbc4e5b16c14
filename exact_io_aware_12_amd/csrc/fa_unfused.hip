// Unfused ("standard") attention for gfx950: the three-step decomposition
// that the fused kernels replace, kept as a measured comparator.
//
// Method: the aiworkagent interview answer on FlashAttention (q15), "standard
// attention" steps, and "FlashAttention and Triton", section 19.2: S = Q K^T
// is written to HBM, read back for a row-wise softmax whose P is written to
// HBM again, and read once more for O = P V. The row softmax is one fused
// pass per row as in section 19.11 of the same chapter (one program per row:
// subtract the row max, exponentiate, divide by the row sum).
//
//   1. S = scale * Q K^T: a plain library GEMM (rocBLAS, bf16 in, fp32 out),
//      S fp32 [BH, N, N] in the caller's workspace.
//   2. fa_row_softmax: one workgroup per row reads S once, applies the
//      causal mask (keys j > i), writes P in bf16 over the first half of the
//      same row's bytes and the row's LSE = max + ln(sum).
//   3. O = P V: a plain library GEMM (bf16 in and out, fp32 accumulate) with
//      P read through a leading dimension of 2N bf16 elements.
#include <rocblas/rocblas.h>

#include <map>
#include <mutex>

#include "fa_common.h"

namespace fa {

namespace {

constexpr int kSmThreads = 256;

// max / sum over the workgroup (4 wave64s): in-wave butterfly, then the four
// wave results through LDS. Contains a barrier: every thread must call it.
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = vmax(v, __shfl_xor(v, s, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return vmax(vmax(red[0], red[1]), vmax(red[2], red[3]));
}
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Row softmax with the row held in registers: 4*IT elements per thread, so
// N <= 1024*IT. VEC: N % 4 == 0, 16-byte loads of 4 consecutive elements.
// Every load happens before the first block reduction (a barrier), so the
// in-place bf16 writes cannot overwrite S elements another thread still
// has to read.
template <int IT, bool VEC>
__global__ __launch_bounds__(kSmThreads) void fa_row_softmax_kernel(float* __restrict__ S,
                                                                    float* __restrict__ LSE,
                                                                    int N, int causal) {
  __shared__ float red[4];
  const long long row = blockIdx.x;
  const int q = (int)(row % N);
  const int valid = causal ? q + 1 : N;   // keys 0 .. valid-1 are admissible
  float* srow = S + row * (long long)N;
  uint16_t* prow = reinterpret_cast<uint16_t*>(srow);
  const int tid = threadIdx.x;

  float x[4 * IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j0 = 4 * (tid + kSmThreads * it);
    if constexpr (VEC) {
      f32x4 v = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (j0 < N) v = *reinterpret_cast<const f32x4*>(srow + j0);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * it + e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * it + e] = (j0 + e < N) ? srow[j0 + e] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j0 + e >= valid) x[4 * it + e] = -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4 * IT; ++i) m = vmax(m, x[i]);
  m = block_max(m, red);   // every row has key 0 admissible: m is finite
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < 4 * IT; ++i) {
    x[i] = fast_exp2((x[i] - m) * kLog2e);
    l += x[i];
  }
  l = block_sum(l, red);
  const float inv = 1.f / l;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j0 = 4 * (tid + kSmThreads * it);
    if constexpr (VEC) {
      if (j0 < N) {
        u32x2 pr = {pack_bf16x2(x[4 * it] * inv, x[4 * it + 1] * inv),
                    pack_bf16x2(x[4 * it + 2] * inv, x[4 * it + 3] * inv)};
        *reinterpret_cast<u32x2*>(prow + j0) = pr;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + e < N) prow[j0 + e] = (uint16_t)(pack_bf16x2(x[4 * it + e] * inv, 0.f) & 0xffffu);
    }
  }
  if (tid == 0) LSE[row] = m + fast_log2(l) * kLn2;
}

// Rows too long for registers: per-thread running (max, sum) over the row,
// combined across the workgroup, then a second pass over the row in chunks of
// 4*256 elements. Each chunk is read, then a barrier, then its P written:
// P bytes of chunk c overlap only S elements of chunks <= c, all of which
// every thread has read by then.
__global__ __launch_bounds__(kSmThreads) void fa_row_softmax_long_kernel(float* __restrict__ S,
                                                                         float* __restrict__ LSE,
                                                                         int N, int causal) {
  __shared__ float red[4];
  const long long row = blockIdx.x;
  const int q = (int)(row % N);
  const int valid = causal ? q + 1 : N;
  float* srow = S + row * (long long)N;
  uint16_t* prow = reinterpret_cast<uint16_t*>(srow);
  const int tid = threadIdx.x;

  float m = -INFINITY, l = 0.f;
  for (int j = tid; j < valid; j += kSmThreads) {
    const float s = srow[j];
    if (s > m) {
      l = l * fast_exp2((m - s) * kLog2e) + 1.f;
      m = s;
    } else {
      l += fast_exp2((s - m) * kLog2e);
    }
  }
  const float mb = block_max(m, red);
  l = block_sum(m == -INFINITY ? 0.f : l * fast_exp2((m - mb) * kLog2e), red);
  const float inv = 1.f / l;
  for (int c0 = 0; c0 < N; c0 += 4 * kSmThreads) {
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = c0 + 4 * tid + e;
      p[e] = (j < valid) ? fast_exp2((srow[j] - mb) * kLog2e) * inv : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = c0 + 4 * tid + e;
      if (j < N) prow[j] = (uint16_t)(pack_bf16x2(p[e], 0.f) & 0xffffu);
    }
  }
  if (tid == 0) LSE[row] = mb + fast_log2(l) * kLn2;
}

// One rocBLAS handle per device, created on first use.
rocblas_handle handle_for_device(hipError_t* err) {
  static std::mutex mu;
  static std::map<int, rocblas_handle> handles;
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = handles.find(dev);
  if (it != handles.end()) return it->second;
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
  handles[dev] = h;
  return h;
}

}  // namespace

// Returns hipSuccess, a HIP error, or hipErrorUnknown when rocBLAS fails
// (*blas_failed is then set).
hipError_t unfused_fwd_dispatch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                uint16_t* o, float* lse, float* ws, int BH, int N, int d,
                                float scale, bool causal, hipStream_t stream, bool* blas_failed) {
  *blas_failed = false;
  hipError_t err = hipSuccess;
  rocblas_handle h = handle_for_device(&err);
  if (err != hipSuccess) return err;
  if (!h) {
    *blas_failed = true;
    return hipErrorUnknown;
  }
  static std::mutex call_mu;   // the handle's stream is per call
  std::lock_guard<std::mutex> lock(call_mu);
  if (rocblas_set_stream(h, stream) != rocblas_status_success) {
    *blas_failed = true;
    return hipErrorUnknown;
  }
  const rocblas_stride sqkv = (rocblas_stride)N * d;
  const rocblas_stride ss = (rocblas_stride)N * N;   // fp32 elements per head
  // 1. Row-major S[q][j] = scale * sum_c Q[q][c] K[j][c]. In rocBLAS's
  //    column-major terms that is S^T (N x N, ld N) = K Q^T with K stored as
  //    the transpose of a d x N column-major matrix and Q^T as a d x N one.
  const float alpha = scale, beta = 0.f, one = 1.f;
  rocblas_status st = rocblas_gemm_strided_batched_ex(
      h, rocblas_operation_transpose, rocblas_operation_none, N, N, d, &alpha, k,
      rocblas_datatype_bf16_r, d, sqkv, q, rocblas_datatype_bf16_r, d, sqkv, &beta, ws,
      rocblas_datatype_f32_r, N, ss, ws, rocblas_datatype_f32_r, N, ss, BH,
      rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success) {
    *blas_failed = true;
    return hipErrorUnknown;
  }
  // 2. Row softmax (and the causal mask), P in place.
  {
    dim3 grid((unsigned)((long long)BH * N)), block(kSmThreads);
    const bool vec = (N % 4) == 0;
    const int c = causal ? 1 : 0;
#define FA_SM_CASE(IT)                                                                        \
  if (N <= 1024 * IT) {                                                                       \
    if (vec)                                                                                  \
      hipLaunchKernelGGL((fa_row_softmax_kernel<IT, true>), grid, block, 0, stream, ws, lse, N, c); \
    else                                                                                      \
      hipLaunchKernelGGL((fa_row_softmax_kernel<IT, false>), grid, block, 0, stream, ws, lse, N, c); \
  } else
    FA_SM_CASE(1) FA_SM_CASE(2) FA_SM_CASE(4) FA_SM_CASE(8) FA_SM_CASE(16)
    hipLaunchKernelGGL(fa_row_softmax_long_kernel, grid, block, 0, stream, ws, lse, N, c);
#undef FA_SM_CASE
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // 3. Row-major O[q][c] = sum_j P[q][j] V[j][c]: column-major O^T (d x N,
  //    ld d) = V^T P^T, with P^T the N x N column-major view of the bf16 P
  //    rows (ld 2N elements: each P row starts at its S row).
  st = rocblas_gemm_strided_batched_ex(
      h, rocblas_operation_none, rocblas_operation_none, d, N, N, &one, v,
      rocblas_datatype_bf16_r, d, sqkv, ws, rocblas_datatype_bf16_r, 2 * N, 2 * ss, &beta, o,
      rocblas_datatype_bf16_r, d, sqkv, o, rocblas_datatype_bf16_r, d, sqkv, BH,
      rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success) {
    *blas_failed = true;
    return hipErrorUnknown;
  }
  return hipSuccess;
}

}  // namespace fa
