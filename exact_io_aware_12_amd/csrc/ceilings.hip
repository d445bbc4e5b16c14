// Ceilings of the units the attention kernels use, measured on the device:
// a calibration program, not part of the library.
//
//   mfma   dense v_mfma_f32_32x32x16_bf16, four independent accumulators per
//          wave (FLOP/s; the MFMA roof)
//   exp    v_exp_f32 chains (8 independent per lane; each step is exp2 then a
//          subtract, as in the softmax)
//   fma    v_fma_f32 chains (8 independent per lane)
//   lds    ds_read_b128 from a 64 KiB tile (bytes/s)
//   mix    four MFMAs plus 8*k exp steps per loop iteration in the same
//          wave, k = 0..4: how much exp work rides free under the MFMAs
//
// Each is timed with HIP events at one and two 4-wave workgroups per CU (one
// and two waves per SIMD), on 256 x {1,2} workgroups. Every kernel writes one
// value per thread so the work is kept; grids and indexes stay in bounds by
// construction (out has 512 * 256 floats; LDS indexes are masked to 4095).
#include <hip/hip_runtime.h>
#include <stdio.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256) void k_mfma(float* out, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f);
    b[i] = (__bf16)(i * 0.01f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma(a, b, c0);
    c1 = mfma(a, b, c1);
    c2 = mfma(a, b, c2);
    c3 = mfma(a, b, c3);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_exp(float* out, int iters) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = -0.001f * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) - 1.0f;
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_fma(float* out, int iters) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = 0.001f * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], 0.999f, 0.0001f);
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_lds(float* out, int iters) {
  __shared__ u32x4 buf[4096];   // 64 KiB
  for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  int idx = threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) acc ^= buf[(idx + r * 256) & 4095];
    idx = (idx + 7) & 4095;
  }
  out[blockIdx.x * 256 + threadIdx.x] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

__global__ __launch_bounds__(256) void k_mix(float* out, int iters, int nexp) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f);
    b[i] = (__bf16)(i * 0.01f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = -0.001f * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
    c0 = mfma(a, b, c0);
    c1 = mfma(a, b, c1);
    c2 = mfma(a, b, c2);
    c3 = mfma(a, b, c3);
    for (int e = 0; e < nexp; ++e)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) - 1.0f;
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Milliseconds of one launch after a short warm-up launch.
template <typename F>
static int timed(F launch, hipEvent_t e0, hipEvent_t e1, float* ms) {
  launch(true);
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0));
  launch(false);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  CHECK(hipEventElapsedTime(ms, e0, e1));
  return 0;
}

int main() {
  int dev = 0, ncu = 0, clk_khz = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  CHECK(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeClockRate, dev));
  if (ncu != 256) {
    fprintf(stderr, "expected 256 CUs, found %d\n", ncu);
    return 1;
  }
  const double clk = clk_khz * 1e3;   // the device's peak engine clock
  float* out = nullptr;
  CHECK(hipMalloc(&out, 512 * 256 * sizeof(float)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  printf("device: %d CUs, peak engine clock %.0f MHz (per-clock figures use it)\n", ncu, clk / 1e6);
  printf("| unit | workgroups per CU | rate | per CU per clock |\n|---|---|---|---|\n");
  for (int wpc = 1; wpc <= 2; ++wpc) {
    const int nb = 256 * wpc;
    float ms = 0.f;
    int it = 20000;
    if (timed([&](bool w) { hipLaunchKernelGGL(k_mfma, dim3(nb), dim3(256), 0, 0, out, w ? 100 : it); }, e0, e1, &ms)) return 1;
    double fl = (double)nb * 4 * it * 4 * 32768.0;
    printf("| mfma 32x32x16 bf16 | %d | %.1f TFLOP/s | %.0f FLOP |\n", wpc, fl / ms / 1e9, fl / (ms * 1e-3) / 256 / clk);
    if (timed([&](bool w) { hipLaunchKernelGGL(k_exp, dim3(nb), dim3(256), 0, 0, out, w ? 100 : it); }, e0, e1, &ms)) return 1;
    double ops = (double)nb * 256 * it * 8;
    printf("| v_exp_f32 + v_sub_f32 | %d | %.2f T lane-steps/s | %.1f lanes |\n", wpc, ops / ms / 1e9, ops / (ms * 1e-3) / 256 / clk);
    if (timed([&](bool w) { hipLaunchKernelGGL(k_fma, dim3(nb), dim3(256), 0, 0, out, w ? 100 : it); }, e0, e1, &ms)) return 1;
    printf("| v_fma_f32 | %d | %.2f T lane-ops/s | %.1f lanes |\n", wpc, ops / ms / 1e9, ops / (ms * 1e-3) / 256 / clk);
    it = 5000;
    if (timed([&](bool w) { hipLaunchKernelGGL(k_lds, dim3(nb), dim3(256), 0, 0, out, w ? 10 : it); }, e0, e1, &ms)) return 1;
    double bytes = (double)nb * 256 * it * 8 * 16;
    printf("| ds_read_b128 | %d | %.1f TB/s | %.0f B |\n", wpc, bytes / ms / 1e9, bytes / (ms * 1e-3) / 256 / clk);
    for (int nexp = 0; nexp <= 4; ++nexp) {
      it = 10000;
      if (timed([&](bool w) { hipLaunchKernelGGL(k_mix, dim3(nb), dim3(256), 0, 0, out, w ? 100 : it, nexp); }, e0, e1, &ms)) return 1;
      double fl2 = (double)nb * 4 * it * 4 * 32768.0;
      printf("| mfma + %d exp steps per 4 MFMAs | %d | %.1f TFLOP/s | %.0f FLOP |\n", 8 * nexp, wpc, fl2 / ms / 1e9, fl2 / (ms * 1e-3) / 256 / clk);
    }
  }
  CHECK(hipFree(out));
  return 0;
}
