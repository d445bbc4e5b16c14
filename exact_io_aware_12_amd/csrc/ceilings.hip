// Ceilings of the units the attention kernels use, measured on the device:
// a calibration program, not part of the library.
//
//   mfma   dense v_mfma_f32_32x32x16_bf16, four (and eight) independent
//          accumulators per wave (FLOP/s; the MFMA roof)
//   exp    v_exp_f32 chains (8 independent per lane; each step is exp2 then a
//          subtract, as in the softmax)
//   fma    v_fma_f32 chains (8 independent per lane)
//   lds    ds_read_b128 from a 64 KiB tile (bytes/s)
//   mix    four MFMAs plus 8*k exp steps per loop iteration in the same
//          wave, k = 0..4, in the compiler's own order (it issues the MFMAs
//          back to back, then the exps)
//   mixil  eight MFMAs per iteration, each followed by E exp steps placed
//          there by scheduling-group barriers: with the VALU mask alone
//          (0x002, which does not take v_exp_f32) and with VALU |
//          transcendental (0x402); how much exp work a wave runs under its
//          own MFMAs when its stream interleaves them
//   ldsmfma MFMAs whose A operand comes from LDS, as the attention kernels
//          read K (ds_read_b128) or V^T (two ds_read_b64_tr_b16), each read
//          feeding one or two MFMAs; the reads run half an iteration ahead
//   full   the forward's steady-state mix: each ds_read_b128 operand feeds R
//          MFMAs, and every MFMA carries one softmax element's VALU work
//          (fma, exp2, add to a row sum, and a bf16 pack every second
//          element), placed after it by scheduling-group barriers. R = 1 at
//          two waves per SIMD is the shape of the kernels (32 rows per
//          wave); R = 2 at one wave per SIMD is a 64-row-per-wave design
//          (twice the output registers, so one wave per SIMD), which halves
//          the LDS bytes per MFMA
//   ldsclk LDS read rate per CU per actual shader clock: one workgroup of
//          4, 8 or 16 waves per CU, R independent reads per lane in flight
//          (ds_read_b128, or ds_read_b64_tr_b16), lane-contiguous 16-byte
//          chunks of a 32 KiB tile; the clock comes from s_memtime against
//          s_memrealtime (100 MHz) between two barriers inside each workgroup
//   hbm    streaming reads of a 2 GiB buffer (global_load_dwordx4, grid
//          stride, U loads in flight per lane, plain or non-temporal), the
//          practical read ceiling of the HBM-bound decode kernel
//   dqacc  fp32 adds into a dQ-shaped accumulator (32 heads x 2048 rows x
//          128 columns) in the pattern a fused dK/dV/dQ kernel would use at
//          B=2, H=16, N=2048, causal: 256 workgroups of 8 waves, each a pair
//          of 128-key tiles (u, 15-u) walking its 34 query tiles of 64 rows and
//          adding one 64 x 128 block per tile (32 lanes of a wave cover 128
//          contiguous bytes of a row). Plain stores of the same blocks
//          against global_atomic_add_f32 at agent and at workgroup scope
//          (the two scopes give the same instruction here). The workgroups of
//          one head sit on one XCD under round-robin placement. Every element
//          of the accumulator is checked against its exact count
//
// Each is timed with HIP events at one and two 4-wave workgroups per CU (one
// and two waves per SIMD), on 256 x {1,2} workgroups. Every kernel writes one
// value per thread so the work is kept; grids and indexes stay in bounds by
// construction (out has 512 * 256 floats; LDS indexes are masked to 4095 in
// k_lds and stay below 32 KiB in k_ldsmfma).
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_mfma8(float* out, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f);
    b[i] = (__bf16)(i * 0.01f);
  }
  f32x16 c[8];
  for (int i = 0; i < 8; ++i) for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int m = 0; m < 8; ++m) c[m] = mfma(a, b, c[m]);
  float s = 0.f;
  for (int i = 0; i < 8; ++i) for (int j = 0; j < 16; ++j) s += c[i][j];
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

template <int E, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_mixil(float* out, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f);
    b[i] = (__bf16)(i * 0.01f);
  }
  f32x16 c[8];
  for (int i = 0; i < 8; ++i) for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = -0.001f * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      c[m] = mfma(a, b, c[m]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int k = (m * E + e) & 15;
        x[k] = __builtin_amdgcn_exp2f(x[k]) - 1.0f;
      }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (E > 0) __builtin_amdgcn_sched_group_barrier(MASK, 2 * E, 0);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) for (int j = 0; j < 16; ++j) s += c[i][j];
  for (int i = 0; i < 16; ++i) s += x[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int R, bool TR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ldsmfma(float* out, int iters) {
  __shared__ __attribute__((aligned(1024))) unsigned char buf[32768];
  for (int i = threadIdx.x; i < 32768 / 4; i += 256) reinterpret_cast<unsigned*>(buf)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, sl = lane & 15;
  bf16x8 b[R];
  for (int r = 0; r < R; ++r) for (int i = 0; i < 8; ++i) b[r][i] = (__bf16)((i + r) * 0.01f);
  f32x16 c[4 * R];
  for (int i = 0; i < 4 * R; ++i) for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  // Operand i of a 16 KiB half: K pattern (row l32 of 32-key block i&1,
  // XOR-swizzled 16-byte chunk 2*(i>>1)+hi) or V^T pattern (16 keys t = i>>2,
  // 32 columns db = i&3, two transposing reads 8 rows apart); all < 16 KiB.
  auto addr = [&](int i, int half) -> int {
    if (!TR) {
      const int kb = i & 1, ks = i >> 1;
      return half * 16384 + (kb * 32 + l32) * 256 + (((2 * ks + hi) ^ (l32 & 15)) << 4);
    } else {
      const int t = i >> 2, db = i & 3;
      const int row = 4 * hi + (sl >> 2), col = 32 * db + 16 * (g & 1) + 4 * (sl & 3);
      const int off = row * 256 + (((col >> 5) ^ (row & 3)) << 6) + (col & 31) * 2;
      return half * 16384 + 16 * t * 256 + off;
    }
  };
  auto rd = [&](int a) -> bf16x8 {
    if (!TR) return *reinterpret_cast<const bf16x8*>(buf + a);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + a));
    const s16x4 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + a + 2048));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, h4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8 a0[8], a1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a0[i] = rd(addr(i, 0));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a1[i] = rd(addr(8 + i, it & 1));
#pragma unroll
      for (int r = 0; r < R; ++r) c[(i & 3) * R + r] = mfma(a0[i], b[r], c[(i & 3) * R + r]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a0[i] = rd(addr(i, (it + 1) & 1));
#pragma unroll
      for (int r = 0; r < R; ++r) c[(i & 3) * R + r] = mfma(a1[i], b[r], c[(i & 3) * R + r]);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 4 * R; ++i) for (int j = 0; j < 16; ++j) s += c[i][j];
  for (int i = 0; i < 8; ++i) s += (float)a0[i][0];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int R, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void k_full(float* out, int iters, float cc) {
  __shared__ __attribute__((aligned(1024))) unsigned char buf[32768];
  for (int i = threadIdx.x; i < 32768 / 4; i += 256) reinterpret_cast<unsigned*>(buf)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  bf16x8 b[R];
  for (int r = 0; r < R; ++r) for (int i = 0; i < 8; ++i) b[r][i] = (__bf16)((i + r) * 0.01f);
  f32x16 c[4 * R];
  for (int i = 0; i < 4 * R; ++i) for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  float x[16], rs[4] = {0.f, 0.f, 0.f, 0.f};
  unsigned pk[8] = {};
  for (int i = 0; i < 16; ++i) x[i] = -0.001f * (threadIdx.x + i);
  // The K pattern of k_ldsmfma: operand i of a 16 KiB half, all < 32 KiB.
  auto addr = [&](int i, int half) -> int {
    const int kb = i & 1, ks = i >> 1;
    return half * 16384 + (kb * 32 + l32) * 256 + (((2 * ks + hi) ^ (l32 & 15)) << 4);
  };
  auto rd = [&](int a) -> bf16x8 { return *reinterpret_cast<const bf16x8*>(buf + a); };
  bf16x8 a0[8], a1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a0[i] = rd(addr(i, 0));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (h == 0) a1[i] = rd(addr(8 + i, it & 1));
        else a0[i] = rd(addr(i, (it + 1) & 1));
#pragma unroll
        for (int r = 0; r < R; ++r) {
          c[(i & 3) * R + r] = mfma(h == 0 ? a0[i] : a1[i], b[r], c[(i & 3) * R + r]);
          const int k = (i * R + r) & 15;
          const float e = __builtin_amdgcn_exp2f(fmaf(x[k], cc, -1.0f));
          rs[k & 3] += e;
          if (k & 1) {
            f32x2 f = {x[k - 1], e};
            pk[(k >> 1) & 7] ^= __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
          }
          x[k] = e;
        }
      }
      // Per operand: its read, then per MFMA the MFMA and 3-4 VALU /
      // transcendental instructions.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
        }
      }
    }
  }
  float s = 0.f;
  for (int i = 0; i < 4 * R; ++i) for (int j = 0; j < 16; ++j) s += c[i][j];
  for (int i = 0; i < 8; ++i) s += (float)a0[i][0] + (float)pk[i];
  for (int i = 0; i < 4; ++i) s += rs[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void k_hbm(const u32x4* __restrict__ src, size_t n16, unsigned* out) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (size_t)(U - 1) * stride < n16; i += (size_t)U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// LDS reads for the per-clock rate (see the header): clk[2b] and clk[2b+1]
// are workgroup b's s_memtime and s_memrealtime deltas between the barriers.
// Indexes stay inside the 32 KiB tile (masked to 2047 chunks).
template <int NT, int R, bool TR>
__global__ __launch_bounds__(NT) void k_ldsclk(unsigned* out, long long* clk, int iters) {
  __shared__ u32x4 buf[2048];
  for (int i = threadIdx.x; i < 2048; i += NT) buf[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  u32x4 acc = {0, 0, 0, 0};
  int idx = threadIdx.x & 2047;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = (idx + r * 64) & 2047;
      if constexpr (TR) {
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS s16x4*)((LDS_AS char*)(LDS_AS void*)buf + c * 16));
        const u32x2 u = __builtin_bit_cast(u32x2, v);
        acc[2 * (r & 1)] ^= u[0];
        acc[2 * (r & 1) + 1] ^= u[1];
      } else {
        acc ^= buf[c];
      }
    }
    idx = (idx + 7) & 2047;
  }
  out[blockIdx.x * NT + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __syncthreads();
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// One block of the dQ-shaped accumulator per (workgroup, query tile): a
// workgroup is a causal pair of 128-key tiles (u, 15 - u) of one head and
// adds into the 64-row query tiles 2*kt .. 31 of each (34 in all). Wave w
// covers rows 32*(w/4) .. +32 and columns 32*(w%4) .. +32 of the block in the
// layout of a 32x32 MFMA accumulator (lane -> column). Heads 4x .. 4x+3 go to
// workgroups b with b % 8 == x. Indexes stay inside 32 x 2048 x 128.
template <int MODE>
__global__ __launch_bounds__(512) void k_dqacc(float* __restrict__ acc) {
  const int b = blockIdx.x, slot = b / 8;
  const int head = (b % 8) * 4 + slot % 4, u = slot / 4;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  float* hp = acc + (size_t)head * 2048 * 128;
  const int col = 32 * (w % 4) + lane % 32;
  for (int part = 0; part < 2; ++part) {
    const int kt = part == 0 ? u : 15 - u;
    for (int qt = 2 * kt; qt < 32; ++qt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 64 * qt + 32 * (w / 4) + 8 * (i / 4) + 4 * (lane / 32) + i % 4;
        float* p = hp + (size_t)row * 128 + col;
        if constexpr (MODE == 0) *p = 1.0f;
        else if constexpr (MODE == 1) __hip_atomic_fetch_add(p, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else __hip_atomic_fetch_add(p, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
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
      printf("| mfma + %d exp steps per 4 MFMAs, compiler order | %d | %.1f TFLOP/s | %.0f FLOP |\n", 8 * nexp, wpc, fl2 / ms / 1e9, fl2 / (ms * 1e-3) / 256 / clk);
    }
    it = 10000;
    const double fl8 = (double)nb * 4 * it * 8 * 32768.0;
    if (timed([&](bool w) { hipLaunchKernelGGL(k_mfma8, dim3(nb), dim3(256), 0, 0, out, w ? 100 : it); }, e0, e1, &ms)) return 1;
    printf("| mfma 32x32x16 bf16, 8 accumulators | %d | %.1f TFLOP/s | %.0f FLOP |\n", wpc, fl8 / ms / 1e9, fl8 / (ms * 1e-3) / 256 / clk);
#define FA_MIXIL(E, M)                                                                              \
    if (timed([&](bool w) { hipLaunchKernelGGL((k_mixil<E, M>), dim3(nb), dim3(256), 0, 0, out, w ? 100 : it); }, e0, e1, &ms)) return 1; \
    printf("| mfma + %d exp steps after each MFMA, sched mask 0x%03x | %d | %.1f TFLOP/s | %.0f FLOP |\n", E, M, wpc, fl8 / ms / 1e9, fl8 / (ms * 1e-3) / 256 / clk);
    FA_MIXIL(1, 0x002) FA_MIXIL(1, 0x402) FA_MIXIL(2, 0x002) FA_MIXIL(2, 0x402)
    FA_MIXIL(3, 0x002) FA_MIXIL(3, 0x402) FA_MIXIL(4, 0x402)
#undef FA_MIXIL
    const double fl16 = (double)nb * 4 * it * 16 * 32768.0;
#define FA_LDSMFMA(R, TR)                                                                           \
    if (timed([&](bool w) { hipLaunchKernelGGL((k_ldsmfma<R, TR>), dim3(nb), dim3(256), 0, 0, out, w ? 100 : it); }, e0, e1, &ms)) return 1; \
    printf("| mfma, A operand from LDS (%s), %d MFMA per operand | %d | %.1f TFLOP/s | %.0f FLOP |\n", TR ? "2 x ds_read_b64_tr_b16" : "ds_read_b128", R, wpc, R * fl16 / ms / 1e9, R * fl16 / (ms * 1e-3) / 256 / clk);
    FA_LDSMFMA(1, false) FA_LDSMFMA(2, false) FA_LDSMFMA(1, true) FA_LDSMFMA(2, true)
#undef FA_LDSMFMA
  }
  // The forward's mix at its two candidate shapes, each at the occupancy its
  // registers allow (256 x WPE workgroups of 4 waves).
  {
    const int it = 5000;
    float ms = 0.f;
#define FA_FULL(R, WPE)                                                                             \
    if (timed([&](bool w) { hipLaunchKernelGGL((k_full<R, WPE>), dim3(256 * WPE), dim3(256), 0, 0, out, w ? 50 : it, 0.5f); }, e0, e1, &ms)) return 1; \
    {                                                                                               \
      const double fl = 256.0 * WPE * 4 * it * 16 * R * 32768.0;                                    \
      printf("| mfma + softmax VALU per MFMA, LDS operand feeding %d MFMA(s) | %d | %.1f TFLOP/s | %.0f FLOP |\n", R, WPE, fl / ms / 1e9, fl / (ms * 1e-3) / 256 / clk); \
    }
    FA_FULL(1, 2) FA_FULL(2, 1) FA_FULL(1, 1) FA_FULL(2, 2)
#undef FA_FULL
  }
  // Streaming HBM reads (one launch reads the whole buffer; its contents do
  // not matter). out2 holds one word per thread of the largest grid.
  {
    const size_t bytes = (size_t)2 << 30, n16 = bytes / 16;
    u32x4* buf = nullptr;
    unsigned* out2 = nullptr;
    CHECK(hipMalloc(&buf, bytes));
    CHECK(hipMalloc(&out2, (size_t)8192 * 256 * sizeof(unsigned)));
    float ms = 0.f;
#define FA_HBM(U, NT)                                                                                   for (int nb = 1024; nb <= 8192; nb *= 2) {                                                            if (timed([&](bool) { hipLaunchKernelGGL((k_hbm<U, NT>), dim3(nb), dim3(256), 0, 0, buf, n16, out2); }, e0, e1, &ms)) return 1;       printf("| HBM read, global_load_dwordx4, %d in flight per lane%s, %d workgroups of 4 waves | %d | %.2f TB/s | |\n", U, NT ? ", non-temporal" : "", nb, nb / 256, bytes / (ms * 1e-3) / 1e12);     }
    FA_HBM(4, false) FA_HBM(8, false) FA_HBM(4, true) FA_HBM(8, true)
#undef FA_HBM
    CHECK(hipFree(out2));
    CHECK(hipFree(buf));
  }
  // LDS read rate per CU per actual clock (one workgroup per CU, 256 CUs).
  {
    unsigned* o3 = nullptr;
    long long* ck = nullptr;
    CHECK(hipMalloc(&o3, 256 * 1024 * sizeof(unsigned)));
    CHECK(hipMalloc(&ck, 2 * 256 * sizeof(long long)));
    long long hk[512];
    printf("| LDS read | waves per CU | reads in flight per lane | rate (all CUs) | per CU per actual clock |\n|---|---|---|---|---|\n");
#define FA_LDSCLK(NT, R, TR)                                                                        \
    {                                                                                               \
      const int it = 4000;                                                                          \
      float ms = 0.f;                                                                               \
      if (timed([&](bool w) { hipLaunchKernelGGL((k_ldsclk<NT, R, TR>), dim3(256), dim3(NT), 0, 0, o3, ck, w ? 10 : it); }, e0, e1, &ms)) return 1; \
      CHECK(hipMemcpy(hk, ck, sizeof(hk), hipMemcpyDeviceToHost));                                  \
      double mc = 0, mr = 0;                                                                        \
      for (int i = 0; i < 256; ++i) { mc += (double)hk[2 * i]; mr += (double)hk[2 * i + 1]; }       \
      const double bytes = (double)NT * it * R * (TR ? 8 : 16);                                     \
      printf("| %s | %d | %d | %.1f TB/s | %.0f B (clock %.0f MHz) |\n", TR ? "ds_read_b64_tr_b16" : "ds_read_b128", \
             NT / 64, R, 256.0 * bytes / (ms * 1e-3) / 1e12, bytes * 256 / mc, mc / mr * 100.0);     \
    }
    FA_LDSCLK(256, 16, false) FA_LDSCLK(512, 16, false) FA_LDSCLK(1024, 16, false)
    FA_LDSCLK(512, 16, true) FA_LDSCLK(1024, 16, true)
#undef FA_LDSCLK
    CHECK(hipFree(ck));
    CHECK(hipFree(o3));
  }
  // fp32 adds into a dQ-shaped accumulator (best of 3 launches, each on a
  // zeroed buffer; every element checked against its exact count).
  {
    const size_t n = (size_t)32 * 2048 * 128;
    float* acc = nullptr;
    CHECK(hipMalloc(&acc, n * sizeof(float)));
    float* host = (float*)malloc(n * sizeof(float));
    if (!host) return 1;
    const double bytes = 256.0 * 34 * 64 * 128 * 4;
    for (int mode = 0; mode < 3; ++mode) {
      float best = 1e30f;
      for (int t = 0; t < 3; ++t) {
        CHECK(hipMemset(acc, 0, n * sizeof(float)));
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(e0));
        if (mode == 0) hipLaunchKernelGGL(k_dqacc<0>, dim3(256), dim3(512), 0, 0, acc);
        if (mode == 1) hipLaunchKernelGGL(k_dqacc<1>, dim3(256), dim3(512), 0, 0, acc);
        if (mode == 2) hipLaunchKernelGGL(k_dqacc<2>, dim3(256), dim3(512), 0, 0, acc);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms = 0.f;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        if (ms < best) best = ms;
      }
      CHECK(hipMemcpy(host, acc, n * sizeof(float), hipMemcpyDeviceToHost));
      long bad = 0;
      for (size_t e = 0; e < n; ++e) {
        const int qt = (int)((e / 128) % 2048) / 64;
        if (host[e] != (mode == 0 ? 1.0f : (float)(qt / 2 + 1))) ++bad;
      }
      printf("| dQ-shaped accumulator, %s, %.1f MB per launch | 1 (8 waves) | %.2f TB/s (%.1f us) | %ld wrong elements |\n",
             mode == 0 ? "plain stores" : mode == 1 ? "global_atomic_add_f32, agent scope" : "global_atomic_add_f32, workgroup scope",
             bytes / 1e6, bytes / (best * 1e-3) / 1e12, best * 1e3, bad);
    }
    free(host);
    CHECK(hipFree(acc));
  }
  CHECK(hipFree(out));
  return 0;
}
