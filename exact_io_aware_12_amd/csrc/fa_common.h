// Device-side building blocks shared by the forward and backward kernels of
// the fused exact attention library (gfx950 / CDNA4 only).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, one
// wave64): for D(32x32) += A(32x16) * B(16x32)
//   * A operand: lane l holds 8 bf16 of row (l % 32), k-slots 8*(l/32)+0..7;
//   * B operand: lane l holds 8 bf16 of column (l % 32), the same k-slots;
//   * accumulator: lane l, register i holds D[row][col] with col = l % 32 and
//     row = 8*(i/4) + 4*(l/32) + (i%4).
// A and B see the k-slots in the same order, so any consistent assignment of
// the contraction index to (half, slot) gives the same sum; the kernels use
// this to feed accumulator registers back in as an operand without moving
// them across lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Race-check build (-DFA_STRICT_SYNC, built as libfa355_strict.so): the wave
// that issues a global -> LDS copy waits for it right away, so no copy is
// ever in flight while the wave or its workgroup goes on. The normal build
// overlaps the copies with MFMA work and relies on its barriers to keep every
// read of a buffer away from a copy into it. Both builds compute the same
// arithmetic in the same order: any difference in their outputs would be a
// copy that raced with a read.
__device__ __forceinline__ void strict_copy_wait() {
#ifdef FA_STRICT_SYNC
  __builtin_amdgcn_s_waitcnt(0x0F70);   // s_waitcnt vmcnt(0)
#endif
}

// NaN-propagating max / min (v_maximum3_f32 / v_minimum3_f32 on gfx950; no
// operand canonicalisation as fmaxf needs in IEEE mode).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max / sum of x over lanes l and l ^ 32, via v_permlane32_swap (one VALU
// exchange, no LDS round trip): swapping x with itself leaves x of the low
// half in one result and x of the high half in the other, on every lane.
__device__ __forceinline__ float halves_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 -> two bf16 (round to nearest even), packed in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// Eight fp32 -> a bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  u32x4 u = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3), pack_bf16x2(a4, a5),
             pack_bf16x2(a6, a7)};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ u32x4 ld_global_16B(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// One wave's 32 output rows (rows 0 .. 31 from `rows`, a row-major [*, D]
// bf16 array), held one row per lane in accumulator layout: lane l has row l % 32
// and d = 32*db + 8*g4 + 4*(l/32) .. +3 in v[db][g4]. Storing them directly
// would scatter each 8-byte store over 32 rows. Instead they go through this
// wave's own LDS slice `stage` (32 rows of 2*D bytes, 16-byte chunks
// XOR-swizzled by the row so that one write's 32 rows spread over the banks)
// and leave as whole rows, 16 bytes per lane, consecutive lanes on
// consecutive chunks of a row. Rows from nvalid on are not stored. A wave's
// LDS operations run in order, so no barrier is needed; no other wave may
// use `stage` meanwhile.
template <int D>
__device__ __forceinline__ void store_rows_staged(uint16_t* rows, int nvalid, uint8_t* stage,
                                                  const u32x2 (&v)[D / 32][4], int lane) {
  constexpr int RB = 2 * D, CPR = RB / 16;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c = (4 * db + g4) ^ (r & (CPR - 1));
      *reinterpret_cast<u32x2*>(stage + r * RB + c * 16 + 8 * h) = v[db][g4];
    }
#pragma unroll
  for (int j = 0; j < 32 * CPR / 64; ++j) {
    const int idx = lane + 64 * j;
    const int rr = idx / CPR, cc = idx % CPR;
    const u32x4 val = *reinterpret_cast<const u32x4*>(stage + rr * RB + ((cc ^ (rr & (CPR - 1))) * 16));
    if (rr < nvalid) *reinterpret_cast<u32x4*>(rows + (size_t)rr * D + cc * 8) = val;
  }
}

}  // namespace fa
