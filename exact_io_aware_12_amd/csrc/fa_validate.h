// Host-side argument checks shared by the C entry points of libfa355.so and
// libfa355_unfused.so. Plain C++ with no HIP calls, so they run (and are
// tested) on a machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/fa355.h"

namespace fa {

constexpr int64_t kMaxElems = 2147483647;  // 2^31 - 1

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// B, H, N >= 1, d in {64, 128}, B*H*N*d < 2^31.
inline int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  const int64_t elems = (int64_t)B * H * N * d;
  if (elems > kMaxElems) return FA_ERR_SHAPE;
  return FA_OK;
}

inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace fa
