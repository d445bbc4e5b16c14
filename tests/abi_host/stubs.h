// What the stand-in launchers of stubs.cpp saw on their last call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct LastCall {
  const char* which = nullptr;
  int BH = 0, N = 0, Nq = 0, d = 0;
  float scale = 0.f;
  bool causal = false;
  const void* ws = nullptr;
  hipStream_t stream = nullptr;
  int calls = 0;
};
extern LastCall g_last;

// The address the no-allocation entry point's scratch lookup returns here.
constexpr uintptr_t kScratchAddr = 0x7f0000000000ull;
