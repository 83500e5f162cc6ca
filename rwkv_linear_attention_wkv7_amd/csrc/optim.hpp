// Multi-tensor parameter updates (optim.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

constexpr int OPT_MAX = 24;  // tensors per launch
struct OptBatch {
  int n;
  float* p[OPT_MAX];
  const float* g[OPT_MAX];
  float* m[OPT_MAX];  // Adam only
  float* v[OPT_MAX];
  size_t count[OPT_MAX];  // elements (a multiple of 4)
};
// adam = 0: SGD; 1: Adam at update index step (>= 1).
hipError_t opt_launch(const OptBatch& t, int adam, float lr, float clip, int step, hipStream_t st);
