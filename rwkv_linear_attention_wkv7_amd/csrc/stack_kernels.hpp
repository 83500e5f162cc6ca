// Launchers of the stack kernels (stack_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>

hipError_t stk_launch_emb_gather(int R, int C, int V, const int* tok, const float* emb, float* out,
                                 hipStream_t st);
hipError_t stk_launch_layernorm(int R, int C, const float* x, const float* w, const float* b,
                                float* y, float* mean, float* rstd, hipStream_t st);
hipError_t stk_launch_cm_shift(int BT, int T, int C, const float* x, const float* x_prev,
                               const float* mu, float* sh, float* x_last, hipStream_t st);
int stk_max_layernorm_width();
