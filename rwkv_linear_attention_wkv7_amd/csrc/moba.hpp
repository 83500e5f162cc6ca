// Launchers of the MoBA attention core (moba.hip).  Token tensors are
// [B][T][H][64] fp32; the selection sel and the row log-sum-exp lse are
// [B][H][T]; kbar holds moba_kbar_floats chunk means; Dbuf B H T floats.
#pragma once
#include <cstdint>

#include <hip/hip_runtime.h>

int moba_num_chunks(int T, int chunk);
size_t moba_kbar_floats(int B, int T, int H, int chunk);
hipError_t moba_launch_forward(int B, int T, int H, int chunk, int topk, const float* q, const float* k,
                               const float* v, float* y, float* lse, uint64_t* sel, float* kbar,
                               hipStream_t st);
hipError_t moba_launch_backward(int B, int T, int H, int chunk, const float* q, const float* k,
                                const float* v, const float* y, const float* lse, const uint64_t* sel,
                                const float* dy, float* dq, float* dk, float* dv, float* Dbuf,
                                hipStream_t st);
