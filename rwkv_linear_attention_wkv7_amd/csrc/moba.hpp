// Launchers of the MoBA attention core (moba.hip).  Token tensors are
// [B][T][H][64] fp32; the selection sel and the row log-sum-exp lse are
// [B][H][T]; ws holds moba_ws_bytes bytes (the same layout in both
// directions).
#pragma once
#include <cstdint>

#include <hip/hip_runtime.h>

int moba_num_chunks(int T, int chunk);
size_t moba_ws_bytes(int B, int T, int H, int chunk, int topk);
hipError_t moba_launch_forward(int B, int T, int H, int chunk, int topk, const float* q, const float* k,
                               const float* v, float* y, float* lse, uint64_t* sel, void* ws,
                               hipStream_t st);
hipError_t moba_launch_backward(int B, int T, int H, int chunk, int topk, const float* q, const float* k,
                                const float* v, const float* y, const float* lse, const uint64_t* sel,
                                const float* dy, float* dq, float* dk, float* dv, void* ws,
                                hipStream_t st);
