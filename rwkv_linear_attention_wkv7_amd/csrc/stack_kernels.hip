// Kernels around the time-mix block in an RWKV-7 stack (gfx950): embedding
// gather, LayerNorm, channel-mix token shift.
//
// Pages: "Foundry/cuda_kernels/fullmodel.cu" (fm_k_emb_fwd: out[t] =
// emb[token[t]]; LayerNorm before each mix and at the output; fm_cm_fwd:
// token shift, sh @ Wk, relu^2, @ Wv) and "infotheory .../rwkv7/model.rs"
// (LayerNorm eps 1e-5; the channel-mix shift state ffn_x_prev).

#include "common.hpp"
#include "stack_kernels.hpp"

namespace stk {

constexpr float LN_EPS = 1e-5f;
constexpr int MAXC4 = 16;  // LayerNorm keeps a row in registers: C <= 64 * 4 * MAXC4

// out[r] = emb[clamp(tok[r])] (float4 per thread)
__global__ __launch_bounds__(256) void emb_gather(int R, int C, int V, const int* __restrict__ tok,
                                                  const float* __restrict__ emb,
                                                  float* __restrict__ out) {
  const size_t n4 = (size_t)R * C / 4;
  const int C4 = C / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t row = i / C4;
    const int c4 = (int)(i - row * C4);
    const int id = min(max(tok[row], 0), V - 1);
    reinterpret_cast<f4*>(out)[i] = reinterpret_cast<const f4*>(emb + (size_t)id * C)[c4];
  }
}

// y = (x - mean) / sqrt(var + eps) * w + b per row; one wave per row, the row
// held in registers (in-place safe).  mean/rstd are optional outputs.
__global__ __launch_bounds__(256) void layernorm_fwd(int R, int C, const float* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ b, float* y,
                                                     float* __restrict__ mean_out,
                                                     float* __restrict__ rstd_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= R) return;
  const int C4 = C / 4;
  const f4* xr = reinterpret_cast<const f4*>(x + (size_t)row * C);
  f4 v[MAXC4];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    const int c4 = lane + 64 * j;
    v[j] = c4 < C4 ? xr[c4] : f4{0.f, 0.f, 0.f, 0.f};
    s += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
  }
  const float mean = wavesum(s) / C;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    const int c4 = lane + 64 * j;
    if (c4 < C4) {
      const f4 d = v[j] - mean;
      q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
  }
  const float rstd = 1.0f / sqrtf(wavesum(q) / C + LN_EPS);
  f4* yr = reinterpret_cast<f4*>(y + (size_t)row * C);
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    const int c4 = lane + 64 * j;
    if (c4 < C4)
      yr[c4] = (v[j] - mean) * rstd * reinterpret_cast<const f4*>(w)[c4] +
               reinterpret_cast<const f4*>(b)[c4];
  }
  if (lane == 0) {
    if (mean_out) mean_out[row] = mean;
    if (rstd_out) rstd_out[row] = rstd;
  }
}

// sh = x + (prev - x) mu, prev = x[t-1] (x_prev or 0 at t = 0); x_last = x[T-1].
// x_last may alias x_prev only when T == 1 (same thread reads then writes).
__global__ __launch_bounds__(256) void cm_shift(int BT, int T, int C, const float* __restrict__ x,
                                                const float* x_prev, const float* __restrict__ mu,
                                                float* __restrict__ sh, float* x_last) {
  const size_t n4 = (size_t)BT * C / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t e = i * 4;
    const size_t bt = e / C;
    const int c = (int)(e - bt * C);
    const int t = (int)(bt % T);
    const f4 xv = *reinterpret_cast<const f4*>(x + e);
    f4 prev = {0.f, 0.f, 0.f, 0.f};
    if (t > 0) prev = *reinterpret_cast<const f4*>(x + e - C);
    else if (x_prev) prev = *reinterpret_cast<const f4*>(x_prev + (bt / T) * C + c);
    *reinterpret_cast<f4*>(sh + e) = xv + (prev - xv) * *reinterpret_cast<const f4*>(mu + c);
    if (x_last && t == T - 1) *reinterpret_cast<f4*>(x_last + (bt / T) * C + c) = xv;
  }
}

}  // namespace stk

static unsigned grid_for(size_t n4) {
  size_t b = (n4 + 255) / 256;
  return (unsigned)(b > 8192 ? 8192 : (b < 1 ? 1 : b));
}

hipError_t stk_launch_emb_gather(int R, int C, int V, const int* tok, const float* emb, float* out,
                                 hipStream_t st) {
  hipLaunchKernelGGL(stk::emb_gather, dim3(grid_for((size_t)R * C / 4)), dim3(256), 0, st, R, C, V,
                     tok, emb, out);
  return hipGetLastError();
}
hipError_t stk_launch_layernorm(int R, int C, const float* x, const float* w, const float* b,
                                float* y, float* mean, float* rstd, hipStream_t st) {
  hipLaunchKernelGGL(stk::layernorm_fwd, dim3((R + 3) / 4), dim3(256), 0, st, R, C, x, w, b, y,
                     mean, rstd);
  return hipGetLastError();
}
hipError_t stk_launch_cm_shift(int BT, int T, int C, const float* x, const float* x_prev,
                               const float* mu, float* sh, float* x_last, hipStream_t st) {
  hipLaunchKernelGGL(stk::cm_shift, dim3(grid_for((size_t)BT * C / 4)), dim3(256), 0, st, BT, T, C,
                     x, x_prev, mu, sh, x_last);
  return hipGetLastError();
}
int stk_max_layernorm_width() { return 64 * 4 * stk::MAXC4; }
