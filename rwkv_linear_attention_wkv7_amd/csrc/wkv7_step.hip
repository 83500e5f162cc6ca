// WKV7 single-token decode step on gfx950 (C-ABI wkv7_step).
//
// The recurrence of the WKV7 kernel on the "Foundry/cuda_kernels/timemix.cu"
// page (composites a = -kk, b = kk*a) for T = 1 with the state updated in
// place: per (b, h), S[i][j] (i value row, j key column),
//     sa = S a ;  S = S diag(w) + sa b^T + v k^T ;  y = S r
// as the streaming state of "infotheory .../rwkv7/model.rs" (att_state per
// layer) is advanced one token.  Bound by HBM: 32 KiB of fp32 state is read
// and written per (b, h) against 9 N^2 flop.

#include "common.hpp"

namespace wkv7k {

constexpr int N = WKV7_N;

// Decode step, bandwidth bound (32 KiB of state per (b,h)).  One workgroup of
// 256 threads per (b,h); thread owns rows rg + 16m (m < 4) x columns 4cg..4cg+3,
// so each load instruction of a wave covers 4 consecutive rows (1 KiB).
template <typename T>
__global__ __launch_bounds__(256) void step_kernel(
    int BH, const T* __restrict__ r, const T* __restrict__ w, const T* __restrict__ k,
    const T* __restrict__ v, const T* __restrict__ a, const T* __restrict__ bv,
    float* __restrict__ state, T* __restrict__ y) {
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x, cg = tid & 15, rg = tid >> 4;
  const size_t vb = (size_t)bh * N;
  float* st = state + (size_t)bh * N * N;
  f4 S[4];
#pragma unroll
  for (int m = 0; m < 4; m++)
    S[m] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(st + (size_t)(rg + 16 * m) * N + cg * 4));
  const f4 av = load4(a + vb + cg * 4), wv = load4(w + vb + cg * 4), kv = load4(k + vb + cg * 4);
  const f4 bb = load4(bv + vb + cg * 4), rv = load4(r + vb + cg * 4);
  float vv[4];
#pragma unroll
  for (int m = 0; m < 4; m++) vv[m] = load1(v + vb + rg + 16 * m);
  float sa[4];
#pragma unroll
  for (int m = 0; m < 4; m++)
    sa[m] = fmaf(S[m][3], av[3], fmaf(S[m][2], av[2], fmaf(S[m][1], av[1], S[m][0] * av[0])));
#pragma unroll
  for (int m = 0; m < 4; m++) sa[m] = rowsum16(sa[m]);
  float yo[4];
#pragma unroll
  for (int m = 0; m < 4; m++) {
#pragma unroll
    for (int c = 0; c < 4; c++) S[m][c] = fmaf(vv[m], kv[c], fmaf(sa[m], bb[c], S[m][c] * wv[c]));
    yo[m] = fmaf(S[m][3], rv[3], fmaf(S[m][2], rv[2], fmaf(S[m][1], rv[1], S[m][0] * rv[0])));
  }
#pragma unroll
  for (int m = 0; m < 4; m++) yo[m] = rowsum16(yo[m]);
#pragma unroll
  for (int m = 0; m < 4; m++)
    __builtin_nontemporal_store(S[m], reinterpret_cast<f4*>(st + (size_t)(rg + 16 * m) * N + cg * 4));
  if (cg < 4) {
    float o = yo[0];
#pragma unroll
    for (int m = 1; m < 4; m++)
      if (cg == m) o = yo[m];
    store1(y + vb + rg + 16 * cg, o);
  }
}

template <typename T>
hipError_t launch_step_t(int B, int H, const void* r, const void* w, const void* k, const void* v,
                         const void* a, const void* b, float* state, void* y, hipStream_t st) {
  hipLaunchKernelGGL((step_kernel<T>), dim3(B * H), dim3(256), 0, st, B * H, (const T*)r,
                     (const T*)w, (const T*)k, (const T*)v, (const T*)a, (const T*)b, state, (T*)y);
  return hipGetLastError();
}

}  // namespace wkv7k

hipError_t wkv7_launch_step(int dtype, int B, int H, const void* r, const void* w, const void* k,
                            const void* v, const void* a, const void* b, float* state, void* y,
                            hipStream_t st) {
  if (dtype == 1) return wkv7k::launch_step_t<bf16_t>(B, H, r, w, k, v, a, b, state, y, st);
  return wkv7k::launch_step_t<float>(B, H, r, w, k, v, a, b, state, y, st);
}
