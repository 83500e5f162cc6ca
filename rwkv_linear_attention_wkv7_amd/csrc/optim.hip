// Parameter updates of the online training segment (SGD and Adam), applied
// to many tensors per launch: a launch takes up to OPT_MAX tensors by value,
// blockIdx.y selects the tensor and the workgroups of blockIdx.x stride over
// its elements (float4; every parameter tensor of the stack has a multiple
// of 4 elements).  Page: "infotheory .../rwkvzip/rwkv7/model.rs",
// apply_full_gradients and AdamStep (b1 = 0.9, b2 = 0.999, eps = 1e-8, bias
// corrections 1 - b^t).  clip > 0 clamps every gradient element to
// [-clip, clip] first; Adam: m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
// p -= lr (m / bc1) / (sqrt(v / bc2) + eps).

#include "common.hpp"
#include "optim.hpp"

namespace optk {

__device__ __forceinline__ float clipf(float g, float c) { return c > 0.f ? fminf(fmaxf(g, -c), c) : g; }

__global__ __launch_bounds__(256) void sgd(OptBatch t, float lr, float clip) {
  const int k = blockIdx.y;
  const size_t n4 = t.count[k] / 4;
  f4* p = reinterpret_cast<f4*>(t.p[k]);
  const f4* g = reinterpret_cast<const f4*>(t.g[k]);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const f4 gv = g[i];
    f4 pv = p[i];
#pragma unroll
    for (int c = 0; c < 4; c++) pv[c] -= lr * clipf(gv[c], clip);
    p[i] = pv;
  }
}

__global__ __launch_bounds__(256) void adam(OptBatch t, float lr, float clip, float b1, float b2,
                                            float eps, float inv_bc1, float inv_bc2) {
  const int k = blockIdx.y;
  const size_t n4 = t.count[k] / 4;
  f4* p = reinterpret_cast<f4*>(t.p[k]);
  const f4* g = reinterpret_cast<const f4*>(t.g[k]);
  f4* m = reinterpret_cast<f4*>(t.m[k]);
  f4* v = reinterpret_cast<f4*>(t.v[k]);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const f4 gv = g[i];
    f4 pv = p[i], mv = m[i], vv = v[i];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const float gc = clipf(gv[c], clip);
      mv[c] = b1 * mv[c] + (1.0f - b1) * gc;
      vv[c] = b2 * vv[c] + (1.0f - b2) * gc * gc;
      pv[c] -= lr * (mv[c] * inv_bc1) / (sqrtf(vv[c] * inv_bc2) + eps);
    }
    p[i] = pv;
    m[i] = mv;
    v[i] = vv;
  }
}

}  // namespace optk

hipError_t opt_launch(const OptBatch& t, int adam, float lr, float clip, int step, hipStream_t st) {
  if (t.n < 1) return hipSuccess;
  size_t most = 0;
  for (int k = 0; k < t.n; k++) most = t.count[k] > most ? t.count[k] : most;
  size_t bx = (most / 4 + 255) / 256;
  bx = bx < 1 ? 1 : (bx > 1024 ? 1024 : bx);
  const dim3 grid((unsigned)bx, (unsigned)t.n);
  if (adam) {
    const double b1 = 0.9, b2 = 0.999;
    const double bc1 = 1.0 - __builtin_pow(b1, step), bc2 = 1.0 - __builtin_pow(b2, step);
    hipLaunchKernelGGL(optk::adam, grid, dim3(256), 0, st, t, lr, clip, (float)b1, (float)b2, 1e-8f,
                       (float)(1.0 / bc1), (float)(1.0 / bc2));
  } else {
    hipLaunchKernelGGL(optk::sgd, grid, dim3(256), 0, st, t, lr, clip);
  }
  return hipGetLastError();
}
