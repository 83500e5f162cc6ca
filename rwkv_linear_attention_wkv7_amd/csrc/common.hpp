// Shared device helpers for the gfx950 (CDNA4, wave64) kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define WKV7_N 64  // head size; the kernels are written for N = 64 only
#define WKV7_CKL 16  // checkpoint interval of the WKV7 forward (tokens)

// The WKV7 checkpoint buffer: the state after every WKV7_CKL tokens,
// [B][H][ceil(T/CKL)][N][N], then the forward's per-token sa = S a_t (old
// state), [B][T][H][N]; all fp32.
__host__ __device__ inline size_t wkv7_ckpt_state_floats(int B, int T, int H) {
  return (size_t)B * H * ((T + WKV7_CKL - 1) / WKV7_CKL) * WKV7_N * WKV7_N;
}
__host__ __device__ inline size_t wkv7_ckpt_total_floats(int B, int T, int H) {
  return wkv7_ckpt_state_floats(B, T, H) + (size_t)B * T * H * WKV7_N;
}
__host__ __device__ inline float* wkv7_ckpt_sa(float* ckpt, int B, int T, int H) {
  return ckpt + wkv7_ckpt_state_floats(B, T, H);
}
__host__ __device__ inline const float* wkv7_ckpt_sa(const float* ckpt, int B, int T, int H) {
  return ckpt + wkv7_ckpt_state_floats(B, T, H);
}

typedef float f4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 ----
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// round to nearest, ties to even (inputs here are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Load 4 consecutive elements (16-byte aligned for fp32, 8-byte for bf16) as fp32.
template <typename T>
__device__ __forceinline__ f4 load4(const T* p);
template <>
__device__ __forceinline__ f4 load4<float>(const float* p) {
  return *reinterpret_cast<const f4*>(p);
}
template <>
__device__ __forceinline__ f4 load4<bf16_t>(const bf16_t* p) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  f4 r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xFFFF0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xFFFF0000u);
  return r;
}

// Raw (unconverted) 4-element and 1-element storage types, used to stage data
// through registers and LDS without converting it on the way.
template <typename T>
struct Raw;
template <>
struct Raw<float> {
  typedef f4 v4;
  typedef float v1;
};
template <>
struct Raw<bf16_t> {
  typedef uint2 v4;
  typedef uint16_t v1;
};
template <typename T>
__device__ __forceinline__ typename Raw<T>::v4 load_raw4(const T* p) {
  return *reinterpret_cast<const typename Raw<T>::v4*>(p);
}
template <typename T>
__device__ __forceinline__ void store_raw4(T* p, typename Raw<T>::v4 x) {
  *reinterpret_cast<typename Raw<T>::v4*>(p) = x;
}
template <typename T>
__device__ __forceinline__ typename Raw<T>::v1 load_raw1(const T* p) {
  return *reinterpret_cast<const typename Raw<T>::v1*>(p);
}
template <typename T>
__device__ __forceinline__ void store_raw1(T* p, typename Raw<T>::v1 x) {
  *reinterpret_cast<typename Raw<T>::v1*>(p) = x;
}

// Raw 4-element value (see Raw) to fp32.
template <typename T>
__device__ __forceinline__ f4 raw4_to_f4(typename Raw<T>::v4 x);
template <>
__device__ __forceinline__ f4 raw4_to_f4<float>(f4 x) { return x; }
template <>
__device__ __forceinline__ f4 raw4_to_f4<bf16_t>(uint2 u) {
  return f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
            __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
}

template <typename T>
__device__ __forceinline__ float raw1_to_f32(typename Raw<T>::v1 x);
template <>
__device__ __forceinline__ float raw1_to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float raw1_to_f32<bf16_t>(uint16_t x) { return bf16_to_f32(x); }

template <typename T>
__device__ __forceinline__ float load1(const T* p);
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load1<bf16_t>(const bf16_t* p) { return bf16_to_f32(p->bits); }

template <typename T>
__device__ __forceinline__ void store4(T* p, f4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, f4 v) {
  *reinterpret_cast<f4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, f4 v) {
  uint2 u;
  u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

template <typename T>
__device__ __forceinline__ void store1(T* p, float v);
template <>
__device__ __forceinline__ void store1<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store1<bf16_t>(bf16_t* p, float v) { p->bits = f32_to_bf16(v); }

// ------------------------------------------------------ cross-lane sums ----
// Sum over the 16 lanes of a DPP row; every lane of the row receives the sum.
__device__ __forceinline__ float rowsum16(float x) {
  x += __builtin_amdgcn_update_dpp(0.0f, x, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0.0f, x, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_update_dpp(0.0f, x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  x += __builtin_amdgcn_update_dpp(0.0f, x, 0x140, 0xF, 0xF, true);  // row_mirror
  return x;
}

// Sum over lanes {l, l^16, l^32, l^48} (the four 16-lane rows of the wave);
// every lane receives the sum of its column position.  gfx950 permlane swaps.
__device__ __forceinline__ float rows4sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Reduce-scatter over the wave's four 16-lane rows.  On entry every lane holds
// 4*NQ values x[cc*NQ + q] (cc < 4 = its column within a float4, q < NQ);
// on exit lane l holds in x[q] (q < NQ) the sum over lanes {l, l^16, l^32, l^48}
// of the values with cc == l/16.  Two permlane-swap rounds, 3*NQ swap+add pairs.
template <int NQ>
__device__ __forceinline__ void rows4_reduce_scatter(float (&x)[4 * NQ]) {
  // stage 1: lanes 0-31 keep cc 0,1 (+ partner's), lanes 32-63 keep cc 2,3
#pragma unroll
  for (int i = 0; i < 2 * NQ; i++) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]), __float_as_uint(x[i + 2 * NQ]),
                                              false, false);
    x[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  // stage 2: within each half, even rows keep the first cc, odd rows the second
#pragma unroll
  for (int i = 0; i < NQ; i++) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]), __float_as_uint(x[i + NQ]),
                                              false, false);
    x[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
}

// Full 64-lane wave sum, result in every lane.
__device__ __forceinline__ float wavesum(float x) { return rows4sum(rowsum16(x)); }

// ------------------------------------------------------------- barrier ----
// Workgroup barrier for LDS traffic only: this wave's LDS operations complete
// (lgkmcnt(0)), then s_barrier; the clobber keeps the compiler from moving
// memory accesses across it.  Unlike __syncthreads() it does not wait for the
// wave's outstanding global loads and stores, so prefetches and result
// stores stay in flight across it.  Only for loops whose waves exchange data
// through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// --------------------------------------------------------------- launch ----
// Workgroups are dispatched round-robin over the 8 XCDs (block g -> XCD g % 8).
// Remap so that consecutive logical ids land on one XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int g, int n) {
  if (n & 7) return g;
  return (g & 7) * (n >> 3) + (g >> 3);
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }
