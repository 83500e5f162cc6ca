// fp32 GEMM on the gfx950 matrix cores (v_mfma_f32_16x16x4_f32).
//
//   C[M][N] = epilogue( op(A)[M][K] . op(B)[K][N] )
//
// Row-major storage.  op(A) = A ([M][K], lda) or A^T (A stored [K][M]);
// op(B) = B ([K][N], ldb) or B^T (B stored [N][K]).  These three layouts are
// all the time-mix block needs: X W (forward), dY W^T (input gradients) and
// X^T dY (weight gradients, reduction over the B*T tokens, split along K).
//
// Tiling: 256 threads = 2x2 waves; each wave owns TI x TJ tiles of 16x16, so
// the workgroup tile is (32 TI) x (32 TJ).  K advances in steps of BK = 32
// through LDS (k-major, rows padded by 16 floats so the four k-rows a wave
// reads land in disjoint bank groups); the next K tile is fetched into
// registers while the current one is multiplied.  Any M is allowed (rows are
// guarded); the dimensions read as float4 (K for A, N for B, or M/N for the
// transposed operands) must be multiples of 4.

#include "common.hpp"

namespace gemmk {

constexpr int BK = 32;
constexpr int PAD = 16;

enum Epi { EPI_NONE = 0, EPI_TANH = 1, EPI_SIGMOID = 2, EPI_TANH_BWD = 3, EPI_SIG_BWD = 4, EPI_SQRELU = 5 };

__device__ __forceinline__ float apply_epi(float acc, int epi, float aux) {
  switch (epi) {
    case EPI_TANH: return tanhf(acc);
    case EPI_SIGMOID: return 1.0f / (1.0f + expf(-acc));
    case EPI_TANH_BWD: return acc * (1.0f - aux * aux);  // aux = tanh(.) of the forward
    case EPI_SIG_BWD: return acc * aux * (1.0f - aux);   // aux = sigmoid(.) of the forward
    case EPI_SQRELU: return acc > 0.f ? acc * acc : 0.f;  // relu(.)^2
    default: return acc;
  }
}

template <int TI, int TJ, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f32(int M, int N, int K, const float* __restrict__ A,
                                                int lda, const float* __restrict__ B, int ldb,
                                                float* __restrict__ C, int ldc, int kslice,
                                                float beta, int epi, const float* __restrict__ aux) {
  constexpr int BM = 32 * TI, BN = 32 * TJ;
  constexpr int A4 = BM * BK / 4 / 256;  // float4 loads per thread for the A tile
  constexpr int B4 = BN * BK / 4 / 256;
  static_assert(A4 >= 1 && B4 >= 1, "tile too small for 256 threads");
  __shared__ float As[BK][BM + PAD];
  __shared__ float Bs[BK][BN + PAD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int kbeg = blockIdx.z * kslice;
  const int kend = min(K, kbeg + kslice);
  C += (size_t)blockIdx.z * M * ldc;  // split-K partials (z = 0 when not split)

  // Tile loads are unconditional from clamped (always valid) addresses, so a
  // whole tile is in flight at once; out-of-range elements are zeroed when the
  // registers are written to LDS.
  f4 ra[A4], rb[B4];
  unsigned oka = 0, okb = 0;

  auto load_tiles = [&](int k0) {
    oka = okb = 0;
#pragma unroll
    for (int q = 0; q < A4; q++) {
      const int idx = tid + 256 * q;
      if (!TA) {  // A[m][k], float4 along k
        const int row = idx / (BK / 4), k4 = idx % (BK / 4);
        const int m = m0 + row, k = k0 + k4 * 4;
        oka |= (unsigned)(m < M && k < kend) << q;
        ra[q] = *reinterpret_cast<const f4*>(A + (size_t)min(m, M - 1) * lda + min(k, kend - 4));
      } else {    // A stored [K][M], float4 along m
        const int kr = idx / (BM / 4), m4 = idx % (BM / 4);
        const int k = k0 + kr, m = m0 + m4 * 4;
        oka |= (unsigned)(k < kend && m < M) << q;
        ra[q] = *reinterpret_cast<const f4*>(A + (size_t)min(k, kend - 1) * lda + min(m, M - 4));
      }
    }
#pragma unroll
    for (int q = 0; q < B4; q++) {
      const int idx = tid + 256 * q;
      if (!TB) {  // B[k][n], float4 along n
        const int kr = idx / (BN / 4), n4 = idx % (BN / 4);
        const int k = k0 + kr, n = n0 + n4 * 4;
        okb |= (unsigned)(k < kend && n < N) << q;
        rb[q] = *reinterpret_cast<const f4*>(B + (size_t)min(k, kend - 1) * ldb + min(n, N - 4));
      } else {    // B stored [N][K], float4 along k
        const int row = idx / (BK / 4), k4 = idx % (BK / 4);
        const int n = n0 + row, k = k0 + k4 * 4;
        okb |= (unsigned)(n < N && k < kend) << q;
        rb[q] = *reinterpret_cast<const f4*>(B + (size_t)min(n, N - 1) * ldb + min(k, kend - 4));
      }
    }
  };
  auto store_tiles = [&]() {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < A4; q++) {
      const int idx = tid + 256 * q;
      const f4 x = (oka >> q) & 1u ? ra[q] : z;
      if (!TA) {
        const int row = idx / (BK / 4), k4 = idx % (BK / 4);
#pragma unroll
        for (int c = 0; c < 4; c++) As[k4 * 4 + c][row] = x[c];
      } else {
        const int kr = idx / (BM / 4), m4 = idx % (BM / 4);
        *reinterpret_cast<f4*>(&As[kr][m4 * 4]) = x;
      }
    }
#pragma unroll
    for (int q = 0; q < B4; q++) {
      const int idx = tid + 256 * q;
      const f4 x = (okb >> q) & 1u ? rb[q] : z;
      if (!TB) {
        const int kr = idx / (BN / 4), n4 = idx % (BN / 4);
        *reinterpret_cast<f4*>(&Bs[kr][n4 * 4]) = x;
      } else {
        const int row = idx / (BK / 4), k4 = idx % (BK / 4);
#pragma unroll
        for (int c = 0; c < 4; c++) Bs[k4 * 4 + c][row] = x[c];
      }
    }
  };

  f4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fk = lane >> 4;
  if (kbeg < kend) load_tiles(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (k0 + BK < kend) load_tiles(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
      float fa[TI], fb[TJ];
#pragma unroll
      for (int i = 0; i < TI; i++) fa[i] = As[kk + fk][wm * 16 * TI + i * 16 + fr];
#pragma unroll
      for (int j = 0; j < TJ; j++) fb[j] = Bs[kk + fk][wn * 16 * TJ + j * 16 + fr];
#pragma unroll
      for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

  // D layout of v_mfma_f32_16x16x4_f32: lane l, element v -> row 4*(l/16)+v, col l%16
#pragma unroll
  for (int i = 0; i < TI; i++) {
#pragma unroll
    for (int j = 0; j < TJ; j++) {
      const int col = n0 + wn * 16 * TJ + j * 16 + fr;
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int row = m0 + wm * 16 * TI + i * 16 + fk * 4 + v;
        if (row >= M) continue;
        const size_t o = (size_t)row * ldc + col;
        float x = acc[i][j][v];
        if (beta != 0.f) x += beta * C[o];
        x = apply_epi(x, epi, aux ? aux[o] : 0.f);
        C[o] = x;
      }
    }
  }
}

// Sum S split-K partials [S][M][N] (leading dim N) into C (ldc), with beta/epilogue.
__global__ __launch_bounds__(256) void splitk_reduce(int M, int N, int S, const float* __restrict__ P,
                                                     float* __restrict__ C, int ldc, float beta,
                                                     int epi, const float* __restrict__ aux) {
  const size_t n4 = (size_t)M * N / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    f4 s = reinterpret_cast<const f4*>(P)[i];
    for (int z = 1; z < S; z++) s += reinterpret_cast<const f4*>(P + (size_t)z * M * N)[i];
    const size_t e = i * 4;
    const int row = (int)(e / N), col = (int)(e % N);
    const size_t o = (size_t)row * ldc + col;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      float x = s[c];
      if (beta != 0.f) x += beta * C[o + c];
      C[o + c] = apply_epi(x, epi, aux ? aux[o + c] : 0.f);
    }
  }
}

template <int TI, int TJ, bool TA, bool TB>
hipError_t launch_t(int M, int N, int K, const float* A, int lda, const float* B, int ldb, float* C,
                    int ldc, int S, int kslice, float beta, int epi, const float* aux,
                    hipStream_t st) {
  dim3 grid((N + 32 * TJ - 1) / (32 * TJ), (M + 32 * TI - 1) / (32 * TI), S);
  hipLaunchKernelGGL((gemm_f32<TI, TJ, TA, TB>), grid, dim3(256), 0, st, M, N, K, A, lda, B, ldb,
                     C, ldc, kslice, beta, epi, aux);
  return hipGetLastError();
}

template <bool TA, bool TB>
hipError_t launch_layout(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                         float* C, int ldc, int S, int kslice, float beta, int epi,
                         const float* aux, hipStream_t st) {
  // Largest tile whose grid still gives every CU work (>= 256 workgroups),
  // else the smallest tile.
  auto blocks = [&](int bm, int bn) { return (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn) * S; };
  if (blocks(128, 128) >= 256 && N >= 128)
    return launch_t<4, 4, TA, TB>(M, N, K, A, lda, B, ldb, C, ldc, S, kslice, beta, epi, aux, st);
  if (blocks(128, 64) >= 256 && N >= 64)
    return launch_t<4, 2, TA, TB>(M, N, K, A, lda, B, ldb, C, ldc, S, kslice, beta, epi, aux, st);
  if (blocks(64, 64) >= 256 && N >= 64)
    return launch_t<2, 2, TA, TB>(M, N, K, A, lda, B, ldb, C, ldc, S, kslice, beta, epi, aux, st);
  if (blocks(64, 32) >= 256)
    return launch_t<2, 1, TA, TB>(M, N, K, A, lda, B, ldb, C, ldc, S, kslice, beta, epi, aux, st);
  return launch_t<1, 1, TA, TB>(M, N, K, A, lda, B, ldb, C, ldc, S, kslice, beta, epi, aux, st);
}

}  // namespace gemmk

// C = epi(op(A) op(B) + beta C).  ws (may be NULL when split == 1) holds
// split*M*N floats of split-K partials.
hipError_t gemm_f32_run(bool transA, bool transB, int M, int N, int K, const float* A, int lda,
                        const float* B, int ldb, float* C, int ldc, float beta, int epi,
                        const float* aux, int split, float* ws, hipStream_t st) {
  using namespace gemmk;
  if (M <= 0 || N <= 0) return hipSuccess;
  if (split <= 1 || ws == nullptr) {
    const int ks = K;
    if (!transA && !transB) return launch_layout<false, false>(M, N, K, A, lda, B, ldb, C, ldc, 1, ks, beta, epi, aux, st);
    if (!transA && transB) return launch_layout<false, true>(M, N, K, A, lda, B, ldb, C, ldc, 1, ks, beta, epi, aux, st);
    if (transA && !transB) return launch_layout<true, false>(M, N, K, A, lda, B, ldb, C, ldc, 1, ks, beta, epi, aux, st);
    return launch_layout<true, true>(M, N, K, A, lda, B, ldb, C, ldc, 1, ks, beta, epi, aux, st);
  }
  int kslice = (K + split - 1) / split;
  kslice = (kslice + BK - 1) / BK * BK;
  const int S = (K + kslice - 1) / kslice;
  hipError_t e;
  if (!transA && !transB) e = launch_layout<false, false>(M, N, K, A, lda, B, ldb, ws, N, S, kslice, 0.f, EPI_NONE, nullptr, st);
  else if (!transA && transB) e = launch_layout<false, true>(M, N, K, A, lda, B, ldb, ws, N, S, kslice, 0.f, EPI_NONE, nullptr, st);
  else if (transA && !transB) e = launch_layout<true, false>(M, N, K, A, lda, B, ldb, ws, N, S, kslice, 0.f, EPI_NONE, nullptr, st);
  else e = launch_layout<true, true>(M, N, K, A, lda, B, ldb, ws, N, S, kslice, 0.f, EPI_NONE, nullptr, st);
  if (e != hipSuccess) return e;
  const size_t n4 = (size_t)M * N / 4;
  int blocks = (int)((n4 + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(splitk_reduce, dim3(blocks), dim3(256), 0, st, M, N, S, ws, C, ldc, beta, epi, aux);
  return hipGetLastError();
}
