// Matrix-core GEMM (gemm.hip): problem descriptors and launchers.  Operands
// and results are fp32 in memory; the products run either in fp32
// (v_mfma_f32_16x16x4_f32) or with bf16-rounded operands and fp32
// accumulation (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_16x16x32_bf16).
#pragma once
#include <hip/hip_runtime.h>

enum GemmEpi {
  EPI_NONE = 0, EPI_TANH = 1, EPI_SIGMOID = 2, EPI_TANH_BWD = 3, EPI_SIG_BWD = 4, EPI_SQRELU = 5,
  EPI_SQRELU_BWD = 6,  // acc * 2 relu(f) with aux = relu(f)^2 (so relu(f) = sqrt(aux))
  EPI_ADD = 7          // acc + aux (a residual from another buffer, same leading dimension)
};

constexpr int GEMM_MAX_BATCH = 8;

enum GemmPrec { GEMM_F32 = 0, GEMM_BF16 = 1 };

// C = epi(op(A) op(B) + beta C); aux (same layout as C) feeds the *_BWD epilogues.
struct GemmProblem {
  int M, N, K;
  const float* A;
  int lda;
  const float* B;
  int ldb;
  float* C;
  int ldc;
  float beta;
  int epi;
  const float* aux;
  float* part;  // split-K partials (internal)
  // optional bf16 copy of the result (dense [M][N], rounded to nearest even),
  // written by every path, for a later product that takes it as its A
  __bf16* C16 = nullptr;
  // optional A already rounded to bf16 (dense [M][K], e.g. an earlier C16):
  // the bf16 matrix-core path then uses it instead of making its own copy
  const __bf16* A16 = nullptr;
};

struct GemmBatch {
  int count;
  GemmProblem p[GEMM_MAX_BATCH];
};

// Up to GEMM_MAX_BATCH independent problems of one layout in one launch.
hipError_t gemm_batch(int prec, bool transA, bool transB, const GemmBatch& b, hipStream_t st);
// One problem, optionally split along K into `split` slices (ws: split*M*N floats).
// Split-K slices gemm_run uses for this shape (it takes the smaller of this
// and the split it is given, which is what its workspace holds).
int gemm_splitk_slices(int prec, int M, int N, int K);
hipError_t gemm_run(int prec, bool transA, bool transB, int M, int N, int K, const float* A,
                    int lda, const float* B, int ldb, float* C, int ldc, float beta, int epi,
                    const float* aux, int split, float* ws, hipStream_t st);
// gemm_run with the optional bf16 operand A16 and result copy C16 (see
// GemmProblem); NULL for either is gemm_run.
hipError_t gemm_run_x(int prec, bool transA, bool transB, int M, int N, int K, const float* A,
                      int lda, const float* B, int ldb, float* C, int ldc, float beta, int epi,
                      const float* aux, int split, float* ws, hipStream_t st, const __bf16* A16,
                      __bf16* C16);
// The split-K products alone: part[s][M][N] (leading dimension N), K cut
// into *slices <= split slices of a multiple of 64 (at least 64 each), left
// for the consumer to add in slice order (no beta, no epilogue).
hipError_t gemm_run_partials(int prec, int M, int N, int K, const float* A, int lda,
                             const float* B, int ldb, int split, float* part, int* slices,
                             hipStream_t st);

// bf16 operand copies.  A bf16 problem that the direct-to-LDS kernel takes
// (M a multiple of 256, N of 128, K of 64), and that is not X^T dY, rounds
// its operands to bf16 once into an arena, stored k-contiguous, and
// multiplies them with no conversion in the loop, when the calling thread
// has set an arena large enough for the whole launch (the sum of
// gemm_pack_need over its problems).  The arena belongs to the caller's
// workspace; the setting lasts until it is cleared (GemmPackScope), and the
// GEMMs that use it must run one after another on one stream.
size_t gemm_pack_need(int M, int N, int K);  // bytes, 0 when the shape does not qualify
// the same when A comes already rounded (GemmProblem::A16): B's copy alone
size_t gemm_pack_need_b(int M, int N, int K);
void gemm_set_pack_arena(void* p, size_t bytes);
struct GemmPackScope {
  GemmPackScope(void* p, size_t bytes) { gemm_set_pack_arena(p, bytes); }
  ~GemmPackScope() { gemm_set_pack_arena(nullptr, 0); }
  GemmPackScope(const GemmPackScope&) = delete;
  GemmPackScope& operator=(const GemmPackScope&) = delete;
};

inline hipError_t gemm_f32_batch(bool transA, bool transB, const GemmBatch& b, hipStream_t st) {
  return gemm_batch(GEMM_F32, transA, transB, b, st);
}
inline hipError_t gemm_f32_run(bool transA, bool transB, int M, int N, int K, const float* A,
                               int lda, const float* B, int ldb, float* C, int ldc, float beta,
                               int epi, const float* aux, int split, float* ws, hipStream_t st) {
  return gemm_run(GEMM_F32, transA, transB, M, N, K, A, lda, B, ldb, C, ldc, beta, epi, aux, split,
                  ws, st);
}
