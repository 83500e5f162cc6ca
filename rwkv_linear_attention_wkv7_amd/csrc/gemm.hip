// fp32 GEMM on the gfx950 matrix cores (v_mfma_f32_16x16x4_f32).
//
//   C[M][N] = epilogue( op(A)[M][K] . op(B)[K][N] + beta C )
//
// Row-major storage.  op(A) = A ([M][K], lda) or A^T (A stored [K][M]);
// op(B) = B ([K][N], ldb) or B^T (B stored [N][K]).  These three layouts are
// all the time-mix block needs: X W (forward), dY W^T (input gradients) and
// X^T dY (weight gradients, reduction over the B*T tokens, split along K).
// This is the contraction the timemix page runs through cuBLAS SGEMM over the
// whole [B*T, *] token batch (rm_gemm).
//
// Tiling: 256 threads = 2x2 waves; each wave owns TI x TJ tiles of 16x16, so
// the workgroup tile is (32 TI) x (32 TJ).  K advances in steps of BK through
// LDS; the next K tile is fetched into registers while the current one is
// multiplied.  Each operand keeps its global orientation in LDS (so every LDS
// store is a 16-byte row segment) with rows padded by 4 floats.  Inside each
// group of 16 k the MFMA steps take k in the order 4g + s (g = lane/16 the
// MFMA k-lane, s = step): the sum is unchanged, and a lane then finds its k
// values of the four steps next to each other, so a row-major operand yields
// its fragments for four MFMAs in one 16-byte LDS read.  Deep K tiles (BK up
// to 128) keep small-tile launches from paying one global round trip per 32 k.  A launch may carry
// up to eight independent problems of the same layout (blockIdx.z selects the
// problem; workgroups outside a smaller problem's grid exit), or one problem
// split along K (blockIdx.z selects the slice, partials summed by
// splitk_reduce).  Any M is allowed; the dimensions read as float4 must be
// multiples of 4.

#include "common.hpp"
#include "gemm.hpp"

namespace gemmk {

constexpr int PAD = 4;  // floats of padding per LDS row

__device__ __forceinline__ float apply_epi(float acc, int epi, float aux) {
  switch (epi) {
    case EPI_TANH: return tanhf(acc);
    case EPI_SIGMOID: return 1.0f / (1.0f + expf(-acc));
    case EPI_TANH_BWD: return acc * (1.0f - aux * aux);  // aux = tanh(.) of the forward
    case EPI_SIG_BWD: return acc * aux * (1.0f - aux);   // aux = sigmoid(.) of the forward
    case EPI_SQRELU: return acc > 0.f ? acc * acc : 0.f;  // relu(.)^2
    case EPI_SQRELU_BWD: return acc * 2.0f * sqrtf(aux);  // aux = relu(f)^2 of the forward
    case EPI_ADD: return acc + aux;
    default: return acc;
  }
}

// Write a wave's TI x TJ accumulator tiles with beta and the epilogue.  D
// layout of both 16x16 MFMAs used here: lane l, element v -> row 4*(l/16)+v,
// column l%16.
template <int TI, int TJ>
__device__ __forceinline__ void store_acc(const GemmProblem& P, bool split, float* __restrict__ C,
                                          int ldc, int m0, int n0, int wm, int wn, int lane,
                                          const f4 (&acc)[TI][TJ]) {
  const int M = P.M, N = P.N, fr = lane & 15, fk = lane >> 4;
  const float beta = split ? 0.f : P.beta;
  const int epi = split ? EPI_NONE : P.epi;
  const float* __restrict__ aux = split ? nullptr : P.aux;
  __bf16* __restrict__ c16 = split ? nullptr : P.C16;
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
        x = apply_epi(x, epi, aux ? aux[(size_t)row * P.ldc + col] : 0.f);
        C[o] = x;
        if (c16) c16[(size_t)row * N + col] = (__bf16)x;
      }
    }
  }
}

// Output tile of this workgroup.  Workgroups go round-robin over the 8 XCDs;
// xcd_remap hands each XCD a contiguous range of logical tile ids, and the
// logical order walks groups of 8 tile rows column by column, so the A row
// panels of a group stay in the XCD's L2 while the B column panels stream
// past once per group.
__device__ __forceinline__ void tile_origin(int BM, int BN, int& m0, int& n0) {
  const int gx = gridDim.x, gy = gridDim.y;
  const int lin = xcd_remap(blockIdx.y * gx + blockIdx.x, gx * gy);
  const int per_group = 8 * gx, gid = lin / per_group, first = gid * 8;
  const int gsz = min(8, gy - first), local = lin - gid * per_group;
  m0 = (first + local % gsz) * BM;
  n0 = (local / gsz) * BN;
}

template <int TI, int TJ, int BK, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f32(GemmBatch batch, int kslice) {
  constexpr int BM = 32 * TI, BN = 32 * TJ;
  constexpr int A4 = BM * BK / 4 / 256;  // float4 loads per thread for the A tile
  constexpr int B4 = BN * BK / 4 / 256;
  static_assert(A4 >= 1 && B4 >= 1, "tile too small for 256 threads");
  static_assert(A4 <= 32 && B4 <= 32, "load masks are 32 bits");
  static_assert(BK % 16 == 0, "K tiles are whole groups of 16");
  // A: [m][k] when A is row-major [M][K], [k][m] when stored [K][M]
  // B: [k][n] when row-major [K][N],      [n][k] when stored [N][K]
  __shared__ __attribute__((aligned(16))) float As[TA ? BK : BM][(TA ? BM : BK) + PAD];
  __shared__ __attribute__((aligned(16))) float Bs[TB ? BN : BK][(TB ? BK : BN) + PAD];

  const bool split = batch.count == 1 && gridDim.z > 1;
  const GemmProblem& P = batch.p[split ? 0 : blockIdx.z];
  const int M = P.M, N = P.N, K = P.K, lda = P.lda, ldb = P.ldb;
  int m0, n0;
  tile_origin(BM, BN, m0, n0);
  if (m0 >= M || n0 >= N) return;  // outside this problem's grid (uniform per workgroup)
  const float* __restrict__ A = P.A;
  const float* __restrict__ B = P.B;
  float* __restrict__ C = P.C;
  const int ldc = split ? N : P.ldc;
  const int kbeg = split ? blockIdx.z * kslice : 0;
  const int kend = split ? min(K, kbeg + kslice) : K;
  if (split) C = P.part + (size_t)blockIdx.z * M * N;  // split-K partials, leading dim N

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

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
        *reinterpret_cast<f4*>(&As[row][k4 * 4]) = x;
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
        *reinterpret_cast<f4*>(&Bs[row][k4 * 4]) = x;
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
    const int klen = min(BK, kend - k0);  // zero-padded beyond klen; skip empty groups
#pragma unroll
    for (int kq = 0; kq < BK; kq += 16) {
      if (kq < klen) {
        const int kb = kq + fk * 4;  // this lane's four k of the group: kb + s, s = step
        f4 fa[TI], fb[TJ];
#pragma unroll
        for (int i = 0; i < TI; i++) {
          const int mr = wm * 16 * TI + i * 16 + fr;
          if (!TA) fa[i] = *reinterpret_cast<const f4*>(&As[mr][kb]);
          else fa[i] = f4{As[kb][mr], As[kb + 1][mr], As[kb + 2][mr], As[kb + 3][mr]};
        }
#pragma unroll
        for (int j = 0; j < TJ; j++) {
          const int nc = wn * 16 * TJ + j * 16 + fr;
          if (TB) fb[j] = *reinterpret_cast<const f4*>(&Bs[nc][kb]);
          else fb[j] = f4{Bs[kb][nc], Bs[kb + 1][nc], Bs[kb + 2][nc], Bs[kb + 3][nc]};
        }
#pragma unroll
        for (int s4 = 0; s4 < 4; s4++)
#pragma unroll
          for (int i = 0; i < TI; i++)
#pragma unroll
            for (int j = 0; j < TJ; j++)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i][s4], fb[j][s4], acc[i][j], 0, 0, 0);
      }
    }
  }

  store_acc<TI, TJ>(P, split, C, ldc, m0, n0, wm, wn, lane, acc);
}

// ------------------------------------------------------------- bf16 path --
// Same tiling and epilogues with v_mfma_f32_16x16x32_bf16: operands are
// rounded to bf16 (round to nearest even, v_cvt_pk_bf16_f32) while they are
// staged into LDS; products accumulate in fp32.  Both operands are stored
// k-contiguous in LDS ([rows][BK + 8] bf16, rows padded by 16 bytes so the
// 16-byte fragment reads of 16 consecutive rows hit distinct banks): a lane's
// MFMA fragment is 8 consecutive k of one row, one 16-byte read.  An operand
// that is k-contiguous in memory is staged as 4-k row pieces (one float4
// load, one 8-byte store) with adjacent lanes on adjacent pieces, so a load
// instruction covers whole 128-byte row segments; a k-strided one is
// transposed inside each thread as 4 k x 4 rows blocks (four float4 loads,
// four 8-byte stores), with adjacent lanes on adjacent k so the stores hit
// distinct banks.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int BPAD = 8;  // bf16 of padding per LDS row

// One operand tile: R rows (of M or N) x BK k, staged global -> registers ->
// LDS.  KC: the operand is k-contiguous in memory (element (row, k) at
// base[row * ld + k]); else element (row, k) is at base[k * ld + row].
template <int R, int BK, bool KC>
struct BfTile {
  static constexpr int UNITS = KC ? R * BK / 4 : (BK / 4) * (R / 4);
  static constexpr int PER = (UNITS + 255) / 256;
  static constexpr int NF = KC ? 1 : 4;  // float4 loads per unit
  static_assert(PER * NF <= 32, "load masks are 32 bits");
  f4 reg[PER][NF];
  unsigned ok;

  // Element offsets of this thread's float4 loads relative to the tile
  // origin (row r0, k0): constant over the K loop, so an interior tile costs
  // one uniform base update per stage and no per-load address arithmetic.
  uint32_t off[PER][NF];
  __device__ __forceinline__ void init(int ld, int tid) {
#pragma unroll
    for (int q = 0; q < PER; q++) {
      const int u = min(tid + 256 * q, UNITS - 1);
      if (KC) {
        const int row = u / (BK / 4), k4 = u % (BK / 4);
        off[q][0] = (uint32_t)(row * ld + k4 * 4);
      } else {
        const int kq = u % (BK / 4), rg = u / (BK / 4);
#pragma unroll
        for (int s = 0; s < 4; s++) off[q][s] = (uint32_t)((kq * 4 + s) * ld + rg * 4);
      }
    }
  }
  // Interior tile (every element inside the matrix): plain loads, all valid.
  __device__ __forceinline__ void load_interior(const float* __restrict__ origin) {
    ok = ~0u;
#pragma unroll
    for (int q = 0; q < PER; q++)
#pragma unroll
      for (int s = 0; s < NF; s++) reg[q][s] = *reinterpret_cast<const f4*>(origin + off[q][s]);
  }

  // Unconditional loads from clamped (always valid) addresses; the mask
  // records which float4 are inside the matrix.
  __device__ __forceinline__ void load(const float* __restrict__ X, int ld, int r0, int rlim,
                                       int k0, int kend, int tid) {
    ok = 0;
#pragma unroll
    for (int q = 0; q < PER; q++) {
      const int u = min(tid + 256 * q, UNITS - 1);
      if (KC) {
        const int row = u / (BK / 4), k4 = u % (BK / 4);
        const int r = r0 + row, k = k0 + k4 * 4;
        ok |= (unsigned)(r < rlim && k < kend) << q;
        reg[q][0] = *reinterpret_cast<const f4*>(X + (size_t)min(r, rlim - 1) * ld + min(k, kend - 4));
      } else {
        const int kq = u % (BK / 4), rg = u / (BK / 4);
        const int r = r0 + rg * 4, k = k0 + kq * 4;
#pragma unroll
        for (int s = 0; s < 4; s++) {
          ok |= (unsigned)(r < rlim && k + s < kend) << (q * NF + s);
          reg[q][s] = *reinterpret_cast<const f4*>(X + (size_t)min(k + s, kend - 1) * ld +
                                                   min(r, rlim - 4));
        }
      }
    }
  }

  template <bool ALL>
  __device__ __forceinline__ void store(__bf16 (*Xs)[BK + BPAD], int tid) const {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < PER; q++) {
      const int u = tid + 256 * q;
      if (UNITS % 256 != 0 && u >= UNITS) continue;
      f4 x[NF];
#pragma unroll
      for (int s = 0; s < NF; s++) x[s] = ALL || ((ok >> (q * NF + s)) & 1u) ? reg[q][s] : z;
      if (KC) {
        const int row = u / (BK / 4), k4 = u % (BK / 4);
        *reinterpret_cast<bf16x4*>(&Xs[row][k4 * 4]) = __builtin_convertvector(x[0], bf16x4);
      } else {
        const int kq = u % (BK / 4), rg = u / (BK / 4);
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const f4 v = {x[0][c], x[1][c], x[2][c], x[3][c]};
          *reinterpret_cast<bf16x4*>(&Xs[rg * 4 + c][kq * 4]) = __builtin_convertvector(v, bf16x4);
        }
      }
    }
  }
};

template <int TI, int TJ, int BK, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_bf16(GemmBatch batch, int kslice) {
  constexpr int BM = 32 * TI, BN = 32 * TJ;
  static_assert(BK % 32 == 0, "K tiles are whole MFMA k steps");
  __shared__ __attribute__((aligned(16))) __bf16 As[2][BM][BK + BPAD];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[2][BN][BK + BPAD];

  const bool split = batch.count == 1 && gridDim.z > 1;
  const GemmProblem& P = batch.p[split ? 0 : blockIdx.z];
  const int M = P.M, N = P.N, K = P.K;
  int m0, n0;
  tile_origin(BM, BN, m0, n0);
  if (m0 >= M || n0 >= N) return;  // outside this problem's grid (uniform per workgroup)
  float* __restrict__ C = P.C;
  const int ldc = split ? N : P.ldc;
  const int kbeg = split ? blockIdx.z * kslice : 0;
  const int kend = split ? min(K, kbeg + kslice) : K;
  if (split) C = P.part + (size_t)blockIdx.z * M * N;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15, fk = lane >> 4;

  BfTile<BM, BK, !TA> ta;  // A[m][k] is k-contiguous unless A is stored [K][M]
  BfTile<BN, BK, TB> tb;   // B stored [N][K] is k-contiguous
  ta.init(P.lda, tid);
  tb.init(P.ldb, tid);
  const float* __restrict__ Ag = P.A;
  const float* __restrict__ Bg = P.B;
  // the M and N extent of this tile is inside the matrices (uniform)
  const bool in_mn = m0 + BM <= M && n0 + BN <= N;

  f4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  // stage k0 -> registers; returns whether every element was inside
  auto load = [&](int k0) -> bool {
    if (in_mn && k0 + BK <= kend) {
      ta.load_interior(TA ? Ag + (size_t)k0 * P.lda + m0 : Ag + (size_t)m0 * P.lda + k0);
      tb.load_interior(TB ? Bg + (size_t)n0 * P.ldb + k0 : Bg + (size_t)k0 * P.ldb + n0);
      return true;
    }
    ta.load(Ag, P.lda, m0, M, k0, kend, tid);
    tb.load(Bg, P.ldb, n0, N, k0, kend, tid);
    return false;
  };
  auto store = [&](bool all, int b) {
    if (all) {
      ta.template store<true>(As[b], tid);
      tb.template store<true>(Bs[b], tid);
    } else {
      ta.template store<false>(As[b], tid);
      tb.template store<false>(Bs[b], tid);
    }
  };

  if (kbeg < kend) store(load(kbeg), 0);
  __syncthreads();
  int buf = 0;
  for (int k0 = kbeg; k0 < kend; k0 += BK, buf ^= 1) {
    const bool more = k0 + BK < kend;
    bool all = true;
    if (more) all = load(k0 + BK);
    const int klen = kend - k0;  // zero-filled beyond klen; skip empty k steps
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      if (ks < klen) {
        bf16x8 fa[TI], fb[TJ];
#pragma unroll
        for (int i = 0; i < TI; i++)
          fa[i] = *reinterpret_cast<const bf16x8*>(&As[buf][wm * 16 * TI + i * 16 + fr][ks + fk * 8]);
#pragma unroll
        for (int j = 0; j < TJ; j++)
          fb[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][wn * 16 * TJ + j * 16 + fr][ks + fk * 8]);
#pragma unroll
        for (int i = 0; i < TI; i++)
#pragma unroll
          for (int j = 0; j < TJ; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
    // the other buffer was last read before the previous barrier
    if (more) store(all, buf ^ 1);
    __syncthreads();
  }

  store_acc<TI, TJ>(P, split, C, ldc, m0, n0, wm, wn, lane, acc);
}

// ------------------------------------------------------------------------
// bf16 matrix-core GEMM with the operands copied global -> LDS by the
// load unit itself (global_load_lds_dwordx4: no registers held while a
// load is in flight), for 256-row tiles whose M, N and K extents are whole
// tiles.  Each of the two LDS stages holds a 32-deep K slice of both
// operands as fp32; fragments are converted to bf16 as they are read.
// The multiply is v_mfma_f32_32x32x16_bf16, which keeps the matrix core
// busy with one wave per SIMD (the 16x16x32 form needs two).
//
// MFMA operands: lane l (i = l % 32, h = l / 32) gives row i of a 32-row
// fragment at 8 k values; in k-step s (16 k) of a stage, lane group h takes
// the k values 16s + 8h + (0..7) on both operands.  Result: lane l, value r
// is row (r & 3) + 8 (r >> 2) + 4 h, column i of the 32x32 block.
//
// LDS layouts (16-byte units "slots"):
//  * k-contiguous operand (KC): LDS row rho is 128 bytes (32 k), its 4-k
//    chunk c stored in slot c ^ key(rho), key(rho) = (rho & 7) ^
//    ((rho >> 3) & 1), so any 8 consecutive rows of a fragment read use 8
//    different 16-byte bank groups of a 128-byte bank row, and 16 rows fill
//    a 256-byte one (even rows take one half, odd rows the other).
//  * row-contiguous operand (stored [K][R]): k-row j holds the R floats in
//    order.  A lane reads 4 adjacent rows at one k with one 16-byte read;
//    those 4 rows feed 4 different fragments (fragment t of a wave takes
//    rows 4i + t, i = 0..31), so the output rows or columns of that side
//    come out interleaved and are put back in place by the store.
//  * The N side always uses the interleaved order (a KC B operand is copied
//    with its rows permuted to match: LDS row rho holds tile row
//    4 (rho % (R/4)) + rho / (R/4)), so each lane ends up holding 4
//    adjacent columns of C and the store is one float4.
// The copy instruction writes 64 consecutive slots (1 KB) per wave; each
// lane fetches the global 16 bytes that belong in its slot.
namespace dmak {

typedef __attribute__((address_space(3))) void lds_void;
typedef float f16v __attribute__((ext_vector_type(16)));
constexpr int BK = 32;  // k per stage

// One global_load_lds_dwordx4: lane i copies the 16 bytes at base + voff to
// LDS address lds + 16 i.  Issued as assembly so that the compiler neither
// tracks these writes to LDS nor adds waits for them: the kernel waits on
// vmcnt itself before the barrier that publishes a stage (the compiler's own
// vmcnt waits stay safe, since extra outstanding copies only make them
// stricter).  m0 holds the LDS address; nothing else here uses m0.  An
// SALU write of m0 needs one wait state before an LDS-DMA load reads it; the
// compiler inserts that nop for its own LDS-DMA but cannot see into this asm,
// so the s_nop is written here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16(const char* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One operand's copy plan: R tile rows, KC or row-contiguous, IL (KC only):
// interleaved row order; NW waves; ES bytes per element (4: fp32, 2: bf16,
// KC only).  Each stage is R rows of 128 bytes (32 fp32 or 64 bf16 k) = R / 8
// copy instructions of 1 KB; wave w issues numbers w, w + NW, ...
template <int R, bool KC, bool IL, int NW, int ES = 4>
struct Copy {
  static_assert(ES == 4 || (ES == 2 && KC), "bf16 operands are copied k-contiguous");
  static constexpr int NI = R / (8 * NW);  // instructions per wave per stage
  uint32_t off[NI];                        // byte offset of this lane's 16 bytes
  __device__ __forceinline__ void init(int ld, int lane, int wave) {
#pragma unroll
    for (int q = 0; q < NI; q++) {
      const int g = q * NW + wave;
      if (KC) {
        const int rho = 8 * g + (lane >> 3), c = (lane & 7) ^ (lane >> 3) ^ (g & 1);
        const int row = IL ? 4 * (rho % (R / 4)) + rho / (R / 4) : rho;
        off[q] = (uint32_t)(row * ld) * (uint32_t)ES + 16u * (uint32_t)c;
      } else {
        const int e = g * 64 + lane;  // float4 index in the stage
        off[q] = (uint32_t)((e / (R / 4)) * ld + 4 * (e % (R / 4))) * 4u;
      }
    }
  }
  // base: global address of the stage's (row 0, k 0) element (uniform);
  // lds: LDS byte address of the stage.
  __device__ __forceinline__ void issue(const char* base, uint32_t lds, int wave) const {
#pragma unroll
    for (int q = 0; q < NI; q++) copy16(base, off[q], lds + (q * NW + wave) * 1024);
  }
};

__device__ __forceinline__ bf16x8 cat8(f4 lo, f4 hi) {
  const bf16x4 a = __builtin_convertvector(lo, bf16x4), b = __builtin_convertvector(hi, bf16x4);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f4 lds4(const char* X, uint32_t byte) {
  return *reinterpret_cast<const f4*>(X + byte);
}

// NF 32-row fragments of one operand side for k-step s of a stage.  Rows of
// fragment f: woff + 32 f + i (KC, natural order) or woff + NF i + f
// (interleaved: row-contiguous operands, NF = 2 or 4, one 8- or 16-byte
// read per k; KC ones copied with IL, NF = 4).
template <int R, bool KC, bool IL, int NF>
__device__ __forceinline__ void frags(const char* X, int s, int woff, int i, int h, bf16x8 (&out)[NF]) {
  static_assert(!(KC && IL) || NF == 4, "the interleaved KC order spans 4 fragments");
  static_assert(KC || NF == 2 || NF == 4, "row-contiguous fragments come in 2s or 4s");
  if (KC) {
    const int key = (i & 7) ^ ((i >> 3) & 1);
    const uint32_t c0 = (uint32_t)(((4 * s + 2 * h) ^ key) * 16), c1 = (uint32_t)(((4 * s + 2 * h + 1) ^ key) * 16);
#pragma unroll
    for (int f = 0; f < NF; f++) {
      const int rho = IL ? f * (R / 4) + woff / 4 + i : woff + 32 * f + i;
      out[f] = cat8(lds4(X, (uint32_t)rho * 128u + c0), lds4(X, (uint32_t)rho * 128u + c1));
    }
  } else if (NF == 4) {
    const uint32_t vb = (uint32_t)((16 * s + 8 * h) * R * 4 + (woff + 4 * i) * 4);
    f4 raw[8];
#pragma unroll
    for (int e = 0; e < 8; e++) raw[e] = lds4(X, vb + e * R * 4);
#pragma unroll
    for (int t = 0; t < NF; t++)
      out[t] = cat8(f4{raw[0][t], raw[1][t], raw[2][t], raw[3][t]},
                    f4{raw[4][t], raw[5][t], raw[6][t], raw[7][t]});
  } else {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const uint32_t vb = (uint32_t)((16 * s + 8 * h) * R * 4 + (woff + 2 * i) * 4);
    f2 raw[8];
#pragma unroll
    for (int e = 0; e < 8; e++) raw[e] = *reinterpret_cast<const f2*>(X + vb + e * R * 4);
#pragma unroll
    for (int t = 0; t < NF; t++)
      out[t] = cat8(f4{raw[0][t], raw[1][t], raw[2][t], raw[3][t]},
                    f4{raw[4][t], raw[5][t], raw[6][t], raw[7][t]});
  }
}

// NF 32-row fragments of a k-contiguous bf16 operand for k-step s of a stage
// (rows as in frags): a 128-byte LDS row holds 64 k as 8 slots of 8 bf16, the
// lane group h of k-step s takes slot 2 s + h, one 16-byte read per fragment.
template <int R, bool IL, int NF>
__device__ __forceinline__ void frags_bf(const char* X, int s, int woff, int i, int h, bf16x8 (&out)[NF]) {
  static_assert(!IL || NF == 4, "the interleaved KC order spans 4 fragments");
  const int key = (i & 7) ^ ((i >> 3) & 1);
  const uint32_t c = (uint32_t)(((2 * s + h) ^ key) * 16);
#pragma unroll
  for (int f = 0; f < NF; f++) {
    const int rho = IL ? f * (R / 4) + woff / 4 + i : woff + 32 * f + i;
    out[f] = *reinterpret_cast<const bf16x8*>(X + (uint32_t)rho * 128u + c);
  }
}

// TJ = 8: 256x256 tile, 8 waves (two per SIMD, so one wave's MFMAs cover
// the other's LDS and barrier waits) as 4 x 2, each 64 x 128 (2 x 4 blocks
// of 32x32).  TJ = 4: 256x128 tile, 4 waves as 4 x 1, each 64 x 128.
// BF: both operands are bf16 in global memory, k-contiguous (A [M][K], B
// [N][K], leading dimensions in bf16 elements), copied as they are: 64 k per
// stage and no conversion in the multiply loop.
// NS: LDS stages (2 or 3).  A stage's copies are issued NS - 1 stages ahead
// of its multiply, so with one wave per SIMD (TJ = 4), where a stage's
// matrix work is shorter than a copy's latency, three stages keep two copies
// in flight behind the one being multiplied.
template <int TJ, bool TA, bool TB, bool BF = false, int NS = 2>
__global__ __launch_bounds__(TJ == 8 ? 512 : 256) void gemm_dma(GemmBatch batch, int kslice) {
  static_assert(!BF || (!TA && TB), "bf16 operands come k-contiguous");
  static_assert(NS == 2 || NS == 3, "two or three stages");
  constexpr int BM = 256, BN = 32 * TJ, NW = TJ == 8 ? 8 : 4;
  constexpr int ES = BF ? 2 : 4, KST = BF ? 64 : BK;  // element bytes, k per stage
  constexpr int FA = 2, FB = 4;  // 32-row fragments per wave
  constexpr bool AKC = !TA, BKC = TB;
  // the N side is always read in the interleaved order (float4 stores along
  // rows of C); the M side only when A is row-contiguous
  constexpr bool AIL = !AKC;
  // each stage: the A tile (BM rows of 128 bytes) then the B tile (BN rows)
  constexpr int SA = BM * 128, SB = BN * 128;
  __shared__ __attribute__((aligned(1024))) char smem[NS * (SA + SB)];

  const bool split = batch.count == 1 && gridDim.z > 1;
  const GemmProblem& P = batch.p[split ? 0 : blockIdx.z];
  const int M = P.M, N = P.N, K = P.K;
  int m0, n0;
  tile_origin(BM, BN, m0, n0);
  if (m0 >= M || n0 >= N) return;  // outside this problem's grid (uniform per workgroup)
  float* __restrict__ C = P.C;
  const int ldc = split ? N : P.ldc;
  const int kbeg = split ? blockIdx.z * kslice : 0;
  const int kend = split ? min(K, kbeg + kslice) : K;
  if (split) C = P.part + (size_t)blockIdx.z * M * N;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wa = TJ == 8 ? (wave >> 1) * 64 : wave * 64;  // wave's first row / column
  const int wb = TJ == 8 ? (wave & 1) * 128 : 0;
  const int i = lane & 31, h = lane >> 5;

  Copy<BM, AKC, false, NW, ES> ca;
  Copy<BN, BKC, true, NW, ES> cb;
  ca.init(P.lda, lane, wave);
  cb.init(P.ldb, lane, wave);
  constexpr int NDMA = Copy<BM, AKC, false, NW, ES>::NI + Copy<BN, BKC, true, NW, ES>::NI;
  // stage origins: (row 0, k0) of each operand tile, in bytes
  const char* Ab = reinterpret_cast<const char*>(P.A) + (AKC ? (size_t)m0 * P.lda * ES : (size_t)m0 * 4);
  const char* Bb = reinterpret_cast<const char*>(P.B) + (BKC ? (size_t)n0 * P.ldb * ES : (size_t)n0 * 4);
  const size_t astep = AKC ? (size_t)KST * ES : (size_t)BK * P.lda * 4;
  const size_t bstep = BKC ? (size_t)KST * ES : (size_t)BK * P.ldb * 4;
  Ab += AKC ? (size_t)kbeg * ES : (size_t)kbeg * P.lda * 4;
  Bb += BKC ? (size_t)kbeg * ES : (size_t)kbeg * P.ldb * 4;

  f16v acc[FA][FB];
#pragma unroll
  for (int a = 0; a < FA; a++)
#pragma unroll
    for (int b = 0; b < FB; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[a][b][r] = 0.f;

  auto compute = [&](const float* Xa, const float* Xb) {
#pragma unroll
    for (int s = 0; s < KST / 16; s++) {
      bf16x8 fa[FA], fb[FB];
      if constexpr (BF) {
        frags_bf<BM, false, FA>(reinterpret_cast<const char*>(Xa), s, wa, i, h, fa);
        frags_bf<BN, true, FB>(reinterpret_cast<const char*>(Xb), s, wb, i, h, fb);
      } else {
        frags<BM, AKC, AIL, FA>(reinterpret_cast<const char*>(Xa), s, wa, i, h, fa);
        frags<BN, BKC, true, FB>(reinterpret_cast<const char*>(Xb), s, wb, i, h, fb);
      }
#pragma unroll
      for (int a = 0; a < FA; a++)
#pragma unroll
        for (int b = 0; b < FB; b++)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
  };

  // NS stages in a ring; the copies of stage s + NS - 1 are issued before
  // stage s is multiplied.  Before a stage is read every wave waits for its
  // own copies into it (vmcnt: the copies of the later stages may stay in
  // flight), then the barrier makes all waves' copies visible; the barrier
  // after the multiply frees the stage for the copy issued next.
  const uint32_t l0 = (uint32_t)(size_t)(lds_void*)smem;
  auto issue = [&](int st) {
    const int bi = st % NS;
    ca.issue(Ab + (size_t)st * astep, l0 + bi * (SA + SB), wave);
    cb.issue(Bb + (size_t)st * bstep, l0 + bi * (SA + SB) + SA, wave);
  };
  const int nk = (kend - kbeg) / KST;
  for (int st = 0; st < NS - 1 && st < nk; st++) issue(st);
  for (int s = 0; s < nk; s++) {
    if (s + NS - 1 < nk) issue(s + NS - 1);
    const int later = min(s + NS - 1, nk - 1) - s;  // stages after s still in flight
    if (NS == 3 && later >= 2)
      wait_vmcnt<2 * NDMA>();
    else if (later >= 1)
      wait_vmcnt<NDMA>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    const char* st_base = smem + (s % NS) * (SA + SB);
    compute(reinterpret_cast<const float*>(st_base), reinterpret_cast<const float*>(st_base + SA));
    lds_barrier();
  }

  // epilogue: fragment rows / columns back to matrix positions; lane i
  // holds columns 4 i + (0..3) of each row, stored as one float4
  const float beta = split ? 0.f : P.beta;
  const int epi = split ? EPI_NONE : P.epi;
  const float* __restrict__ aux = split ? nullptr : P.aux;
  __bf16* __restrict__ c16 = split ? nullptr : P.C16;
  const int col = n0 + wb + 4 * i;
#pragma unroll
  for (int a = 0; a < FA; a++) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int rr = (r & 3) + 8 * (r >> 2) + 4 * h;  // row within the 32x32 block
      const int row = m0 + wa + (AKC ? 32 * a + rr : FA * rr + a);
      float* o = C + (size_t)row * ldc + col;
      f4 x = {acc[a][0][r], acc[a][1][r], acc[a][2][r], acc[a][3][r]};
      if (beta != 0.f) x += beta * *reinterpret_cast<const f4*>(o);
      if (epi != EPI_NONE) {
        const f4 ax = aux ? *reinterpret_cast<const f4*>(aux + (size_t)row * P.ldc + col) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; t++) x[t] = apply_epi(x[t], epi, ax[t]);
      }
      *reinterpret_cast<f4*>(o) = x;
      if (c16) *reinterpret_cast<bf16x4*>(c16 + (size_t)row * P.N + col) = __builtin_convertvector(x, bf16x4);
    }
  }
}

}  // namespace dmak

// ------------------------------------------------------------------ packs --
// Operands rounded to bf16 (round to nearest even) once and stored
// k-contiguous for the bf16 mode of gemm_dma.
// dst[r][c] = bf16(src[r][c]), R x K (K a multiple of 8), dst leading dim K.
__global__ __launch_bounds__(256) void pack_bf16(int R, int K, const float* __restrict__ src, int lds,
                                                 __bf16* __restrict__ dst) {
  const int K8 = K / 8;
  const size_t n = (size_t)R * K8;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int r = (int)(i / K8), c = (int)(i - (size_t)r * K8) * 8;
    const f4* p = reinterpret_cast<const f4*>(src + (size_t)r * lds + c);
    const bf16x4 lo = __builtin_convertvector(p[0], bf16x4), hi = __builtin_convertvector(p[1], bf16x4);
    *reinterpret_cast<bf16x8*>(dst + (size_t)r * K + c) =
        bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// dst[n][k] = bf16(src[k][n]) for a K x N source (K and N multiples of 64),
// dst leading dim K.  A 64 x 64 tile per workgroup through LDS: rows of the
// source read as float4, rows of the result written as 16 bytes.
__global__ __launch_bounds__(256) void pack_bf16_t(int K, int N, const float* __restrict__ src, int lds,
                                                   __bf16* __restrict__ dst) {
  __shared__ float tile[64][65];
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64, tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int k = tid / 16 + 16 * j, c = (tid % 16) * 4;
    const f4 v = *reinterpret_cast<const f4*>(src + (size_t)(k0 + k) * lds + n0 + c);
    tile[k][c] = v[0];
    tile[k][c + 1] = v[1];
    tile[k][c + 2] = v[2];
    tile[k][c + 3] = v[3];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int n = tid / 8 + 32 * j, kq = (tid % 8) * 8;
    const f4 lo = {tile[kq][n], tile[kq + 1][n], tile[kq + 2][n], tile[kq + 3][n]};
    const f4 hi = {tile[kq + 4][n], tile[kq + 5][n], tile[kq + 6][n], tile[kq + 7][n]};
    const bf16x4 a = __builtin_convertvector(lo, bf16x4), b = __builtin_convertvector(hi, bf16x4);
    *reinterpret_cast<bf16x8*>(dst + (size_t)(n0 + n) * K + k0 + kq) =
        bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// Sum S split-K partials [S][M][N] (leading dim N) into C (ldc), with beta/epilogue.
// The partials are added in slice order; each thread issues the loads of up
// to eight slices before the first add, so that enough reads are in flight to
// cover the memory latency (one load per add leaves the pass latency bound).
__global__ __launch_bounds__(256) void splitk_reduce(int M, int N, int S, const float* __restrict__ P,
                                                     float* __restrict__ C, int ldc, float beta,
                                                     int epi, const float* __restrict__ aux,
                                                     __bf16* __restrict__ c16) {
  const size_t n4 = (size_t)M * N / 4, zs = (size_t)M * N / 4;
  const f4* __restrict__ P4 = reinterpret_cast<const f4*>(P);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    f4 s = P4[i];
    int z = 1;
    for (; z + 8 <= S; z += 8) {
      f4 x[8];
#pragma unroll
      for (int u = 0; u < 8; u++) x[u] = P4[(size_t)(z + u) * zs + i];
#pragma unroll
      for (int u = 0; u < 8; u++) s += x[u];
    }
    for (; z + 4 <= S; z += 4) {
      f4 x[4];
#pragma unroll
      for (int u = 0; u < 4; u++) x[u] = P4[(size_t)(z + u) * zs + i];
#pragma unroll
      for (int u = 0; u < 4; u++) s += x[u];
    }
    for (; z < S; z++) s += P4[(size_t)z * zs + i];
    const size_t e = i * 4;
    const int row = (int)(e / N), col = (int)(e % N);
    const size_t o = (size_t)row * ldc + col;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      float x = s[c];
      if (beta != 0.f) x += beta * C[o + c];
      x = apply_epi(x, epi, aux ? aux[o + c] : 0.f);
      C[o + c] = x;
      if (c16) c16[e + c] = (__bf16)x;
    }
  }
}

template <int PREC, int TI, int TJ, int BK, bool TA, bool TB>
hipError_t launch_t(const GemmBatch& b, int gz, int kslice, hipStream_t st) {
  int maxM = 0, maxN = 0;
  for (int i = 0; i < b.count; i++) {
    maxM = max(maxM, b.p[i].M);
    maxN = max(maxN, b.p[i].N);
  }
  dim3 grid((maxN + 32 * TJ - 1) / (32 * TJ), (maxM + 32 * TI - 1) / (32 * TI), gz);
  if (PREC == GEMM_BF16)
    hipLaunchKernelGGL((gemm_bf16<TI, TJ, BK, TA, TB>), grid, dim3(256), 0, st, b, kslice);
  else
    hipLaunchKernelGGL((gemm_f32<TI, TJ, BK, TA, TB>), grid, dim3(256), 0, st, b, kslice);
  return hipGetLastError();
}

template <int PREC, int TI, int TJ, bool TA, bool TB>
hipError_t launch_bk(const GemmBatch& b, int gz, int kslice, int klen, hipStream_t st) {
  // K tile depth: shallow for big tiles (plenty of MFMA work per K step),
  // deep for small tiles so few global round trips remain.
  if (TI * TJ >= 8 || klen <= 32) return launch_t<PREC, TI, TJ, 32, TA, TB>(b, gz, kslice, st);
  if (klen <= 64 || TI * TJ >= 4) return launch_t<PREC, TI, TJ, 64, TA, TB>(b, gz, kslice, st);
  return launch_t<PREC, TI, TJ, 128, TA, TB>(b, gz, kslice, st);
}

// Direct-to-LDS bf16 kernel: every problem's M a multiple of 256, N of the
// tile width, K (and the split-K slice) of 32, leading dimensions and
// pointers 16-byte aligned.  Returns the fragment count per wave in N (8 or
// 4), or 0 when the batch does not qualify.
int dma_tj(const GemmBatch& b, bool transA, int gz, int kslice) {
  if (kslice % (2 * dmak::BK) != 0 || kslice <= 0) return 0;
  bool n256 = true;
  long tiles = 0;
  auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  for (int i = 0; i < b.count; i++) {
    const GemmProblem& q = b.p[i];
    if (q.M % 256 || q.N % 128 || q.K % (2 * dmak::BK) || q.lda % 4 || q.ldb % 4 || q.ldc % 4) return 0;
    if (!al(q.A) || !al(q.B) || !al(q.C) || (q.aux && !al(q.aux)) || (q.part && !al(q.part))) return 0;
    n256 = n256 && q.N % 256 == 0;
    tiles = std::max(tiles, (long)(q.M / 256) * (q.N / 256));
  }
  // below half the CUs (the decode stack's small products) the
  // register-staged tiles, which come in smaller sizes, do better
  long t128 = 0;
  for (int i = 0; i < b.count; i++) t128 = std::max(t128, (long)(b.p[i].M / 256) * (b.p[i].N / 128));
  if (t128 * gz < 128) return 0;
  (void)transA;
  return n256 && tiles * gz >= 256 ? 8 : 4;
}

template <int TJ, bool TA, bool TB>
hipError_t launch_dma_t(const GemmBatch& b, int gz, int kslice, hipStream_t st) {
  int maxM = 0, maxN = 0;
  for (int i = 0; i < b.count; i++) {
    maxM = max(maxM, b.p[i].M);
    maxN = max(maxN, b.p[i].N);
  }
  dim3 grid(maxN / (32 * TJ), maxM / 256, gz);
  hipLaunchKernelGGL((dmak::gemm_dma<TJ, TA, TB>), grid, dim3(TJ == 8 ? 512 : 256), 0, st, b, kslice);
  return hipGetLastError();
}

template <bool TA, bool TB>
hipError_t launch_dma(const GemmBatch& b, int tj, int gz, int kslice, hipStream_t st) {
  return tj == 8 ? launch_dma_t<8, TA, TB>(b, gz, kslice, st) : launch_dma_t<4, TA, TB>(b, gz, kslice, st);
}

// The caller's arena for bf16 operand copies (set for the duration of one
// library call on the calling thread; null: operands are converted in LDS).
thread_local char* tl_pack = nullptr;
thread_local size_t tl_pack_bytes = 0;

constexpr size_t PACK_MAX_A = (size_t)64 << 20;   // elements: larger activations are read as fp32
constexpr size_t PACK_MAX_B = (size_t)128 << 20;  // elements of a packed weight

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The bf16 mode of gemm_dma: every operand of the batch is rounded to bf16
// once into the arena, k-contiguous (A [M][K] as is, B to [N][K]: as is when
// it is stored [N][K], transposed otherwise), then multiplied without any
// conversion in the loop.  Returns hipErrorNotSupported when the batch does
// not take this path.
hipError_t launch_dma_packed(const GemmBatch& b, bool transB, int tj, int gz, int kslice,
                             hipStream_t st) {
  size_t need = 0;
  for (int i = 0; i < b.count; i++) {
    const GemmProblem& q = b.p[i];
    const size_t n = q.A16 ? gemm_pack_need_b(q.M, q.N, q.K) : gemm_pack_need(q.M, q.N, q.K);
    if (n == 0) return hipErrorNotSupported;
    need += n;
  }
  if (!tl_pack || need > tl_pack_bytes) return hipErrorNotSupported;
  GemmBatch pb = b;
  char* cur = tl_pack;
  for (int i = 0; i < b.count; i++) {
    const GemmProblem& q = b.p[i];
    const __bf16* pa = q.A16;  // an A rounded to bf16 by its producer: no copy, no arena
    if (!pa) {
      __bf16* pw = reinterpret_cast<__bf16*>(cur);
      pa = pw;
      const size_t n8 = (size_t)q.M * q.K / 8;
      hipLaunchKernelGGL(pack_bf16, dim3((int)std::min<size_t>((n8 + 255) / 256, 4096)), dim3(256), 0,
                         st, q.M, q.K, q.A, q.lda, pw);
      cur += align256((size_t)q.M * q.K * 2);
    }
    __bf16* pbm = reinterpret_cast<__bf16*>(cur);
    cur += align256((size_t)q.N * q.K * 2);
    auto blocks = [](size_t n8) { return (int)std::min<size_t>((n8 + 255) / 256, 4096); };
    if (transB)
      hipLaunchKernelGGL(pack_bf16, dim3(blocks((size_t)q.N * q.K / 8)), dim3(256), 0, st, q.N, q.K,
                         q.B, q.ldb, pbm);
    else
      hipLaunchKernelGGL(pack_bf16_t, dim3(q.N / 64, q.K / 64), dim3(256), 0, st, q.K, q.N, q.B, q.ldb,
                         pbm);
    pb.p[i].A = reinterpret_cast<const float*>(pa);
    pb.p[i].lda = q.K;
    pb.p[i].B = reinterpret_cast<const float*>(pbm);
    pb.p[i].ldb = q.K;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int maxM = 0, maxN = 0;
  for (int i = 0; i < pb.count; i++) {
    maxM = max(maxM, pb.p[i].M);
    maxN = max(maxN, pb.p[i].N);
  }
  dim3 grid(maxN / (32 * tj), maxM / 256, gz);
  if (tj == 8)
    hipLaunchKernelGGL((dmak::gemm_dma<8, false, true, true>), grid, dim3(512), 0, st, pb, kslice);
  else
    hipLaunchKernelGGL((dmak::gemm_dma<4, false, true, true, 3>), grid, dim3(256), 0, st, pb, kslice);
  return hipGetLastError();
}

template <int PREC, bool TA, bool TB>
hipError_t launch_layout(const GemmBatch& b, int gz, int kslice, int klen, hipStream_t st) {
  // Largest tile whose grid reaches 512 workgroups, or 256 when each workgroup
  // still has >= 8M multiply-adds; else the smallest tile.  Small problems
  // (the decode stack's 2048-row products) are latency bound and gain from
  // more, smaller workgroups; large ones keep the 128x128 tile.  Measured on
  // MI355X, fp32: 2048x256x256 7.2 us at 32x32 vs 8.6 at 64x32 and 11.6 at
  // 64x64; 2048x1024x256 17.5 us at 64x64 vs 20.0 at 128x64; 8192x768x768
  // 120 us at 128x128 (384 workgroups) vs 95 at 128x64 (768).
  int maxM = 0, maxN = 0;
  for (int i = 0; i < b.count; i++) {
    maxM = max(maxM, b.p[i].M);
    maxN = max(maxN, b.p[i].N);
  }
  auto fits = [&](int bm, int bn) {
    const long wg = (long)((maxM + bm - 1) / bm) * ((maxN + bn - 1) / bn) * gz;
    return maxN >= bn && (wg >= 512 || (wg >= 256 && (long)bm * bn * klen >= (8l << 20)));
  };
  // a 128x128 grid that only part-fills a second round of the 256 CUs leaves
  // the CUs holding two tiles to set the time: the 128x64 tiles then spread
  // evenly (three per CU at 768 workgroups)
  const long wg128 = (long)((maxM + 127) / 128) * ((maxN + 127) / 128) * gz;
  const bool ragged = wg128 > 256 && wg128 < 512 && wg128 % 256 != 0;
  if (fits(128, 128) && !(ragged && fits(128, 64))) return launch_bk<PREC, 4, 4, TA, TB>(b, gz, kslice, klen, st);
  if (fits(128, 64)) return launch_bk<PREC, 4, 2, TA, TB>(b, gz, kslice, klen, st);
  if (fits(64, 64)) return launch_bk<PREC, 2, 2, TA, TB>(b, gz, kslice, klen, st);
  if (fits(64, 32)) return launch_bk<PREC, 2, 1, TA, TB>(b, gz, kslice, klen, st);
  return launch_bk<PREC, 1, 1, TA, TB>(b, gz, kslice, klen, st);
}

template <int PREC>
hipError_t dispatch_p(bool transA, bool transB, const GemmBatch& b, int gz, int kslice, int klen,
                      hipStream_t st) {
  if (!transA && !transB) return launch_layout<PREC, false, false>(b, gz, kslice, klen, st);
  if (!transA && transB) return launch_layout<PREC, false, true>(b, gz, kslice, klen, st);
  if (transA && !transB) return launch_layout<PREC, true, false>(b, gz, kslice, klen, st);
  return launch_layout<PREC, true, true>(b, gz, kslice, klen, st);
}

hipError_t dispatch(int prec, bool transA, bool transB, const GemmBatch& b, int gz, int kslice,
                    int klen, hipStream_t st) {
  if (prec == GEMM_BF16) {
    const int tj = dma_tj(b, transA, gz, kslice);
    if (tj && !transA) {
      const hipError_t e = launch_dma_packed(b, transB, tj, gz, kslice, st);
      if (e != hipErrorNotSupported) return e;
    }
    if (tj && !transA && !transB) return launch_dma<false, false>(b, tj, gz, kslice, st);
    if (tj && !transA && transB) return launch_dma<false, true>(b, tj, gz, kslice, st);
    if (tj && transA && !transB) return launch_dma<true, false>(b, tj, gz, kslice, st);
    if (tj) return launch_dma<true, true>(b, tj, gz, kslice, st);
    return dispatch_p<GEMM_BF16>(transA, transB, b, gz, kslice, klen, st);
  }
  return dispatch_p<GEMM_F32>(transA, transB, b, gz, kslice, klen, st);
}

}  // namespace gemmk

size_t gemm_pack_need_b(int M, int N, int K) {
  using namespace gemmk;
  if (M % 256 || N % 128 || K % 64 || M <= 0 || N <= 0 || K <= 0) return 0;
  if ((size_t)N * K > PACK_MAX_B) return 0;
  return align256((size_t)N * K * 2);
}

size_t gemm_pack_need(int M, int N, int K) {
  using namespace gemmk;
  if (M % 256 || N % 128 || K % 64 || M <= 0 || N <= 0 || K <= 0) return 0;
  if ((size_t)M * K > PACK_MAX_A || (size_t)N * K > PACK_MAX_B) return 0;
  return align256((size_t)M * K * 2) + align256((size_t)N * K * 2);
}

void gemm_set_pack_arena(void* p, size_t bytes) {
  gemmk::tl_pack = reinterpret_cast<char*>(p);
  gemmk::tl_pack_bytes = p ? bytes : 0;
}

hipError_t gemm_batch(int prec, bool transA, bool transB, const GemmBatch& b, hipStream_t st) {
  if (b.count < 1 || b.count > GEMM_MAX_BATCH) return hipErrorInvalidValue;
  int maxK = 0;
  for (int i = 0; i < b.count; i++) maxK = max(maxK, b.p[i].K);
  return gemmk::dispatch(prec, transA, transB, b, b.count, maxK, maxK, st);
}

// K slices for a product split along K (the weight gradients X^T dY, which run
// beside the rest of the backward on a second stream): about 64 workgroups
// of the 256-row direct-to-LDS bf16 tiles, 256 of the 128x128 ones, each
// slice at least 256 deep.  Fewer slices than one workgroup per CU measured
// faster in the training step and the online segment (less partial traffic,
// and the products leave more CUs to the other stream); far fewer leave
// single long products on the critical path.
int gemm_splitk_slices(int prec, int M, int N, int K) {
  long want;
  if (prec == GEMM_BF16 && M % 256 == 0 && N % 128 == 0 && K % (2 * gemmk::dmak::BK) == 0) {
    const long tiles = (long)(M / 256) * (N % 256 == 0 ? N / 256 : N / 128);
    want = (64 + tiles - 1) / tiles;
  } else {
    const long tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
    want = (256 + tiles - 1) / tiles;
  }
  want = std::min(want, (long)(K / 256));
  return want < 1 ? 1 : (int)want;
}

hipError_t gemm_run_partials(int prec, int M, int N, int K, const float* A, int lda,
                             const float* B, int ldb, int split, float* part, int* slices,
                             hipStream_t st) {
  using namespace gemmk;
  split = std::max(1, std::min(split, K / 64));
  int kslice = (K + split - 1) / split;
  kslice = (kslice + 63) / 64 * 64;
  const int S = (K + kslice - 1) / kslice;
  *slices = S;
  if (M <= 0 || N <= 0) return hipSuccess;
  GemmBatch b;
  b.count = 1;
  b.p[0] = GemmProblem{M, N, K, A, lda, B, ldb, part, N, 0.f, EPI_NONE, nullptr, part};
  return dispatch(prec, false, false, b, S, kslice, kslice, st);
}

// C = epi(op(A) op(B) + beta C).  ws (may be NULL when split == 1) holds
// split*M*N floats of split-K partials.
hipError_t gemm_run_x(int prec, bool transA, bool transB, int M, int N, int K, const float* A,
                      int lda, const float* B, int ldb, float* C, int ldc, float beta, int epi,
                      const float* aux, int split, float* ws, hipStream_t st, const __bf16* A16,
                      __bf16* C16) {
  using namespace gemmk;
  if (M <= 0 || N <= 0) return hipSuccess;
  GemmBatch b;
  b.count = 1;
  b.p[0] = GemmProblem{M, N, K, A, lda, B, ldb, C, ldc, beta, epi, aux, nullptr, C16, A16};
  if (split > 1 && ws != nullptr) split = std::min(split, gemm_splitk_slices(prec, M, N, K));
  if (split <= 1 || ws == nullptr) return dispatch(prec, transA, transB, b, 1, K, K, st);
  int kslice = (K + split - 1) / split;
  kslice = (kslice + 63) / 64 * 64;
  const int S = (K + kslice - 1) / kslice;
  b.p[0].part = ws;
  hipError_t e = dispatch(prec, transA, transB, b, S, kslice, kslice, st);
  if (e != hipSuccess) return e;
  const size_t n4 = (size_t)M * N / 4;
  int blocks = (int)((n4 + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(splitk_reduce, dim3(blocks), dim3(256), 0, st, M, N, S, ws, C, ldc, beta, epi, aux, C16);
  return hipGetLastError();
}

hipError_t gemm_run(int prec, bool transA, bool transB, int M, int N, int K, const float* A,
                    int lda, const float* B, int ldb, float* C, int ldc, float beta, int epi,
                    const float* aux, int split, float* ws, hipStream_t st) {
  return gemm_run_x(prec, transA, transB, M, N, K, A, lda, B, ldb, C, ldc, beta, epi, aux, split,
                    ws, st, nullptr, nullptr);
}
