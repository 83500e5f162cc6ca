// Chunked WKV7 forward on the gfx950 matrix cores (v_mfma_f32_16x16x4_f32).
//
// Same recurrence as the token-sequential kernel (per batch b, head h, token
// t; S is 64x64 fp32, S[i][j] with i = value row, j = key column):
//     sa_t = S a_t ;  S = S diag(w_t) + sa_t b_t^T + v_t k_t^T ;  y_t = S r_t
// ("Foundry/cuda_kernels/timemix.cu", the WKV7 kernel and its composites
// a = -kk, b = kk*a).  The recurrence is unrolled over chunks of L = 16
// tokens (a derivation of ours; the pages only run it token by token).  With
// g_t[j] = sum_{tau<=t} ln w_tau[j] (cumulative log-decay from the chunk
// start, g_{-1} = 0) and the chunk's entry state S0:
//   sa_t = S0 (a_t e^{g_{t-1}}) + sum_{tau<t} [ sa_tau <b_tau, a_t e^{g_{t-1}-g_tau}>
//                                             + v_tau  <k_tau, a_t e^{g_{t-1}-g_tau}> ]
//   y_t  = S0 (r_t e^{g_t})     + sum_{tau<=t} [ sa_tau <b_tau, r_t e^{g_t-g_tau}>
//                                              + v_tau  <k_tau, r_t e^{g_t-g_tau}> ]
//   S_L  = S0 diag(e^{g_L}) + sum_tau [ sa_tau (b_tau e^{g_L-g_tau})^T
//                                     + v_tau  (k_tau e^{g_L-g_tau})^T ]
// Stacking tokens as rows (L x 64 matrices SA, V; L x L matrices P, Q, Rb, Rk
// of the bracketed inner products, strictly lower for P, Q, lower for Rb, Rk):
//   (I - P) SA = AS S0^T + Q V,  so  SA = At S0^T + Qt V  with At = M AS, Qt = M Q,
//   M = (I - P)^-1 (unit lower triangular),
//   Y = Rt S0^T + Wt V  with Rt = RS + Rb At, Wt = Rb Qt + Rk,
//   S_L^T = diag(e^{g_L}) S0^T + BH^T SA + KH^T V.
// The inner products with e^{g_{t-1}-g_tau} are formed as products of
// a e^{g_{t-1}-g_ref} and b e^{g_ref-g_tau} around the chunk midpoint g_ref;
// a chunk whose exponents would leave [-40, 40] (cumulative decay below
// about e^-40 over half a chunk, or any growth) is run token by token
// instead, so the kernel is exact for every w.
//
// Everything but the state pass depends on the chunk's own inputs only, so
// it runs for all chunks at once.  fwd_prep (one workgroup per (b, h,
// chunk)): (1) all 256 threads form the scaled vectors from the cumulative
// log-decay; (2) each wave forms one of P, Q, Rb, Rk (16 MFMAs); (3) each
// wave applies (I - P)^-1 to a 16-column tile through the product form
// (I + P)(I + P^2)(I + P^4)(I + P^8) of the nilpotent P (about 30 MFMAs);
// the chunk's At, Rt, BH^T, KH^T, V^T, Qt, Wt, e^{g_L} go to a workspace
// record.  fwd_scan (one workgroup per (b, h), chunks in order, records
// double-buffered through LDS): wave q advances state rows 16q..16q+15 with
// 72 MFMAs per chunk.  The state lives in MFMA accumulator registers as S^T
// tiles: lane l of wave q, tile jt, element v holds
// S[16q + l%16][16jt + 4(l/16) + v].  That layout is at once the B operand
// of the products with S0^T (k = j taken in the order 4(l/16) + step inside
// each group of 16) and the accumulator of the state update, and the SA
// accumulator is the B operand of BH^T SA the same way, so the chain never
// leaves registers.  Checkpoints (every 16 tokens) are the chunk entry
// states, in the layout the checkpoint-recomputing backward reads.

#include "common.hpp"

namespace wkv7c {

constexpr int N = WKV7_N;
constexpr int L = WKV7_CKL;  // chunk length = checkpoint interval
constexpr int RS = N + 4;  // padded row stride of [L][N] arrays (floats)
constexpr int TS = L + 4;  // padded row stride of [N][L] and [L][L] arrays
constexpr float EXP_LIMIT = 40.f;

// Workspace record of one (b, h, chunk), dense fp32: At, Rt [L][N]; BH^T,
// KH^T, V^T [N][L]; Qt, Wt [L][L]; e^{g_L} [N]; flag (1 = run token by token).
constexpr int O_AT = 0, O_RT = 1024, O_BH = 2048, O_KH = 3072, O_VT = 4096, O_QT = 5120,
              O_WT = 5376, O_LAM = 5632, O_FLAG = 5696, REC = 5760;
constexpr int REC4 = REC / 4;
// scan scratch per head after the records: L*N (y of tail tokens), N*N
// (checkpoint stores when none are wanted), L*N (sa of tail tokens, and all
// of it when no checkpoints are wanted)
constexpr int SINK = L * N + N * N + L * N;

// The same data in LDS, rows padded for conflict-free 16-byte fragment reads.
struct ChunkLds {
  float A[2][L][RS];   // At, Rt
  float T3[3][N][TS];  // BH^T, KH^T, V^T
  float QW[2][L][TS];  // Qt, Wt
  float lam[N];
  float flag[64];
};

// LDS address of the float4 at record offset o (a multiple of 4).
__device__ __forceinline__ float* rec_lds(ChunkLds& d, int o) {
  if (o < O_BH) {
    const int m = o >> 10, rem = o & 1023;
    return &d.A[m][rem >> 6][rem & 63];
  }
  if (o < O_QT) {
    const int m = (o - O_BH) >> 10, rem = (o - O_BH) & 1023;
    return &d.T3[m][rem >> 4][rem & 15];
  }
  if (o < O_LAM) {
    const int m = (o - O_QT) >> 8, rem = (o - O_QT) & 255;
    return &d.QW[m][rem >> 4][rem & 15];
  }
  if (o < O_FLAG) return &d.lam[o - O_LAM];
  return &d.flag[o - O_FLAG];
}

// c += A B over one group of 16 k: A fragment a (lane: row l%16, k 4(l/16)+s),
// B fragment b (lane: k 4(l/16)+s, column l%16), s = MFMA step.
__device__ __forceinline__ f4 mma16(f4 a, f4 b, f4 c) {
#pragma unroll
  for (int s = 0; s < 4; s++) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }

template <typename T>
__device__ __forceinline__ const T* vec_ptr(int vi, const T* r, const T* w, const T* k,
                                           const T* a, const T* bv, const T* v) {
  return vi == 0 ? r : vi == 1 ? w : vi == 2 ? k : vi == 3 ? a : vi == 4 ? bv : v;
}

// ------------------------------------------------------------------ prep --
template <typename T>
__global__ __launch_bounds__(256) void fwd_prep(int Tn, int H, int nck, const T* __restrict__ r,
                                                const T* __restrict__ w, const T* __restrict__ k,
                                                const T* __restrict__ v, const T* __restrict__ a,
                                                const T* __restrict__ bv, float* __restrict__ rec) {
  __shared__ __attribute__((aligned(16))) ChunkLds out;
  // chunk inputs (0 r, 1 w, 2 k, 3 a, 4 b, 5 v), dead after (1); the powers
  // of P of (3) reuse the space
  __shared__ __attribute__((aligned(16))) union {
    float xin[6][L][N];
    float pow[4][3][L][TS];
  } u;
  // a e^{g_{t-1}} and r e^{g_t} live where At and Rt go: in (3) each wave
  // reads a column tile and writes the same tile back
  float(*sAS)[RS] = out.A[0];
  float(*sRS)[RS] = out.A[1];
  __shared__ __attribute__((aligned(16))) float sAP[L][RS];  // a e^{g_{t-1}-gref}
  __shared__ __attribute__((aligned(16))) float sRP[L][RS];  // r e^{g_t-gref}
  __shared__ __attribute__((aligned(16))) float sBB[L][RS];  // b e^{gref-g_t}
  __shared__ __attribute__((aligned(16))) float sKB[L][RS];  // k e^{gref-g_t}
  __shared__ __attribute__((aligned(16))) float sP[L][TS];
  __shared__ __attribute__((aligned(16))) float sQ[L][TS];
  __shared__ __attribute__((aligned(16))) float sRb[L][TS];
  __shared__ __attribute__((aligned(16))) float sRk[L][TS];
  __shared__ float sPart[4][N];
  __shared__ int sSlow;

  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = g / nck, c = g - bh * nck;
  const int H_ = H, b = bh / H_, h = bh - b * H_;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const size_t C = (size_t)H * N;
  const size_t vbase = (size_t)b * Tn * C + (size_t)h * N;
  const int t0 = c * L;

  {
    // thread -> (vector q, token tid/16, column group tid%16); tokens past the
    // end become identity steps (w = 1, everything else 0)
    const int tok = tid >> 4, c4 = (tid & 15) * 4;
    const bool in = t0 + tok < Tn;
    const int tc = min(t0 + tok, Tn - 1);
    typename Raw<T>::v4 pre[6];
#pragma unroll
    for (int q = 0; q < 6; q++) pre[q] = load_raw4(vec_ptr(q, r, w, k, a, bv, v) + vbase + (size_t)tc * C + c4);
#pragma unroll
    for (int q = 0; q < 6; q++) {
      f4 x = raw4_to_f4<T>(pre[q]);
      if (!in) x = q == 1 ? f4{1.f, 1.f, 1.f, 1.f} : f4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f4*>(&u.xin[q][tok][c4]) = x;
    }
  }
  if (tid == 0) sSlow = 0;
  __syncthreads();

  // ---- (1) cumulative log-decay and scaled vectors; thread = (column j, tokens 4q..4q+3)
  {
    const int j = tid & 63, qd = wave;
    float gl[4];
    float acc = 0.f;
#pragma unroll
    for (int uu = 0; uu < 4; uu++) {
      acc += __logf(u.xin[1][4 * qd + uu][j]);
      gl[uu] = acc;
    }
    sPart[qd][j] = acc;
    __syncthreads();
    const float p0 = sPart[0][j], p1 = sPart[1][j], p2 = sPart[2][j], p3 = sPart[3][j];
    const float base = qd == 0 ? 0.f : qd == 1 ? p0 : qd == 2 ? p0 + p1 : p0 + p1 + p2;
    const float gref = p0 + p1;  // g after token 7
    const float gL = p0 + p1 + p2 + p3;
    // |exponent| <= EXP_LIMIT everywhere below is checked first; then
    // e^{g_t} and e^{-g_t} per token and e^{+-gref}, e^{gL} per column give
    // every factor as a product of two.
    bool slow = !(fabsf(gref) <= EXP_LIMIT && fabsf(gL - gref) <= EXP_LIMIT);
    const float egr = __expf(gref), emgr = __expf(-gref), egL = __expf(gL);
    float ep = __expf(base);
#pragma unroll
    for (int uu = 0; uu < 4; uu++) {
      const int t = 4 * qd + uu;
      const float gg = base + gl[uu];
      slow |= !(fabsf(gg - gref) <= EXP_LIMIT && gg <= EXP_LIMIT);
      const float e = __expf(gg), em = __expf(-gg);
      const float av = u.xin[3][t][j], rv = u.xin[0][t][j], bb = u.xin[4][t][j], kv = u.xin[2][t][j];
      sAS[t][j] = av * ep;
      sAP[t][j] = av * (ep * emgr);
      sRS[t][j] = rv * e;
      sRP[t][j] = rv * (e * emgr);
      const float eb = egr * em;
      sBB[t][j] = bb * eb;
      sKB[t][j] = kv * eb;
      const float eL = egL * em;
      out.T3[0][j][t] = bb * eL;
      out.T3[1][j][t] = kv * eL;
      out.T3[2][j][t] = u.xin[5][t][j];
      ep = e;
    }
    if (qd == 0) out.lam[j] = egL;
    if (slow) sSlow = 1;  // benign race: every writer stores 1
  }
  __syncthreads();
  const bool slow = sSlow != 0;
  if (tid == 0) out.flag[0] = slow ? 1.f : 0.f;

  if (!slow) {
    // ---- (2) wave 0: P = AP BB^T, 1: Q = AP KB^T, 2: Rb = RP BB^T, 3: Rk = RP KB^T
    {
      const float(*X)[RS] = wave < 2 ? sAP : sRP;
      const float(*Y)[RS] = (wave & 1) ? sKB : sBB;
      float(*D)[TS] = wave == 0 ? sP : wave == 1 ? sQ : wave == 2 ? sRb : sRk;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = 0; jb < 4; jb++)
        acc = mma16(ld4(&X[fr][16 * jb + 4 * fg]), ld4(&Y[fr][16 * jb + 4 * fg]), acc);
      const bool strict = wave < 2;
#pragma unroll
      for (int uu = 0; uu < 4; uu++) {
        const int t = 4 * fg + uu, tau = fr;
        D[t][tau] = (strict ? tau < t : tau <= t) ? acc[uu] : 0.f;
      }
    }
    __syncthreads();

    // ---- (3) M = (I - P)^-1 = (I + P)(I + P^2)(I + P^4)(I + P^8) (P is
    //          strictly lower, P^16 = 0), applied right to left to 16-column
    //          tiles X: X += P^8 X, X += P^4 X, X += P^2 X, X += P X.  Wave q
    //          takes AS columns 16q.. (-> At), wave 0 also Q (-> Qt); then
    //          Rt = RS + Rb At, Wt = Rk + Rb Qt.  Each wave forms the powers
    //          itself in its own LDS rows (no cross-wave wait).
    float(*Pw)[L][TS] = u.pow[wave];
    const f4 pa = ld4(&sP[fr][4 * fg]);  // A layout: P[l%16][4g+s]
    f4 pb;                               // B layout: P[4g+s][l%16]
#pragma unroll
    for (int s2 = 0; s2 < 4; s2++) pb[s2] = sP[4 * fg + s2][fr];
    f4 pw = mma16(pa, pb, f4{0.f, 0.f, 0.f, 0.f});  // C layout: P^2[4g+v][l%16]
#pragma unroll
    for (int e = 0; e < 3; e++) {
#pragma unroll
      for (int uu = 0; uu < 4; uu++) Pw[e][4 * fg + uu][fr] = pw[uu];
      if (e < 2) pw = mma16(ld4(&Pw[e][fr][4 * fg]), pw, f4{0.f, 0.f, 0.f, 0.f});  // square
    }
    const f4 a8 = ld4(&Pw[2][fr][4 * fg]), a4 = ld4(&Pw[1][fr][4 * fg]);
    const f4 a2 = ld4(&Pw[0][fr][4 * fg]);
    const f4 rb = ld4(&sRb[fr][4 * fg]);
    auto solve = [&](f4 x) {
      x = mma16(a8, x, x);
      x = mma16(a4, x, x);
      x = mma16(a2, x, x);
      return mma16(pa, x, x);
    };
    const int col = 16 * wave + fr;
    f4 x, rr;
#pragma unroll
    for (int uu = 0; uu < 4; uu++) {
      x[uu] = sAS[4 * fg + uu][col];
      rr[uu] = sRS[4 * fg + uu][col];
    }
    if (wave == 0) {
      // two independent chains (AS tile 0 and Q), interleaved
      f4 xq, wq;
#pragma unroll
      for (int uu = 0; uu < 4; uu++) {
        xq[uu] = sQ[4 * fg + uu][fr];
        wq[uu] = sRk[4 * fg + uu][fr];
      }
      x = mma16(a8, x, x);
      xq = mma16(a8, xq, xq);
      x = mma16(a4, x, x);
      xq = mma16(a4, xq, xq);
      x = mma16(a2, x, x);
      xq = mma16(a2, xq, xq);
      x = mma16(pa, x, x);
      xq = mma16(pa, xq, xq);
      rr = mma16(rb, x, rr);
      wq = mma16(rb, xq, wq);
#pragma unroll
      for (int uu = 0; uu < 4; uu++) {
        out.QW[0][4 * fg + uu][fr] = xq[uu];
        out.QW[1][4 * fg + uu][fr] = wq[uu];
      }
    } else {
      x = solve(x);
      rr = mma16(rb, x, rr);
    }
#pragma unroll
    for (int uu = 0; uu < 4; uu++) {
      out.A[0][4 * fg + uu][col] = x[uu];
      out.A[1][4 * fg + uu][col] = rr[uu];
    }
  }
  __syncthreads();

  // record -> workspace (a slow chunk's record carries only its flag)
  float* dst = rec + ((size_t)bh * nck + c) * REC;
  for (int i4 = tid; i4 < REC4; i4 += 256) {
    const int o = 4 * i4;
    if (slow && o < O_FLAG) continue;
    *reinterpret_cast<f4*>(dst + o) = ld4(rec_lds(out, o));
  }
}

// ------------------------------------------------------------------ scan --
// HAS_Y: y is written.  The chunk loop keeps its stores free of branches
// (y presence is a compile-time switch, tail tokens store to a sink): with
// straight-line stores the compiler's memory-counter waits stay exact, so the
// stores of one chunk are not waited for at the next barrier.
template <typename T, bool HAS_Y>
__global__ __launch_bounds__(256) void fwd_scan(
    int Tn, int H, const T* __restrict__ r, const T* __restrict__ w, const T* __restrict__ k,
    const T* __restrict__ v, const T* __restrict__ a, const T* __restrict__ bv,
    float* __restrict__ rec, const float* __restrict__ s0, T* __restrict__ y,
    float* __restrict__ sT, float* __restrict__ ckpt, float* __restrict__ sa_all) {
  __shared__ __attribute__((aligned(16))) ChunkLds buf[2];
  constexpr int PER = (REC4 + 255) / 256;

  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int row = 16 * wave + fr;  // state row i owned by this lane
  const size_t C = (size_t)H * N;
  const size_t vbase = (size_t)b * Tn * C + (size_t)h * N;
  const size_t sbase = (size_t)bh * N * N;
  const int nck = (Tn + L - 1) / L;
  const float* recs = rec + (size_t)bh * nck * REC;
  // per-head scratch after all records: the y of tail tokens (L x N of T),
  // then the checkpoint stores when no checkpoints are wanted (N x N fp32)
  float* sinkh = rec + (size_t)gridDim.x * nck * REC + (size_t)bh * SINK;
  T* sink = reinterpret_cast<T*>(sinkh);
  float* ckb = ckpt ? ckpt + (size_t)bh * nck * N * N : sinkh + L * N;
  const size_t ck_stride = ckpt ? (size_t)N * N : 0;
  // sa of token t: sa_all[vbase + t*C + i] when wanted, else the sink
  float* sa_sink = sinkh + L * N + N * N;

  f4 ST[4];
#pragma unroll
  for (int jt = 0; jt < 4; jt++)
    ST[jt] = s0 ? ld4(s0 + sbase + (size_t)row * N + 16 * jt + 4 * fg) : f4{0.f, 0.f, 0.f, 0.f};

  // Records travel global -> registers -> LDS two chunks ahead (the loads of
  // chunk c+2 are issued at chunk c and land in LDS at chunk c+1).  Every
  // memory access of the loop is unconditional (clamped chunk index,
  // precomputed LDS slots, sinks for unwanted stores), so the compiler's
  // memory-counter waits stay exact and no barrier waits for stores.
  int loff[PER];  // LDS float offset of each of this thread's record float4
#pragma unroll
  for (int q = 0; q < PER; q++) {
    const int i4 = tid + 256 * q;
    float* p = i4 < REC4 ? rec_lds(buf[0], 4 * i4) : &buf[0].flag[4];  // spare slot
    loff[q] = (int)(p - reinterpret_cast<float*>(&buf[0]));
  }
  f4 preA[PER], preB[PER];
  auto fetch = [&](f4 (&pre)[PER], int c) {
    const float* src = recs + (size_t)min(c, nck - 1) * REC;
#pragma unroll
    for (int q = 0; q < PER; q++) pre[q] = ld4(src + 4 * min(tid + 256 * q, REC4 - 1));
  };
  auto commit = [&](const f4 (&pre)[PER], int bi) {
    float* base = reinterpret_cast<float*>(&buf[bi]);
#pragma unroll
    for (int q = 0; q < PER; q++) *reinterpret_cast<f4*>(base + loff[q]) = pre[q];
  };

  auto chunk = [&](int c) {
    const int t0 = c * L;
    ChunkLds& d = buf[c & 1];
    {
      float* cp = ckb + (size_t)c * ck_stride + (size_t)row * N + 4 * fg;
#pragma unroll
      for (int jt = 0; jt < 4; jt++) *reinterpret_cast<f4*>(cp + 16 * jt) = ST[jt];
    }
    if (d.flag[0] == 0.f) {
      const f4 vt = ld4(&d.T3[2][row][4 * fg]);  // V[4g+s][row]
      const f4 z = {0.f, 0.f, 0.f, 0.f};
      // two half chains per product, summed at the end
      f4 sa0 = mma16(ld4(&d.QW[0][fr][4 * fg]), vt, z), sa1 = z;
      f4 yv0 = mma16(ld4(&d.QW[1][fr][4 * fg]), vt, z), yv1 = z;
#pragma unroll
      for (int jt = 0; jt < 4; jt += 2) {
        sa0 = mma16(ld4(&d.A[0][fr][16 * jt + 4 * fg]), ST[jt], sa0);
        sa1 = mma16(ld4(&d.A[0][fr][16 * jt + 16 + 4 * fg]), ST[jt + 1], sa1);
        yv0 = mma16(ld4(&d.A[1][fr][16 * jt + 4 * fg]), ST[jt], yv0);
        yv1 = mma16(ld4(&d.A[1][fr][16 * jt + 16 + 4 * fg]), ST[jt + 1], yv1);
      }
      const f4 sa = sa0 + sa1, yv = yv0 + yv1;
#pragma unroll
      for (int jt = 0; jt < 4; jt++) {
        f4 s = ST[jt] * ld4(&d.lam[16 * jt + 4 * fg]);
        s = mma16(ld4(&d.T3[1][16 * jt + fr][4 * fg]), vt, s);
        ST[jt] = mma16(ld4(&d.T3[0][16 * jt + fr][4 * fg]), sa, s);
      }
      if (HAS_Y) {
        // yv: lane holds Y[t = 4g+u][i = row]; tokens past the end go to
        // this head's sink instead (a select, not a branch)
#pragma unroll
        for (int uu = 0; uu < 4; uu++) {
          const int t = t0 + 4 * fg + uu;
          T* dst = t < Tn ? y + vbase + (size_t)t * C + row : sink + (4 * fg + uu) * N + row;
          store1(dst, yv[uu]);
        }
      }
      // sa, laid out like yv
#pragma unroll
      for (int uu = 0; uu < 4; uu++) {
        const int t = t0 + 4 * fg + uu;
        float* dst = (sa_all && t < Tn) ? sa_all + vbase + (size_t)t * C + row : sa_sink + (4 * fg + uu) * N + row;
        *dst = sa[uu];
      }
    } else {
      // token by token (extreme decay), inputs straight from memory
      const int ns = min(L, Tn - t0);
      for (int t = t0; t < t0 + ns; t++) {
        const size_t o = vbase + (size_t)t * C;
        float part = 0.f;
#pragma unroll
        for (int jt = 0; jt < 4; jt++) {
          const f4 av = load4(a + o + 16 * jt + 4 * fg);
#pragma unroll
          for (int uu = 0; uu < 4; uu++) part = fmaf(ST[jt][uu], av[uu], part);
        }
        const float sav = rows4sum(part);
        if (sa_all && fg == 0) sa_all[o + row] = sav;
        const float vv = load1(v + o + row);
        float yp = 0.f;
#pragma unroll
        for (int jt = 0; jt < 4; jt++) {
          const f4 wv = load4(w + o + 16 * jt + 4 * fg), bb = load4(bv + o + 16 * jt + 4 * fg);
          const f4 kv = load4(k + o + 16 * jt + 4 * fg), rv = load4(r + o + 16 * jt + 4 * fg);
#pragma unroll
          for (int uu = 0; uu < 4; uu++) {
            ST[jt][uu] = fmaf(vv, kv[uu], fmaf(sav, bb[uu], ST[jt][uu] * wv[uu]));
            yp = fmaf(ST[jt][uu], rv[uu], yp);
          }
        }
        const float yt = rows4sum(yp);
        if (HAS_Y && fg == 0) store1(y + o + row, yt);
      }
    }
  };

  fetch(preA, 0);
  fetch(preB, 1);
  commit(preA, 0);
  __syncthreads();
  // chunk c reads buf[c & 1]; preB holds chunk c+1 when c is even, preA when
  // c is odd.  A commit into the other buffer comes after every read of it
  // (those were before the previous barrier).
  for (int c = 0; c < nck; c += 2) {
    fetch(preA, c + 2);
    chunk(c);
    commit(preB, 1);
    lds_barrier();
    if (c + 1 >= nck) break;
    fetch(preB, c + 3);
    chunk(c + 1);
    commit(preA, 0);
    lds_barrier();
  }

  if (sT) {
    float* sp = sT + sbase + (size_t)row * N + 4 * fg;
#pragma unroll
    for (int jt = 0; jt < 4; jt++) *reinterpret_cast<f4*>(sp + 16 * jt) = ST[jt];
  }
}

}  // namespace wkv7c

size_t wkv7_chunk_ws_floats(int B, int T, int H) {
  // records, then the scan's per-head sink
  return (size_t)B * H * (((T + wkv7c::L - 1) / wkv7c::L) * wkv7c::REC + wkv7c::SINK);
}

hipError_t wkv7_launch_forward_chunked(int dtype, int B, int T, int H, const void* r, const void* w,
                                       const void* k, const void* v, const void* a, const void* b,
                                       const float* s0, void* y, float* sT, float* ckpt, float* ws,
                                       hipStream_t st) {
  const int nck = (T + wkv7c::L - 1) / wkv7c::L;
  const dim3 block(256);
  float* sa = ckpt ? wkv7_ckpt_sa(ckpt, B, T, H) : nullptr;
  if (dtype == 1) {
    typedef bf16_t X;
    hipLaunchKernelGGL((wkv7c::fwd_prep<X>), dim3(B * H * nck), block, 0, st, T, H, nck,
                       (const X*)r, (const X*)w, (const X*)k, (const X*)v, (const X*)a,
                       (const X*)b, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (y)
      hipLaunchKernelGGL((wkv7c::fwd_scan<X, true>), dim3(B * H), block, 0, st, T, H, (const X*)r,
                         (const X*)w, (const X*)k, (const X*)v, (const X*)a, (const X*)b, ws, s0,
                         (X*)y, sT, ckpt, sa);
    else
      hipLaunchKernelGGL((wkv7c::fwd_scan<X, false>), dim3(B * H), block, 0, st, T, H, (const X*)r,
                         (const X*)w, (const X*)k, (const X*)v, (const X*)a, (const X*)b, ws, s0,
                         (X*)y, sT, ckpt, sa);
  } else {
    typedef float X;
    hipLaunchKernelGGL((wkv7c::fwd_prep<X>), dim3(B * H * nck), block, 0, st, T, H, nck,
                       (const X*)r, (const X*)w, (const X*)k, (const X*)v, (const X*)a,
                       (const X*)b, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (y)
      hipLaunchKernelGGL((wkv7c::fwd_scan<X, true>), dim3(B * H), block, 0, st, T, H, (const X*)r,
                         (const X*)w, (const X*)k, (const X*)v, (const X*)a, (const X*)b, ws, s0,
                         (X*)y, sT, ckpt, sa);
    else
      hipLaunchKernelGGL((wkv7c::fwd_scan<X, false>), dim3(B * H), block, 0, st, T, H, (const X*)r,
                         (const X*)w, (const X*)k, (const X*)v, (const X*)a, (const X*)b, ws, s0,
                         (X*)y, sT, ckpt, sa);
  }
  return hipGetLastError();
}
