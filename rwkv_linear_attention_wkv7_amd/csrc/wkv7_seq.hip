// WKV7 recurrence on gfx950: token-sequential forward and the
// checkpoint-recomputing backward (the single-token decode step is in
// wkv7_step.hip, the chunked matrix-core forward in wkv7_chunk.hip).
//
// The recurrence (per batch b, head h, token t; S is 64x64 fp32, S[i][j] with
// i = value row, j = key column), as passed to the WKV7 kernel on the
// "Foundry/cuda_kernels/timemix.cu" page (k_composites: a = -kk, b = kk*a)
// and differentiated in the WKV state-backward block of "infotheory
// .../rwkv7/model.rs":
//     sa  = S a_t ;  S = S diag(w_t) + sa b_t^T + v_t k_t^T ;  y_t = S r_t
//
// Every state row evolves independently of the others (row i only needs
// v_t[i] and its own sa[i]), so rows are spread over lanes and workgroups: a
// lane owns RPT rows x 4 adjacent columns, 16 lanes (one DPP row) cover the 64
// columns of a state row, and the row dot products (S a, S r) are 16-lane DPP
// sums.  The per-token vectors are staged through LDS in blocks of 16 tokens
// and read as float4 by every row a lane owns.
//
// Backward: with G = dL/dS_t the reverse step is row-local too (G rows evolve
// independently), except for the column sums dr, dk, db, dw, da over the 64
// rows.  Those are reduced in-thread over a lane's rows, across the wave's
// four 16-lane rows with gfx950 permlane swaps, across the workgroup's waves
// through LDS once per 16-token chunk, and across the workgroups that share a
// head through fp32 partial buffers summed by a second kernel in fixed order.

#include <type_traits>

#include "common.hpp"

namespace wkv7k {

constexpr int N = WKV7_N;
constexpr int TT = 16;    // tokens per LDS staging block
constexpr int CKL = WKV7_CKL;  // checkpoint interval (tokens) = backward chunk
static_assert(CKL == TT, "checkpoints are taken at block starts");

__device__ __forceinline__ float dot4(const float (&s)[4], f4 v) {
  return fmaf(s[3], v[3], fmaf(s[2], v[2], fmaf(s[1], v[1], s[0] * v[0])));
}

// ------------------------------------------------------------------ forward
// Grid: B*H*(64/(16*RPT)) workgroups of 256 threads; workgroup -> (b, h, row
// block of 16*RPT rows).  Thread: column group cg = tid%16 (columns 4cg..4cg+3),
// row group rg = tid/16 owning rows rb*16*RPT + rg*RPT + m, m < RPT.
template <int RPT, typename T>
__global__ __launch_bounds__(256) void fwd_seq(
    int B, int Tn, int H, const T* __restrict__ r, const T* __restrict__ w,
    const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ a,
    const T* __restrict__ bv, const float* __restrict__ s0, T* __restrict__ y,
    float* __restrict__ sT, float* __restrict__ ckpt, float* __restrict__ sa_out) {
  constexpr int ROWS = 16 * RPT;
  constexpr int NRB = N / ROWS;
  // staging: r, w, k, a, b of each token and v of this slice travel raw
  // (unconverted) through registers and are widened to fp32 once, when the
  // block is written to LDS (every value is read by all 16 row groups)
  __shared__ __attribute__((aligned(16))) float sv[2][TT][5][N];
  __shared__ __attribute__((aligned(16))) float svv[2][TT][ROWS];
  typedef typename Raw<T>::v4 R4;
  typedef typename Raw<T>::v1 R1;

  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = g / NRB, rb = g - bh * NRB;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, cg = tid & 15, rg = tid >> 4;
  const int rloc0 = rg * RPT;
  const int row0 = rb * ROWS + rloc0;
  const size_t C = (size_t)H * N;
  const size_t vbase = (size_t)b * Tn * C + (size_t)h * N;
  const size_t sbase = ((size_t)b * H + h) * N * N;
  const int nck = (Tn + CKL - 1) / CKL;

  float S[RPT][4];
#pragma unroll
  for (int m = 0; m < RPT; m++) {
    f4 x = {0.f, 0.f, 0.f, 0.f};
    if (s0) x = *reinterpret_cast<const f4*>(s0 + sbase + (size_t)(row0 + m) * N + cg * 4);
#pragma unroll
    for (int c = 0; c < 4; c++) S[m][c] = x[c];
  }

  auto vec_ptr = [&](int vi) -> const T* {
    return vi == 0 ? r : vi == 1 ? w : vi == 2 ? k : vi == 3 ? a : bv;
  };
  constexpr int NV4 = TT * 5 * 16;  // float4 slots per block
  constexpr int NV4_PER = NV4 / 256;
  static_assert(NV4 % 256 == 0, "block staging assumes 256 threads");
  constexpr int NVV_PER = (TT * ROWS + 255) / 256;
  R4 pre[NV4_PER];
  R1 prev[NVV_PER];

  // thread -> (token, vector, column group) slots of the staged block, fixed
  // for the whole kernel: the source rows are resolved once.  Loads are
  // unconditional from clamped (always valid) token indices so that all of
  // them are in flight together; tokens past the end are never used.
  const T* src4[NV4_PER];
  int tok4[NV4_PER];
#pragma unroll
  for (int q = 0; q < NV4_PER; q++) {
    const int f = tid + 256 * q;
    const int tok = f / 80, rem = f - tok * 80, vi = rem >> 4, c4 = rem & 15;
    src4[q] = vec_ptr(vi) + vbase + c4 * 4;
    tok4[q] = tok;
  }
  auto load_block = [&](int t0) {
#pragma unroll
    for (int q = 0; q < NV4_PER; q++)
      pre[q] = load_raw4(src4[q] + (size_t)min(t0 + tok4[q], Tn - 1) * C);
#pragma unroll
    for (int q = 0; q < NVV_PER; q++) {
      const int f = min(tid + 256 * q, TT * ROWS - 1);
      const int tok = f / ROWS, rr = f - tok * ROWS;
      const int tc = min(t0 + tok, Tn - 1);
      prev[q] = load_raw1(v + vbase + (size_t)tc * C + rb * ROWS + rr);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int q = 0; q < NV4_PER; q++) {
      const int f = tid + 256 * q;
      const int tok = f / 80, rem = f - tok * 80, vi = rem >> 4, c4 = rem & 15;
      *reinterpret_cast<f4*>(&sv[buf][tok][vi][c4 * 4]) = raw4_to_f4<T>(pre[q]);
    }
#pragma unroll
    for (int q = 0; q < NVV_PER; q++) {
      const int f = tid + 256 * q;
      if (f < TT * ROWS) {
        const int tok = f / ROWS, rr = f - tok * ROWS;
        svv[buf][tok][rr] = raw1_to_f32<T>(prev[q]);
      }
    }
  };

  // one token; the row sums of y (and sa) stay with the lane whose cg equals tt
  float yb[RPT], sab[RPT];
  struct Tok {
    f4 av, wv, kv, bb, rv;
    float vv[RPT];
  };
  auto ldtok = [&](int buf, int tt, Tok& o) {
    o.av = load4(&sv[buf][tt][3][cg * 4]);
    o.wv = load4(&sv[buf][tt][1][cg * 4]);
    o.kv = load4(&sv[buf][tt][2][cg * 4]);
    o.bb = load4(&sv[buf][tt][4][cg * 4]);
    o.rv = load4(&sv[buf][tt][0][cg * 4]);
#pragma unroll
    for (int m = 0; m < RPT; m++) o.vv[m] = load1(&svv[buf][tt][rloc0 + m]);
  };
  auto token_in = [&](const Tok& in, int tt) {
    const f4 av = in.av, wv = in.wv, kv = in.kv, bb = in.bb, rv = in.rv;
    float sa[RPT];
#pragma unroll
    for (int m = 0; m < RPT; m++) sa[m] = dot4(S[m], av);
#pragma unroll
    for (int m = 0; m < RPT; m++) sa[m] = rowsum16(sa[m]);
#pragma unroll
    for (int m = 0; m < RPT; m++) {
      sab[m] = (cg == tt) ? sa[m] : sab[m];
#pragma unroll
      for (int c = 0; c < 4; c++) S[m][c] = fmaf(in.vv[m], kv[c], fmaf(sa[m], bb[c], S[m][c] * wv[c]));
    }
    float yy[RPT];
#pragma unroll
    for (int m = 0; m < RPT; m++) yy[m] = dot4(S[m], rv);
#pragma unroll
    for (int m = 0; m < RPT; m++) {
      yy[m] = rowsum16(yy[m]);
      yb[m] = (cg == tt) ? yy[m] : yb[m];
    }
  };
  auto token = [&](int buf, int tt) {
    const f4 av = load4(&sv[buf][tt][3][cg * 4]);
    const f4 wv = load4(&sv[buf][tt][1][cg * 4]), kv = load4(&sv[buf][tt][2][cg * 4]);
    const f4 bb = load4(&sv[buf][tt][4][cg * 4]), rv = load4(&sv[buf][tt][0][cg * 4]);
    float sa[RPT];
#pragma unroll
    for (int m = 0; m < RPT; m++) sa[m] = dot4(S[m], av);
#pragma unroll
    for (int m = 0; m < RPT; m++) sa[m] = rowsum16(sa[m]);
#pragma unroll
    for (int m = 0; m < RPT; m++) {
      const float vv = load1(&svv[buf][tt][rloc0 + m]);
      sab[m] = (cg == tt) ? sa[m] : sab[m];
#pragma unroll
      for (int c = 0; c < 4; c++) S[m][c] = fmaf(vv, kv[c], fmaf(sa[m], bb[c], S[m][c] * wv[c]));
    }
    float yy[RPT];
#pragma unroll
    for (int m = 0; m < RPT; m++) yy[m] = dot4(S[m], rv);
#pragma unroll
    for (int m = 0; m < RPT; m++) {
      yy[m] = rowsum16(yy[m]);
      yb[m] = (cg == tt) ? yy[m] : yb[m];
    }
  };

  load_block(0);
  store_block(0);
  __syncthreads();
  int buf = 0;
  for (int t0 = 0; t0 < Tn; t0 += TT, buf ^= 1) {
    const bool more = t0 + TT < Tn;
    if (more) load_block(t0 + TT);
    if (ckpt) {
      float* cp = ckpt + (((size_t)bh * nck + t0 / CKL) * N + row0) * N + cg * 4;
#pragma unroll
      for (int m = 0; m < RPT; m++)
        *reinterpret_cast<f4*>(cp + (size_t)m * N) = f4{S[m][0], S[m][1], S[m][2], S[m][3]};
    }
    const int nt = min(TT, Tn - t0);
#pragma unroll
    for (int m = 0; m < RPT; m++) yb[m] = sab[m] = 0.f;
    if (nt == TT) {
      // The next token's inputs are read from LDS while this one runs.  The
      // state after token tt - 1 gives both y_{tt-1} (with r_{tt-1}) and
      // sa_tt (with a_tt): the two dot products and row sums are formed
      // together, so the read-out of one token overlaps the state step of
      // the next instead of following it.
      Tok tc, tn, tn2;
      ldtok(buf, 0, tc);
      ldtok(buf, 1, tn);
      f4 rprev = tc.rv;
#pragma unroll
      for (int tt = 0; tt < TT; tt++) {
        if (tt + 2 < TT) ldtok(buf, tt + 2, tn2);
        __builtin_amdgcn_sched_barrier(0);
        float sa[RPT], yy[RPT];
#pragma unroll
        for (int m = 0; m < RPT; m++) {
          sa[m] = dot4(S[m], tc.av);
          if (tt > 0) yy[m] = dot4(S[m], rprev);
        }
#pragma unroll
        for (int m = 0; m < RPT; m++) {
          sa[m] = rowsum16(sa[m]);
          if (tt > 0) yy[m] = rowsum16(yy[m]);
        }
#pragma unroll
        for (int m = 0; m < RPT; m++) {
          sab[m] = (cg == tt) ? sa[m] : sab[m];
          if (tt > 0) yb[m] = (cg == tt - 1) ? yy[m] : yb[m];
#pragma unroll
          for (int c = 0; c < 4; c++)
            S[m][c] = fmaf(tc.vv[m], tc.kv[c], fmaf(sa[m], tc.bb[c], S[m][c] * tc.wv[c]));
        }
        rprev = tc.rv;
        tc = tn;
        tn = tn2;
      }
#pragma unroll
      for (int m = 0; m < RPT; m++) {
        const float y15 = rowsum16(dot4(S[m], rprev));
        yb[m] = (cg == TT - 1) ? y15 : yb[m];
      }
    } else {
      for (int tt = 0; tt < nt; tt++) token(buf, tt);
    }
    if (y && cg < nt) {
      T* yp = y + vbase + (size_t)(t0 + cg) * C + row0;
#pragma unroll
      for (int m = 0; m < RPT; m++) store1(yp + m, yb[m]);
    }
    if (sa_out && cg < nt) {
      float* sp = sa_out + vbase + (size_t)(t0 + cg) * C + row0;
#pragma unroll
      for (int m = 0; m < RPT; m++) sp[m] = sab[m];
    }
    if (more) store_block(buf ^ 1);
    lds_barrier();
  }

  if (sT) {
#pragma unroll
    for (int m = 0; m < RPT; m++)
      *reinterpret_cast<f4*>(sT + sbase + (size_t)(row0 + m) * N + cg * 4) =
          f4{S[m][0], S[m][1], S[m][2], S[m][3]};
  }
}

// ----------------------------------------------------------------- backward
// Workgroup = (b, h, one of NSPLIT row slices of ROWS = RPT*RG rows), 16*RG
// threads.  Thread: column group cg = tid%16, rows slice*ROWS + rg*RPT + m.
// Chunks of CKL tokens are processed last to first; each is recomputed from
// its checkpoint with the states before every token kept in registers.
// Output: fp32 column partials part[slice][vec][B][T][H][N] for vec = dr, dk,
// db, dw, da (summed over the slices by reduce_partials), dv directly.
template <int RPT, int RG, typename T>
__global__ __launch_bounds__(16 * RG) void bwd_seq(
    int B, int Tn, int H, const T* __restrict__ r, const T* __restrict__ w,
    const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ a,
    const T* __restrict__ bv, const T* __restrict__ dy, const float* __restrict__ ckpt,
    const float* __restrict__ dsT, float* __restrict__ part, T* __restrict__ dv,
    float* __restrict__ ds0, int c_lo, int c_hi, const int* __restrict__ gate) {
  // chunks [c_lo, c_hi) of the sequence are processed (last to first); G
  // enters as dsT (the gradient of the state after chunk c_hi - 1) and leaves
  // as ds0 (before chunk c_lo), so a long sequence can run as several launches.
  // gate: NULL, or a flag that is nonzero when this kernel (rather than the
  // two-pass backward) is to produce the results; zero: return at once.
  if (gate && !*gate) return;
  constexpr int ROWS = RPT * RG, NSPLIT = N / ROWS, NW = RG / 4, NT = 16 * RG;
  static_assert(RG % 4 == 0, "whole waves");
  // staging, double-buffered, widened to fp32 once on the way into LDS: the
  // next (earlier) chunk is fetched raw into registers while the current one
  // is processed
  __shared__ __attribute__((aligned(16))) float sv[2][CKL][5][N];   // r, w, k, a, b
  __shared__ __attribute__((aligned(16))) float svr[2][CKL][2][ROWS];  // v, dy of this slice
  __shared__ __attribute__((aligned(16))) float red[NW][CKL][5][N];  // per-wave column partials
  typedef typename Raw<T>::v4 R4;
  typedef typename Raw<T>::v1 R1;

  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = g / NSPLIT, sp = g - bh * NSPLIT;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, cg = tid & 15, rg = tid >> 4;
  const int lane = tid & 63, wave = tid >> 6;
  const int rloc0 = rg * RPT;
  const int row0 = sp * ROWS + rloc0;
  const size_t C = (size_t)H * N;
  const size_t vbase = (size_t)b * Tn * C + (size_t)h * N;
  const size_t sbase = ((size_t)b * H + h) * N * N;
  const size_t plane = (size_t)B * Tn * C;  // elements of one gradient tensor
  const int nck = (Tn + CKL - 1) / CKL;
  auto vec_ptr = [&](int vi) -> const T* {
    return vi == 0 ? r : vi == 1 ? w : vi == 2 ? k : vi == 3 ? a : bv;
  };

  float G[RPT][4];
#pragma unroll
  for (int m = 0; m < RPT; m++) {
    f4 x = {0.f, 0.f, 0.f, 0.f};
    if (dsT) x = *reinterpret_cast<const f4*>(dsT + sbase + (size_t)(row0 + m) * N + cg * 4);
#pragma unroll
    for (int c = 0; c < 4; c++) G[m][c] = x[c];
  }

  // unconditional loads from clamped token indices (all in flight together).
  // Each thread's staging slots are fixed for the whole kernel, so their
  // source rows (tensor, column group) are resolved once here; a chunk only
  // adds its token offset.  The chunk's checkpoint rows are fetched first,
  // with its vectors, one chunk ahead: a wait for any staged value then
  // covers them, and no wait ever has to reach past the column-partial
  // stores of the chunk before (the memory counter is in order and counts
  // stores too).
  constexpr int NA = (CKL * 80 + NT - 1) / NT, NB = (CKL * 2 * ROWS + NT - 1) / NT;
  R4 xa[NA];
  R1 xb[NB];
  f4 xck[RPT];
  const T* srca[NA];
  int toka[NA];
  const T* srcb[NB];
  int tokb[NB];
#pragma unroll
  for (int q = 0; q < NA; q++) {
    const int f = min(tid + NT * q, CKL * 80 - 1);
    const int tok = f / 80, rem = f - tok * 80, vi = rem >> 4, c4 = rem & 15;
    srca[q] = vec_ptr(vi) + vbase + c4 * 4;
    toka[q] = tok;
  }
#pragma unroll
  for (int q = 0; q < NB; q++) {
    const int f = min(tid + NT * q, CKL * 2 * ROWS - 1);
    const int tok = f / (2 * ROWS), rem = f - tok * 2 * ROWS, vi = rem / ROWS, i = rem - vi * ROWS;
    srcb[q] = (vi ? dy : v) + vbase + sp * ROWS + i;
    tokb[q] = tok;
  }
  const float* ckrow = ckpt + ((size_t)bh * nck * N + row0) * N + cg * 4;
  auto fetch = [&](int c) {
    const int tc0 = c * CKL, ns = min(CKL, Tn - tc0);
#pragma unroll
    for (int m = 0; m < RPT; m++)
      xck[m] = *reinterpret_cast<const f4*>(ckrow + ((size_t)c * N + m) * N);
#pragma unroll
    for (int q = 0; q < NA; q++) xa[q] = load_raw4(srca[q] + (size_t)(tc0 + min(toka[q], ns - 1)) * C);
#pragma unroll
    for (int q = 0; q < NB; q++) xb[q] = load_raw1(srcb[q] + (size_t)(tc0 + min(tokb[q], ns - 1)) * C);
  };
  // Tokens past the end of a partial chunk are staged as identity steps
  // (w = 1; r, k, v, a, b, dy = 0): the state and its gradient pass through
  // them unchanged and contribute nothing, so the token loops need no guards.
  auto commit = [&](int buf, int ns) {
#pragma unroll
    for (int q = 0; q < NA; q++) {
      const int f = tid + NT * q;
      if (f < CKL * 80) {
        const int tok = f / 80, rem = f - tok * 80, vi = rem >> 4, c4 = rem & 15;
        const float pad = vi == 1 ? 1.f : 0.f;
        *reinterpret_cast<f4*>(&sv[buf][tok][vi][c4 * 4]) =
            tok < ns ? raw4_to_f4<T>(xa[q]) : f4{pad, pad, pad, pad};
      }
    }
#pragma unroll
    for (int q = 0; q < NB; q++) {
      const int f = tid + NT * q;
      if (f < CKL * 2 * ROWS) {
        const int tok = f / (2 * ROWS), rem = f - tok * 2 * ROWS, vi = rem / ROWS, i = rem - vi * ROWS;
        svr[buf][tok][vi][i] = tok < ns ? raw1_to_f32<T>(xb[q]) : 0.f;
      }
    }
  };

  // One chunk of ns valid tokens, all CKL staged ones processed (identity
  // padding), so the unrolled tokens are scheduled together.  Sh[0] is the
  // chunk's checkpoint on entry.
  float Sh[CKL + 1][RPT][4];
  auto chunk = [&](int buf, int tc0, int ns) {
    // recompute: Sh[tt] = state before token tt, sah[tt] = S a_tt (the next
    // token's inputs are read while the current one is processed)
    float sah[CKL][RPT];
    struct Fw {
      f4 av, wv, kv, bb;
      float vv[RPT];
    };
    auto ldfw = [&](int tt, Fw& o) {
      o.av = load4(&sv[buf][tt][3][cg * 4]);
      o.wv = load4(&sv[buf][tt][1][cg * 4]);
      o.kv = load4(&sv[buf][tt][2][cg * 4]);
      o.bb = load4(&sv[buf][tt][4][cg * 4]);
#pragma unroll
      for (int m = 0; m < RPT; m++) o.vv[m] = load1(&svr[buf][tt][0][rloc0 + m]);
    };
    {
      Fw fc, fn;
      ldfw(0, fc);
#pragma unroll
      for (int tt = 0; tt < CKL; tt++) {
        if (tt + 1 < CKL) ldfw(tt + 1, fn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < RPT; m++) sah[tt][m] = dot4(Sh[tt][m], fc.av);
#pragma unroll
        for (int m = 0; m < RPT; m++) sah[tt][m] = rowsum16(sah[tt][m]);
#pragma unroll
        for (int m = 0; m < RPT; m++) {
#pragma unroll
          for (int cc = 0; cc < 4; cc++)
            Sh[tt + 1][m][cc] =
                fmaf(fc.vv[m], fc.kv[cc], fmaf(sah[tt][m], fc.bb[cc], Sh[tt][m][cc] * fc.wv[cc]));
        }
        fc = fn;
      }
    }

    float dvb[RPT];
#pragma unroll
    for (int m = 0; m < RPT; m++) dvb[m] = 0.f;
    // one token's staged inputs; the next (earlier) token's are read from
    // LDS while the current one is processed
    struct Tok {
      f4 rv, wv, kv, av, bb;
      float vv[RPT], dyv[RPT];
    };
    auto ldtok = [&](int tt, Tok& o) {
      o.rv = load4(&sv[buf][tt][0][cg * 4]);
      o.wv = load4(&sv[buf][tt][1][cg * 4]);
      o.kv = load4(&sv[buf][tt][2][cg * 4]);
      o.av = load4(&sv[buf][tt][3][cg * 4]);
      o.bb = load4(&sv[buf][tt][4][cg * 4]);
#pragma unroll
      for (int m = 0; m < RPT; m++) {
        o.vv[m] = load1(&svr[buf][tt][0][rloc0 + m]);
        o.dyv[m] = load1(&svr[buf][tt][1][rloc0 + m]);
      }
    };
    Tok cur, nxt;
    ldtok(CKL - 1, cur);
#pragma unroll
    for (int tt = CKL - 1; tt >= 0; tt--) {
      {
        if (tt > 0) ldtok(tt - 1, nxt);
        // keep those reads here, ahead of this token's work (the scheduler
        // would otherwise sink them below this token's LDS writes)
        __builtin_amdgcn_sched_barrier(0);
        const f4 rv = cur.rv, wv = cur.wv, kv = cur.kv, av = cur.av, bb = cur.bb;
        float vv[RPT], dyv[RPT], dvv[RPT], dsa[RPT];
#pragma unroll
        for (int m = 0; m < RPT; m++) {
          vv[m] = cur.vv[m];
          dyv[m] = cur.dyv[m];
        }
#pragma unroll
        for (int m = 0; m < RPT; m++)
#pragma unroll
          for (int cc = 0; cc < 4; cc++) G[m][cc] = fmaf(dyv[m], rv[cc], G[m][cc]);
#pragma unroll
        for (int m = 0; m < RPT; m++) {
          dvv[m] = dot4(G[m], kv);
          dsa[m] = dot4(G[m], bb);
        }
#pragma unroll
        for (int m = 0; m < RPT; m++) {
          dvv[m] = rowsum16(dvv[m]);
          dsa[m] = rowsum16(dsa[m]);
          dvb[m] = (cg == tt) ? dvv[m] : dvb[m];
        }
        // column partials over this lane's rows: x[cc*5 + vec], vec = dr, dk, db, dw, da
        float x[20];
#pragma unroll
        for (int cc = 0; cc < 4; cc++) {
          float xr = 0.f, xk = 0.f, xb = 0.f, xw = 0.f, xa = 0.f;
#pragma unroll
          for (int m = 0; m < RPT; m++) {
            xr = fmaf(Sh[tt + 1][m][cc], dyv[m], xr);
            xk = fmaf(G[m][cc], vv[m], xk);
            xb = fmaf(G[m][cc], sah[tt][m], xb);
            xw = fmaf(G[m][cc], Sh[tt][m][cc], xw);
            xa = fmaf(dsa[m], Sh[tt][m][cc], xa);
          }
          x[cc * 5 + 0] = xr; x[cc * 5 + 1] = xk; x[cc * 5 + 2] = xb;
          x[cc * 5 + 3] = xw; x[cc * 5 + 4] = xa;
        }
#pragma unroll
        for (int m = 0; m < RPT; m++)
#pragma unroll
          for (int cc = 0; cc < 4; cc++) G[m][cc] = fmaf(dsa[m], av[cc], G[m][cc] * wv[cc]);
        // after the reduce-scatter lane (row-in-wave q, cg) holds the wave's sums
        // for column 4*cg + q
        rows4_reduce_scatter<5>(x);
        const int col = cg * 4 + ((lane >> 4) & 3);
#pragma unroll
        for (int vi = 0; vi < 5; vi++) red[wave][tt][vi][col] = x[vi];
        cur = nxt;
      }
    }
    if (cg < ns) {
      T* dp = dv + vbase + (size_t)(tc0 + cg) * C + row0;
#pragma unroll
      for (int m = 0; m < RPT; m++) store1(dp + m, dvb[m]);
    }
    lds_barrier();
    constexpr int NRED = (CKL * 80 + NT - 1) / NT;
#pragma unroll
    for (int q = 0; q < NRED; q++) {
      const int f = tid + NT * q;
      if (f < ns * 80) {
        const int tok = f / 80, rem = f - tok * 80, vi = rem >> 4, c4 = rem & 15;
        f4 s4 = *reinterpret_cast<const f4*>(&red[0][tok][vi][c4 * 4]);
#pragma unroll
        for (int wv = 1; wv < NW; wv++) s4 += *reinterpret_cast<const f4*>(&red[wv][tok][vi][c4 * 4]);
        *reinterpret_cast<f4*>(part + ((size_t)sp * 5 + vi) * plane + vbase +
                               (size_t)(tc0 + tok) * C + c4 * 4) = s4;
      }
    }
  };

  fetch(c_hi - 1);
  commit(0, min(CKL, Tn - (c_hi - 1) * CKL));
  int buf = 0;
  for (int c = c_hi - 1; c >= c_lo; c--, buf ^= 1) {
    const int tc0 = c * CKL, ns = min(CKL, Tn - tc0);
#pragma unroll
    for (int m = 0; m < RPT; m++)
#pragma unroll
      for (int cc = 0; cc < 4; cc++) Sh[0][m][cc] = xck[m][cc];
    lds_barrier();  // staged chunk visible; previous readers of the other buffer done
    if (c > c_lo) fetch(c - 1);
    chunk(buf, tc0, ns);
    if (c > c_lo) commit(buf ^ 1, CKL);
  }
  if (ds0) {
#pragma unroll
    for (int m = 0; m < RPT; m++)
      *reinterpret_cast<f4*>(ds0 + sbase + (size_t)(row0 + m) * N + cg * 4) =
          f4{G[m][0], G[m][1], G[m][2], G[m][3]};
  }
}

// out_vec = sum over slices of part[slice][vec] (fixed order), cast to T,
// for tokens [t_lo, t_lo + t_len) of every sequence (rows of C4 float4).
template <typename T, int NS>
__global__ __launch_bounds__(256) void reduce_bwd_partials(size_t plane4, int Tn, int t_lo, int t_len,
                                                           int C4, const float* __restrict__ part,
                                                           T* dr, T* dk, T* db, T* dw, T* da,
                                                           const int* __restrict__ gate) {
  if (gate && !*gate) return;  // as in bwd_seq
  // U float4 per thread per pass, every slice's loads issued together
  // (clamped indices, guarded stores): enough loads in flight to stream the
  // partials at HBM rate.  The slices are summed in slice order.
  constexpr int U = 4;
  const size_t seq4 = (size_t)t_len * C4;                  // float4 per sequence in range
  const size_t seg4 = plane4 / ((size_t)Tn * C4) * seq4;   // float4 per vector in range
  const size_t n4 = seg4 * 5, stride = (size_t)gridDim.x * 256;
  const f4* P = reinterpret_cast<const f4*>(part);
  auto elem = [&](size_t i, int& vi) {
    vi = (int)(i / seg4);
    const size_t r = i - (size_t)vi * seg4, b = r / seq4;
    return (b * Tn + t_lo) * C4 + (r - b * seq4);
  };
  for (size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x; i0 < n4; i0 += stride * U) {
    f4 s[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      int vi;
      const size_t e4 = elem(min(i0 + u * stride, n4 - 1), vi);
      f4 x[NS];
#pragma unroll
      for (int sp = 0; sp < NS; sp++)
        x[sp] = __builtin_nontemporal_load(P + ((size_t)sp * 5 + vi) * plane4 + e4);
      s[u] = x[0];
#pragma unroll
      for (int sp = 1; sp < NS; sp++) s[u] += x[sp];
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const size_t i = i0 + u * stride;
      if (i < n4) {
        int vi;
        const size_t e4 = elem(i, vi);
        T* o = vi == 0 ? dr : vi == 1 ? dk : vi == 2 ? db : vi == 3 ? dw : da;
        store4(o + e4 * 4, s[u]);
      }
    }
  }
}

// Row slices per head.  A 256-thread workgroup's LDS (sv, svr, red: ~122-128
// KiB) leaves one workgroup per CU, so slices only pay while the grid still
// fits in one pass over the 256 CUs: four 16-row slices when B*H*4 <= 256
// (the recurrence is latency bound, so a slice of half the rows takes well
// over half the time and the idle CUs are the larger loss), else two 32-row
// slices (more slices would double the partial traffic and add passes).
int bwd_nsplit(int B, int H) { return (long)B * H * 4 <= 256 ? 4 : 2; }

// Forward rows per thread: 16-row workgroups (RPT = 1, four per head) when
// they fit one workgroup per CU, or fill whole rounds of the 256 CUs (up to
// two per CU); else 32-row ones.  A part-filled second round leaves the CUs
// that hold two 16-row workgroups to set the time: measured on MI355X, fp32,
// B=8 T=1024 H=12 (384 or 192 workgroups) 215 us at 16 rows, 193 at 32;
// B=4 T=2048 H=16 (256 / 128) 310 vs 371; bf16 B=4 T=8192 H=32 (512 / 256)
// 1509 vs 1550.
int fwd_rpt(int B, int H) {
  const long wg = (long)B * H * 4;
  return wg <= 256 || (wg <= 512 && wg % 256 == 0) ? 1 : 2;
}

}  // namespace wkv7k

// ------------------------------------------------------------ launchers ----
// (called from the C-ABI after argument validation)
namespace wkv7k {

template <typename T>
hipError_t launch_forward_t(int B, int T_, int H, const void* r, const void* w, const void* k,
                            const void* v, const void* a, const void* b, const float* s0, void* y,
                            float* sT, float* ckpt, hipStream_t st) {
  float* sa = ckpt ? wkv7_ckpt_sa(ckpt, B, T_, H) : nullptr;
  if (fwd_rpt(B, H) == 1)
    hipLaunchKernelGGL((fwd_seq<1, T>), dim3(B * H * 4), dim3(256), 0, st, B, T_, H, (const T*)r,
                       (const T*)w, (const T*)k, (const T*)v, (const T*)a, (const T*)b, s0, (T*)y,
                       sT, ckpt, sa);
  else
    hipLaunchKernelGGL((fwd_seq<2, T>), dim3(B * H * 2), dim3(256), 0, st, B, T_, H, (const T*)r,
                       (const T*)w, (const T*)k, (const T*)v, (const T*)a, (const T*)b, s0, (T*)y,
                       sT, ckpt, sa);
  return hipGetLastError();
}

// The reverse pass over chunks [c_lo, c_hi), then (on `rst`) the reduction
// of its column partials for those chunks' tokens.
template <typename T>
hipError_t launch_backward_t(int B, int T_, int H, const void* r, const void* w, const void* k,
                             const void* v, const void* a, const void* b, const void* dy,
                             const float* ckpt, const float* dsT, void* dr, void* dw, void* dk,
                             void* dv, void* da, void* db, float* ds0, float* part, int c_lo,
                             int c_hi, hipStream_t st, hipStream_t rst, hipEvent_t ready,
                             const int* gate) {
  const int ns = bwd_nsplit(B, H);
  const dim3 grid(B * H * ns);
  if (ns == 4)
    hipLaunchKernelGGL((bwd_seq<1, 16, T>), grid, dim3(256), 0, st, B, T_, H, (const T*)r,
                       (const T*)w, (const T*)k, (const T*)v, (const T*)a, (const T*)b,
                       (const T*)dy, ckpt, dsT, part, (T*)dv, ds0, c_lo, c_hi, gate);
  else
    hipLaunchKernelGGL((bwd_seq<2, 16, T>), grid, dim3(256), 0, st, B, T_, H, (const T*)r,
                       (const T*)w, (const T*)k, (const T*)v, (const T*)a, (const T*)b,
                       (const T*)dy, ckpt, dsT, part, (T*)dv, ds0, c_lo, c_hi, gate);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (rst != st) {
    if ((e = hipEventRecord(ready, st)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(rst, ready, 0)) != hipSuccess) return e;
  }
  const int t_lo = c_lo * CKL, t_len = min(T_, c_hi * CKL) - t_lo;
  const int C4 = H * N / 4;
  const size_t plane4 = (size_t)B * T_ * C4;
  size_t blocks = ((size_t)B * t_len * C4 * 5 + 1023) / 1024;
  if (blocks > 4096) blocks = 4096;
  if (ns == 4)
    hipLaunchKernelGGL((reduce_bwd_partials<T, 4>), dim3((unsigned)blocks), dim3(256), 0, rst,
                       plane4, T_, t_lo, t_len, C4, part, (T*)dr, (T*)dk, (T*)db, (T*)dw, (T*)da, gate);
  else
    hipLaunchKernelGGL((reduce_bwd_partials<T, 2>), dim3((unsigned)blocks), dim3(256), 0, rst,
                       plane4, T_, t_lo, t_len, C4, part, (T*)dr, (T*)dk, (T*)db, (T*)dw, (T*)da, gate);
  return hipGetLastError();
}


}  // namespace wkv7k

hipError_t wkv7_launch_forward_chunked(int dtype, int B, int T, int H, const void* r, const void* w,
                                       const void* k, const void* v, const void* a, const void* b,
                                       const float* s0, void* y, float* sT, float* ckpt, float* ws,
                                       hipStream_t st);

// Path choice.  The chunked matrix-core kernels run when the caller hands
// over a chunk workspace and T >= 2 chunks; otherwise (and for every forward
// the library runs internally) the token-sequential kernel.  Measured on
// MI355X, fp32 forward alone, chunked / sequential: 1.23 / 1.00 ms at B = 1,
// T = 8192, H = 16; 1.45 / 1.02 ms at B*H = 48; 0.28 / 0.28 ms at B = 4,
// T = 2048, H = 16: the chunk scan is a dependent chain of about 6 000
// cycles per 16-token chunk and head, longer than 16 sequential tokens of a
// head whose rows are spread over four workgroups.
bool wkv7_use_chunked(int T) { return T >= 2 * wkv7k::CKL; }

hipError_t wkv7_launch_forward(int dtype, int B, int T, int H, const void* r, const void* w,
                               const void* k, const void* v, const void* a, const void* b,
                               const float* s0, void* y, float* sT, float* ckpt, float* chunk_ws,
                               hipStream_t st) {
  if (chunk_ws && wkv7_use_chunked(T))
    return wkv7_launch_forward_chunked(dtype, B, T, H, r, w, k, v, a, b, s0, y, sT, ckpt, chunk_ws,
                                       st);
  if (dtype == 1)
    return wkv7k::launch_forward_t<bf16_t>(B, T, H, r, w, k, v, a, b, s0, y, sT, ckpt, st);
  return wkv7k::launch_forward_t<float>(B, T, H, r, w, k, v, a, b, s0, y, sT, ckpt, st);
}

size_t wkv7_bwd_partial_floats(int B, int T, int H) {
  return (size_t)wkv7k::bwd_nsplit(B, H) * 5 * B * T * H * WKV7_N;
}

hipError_t wkv7_launch_backward(int dtype, int B, int T, int H, const void* r, const void* w,
                                const void* k, const void* v, const void* a, const void* b,
                                const void* dy, const float* ckpt, const float* dsT, void* dr,
                                void* dw, void* dk, void* dv, void* da, void* db, float* ds0,
                                float* part, const int* gate, hipStream_t st) {
  const int nck = (T + wkv7k::CKL - 1) / wkv7k::CKL;
  if (dtype == 1)
    return wkv7k::launch_backward_t<bf16_t>(B, T, H, r, w, k, v, a, b, dy, ckpt, dsT, dr, dw, dk,
                                            dv, da, db, ds0, part, 0, nck, st, st, nullptr, gate);
  return wkv7k::launch_backward_t<float>(B, T, H, r, w, k, v, a, b, dy, ckpt, dsT, dr, dw, dk, dv,
                                         da, db, ds0, part, 0, nck, st, st, nullptr, gate);
}

int wkv7_ckpt_interval_const() { return wkv7k::CKL; }
