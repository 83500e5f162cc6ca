// WKV7 recurrence on gfx950: token-sequential forward, checkpoint-recomputing
// backward, and the single-token decode step.
//
// The recurrence (per batch b, head h, token t; S is 64x64 fp32, S[i][j] with
// i = value row, j = key column), as passed to the WKV7 kernel on the
// "Foundry/cuda_kernels/timemix.cu" page (k_composites: a = -kk, b = kk*a)
// and differentiated in the WKV state-backward block of "infotheory
// .../rwkv7/model.rs":
//     sa  = S a_t ;  S = S diag(w_t) + sa b_t^T + v_t k_t^T ;  y_t = S r_t
//
// Every state row evolves independently of the others (row i only needs
// v_t[i] and its own sa[i]), so rows are spread over lanes: a lane owns RPT
// rows x 4 adjacent columns, 16 lanes (one DPP row) cover the 64 columns of a
// state row, and the row dot products (S a, S r) are 16-lane DPP sums.  The
// per-token vectors are staged through LDS in blocks of tokens and read as
// float4 by every row that needs them.

#include "common.hpp"

namespace wkv7k {

constexpr int N = WKV7_N;
constexpr int TT = 16;    // tokens per LDS staging block (forward)
constexpr int CKL = 16;   // checkpoint interval (tokens)
constexpr int SUB = 8;    // backward sub-chunk kept as register history
static_assert(CKL == 2 * SUB, "backward assumes two sub-chunks per checkpoint");

// ------------------------------------------------------------------ forward
// Grid: B*H*(64/(16*RPT)) workgroups of 256 threads; workgroup -> (b, h, row
// block of 16*RPT rows).  Thread: column group cg = tid%16 (columns 4cg..4cg+3),
// row group rg = tid/16 owning rows rb*16*RPT + rg*RPT + m, m < RPT.
template <int RPT, typename T>
__global__ __launch_bounds__(256) void fwd_seq(
    int B, int Tn, int H, const T* __restrict__ r, const T* __restrict__ w,
    const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ a,
    const T* __restrict__ bv, const float* __restrict__ s0, T* __restrict__ y,
    float* __restrict__ sT, float* __restrict__ ckpt) {
  constexpr int ROWS = 16 * RPT;
  constexpr int NRB = N / ROWS;
  __shared__ f4 sv[2][TT][5][16];     // r, w, k, a, b of each staged token
  __shared__ float svv[2][TT][ROWS];  // v of this workgroup's rows

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
  constexpr int NV4 = TT * 5 * 16;        // float4 slots per block
  constexpr int NV4_PER = (NV4 + 255) / 256;
  constexpr int NVV_PER = (TT * ROWS + 255) / 256;
  f4 pre[NV4_PER];
  float prev[NVV_PER];

  auto load_block = [&](int t0) {
#pragma unroll
    for (int q = 0; q < NV4_PER; q++) {
      const int f = tid + 256 * q;
      f4 x = {0.f, 0.f, 0.f, 0.f};
      if (f < NV4) {
        const int tok = f / 80, rem = f - tok * 80, vi = rem >> 4, c4 = rem & 15;
        if (t0 + tok < Tn) x = load4(vec_ptr(vi) + vbase + (size_t)(t0 + tok) * C + c4 * 4);
      }
      pre[q] = x;
    }
#pragma unroll
    for (int q = 0; q < NVV_PER; q++) {
      const int f = tid + 256 * q;
      float x = 0.f;
      if (f < TT * ROWS) {
        const int tok = f / ROWS, rr = f - tok * ROWS;
        if (t0 + tok < Tn) x = load1(v + vbase + (size_t)(t0 + tok) * C + rb * ROWS + rr);
      }
      prev[q] = x;
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int q = 0; q < NV4_PER; q++) {
      const int f = tid + 256 * q;
      if (f < NV4) {
        const int tok = f / 80, rem = f - tok * 80, vi = rem >> 4, c4 = rem & 15;
        sv[buf][tok][vi][c4] = pre[q];
      }
    }
#pragma unroll
    for (int q = 0; q < NVV_PER; q++) {
      const int f = tid + 256 * q;
      if (f < TT * ROWS) {
        const int tok = f / ROWS, rr = f - tok * ROWS;
        svv[buf][tok][rr] = prev[q];
      }
    }
  };

  load_block(0);
  store_block(0);
  __syncthreads();
  int buf = 0;
  for (int t0 = 0; t0 < Tn; t0 += TT, buf ^= 1) {
    const bool more = t0 + TT < Tn;
    if (more) load_block(t0 + TT);
    const int nt = min(TT, Tn - t0);
    for (int tt = 0; tt < nt; tt++) {
      const int t = t0 + tt;
      if (ckpt && (t % CKL) == 0) {
        float* cp = ckpt + (((size_t)bh * nck + t / CKL) * N + row0) * N + cg * 4;
#pragma unroll
        for (int m = 0; m < RPT; m++) {
          f4 x = {S[m][0], S[m][1], S[m][2], S[m][3]};
          *reinterpret_cast<f4*>(cp + (size_t)m * N) = x;
        }
      }
      const f4 av = sv[buf][tt][3][cg];
      float sa[RPT];
#pragma unroll
      for (int m = 0; m < RPT; m++)
        sa[m] = fmaf(S[m][3], av[3], fmaf(S[m][2], av[2], fmaf(S[m][1], av[1], S[m][0] * av[0])));
#pragma unroll
      for (int m = 0; m < RPT; m++) sa[m] = rowsum16(sa[m]);
      const f4 wv = sv[buf][tt][1][cg], kv = sv[buf][tt][2][cg], bb = sv[buf][tt][4][cg];
#pragma unroll
      for (int m = 0; m < RPT; m++) {
        const float vv = svv[buf][tt][rloc0 + m];
#pragma unroll
        for (int c = 0; c < 4; c++) S[m][c] = fmaf(vv, kv[c], fmaf(sa[m], bb[c], S[m][c] * wv[c]));
      }
      if (y) {
        const f4 rv = sv[buf][tt][0][cg];
        float yo = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; m++) {
          float d = fmaf(S[m][3], rv[3], fmaf(S[m][2], rv[2], fmaf(S[m][1], rv[1], S[m][0] * rv[0])));
          d = rowsum16(d);
          if (cg == m) yo = d;
        }
        if (cg < RPT) store1(y + vbase + (size_t)t * C + row0 + cg, yo);
      }
    }
    if (more) store_block(buf ^ 1);
    __syncthreads();
  }

  if (sT) {
#pragma unroll
    for (int m = 0; m < RPT; m++) {
      f4 x = {S[m][0], S[m][1], S[m][2], S[m][3]};
      *reinterpret_cast<f4*>(sT + sbase + (size_t)(row0 + m) * N + cg * 4) = x;
    }
  }
}

// --------------------------------------------------------------------- step
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

// ----------------------------------------------------------------- backward
// One workgroup (256 threads) per (b,h).  Thread: column group cg = tid%16,
// rows 4*rg .. 4*rg+3 with rg = tid/16 (each wave holds 16 rows).
// Checkpoint chunks of CKL tokens are processed last to first; each chunk is
// recomputed from its checkpoint in two sub-chunks of SUB tokens whose states
// are kept in registers.  Per token the column reductions (dr, dk, db, dw,
// da: sums over the 64 rows) go in-thread over 4 rows, across the wave's
// four 16-lane rows with permlane swaps, and across the 4 waves through LDS.
template <typename T>
__global__ __launch_bounds__(256) void bwd_seq(
    int B, int Tn, int H, const T* __restrict__ r, const T* __restrict__ w,
    const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ a,
    const T* __restrict__ bv, const T* __restrict__ dy, const float* __restrict__ ckpt,
    const float* __restrict__ dsT, T* __restrict__ dr, T* __restrict__ dw,
    T* __restrict__ dk, T* __restrict__ dv, T* __restrict__ da, T* __restrict__ db,
    float* __restrict__ ds0) {
  __shared__ f4 sv[SUB][5][16];     // r, w, k, a, b
  __shared__ float svr[SUB][2][N];  // v, dy
  __shared__ f4 red[2][4][5][16];   // per-wave column partials: dr, dk, db, dw, da

  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, cg = tid & 15, rg = tid >> 4;
  const int lane = tid & 63, wave = tid >> 6;
  const int row0 = rg * 4;
  const size_t C = (size_t)H * N;
  const size_t vbase = (size_t)b * Tn * C + (size_t)h * N;
  const size_t sbase = ((size_t)b * H + h) * N * N;
  const int nck = (Tn + CKL - 1) / CKL;
  auto vec_ptr = [&](int vi) -> const T* {
    return vi == 0 ? r : vi == 1 ? w : vi == 2 ? k : vi == 3 ? a : bv;
  };
  auto out_ptr = [&](int vi) -> T* {
    return vi == 0 ? dr : vi == 1 ? dk : vi == 2 ? db : vi == 3 ? dw : da;
  };

  float G[4][4];
#pragma unroll
  for (int m = 0; m < 4; m++) {
    f4 x = {0.f, 0.f, 0.f, 0.f};
    if (dsT) x = *reinterpret_cast<const f4*>(dsT + sbase + (size_t)(row0 + m) * N + cg * 4);
#pragma unroll
    for (int c = 0; c < 4; c++) G[m][c] = x[c];
  }

  auto stage = [&](int ts0, int ns) {
    for (int f = tid; f < SUB * 80; f += 256) {
      const int tok = f / 80, rem = f - tok * 80, vi = rem >> 4, c4 = rem & 15;
      f4 x = {0.f, 0.f, 0.f, 0.f};
      if (tok < ns) x = load4(vec_ptr(vi) + vbase + (size_t)(ts0 + tok) * C + c4 * 4);
      sv[tok][vi][c4] = x;
    }
    for (int f = tid; f < SUB * 2 * N; f += 256) {
      const int tok = f / (2 * N), rem = f - tok * 2 * N, vi = rem / N, i = rem - vi * N;
      float x = 0.f;
      if (tok < ns) x = load1((vi ? dy : v) + vbase + (size_t)(ts0 + tok) * C + i);
      svr[tok][vi][i] = x;
    }
  };
  auto load_ckpt = [&](int c, float (&S)[4][4]) {
    const float* cp = ckpt + (((size_t)bh * nck + c) * N + row0) * N + cg * 4;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      f4 x = *reinterpret_cast<const f4*>(cp + (size_t)m * N);
#pragma unroll
      for (int cc = 0; cc < 4; cc++) S[m][cc] = x[cc];
    }
  };
  // one forward token from S (in place); returns sa (full row sums) in sa[]
  auto fwd_tok = [&](int tt, float (&S)[4][4], float (&sa)[4]) {
    const f4 av = sv[tt][3][cg];
#pragma unroll
    for (int m = 0; m < 4; m++)
      sa[m] = rowsum16(fmaf(S[m][3], av[3], fmaf(S[m][2], av[2], fmaf(S[m][1], av[1], S[m][0] * av[0]))));
    const f4 wv = sv[tt][1][cg], kv = sv[tt][2][cg], bb = sv[tt][4][cg];
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const float vv = svr[tt][0][row0 + m];
#pragma unroll
      for (int c = 0; c < 4; c++) S[m][c] = fmaf(vv, kv[c], fmaf(sa[m], bb[c], S[m][c] * wv[c]));
    }
  };

  int rbuf = 0;
  for (int c = nck - 1; c >= 0; c--) {
    const int tc0 = c * CKL, tc1 = min(Tn, tc0 + CKL);
    const int nsub = (tc1 - tc0 + SUB - 1) / SUB;
    // state at the start of the second sub-chunk
    float S1[4][4];
    if (nsub == 2) {
      load_ckpt(c, S1);
      __syncthreads();
      stage(tc0, SUB);
      __syncthreads();
      float sa[4];
#pragma unroll
      for (int tt = 0; tt < SUB; tt++) fwd_tok(tt, S1, sa);
    }
    for (int s = nsub - 1; s >= 0; s--) {
      const int ts0 = tc0 + s * SUB, ns = min(SUB, tc1 - ts0);
      __syncthreads();
      stage(ts0, ns);
      __syncthreads();
      float Sh[SUB + 1][4][4];
      float sah[SUB][4];
      if (s == 1) {
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
          for (int cc = 0; cc < 4; cc++) Sh[0][m][cc] = S1[m][cc];
      } else {
        load_ckpt(c, Sh[0]);
      }
#pragma unroll
      for (int tt = 0; tt < SUB; tt++) {
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
          for (int cc = 0; cc < 4; cc++) Sh[tt + 1][m][cc] = Sh[tt][m][cc];
        if (tt < ns) fwd_tok(tt, Sh[tt + 1], sah[tt]);
      }
#pragma unroll
      for (int tt = SUB - 1; tt >= 0; tt--) {
        if (tt < ns) {
          const int t = ts0 + tt;
          const f4 rv = sv[tt][0][cg], wv = sv[tt][1][cg], kv = sv[tt][2][cg];
          const f4 av = sv[tt][3][cg], bb = sv[tt][4][cg];
          float vv[4], dyv[4];
#pragma unroll
          for (int m = 0; m < 4; m++) {
            vv[m] = svr[tt][0][row0 + m];
            dyv[m] = svr[tt][1][row0 + m];
          }
          float pr[4], pk[4], pb[4], pw[4], pa[4], dvv[4], dsa[4];
#pragma unroll
          for (int m = 0; m < 4; m++)
#pragma unroll
            for (int cc = 0; cc < 4; cc++) G[m][cc] = fmaf(dyv[m], rv[cc], G[m][cc]);
#pragma unroll
          for (int m = 0; m < 4; m++) {
            dvv[m] = fmaf(G[m][3], kv[3], fmaf(G[m][2], kv[2], fmaf(G[m][1], kv[1], G[m][0] * kv[0])));
            dsa[m] = fmaf(G[m][3], bb[3], fmaf(G[m][2], bb[2], fmaf(G[m][1], bb[1], G[m][0] * bb[0])));
          }
#pragma unroll
          for (int m = 0; m < 4; m++) {
            dvv[m] = rowsum16(dvv[m]);
            dsa[m] = rowsum16(dsa[m]);
          }
#pragma unroll
          for (int cc = 0; cc < 4; cc++) {
            float xr = 0.f, xk = 0.f, xb = 0.f, xw = 0.f, xa = 0.f;
#pragma unroll
            for (int m = 0; m < 4; m++) {
              xr = fmaf(Sh[tt + 1][m][cc], dyv[m], xr);
              xk = fmaf(G[m][cc], vv[m], xk);
              xb = fmaf(G[m][cc], sah[tt][m], xb);
              xw = fmaf(G[m][cc], Sh[tt][m][cc], xw);
              xa = fmaf(dsa[m], Sh[tt][m][cc], xa);
            }
            pr[cc] = xr; pk[cc] = xk; pb[cc] = xb; pw[cc] = xw; pa[cc] = xa;
          }
#pragma unroll
          for (int m = 0; m < 4; m++)
#pragma unroll
            for (int cc = 0; cc < 4; cc++) G[m][cc] = fmaf(dsa[m], av[cc], G[m][cc] * wv[cc]);
#pragma unroll
          for (int cc = 0; cc < 4; cc++) {
            pr[cc] = rows4sum(pr[cc]);
            pk[cc] = rows4sum(pk[cc]);
            pb[cc] = rows4sum(pb[cc]);
            pw[cc] = rows4sum(pw[cc]);
            pa[cc] = rows4sum(pa[cc]);
          }
          if (lane < 16) {
            red[rbuf][wave][0][cg] = f4{pr[0], pr[1], pr[2], pr[3]};
            red[rbuf][wave][1][cg] = f4{pk[0], pk[1], pk[2], pk[3]};
            red[rbuf][wave][2][cg] = f4{pb[0], pb[1], pb[2], pb[3]};
            red[rbuf][wave][3][cg] = f4{pw[0], pw[1], pw[2], pw[3]};
            red[rbuf][wave][4][cg] = f4{pa[0], pa[1], pa[2], pa[3]};
          }
          if (cg < 4) {
            float o = dvv[0];
#pragma unroll
            for (int m = 1; m < 4; m++)
              if (cg == m) o = dvv[m];
            store1(dv + vbase + (size_t)t * C + row0 + cg, o);
          }
          __syncthreads();
          if (tid < 80) {
            const int vi = tid >> 4, c4 = tid & 15;
            f4 s4 = red[rbuf][0][vi][c4];
            s4 += red[rbuf][1][vi][c4];
            s4 += red[rbuf][2][vi][c4];
            s4 += red[rbuf][3][vi][c4];
            store4(out_ptr(vi) + vbase + (size_t)t * C + c4 * 4, s4);
          }
          rbuf ^= 1;
        }
      }
    }
  }
  if (ds0) {
#pragma unroll
    for (int m = 0; m < 4; m++) {
      f4 x = {G[m][0], G[m][1], G[m][2], G[m][3]};
      *reinterpret_cast<f4*>(ds0 + sbase + (size_t)(row0 + m) * N + cg * 4) = x;
    }
  }
}

}  // namespace wkv7k

// ------------------------------------------------------------ launchers ----
// (called from the C-ABI after argument validation)
namespace wkv7k {

template <typename T>
hipError_t launch_forward_t(int B, int T_, int H, const void* r, const void* w, const void* k,
                            const void* v, const void* a, const void* b, const float* s0, void* y,
                            float* sT, float* ckpt, hipStream_t st) {
  constexpr int RPT = 1;
  const int nblk = B * H * (N / (16 * RPT));
  hipLaunchKernelGGL((fwd_seq<RPT, T>), dim3(nblk), dim3(256), 0, st, B, T_, H,
                     (const T*)r, (const T*)w, (const T*)k, (const T*)v, (const T*)a,
                     (const T*)b, s0, (T*)y, sT, ckpt);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_backward_t(int B, int T_, int H, const void* r, const void* w, const void* k,
                             const void* v, const void* a, const void* b, const void* dy,
                             const float* ckpt, const float* dsT, void* dr, void* dw, void* dk,
                             void* dv, void* da, void* db, float* ds0, hipStream_t st) {
  hipLaunchKernelGGL((bwd_seq<T>), dim3(B * H), dim3(256), 0, st, B, T_, H, (const T*)r,
                     (const T*)w, (const T*)k, (const T*)v, (const T*)a, (const T*)b,
                     (const T*)dy, ckpt, dsT, (T*)dr, (T*)dw, (T*)dk, (T*)dv, (T*)da, (T*)db, ds0);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_step_t(int B, int H, const void* r, const void* w, const void* k, const void* v,
                         const void* a, const void* b, float* state, void* y, hipStream_t st) {
  hipLaunchKernelGGL((step_kernel<T>), dim3(B * H), dim3(256), 0, st, B * H, (const T*)r,
                     (const T*)w, (const T*)k, (const T*)v, (const T*)a, (const T*)b, state, (T*)y);
  return hipGetLastError();
}

}  // namespace wkv7k

hipError_t wkv7_launch_forward(int dtype, int B, int T, int H, const void* r, const void* w,
                               const void* k, const void* v, const void* a, const void* b,
                               const float* s0, void* y, float* sT, float* ckpt, hipStream_t st) {
  if (dtype == 1)
    return wkv7k::launch_forward_t<bf16_t>(B, T, H, r, w, k, v, a, b, s0, y, sT, ckpt, st);
  return wkv7k::launch_forward_t<float>(B, T, H, r, w, k, v, a, b, s0, y, sT, ckpt, st);
}

hipError_t wkv7_launch_backward(int dtype, int B, int T, int H, const void* r, const void* w,
                                const void* k, const void* v, const void* a, const void* b,
                                const void* dy, const float* ckpt, const float* dsT, void* dr,
                                void* dw, void* dk, void* dv, void* da, void* db, float* ds0,
                                hipStream_t st) {
  if (dtype == 1)
    return wkv7k::launch_backward_t<bf16_t>(B, T, H, r, w, k, v, a, b, dy, ckpt, dsT, dr, dw, dk,
                                            dv, da, db, ds0, st);
  return wkv7k::launch_backward_t<float>(B, T, H, r, w, k, v, a, b, dy, ckpt, dsT, dr, dw, dk, dv,
                                         da, db, ds0, st);
}

hipError_t wkv7_launch_step(int dtype, int B, int H, const void* r, const void* w, const void* k,
                            const void* v, const void* a, const void* b, float* state, void* y,
                            hipStream_t st) {
  if (dtype == 1) return wkv7k::launch_step_t<bf16_t>(B, H, r, w, k, v, a, b, state, y, st);
  return wkv7k::launch_step_t<float>(B, H, r, w, k, v, a, b, state, y, st);
}

int wkv7_ckpt_interval_const() { return wkv7k::CKL; }
