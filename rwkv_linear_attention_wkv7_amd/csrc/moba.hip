// MoBA sparse attention core on gfx950: chunk selection, forward and the
// backward with the selection held fixed ("Foundry/cuda_kernels/
// fullmodel.cu", fm_attn_core_fwd and the attention-core part of
// fm_attn_bwd).  Per (batch, head), head size 64, scale 1/8:
//   chunks of `chunk` keys; query t (chunk cur = t / chunk) always attends
//   to its own chunk up to itself; earlier chunks are scored by
//   q_t . mean(k over the chunk) and the top (topk - 1) are attended too
//   (ties: the lower chunk index); y_t = softmax(q_t K^T / 8 over the
//   attended keys) V.
//
// Selection: one wave per (b, t, h), lane c scoring chunk c; the chosen
// chunks are one 64-bit mask per query (at most 64 chunks).  The forward is
// a flash-style pass: a workgroup per (b, h, 64-query tile) walks the
// 64-key tiles up to its own, skipping tiles no query of the tile selected;
// S = Q K^T and P V run as 64x64x64 register-tiled products from LDS
// (thread (ty, tx) owns rows 4 ty.. and columns 4 tx..), with an online
// softmax whose row reductions are 16-lane shuffles.  It writes y and the
// row log-sum-exp.  The backward recomputes P from the log-sum-exp: a dQ
// pass per query tile (dS = P (dP - D), D = rowsum(dY Y), dQ = dS K / 8)
// and a dK / dV pass per key tile over the query tiles that selected it
// (dV = P^T dY, dK = dS^T Q / 8), so every output is summed in a fixed
// order by one workgroup (no atomics).

#include <cstdint>

#include "common.hpp"
#include "moba.hpp"

namespace mobak {

constexpr int HN = 64;   // head size
constexpr int TS = 64;   // query and key tile
constexpr int LP = 68;   // padded LDS row (floats)
constexpr float SCALE = 0.125f;  // 1 / sqrt(64)

// Mean of k over each chunk: kbar[b][h][c][n].  Grid (nchunks, B H), 64 threads.
__global__ __launch_bounds__(64) void kbar(int T, int H, int chunk, const float* __restrict__ k,
                                           float* __restrict__ kb) {
  const int c = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh - b * H, n = threadIdx.x;
  const int C = H * HN, t0 = c * chunk, t1 = min(T, t0 + chunk);
  float s = 0.f;
  for (int t = t0; t < t1; t++) s += k[((size_t)b * T + t) * C + h * HN + n];
  kb[((size_t)bh * gridDim.x + c) * HN + n] = s / (float)(t1 - t0);
}

// One wave per (b, t, h): lane c < cur scores chunk c; the top (topk - 1)
// by (score desc, chunk asc) are selected, plus the current chunk.
// sel[b][h][t] (64-bit).  Grid: B T H / 4 workgroups of 256 threads.
__global__ __launch_bounds__(256) void select(int B, int T, int H, int chunk, int nc, int topk,
                                              const float* __restrict__ q, const float* __restrict__ kb,
                                              uint64_t* __restrict__ sel) {
  const int lane = threadIdx.x & 63;
  const size_t w = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (size_t)B * T * H) return;  // uniform per wave
  const int h = (int)(w % H);
  const size_t bt = w / H;
  const int b = (int)(bt / T), t = (int)(bt - (size_t)b * T);
  const int cur = t / chunk, C = H * HN;
  const f4* qv = reinterpret_cast<const f4*>(q + bt * C + h * HN);
  float s = -INFINITY;
  if (lane < cur) {
    const f4* kv = reinterpret_cast<const f4*>(kb + (((size_t)b * H + h) * nc + lane) * HN);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < HN / 4; i++) {
      const f4 x = qv[i], y = kv[i];
      a += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
    }
    s = a;
  }
  uint64_t m = (uint64_t)1 << cur;
  bool taken = lane >= cur;
  for (int r = 0; r < topk - 1 && r < cur; r++) {
    float bv = taken ? -INFINITY : s;
    int bi = taken ? 64 : lane;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi >= 64) break;  // no candidate left (uniform)
    m |= (uint64_t)1 << bi;
    if (lane == bi) taken = true;
  }
  if (lane == 0) sel[((size_t)b * H + h) * T + t] = m;
}

// LDS tile helpers.  A tile holds 64 rows (positions r0 .. r0 + 63 of one
// head) of a [B][T][C] tensor; rows past T are zeros.
// Transposed: X[c][row].
__device__ __forceinline__ void load_T(float (*X)[LP], const float* __restrict__ src, int b, int T,
                                       int C, int h, int r0) {
  for (int i = threadIdx.x; i < TS * HN / 4; i += 256) {
    const int row = i / (HN / 4), c = (i % (HN / 4)) * 4, t = r0 + row;
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (t < T) v = *reinterpret_cast<const f4*>(src + ((size_t)b * T + t) * C + h * HN + c);
    X[c][row] = v[0];
    X[c + 1][row] = v[1];
    X[c + 2][row] = v[2];
    X[c + 3][row] = v[3];
  }
}
// Row layout: X[row][c].
__device__ __forceinline__ void load_R(float (*X)[LP], const float* __restrict__ src, int b, int T,
                                       int C, int h, int r0) {
  for (int i = threadIdx.x; i < TS * HN / 4; i += 256) {
    const int row = i / (HN / 4), c = (i % (HN / 4)) * 4, t = r0 + row;
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (t < T) v = *reinterpret_cast<const f4*>(src + ((size_t)b * T + t) * C + h * HN + c);
    *reinterpret_cast<f4*>(&X[row][c]) = v;
  }
}

// acc[i][j] += sum_c A[c][4 ty + i] B[c][4 tx + j]  (A, B transposed tiles)
__device__ __forceinline__ void mm_tt(const float (*A)[LP], const float (*Bm)[LP], int ty, int tx,
                                      float (&acc)[4][4]) {
#pragma unroll 8
  for (int c = 0; c < HN; c++) {
    const f4 a = *reinterpret_cast<const f4*>(&A[c][4 * ty]);
    const f4 bb = *reinterpret_cast<const f4*>(&Bm[c][4 * tx]);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] += a[i] * bb[j];
  }
}

// acc[i][j] += sum_r A[r][4 ty + i] Bm[r][4 tx + j] over 64 rows r (A
// indexed [r][row of the result], Bm in row layout [r][column]).
__device__ __forceinline__ void mm_rr(const float (*A)[LP], const float (*Bm)[LP], int ty, int tx,
                                      float (&acc)[4][4]) {
#pragma unroll 8
  for (int r = 0; r < TS; r++) {
    const f4 a = *reinterpret_cast<const f4*>(&A[r][4 * ty]);
    const f4 bb = *reinterpret_cast<const f4*>(&Bm[r][4 * tx]);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] += a[i] * bb[j];
  }
}

__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float max16(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Bits of the chunks that overlap key tile kt.
__device__ __forceinline__ uint64_t tile_chunks(int kt, int chunk, int nc) {
  const int lo = kt * TS / chunk, hi = min(nc - 1, (kt * TS + TS - 1) / chunk);
  const int n = hi - lo + 1;
  return (n >= 64 ? ~(uint64_t)0 : (((uint64_t)1 << n) - 1)) << lo;
}

// OR of the selection masks of query tile qt (every thread gets it).
__device__ __forceinline__ uint64_t tile_or(const uint64_t* __restrict__ sel_bh, int T, int qt,
                                            uint64_t* red) {
  const int tid = threadIdx.x, t = qt * TS + (tid & 63);
  uint64_t m = (tid < 64 && t < T) ? sel_bh[t] : 0;
  uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo |= __shfl_xor(lo, o);
    hi |= __shfl_xor(hi, o);
  }
  if (tid == 0) *red = ((uint64_t)hi << 32) | lo;
  __syncthreads();
  const uint64_t r = *red;
  __syncthreads();
  return r;
}

// Forward: grid (query tiles, B H), 256 threads.
__global__ __launch_bounds__(256) void fwd(int T, int H, int chunk, int nc, const float* __restrict__ q,
                                           const float* __restrict__ k, const float* __restrict__ v,
                                           const uint64_t* __restrict__ sel, float* __restrict__ y,
                                           float* __restrict__ lse) {
  __shared__ float qT[HN][LP], kT[HN][LP], vR[TS][LP], pT[TS][LP];
  __shared__ uint64_t red;
  const int qt = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh - b * H, C = H * HN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const uint64_t* sb = sel + (size_t)bh * T;
  int tr[4];
  uint64_t mr[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    tr[i] = qt * TS + 4 * ty + i;
    mr[i] = tr[i] < T ? sb[tr[i]] : 0;
  }
  const uint64_t tor = tile_or(sb, T, qt, &red);
  load_T(qT, q, b, T, C, h, qt * TS);
  float m[4], l[4], o[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    m[i] = -1e30f;
    l[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) o[i][j] = 0.f;
  }
  for (int kt = 0; kt <= qt; kt++) {
    if (!(tor & tile_chunks(kt, chunk, nc))) continue;  // uniform
    __syncthreads();  // previous tile's readers are done
    load_T(kT, k, b, T, C, h, kt * TS);
    load_R(vR, v, b, T, C, h, kt * TS);
    __syncthreads();
    float s[4][4] = {};
    mm_tt(qT, kT, ty, tx, s);
    int kc[4];
#pragma unroll
    for (int j = 0; j < 4; j++) kc[j] = (kt * TS + 4 * tx + j) / chunk;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int key = kt * TS + 4 * tx + j;
        const bool ok = key <= tr[i] && tr[i] < T && ((mr[i] >> kc[j]) & 1);
        s[i][j] = ok ? s[i][j] * SCALE : -INFINITY;
        mx = fmaxf(mx, s[i][j]);
      }
      const float mn = fmaxf(m[i], max16(mx));
      const float alpha = expf(m[i] - mn);
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        s[i][j] = expf(s[i][j] - mn);  // 0 where masked
        rs += s[i][j];
      }
      l[i] = l[i] * alpha + sum16(rs);
      m[i] = mn;
#pragma unroll
      for (int j = 0; j < 4; j++) o[i][j] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) pT[4 * tx + j][4 * ty + i] = s[i][j];
    __syncthreads();
    mm_rr(pT, vR, ty, tx, o);
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (tr[i] >= T) continue;
    const float inv = 1.0f / l[i];
    *reinterpret_cast<f4*>(y + ((size_t)b * T + tr[i]) * C + h * HN + 4 * tx) =
        f4{o[i][0] * inv, o[i][1] * inv, o[i][2] * inv, o[i][3] * inv};
    if (tx == 0) lse[(size_t)bh * T + tr[i]] = m[i] + logf(l[i]);
  }
}

// Backward, query side: grid (query tiles, B H).  Writes dq and D = rowsum(dy y).
__global__ __launch_bounds__(256) void bwd_dq(int T, int H, int chunk, int nc, const float* __restrict__ q,
                                              const float* __restrict__ k, const float* __restrict__ v,
                                              const float* __restrict__ y, const float* __restrict__ lse,
                                              const uint64_t* __restrict__ sel, const float* __restrict__ dy,
                                              float* __restrict__ dq, float* __restrict__ Dout) {
  __shared__ float qT[HN][LP], doT[HN][LP], kT[HN][LP], vT[HN][LP], kR[TS][LP], dsT[TS][LP];
  __shared__ uint64_t red;
  const int qt = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh - b * H, C = H * HN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const uint64_t* sb = sel + (size_t)bh * T;
  int tr[4];
  uint64_t mr[4];
  float Lr[4], Dr[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    tr[i] = qt * TS + 4 * ty + i;
    const bool in = tr[i] < T;
    mr[i] = in ? sb[tr[i]] : 0;
    Lr[i] = in ? lse[(size_t)bh * T + tr[i]] : 0.f;
    float d = 0.f;
    if (in) {
      const size_t e = ((size_t)b * T + tr[i]) * C + h * HN + 4 * tx;
      const f4 a = *reinterpret_cast<const f4*>(dy + e), c = *reinterpret_cast<const f4*>(y + e);
      d = a[0] * c[0] + a[1] * c[1] + a[2] * c[2] + a[3] * c[3];
    }
    Dr[i] = sum16(d);
    if (in && tx == 0) Dout[(size_t)bh * T + tr[i]] = Dr[i];
  }
  const uint64_t tor = tile_or(sb, T, qt, &red);
  load_T(qT, q, b, T, C, h, qt * TS);
  load_T(doT, dy, b, T, C, h, qt * TS);
  float acc[4][4] = {};
  for (int kt = 0; kt <= qt; kt++) {
    if (!(tor & tile_chunks(kt, chunk, nc))) continue;  // uniform
    __syncthreads();
    load_T(kT, k, b, T, C, h, kt * TS);
    load_T(vT, v, b, T, C, h, kt * TS);
    load_R(kR, k, b, T, C, h, kt * TS);
    __syncthreads();
    float s[4][4] = {}, dp[4][4] = {};
    mm_tt(qT, kT, ty, tx, s);
    mm_tt(doT, vT, ty, tx, dp);
    int kc[4];
#pragma unroll
    for (int j = 0; j < 4; j++) kc[j] = (kt * TS + 4 * tx + j) / chunk;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int key = kt * TS + 4 * tx + j;
        const bool ok = key <= tr[i] && tr[i] < T && ((mr[i] >> kc[j]) & 1);
        const float p = ok ? expf(s[i][j] * SCALE - Lr[i]) : 0.f;
        dsT[4 * tx + j][4 * ty + i] = p * (dp[i][j] - Dr[i]);
      }
    __syncthreads();
    mm_rr(dsT, kR, ty, tx, acc);
  }
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (tr[i] < T)
      *reinterpret_cast<f4*>(dq + ((size_t)b * T + tr[i]) * C + h * HN + 4 * tx) =
          f4{acc[i][0] * SCALE, acc[i][1] * SCALE, acc[i][2] * SCALE, acc[i][3] * SCALE};
}

// Backward, key side: grid (key tiles, B H).  dv = P^T dy, dk = dS^T q / 8
// over the query tiles at or after this key tile whose queries selected it.
__global__ __launch_bounds__(256) void bwd_dkv(int T, int H, int chunk, int nc, const float* __restrict__ q,
                                               const float* __restrict__ k, const float* __restrict__ v,
                                               const float* __restrict__ lse, const float* __restrict__ Din,
                                               const uint64_t* __restrict__ sel, const float* __restrict__ dy,
                                               float* __restrict__ dk, float* __restrict__ dv) {
  __shared__ float kT[HN][LP], vT[HN][LP], qT[HN][LP], doT[HN][LP], qR[TS][LP], doR[TS][LP];
  __shared__ float pS[TS][LP], dsS[TS][LP];
  __shared__ uint64_t msk[TS];
  __shared__ float Ls[TS], Ds[TS];
  __shared__ uint64_t red;
  const int kt = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh - b * H, C = H * HN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const uint64_t* sb = sel + (size_t)bh * T;
  const uint64_t mine = tile_chunks(kt, chunk, nc);
  load_T(kT, k, b, T, C, h, kt * TS);
  load_T(vT, v, b, T, C, h, kt * TS);
  int kc[4];
#pragma unroll
  for (int i = 0; i < 4; i++) kc[i] = (kt * TS + 4 * ty + i) / chunk;
  float adk[4][4] = {}, adv[4][4] = {};
  const int nqt = (T + TS - 1) / TS;
  for (int qt = kt; qt < nqt; qt++) {
    if (!(tile_or(sb, T, qt, &red) & mine)) continue;  // uniform
    load_T(qT, q, b, T, C, h, qt * TS);
    load_T(doT, dy, b, T, C, h, qt * TS);
    load_R(qR, q, b, T, C, h, qt * TS);
    load_R(doR, dy, b, T, C, h, qt * TS);
    if (tid < TS) {
      const int t = qt * TS + tid;
      msk[tid] = t < T ? sb[t] : 0;
      Ls[tid] = t < T ? lse[(size_t)bh * T + t] : 0.f;
      Ds[tid] = t < T ? Din[(size_t)bh * T + t] : 0.f;
    }
    __syncthreads();
    // rows of S^T: keys 4 ty + i; columns: queries 4 tx + j
    float s[4][4] = {}, dp[4][4] = {};
    mm_tt(kT, qT, ty, tx, s);
    mm_tt(vT, doT, ty, tx, dp);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int qi = 4 * tx + j, t = qt * TS + qi;
      const uint64_t mq = msk[qi];
      const float L = Ls[qi], D = Ds[qi];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int key = kt * TS + 4 * ty + i;
        const bool ok = t < T && key <= t && ((mq >> kc[i]) & 1);
        const float p = ok ? expf(s[i][j] * SCALE - L) : 0.f;
        pS[qi][4 * ty + i] = p;
        dsS[qi][4 * ty + i] = p * (dp[i][j] - D);
      }
    }
    __syncthreads();
    mm_rr(pS, doR, ty, tx, adv);
    mm_rr(dsS, qR, ty, tx, adk);
    __syncthreads();  // before the next query tile overwrites the tiles
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int key = kt * TS + 4 * ty + i;
    if (key >= T) continue;
    const size_t e = ((size_t)b * T + key) * C + h * HN + 4 * tx;
    *reinterpret_cast<f4*>(dk + e) = f4{adk[i][0] * SCALE, adk[i][1] * SCALE, adk[i][2] * SCALE, adk[i][3] * SCALE};
    *reinterpret_cast<f4*>(dv + e) = f4{adv[i][0], adv[i][1], adv[i][2], adv[i][3]};
  }
}

}  // namespace mobak

int moba_num_chunks(int T, int chunk) { return (T + chunk - 1) / chunk; }

size_t moba_kbar_floats(int B, int T, int H, int chunk) {
  return (size_t)B * H * moba_num_chunks(T, chunk) * mobak::HN;
}

hipError_t moba_launch_forward(int B, int T, int H, int chunk, int topk, const float* q, const float* k,
                               const float* v, float* y, float* lse, uint64_t* sel, float* kbar,
                               hipStream_t st) {
  const int nc = moba_num_chunks(T, chunk);
  hipLaunchKernelGGL(mobak::kbar, dim3(nc, B * H), dim3(64), 0, st, T, H, chunk, k, kbar);
  const size_t waves = (size_t)B * T * H;
  hipLaunchKernelGGL(mobak::select, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, B, T, H, chunk, nc,
                     topk, q, kbar, sel);
  const int nqt = (T + mobak::TS - 1) / mobak::TS;
  hipLaunchKernelGGL(mobak::fwd, dim3(nqt, B * H), dim3(256), 0, st, T, H, chunk, nc, q, k, v, sel, y, lse);
  return hipGetLastError();
}

hipError_t moba_launch_backward(int B, int T, int H, int chunk, const float* q, const float* k,
                                const float* v, const float* y, const float* lse, const uint64_t* sel,
                                const float* dy, float* dq, float* dk, float* dv, float* Dbuf,
                                hipStream_t st) {
  const int nc = moba_num_chunks(T, chunk);
  const int nt = (T + mobak::TS - 1) / mobak::TS;
  hipLaunchKernelGGL(mobak::bwd_dq, dim3(nt, B * H), dim3(256), 0, st, T, H, chunk, nc, q, k, v, y, lse,
                     sel, dy, dq, Dbuf);
  hipLaunchKernelGGL(mobak::bwd_dkv, dim3(nt, B * H), dim3(256), 0, st, T, H, chunk, nc, q, k, v, lse, Dbuf,
                     sel, dy, dk, dv);
  return hipGetLastError();
}
