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
// chunks are one 64-bit mask per query (at most 64 chunks).  Chunks of 64
// keys take the gathered path further below, which computes only the
// selected (query, chunk) pairs.  Other chunk lengths use tile kernels: the
// forward is a flash-style pass: a workgroup per (b, h, 64-query tile) walks the
// 64-key tiles up to its own, skipping tiles no query of the tile selected;
// S = Q K^T and P V run as 64x64x64 register-tiled products from LDS
// (thread (ty, tx) owns rows 4 ty.. and columns 4 tx..), with an online
// softmax whose row reductions are 16-lane shuffles.  It writes y and the
// row log-sum-exp.  The backward recomputes P from the log-sum-exp: a dQ
// pass per query tile (dS = P (dP - D), D = rowsum(dY Y), dQ = dS K / 8)
// and a dK / dV pass per key tile over the query tiles that selected it
// (dV = P^T dY, dK = dS^T Q / 8), so every output is summed in a fixed
// order by one workgroup (no atomics).

#include <algorithm>
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

// ---------------------------------------------------------------------------
// Sparse path for chunks of 64 keys (one key tile per chunk).  Per (b, h,
// chunk c) the queries that selected c are gathered into an ordered list
// (ascending position), and only those (query, chunk) pairs are computed, 64
// gathered queries at a time:
//   forward: per pair the chunk's softmax partial (row max m, sum l and the
//   unnormalised P V) goes to slot j of the query (j = rank of c among the
//   query's chunks); a merge combines the slots in chunk order into y and
//   the log-sum-exp;
//   backward: one workgroup per chunk walks its list: dV and dK of the chunk
//   are summed over the gathered queries in list order, and each pair's dQ
//   share goes to the query's slot j; a merge sums the slots in chunk order.

// list[bh][c][0 .. cnt) = the positions t >= 64 c whose mask has bit c, in
// ascending order.  Grid (chunks, B H), 256 threads.
__global__ __launch_bounds__(256) void sp_list(int T, int nc, const uint64_t* __restrict__ sel,
                                               int* __restrict__ list, int* __restrict__ cnt) {
  __shared__ int wsum[4];
  __shared__ int base;
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t* sb = sel + (size_t)bh * T;
  int* out = list + ((size_t)bh * nc + c) * T;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int t0 = c * TS; t0 < T; t0 += 256) {
    const int t = t0 + tid;
    const bool on = t < T && ((sb[t] >> c) & 1);
    const uint64_t bal = __ballot(on);
    const int before = __popcll(bal & ((lane ? (~(uint64_t)0 >> (64 - lane)) : (uint64_t)0)));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; w++) off += wsum[w];
    if (on) out[off + before] = t;
    __syncthreads();
    if (tid == 0) base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (tid == 0) cnt[(size_t)bh * nc + c] = base;
}

// Gathered tile loads: rows are the listed positions idx[0 .. n), rows past
// n are zeros.
__device__ __forceinline__ void gather_T(float (*X)[LP], const float* __restrict__ src, const int* idx,
                                         int n, int b, int T, int C, int h) {
  for (int i = threadIdx.x; i < TS * HN / 4; i += 256) {
    const int row = i / (HN / 4), c = (i % (HN / 4)) * 4;
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < n) v = *reinterpret_cast<const f4*>(src + ((size_t)b * T + idx[row]) * C + h * HN + c);
    X[c][row] = v[0];
    X[c + 1][row] = v[1];
    X[c + 2][row] = v[2];
    X[c + 3][row] = v[3];
  }
}
__device__ __forceinline__ void gather_R(float (*X)[LP], const float* __restrict__ src, const int* idx,
                                         int n, int b, int T, int C, int h) {
  for (int i = threadIdx.x; i < TS * HN / 4; i += 256) {
    const int row = i / (HN / 4), c = (i % (HN / 4)) * 4;
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < n) v = *reinterpret_cast<const f4*>(src + ((size_t)b * T + idx[row]) * C + h * HN + c);
    *reinterpret_cast<f4*>(&X[row][c]) = v;
  }
}

// Slot of chunk c among the chunks of mask m (their rank in ascending order).
__device__ __forceinline__ int slot_of(uint64_t m, int c) {
  return __popcll(m & (c ? (~(uint64_t)0 >> (64 - c)) : (uint64_t)0));
}

// Matrix-core helpers of the gathered kernels (v_mfma_f32_16x16x4_f32).
// c += A B over one group of 16 k: lane l supplies A[l%16][4(l/16)+s] in
// a[s] and B[4(l/16)+s][l%16] in b[s]; the result tile: lane l element v
// holds C[4(l/16)+v][l%16].
__device__ __forceinline__ f4 mma16(f4 a, f4 b, f4 c) {
#pragma unroll
  for (int s = 0; s < 4; s++) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f4 ldf4(const float* p) { return *reinterpret_cast<const f4*>(p); }
// B fragment from a row-layout tile X[k][n]: X[k0 + 4 fg + s][n] for s < 4.
__device__ __forceinline__ f4 colf4(const float (*X)[LP], int k0, int fg, int n) {
  return f4{X[k0 + 4 * fg][n], X[k0 + 4 * fg + 1][n], X[k0 + 4 * fg + 2][n], X[k0 + 4 * fg + 3][n]};
}
// Max over the 16 lanes of a DPP row (every lane of the row receives it).
__device__ __forceinline__ float rowmax16(float x) {
  x = fmaxf(x, __builtin_amdgcn_update_dpp(-INFINITY, x, 0xB1, 0xF, 0xF, false));
  x = fmaxf(x, __builtin_amdgcn_update_dpp(-INFINITY, x, 0x4E, 0xF, 0xF, false));
  x = fmaxf(x, __builtin_amdgcn_update_dpp(-INFINITY, x, 0x141, 0xF, 0xF, false));
  x = fmaxf(x, __builtin_amdgcn_update_dpp(-INFINITY, x, 0x140, 0xF, 0xF, false));
  return x;
}
// Gathered rows (row layout X[row][c]) with any block size.
template <int NT>
__device__ __forceinline__ void gather_rows(float (*X)[LP], const float* __restrict__ src,
                                            const int* idx, int n, int b, int T, int C, int h) {
  for (int i = threadIdx.x; i < TS * HN / 4; i += NT) {
    const int row = i / (HN / 4), c = (i % (HN / 4)) * 4;
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < n) v = *reinterpret_cast<const f4*>(src + ((size_t)b * T + idx[row]) * C + h * HN + c);
    *reinterpret_cast<f4*>(&X[row][c]) = v;
  }
}
template <int NT>
__device__ __forceinline__ void load_rows(float (*X)[LP], const float* __restrict__ src, int b, int T,
                                          int C, int h, int r0) {
  for (int i = threadIdx.x; i < TS * HN / 4; i += NT) {
    const int row = i / (HN / 4), c = (i % (HN / 4)) * 4, t = r0 + row;
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (t < T) v = *reinterpret_cast<const f4*>(src + ((size_t)b * T + t) * C + h * HN + c);
    *reinterpret_cast<f4*>(&X[row][c]) = v;
  }
}

// Forward partials: grid (half the chunks, B H), 4 waves; the workgroup walks
// the lists of two chunks in blocks of 64 queries (K and V of a chunk loaded
// once).
// Wave w owns gathered queries 16w..16w+15: S = Q K^T and O = P V on the
// matrix cores, the row max and sum over the chunk's 64 keys in-lane and
// across the lanes of a DPP row.
// po[bh][t][j][64] = sum_key e^(s - m) v, pm / pl[bh][t][j] = m and the sum of
// e^(s - m) over the chunk's allowed keys (s = q.k / 8).
__global__ __launch_bounds__(256) void sp_fwd(int T, int H, int nc, int K, const float* __restrict__ q,
                                              const float* __restrict__ k, const float* __restrict__ v,
                                              const uint64_t* __restrict__ sel, const int* __restrict__ list,
                                              const int* __restrict__ cnt, float* __restrict__ po,
                                              float* __restrict__ pm, float* __restrict__ pl) {
  __shared__ __attribute__((aligned(16))) float qR[TS][LP], kR[TS][LP], vR[TS][LP], pN[TS][LP];
  __shared__ int idx[TS];
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H, C = H * HN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, fr = lane & 15, fg = lane >> 4;
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  // chunks x and nc-1-x: an early chunk (selected by many later queries)
  // with a late one, so the workgroups carry similar work
  for (int pass = 0; pass < 2; pass++) {
  const int c = pass == 0 ? blockIdx.x : nc - 1 - blockIdx.x;
  if (pass == 1 && c == blockIdx.x) break;
  const int n_all = cnt[(size_t)bh * nc + c];
  const int* lst = list + ((size_t)bh * nc + c) * T;
  __syncthreads();  // the previous chunk's readers are done
  load_rows<256>(kR, k, b, T, C, h, c * TS);
  load_rows<256>(vR, v, b, T, C, h, c * TS);
  // Block b0's list entries and gathered q rows are fetched into registers
  // while block b0 - 64 runs (thread: list entry tid; rows tid/16 + 16 j,
  // 4 columns at 4 (tid%16)).
  int pt = 0;
  f4 pq4[4];
  auto fetch = [&](int b0) {
    const int n = min(TS, n_all - b0);
    if (tid < TS) pt = tid < n ? lst[b0 + tid] : 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int row = (tid >> 4) + 16 * j, cc = (tid & 15) * 4;
      pq4[j] = row < n ? *reinterpret_cast<const f4*>(q + ((size_t)b * T + lst[b0 + row]) * C + h * HN + cc) : z;
    }
  };
  if (n_all > 0) fetch(0);
  for (int b0 = 0; b0 < n_all; b0 += TS) {
    const int n = min(TS, n_all - b0);
    __syncthreads();  // the previous block's readers are done
    if (tid < TS) idx[tid] = pt;
#pragma unroll
    for (int j = 0; j < 4; j++)
      *reinterpret_cast<f4*>(&qR[(tid >> 4) + 16 * j][(tid & 15) * 4]) = pq4[j];
    __syncthreads();
    if (b0 + TS < n_all) fetch(b0 + TS);
    // s[jt][vv] = S[query 16w + 4fg + vv][key 16jt + fr]
    f4 s[4] = {z, z, z, z};
#pragma unroll
    for (int kg = 0; kg < 4; kg++) {
      const f4 a = ldf4(&qR[16 * w + fr][16 * kg + 4 * fg]);
#pragma unroll
      for (int jt = 0; jt < 4; jt++) s[jt] = mma16(a, ldf4(&kR[16 * jt + fr][16 * kg + 4 * fg]), s[jt]);
    }
    float m[4], l[4];
#pragma unroll
    for (int vv = 0; vv < 4; vv++) {
      const int r = 16 * w + 4 * fg + vv;
      const int t = r < n ? idx[r] : -1;
      float mx = -INFINITY;
#pragma unroll
      for (int jt = 0; jt < 4; jt++) {
        const int key = c * TS + 16 * jt + fr;
        const bool ok = t >= 0 && key <= t;  // key <= t < T
        s[jt][vv] = ok ? s[jt][vv] * SCALE : -INFINITY;
        mx = fmaxf(mx, s[jt][vv]);
      }
      m[vv] = fmaxf(rowmax16(mx), -1e30f);
      float rs = 0.f;
#pragma unroll
      for (int jt = 0; jt < 4; jt++) {
        s[jt][vv] = expf(s[jt][vv] - m[vv]);
        rs += s[jt][vv];
        pN[r][16 * jt + fr] = s[jt][vv];
      }
      l[vv] = rowsum16(rs);
    }
    __syncthreads();
    // o[jt][vv] = O[query 16w + 4fg + vv][d 16jt + fr] = sum_key P V
    f4 o[4] = {z, z, z, z};
#pragma unroll
    for (int kg = 0; kg < 4; kg++) {
      const f4 a = ldf4(&pN[16 * w + fr][16 * kg + 4 * fg]);
#pragma unroll
      for (int jt = 0; jt < 4; jt++) o[jt] = mma16(a, colf4(vR, 16 * kg, fg, 16 * jt + fr), o[jt]);
    }
#pragma unroll
    for (int vv = 0; vv < 4; vv++) {
      const int r = 16 * w + 4 * fg + vv;
      if (r >= n) continue;
      const int t = idx[r];
      const int j = slot_of(sel[(size_t)bh * T + t], c);
      if (j >= K) continue;  // a mask with more chunks than topk (not one the selection wrote)
      const size_t e = ((size_t)bh * T + t) * K + j;
#pragma unroll
      for (int jt = 0; jt < 4; jt++) po[e * HN + 16 * jt + fr] = o[jt][vv];
      if (fr == 0) {
        pm[e] = m[vv];
        pl[e] = l[vv];
      }
    }
  }
  }
}

// Merge: 16 lanes per (b, h, t); the query's slots combined in chunk order.
__global__ __launch_bounds__(256) void sp_merge(int BHT, int T, int H, int K, const uint64_t* __restrict__ sel,
                                                const float* __restrict__ po, const float* __restrict__ pm,
                                                const float* __restrict__ pl, float* __restrict__ y,
                                                float* __restrict__ lse) {
  const int g = blockIdx.x * 16 + (threadIdx.x >> 4), l16 = threadIdx.x & 15;
  if (g >= BHT) return;
  const int bh = g / T, t = g - bh * T, b = bh / H, h = bh - b * H, C = H * HN;
  const int ns = min(__popcll(sel[g]), K);
  const size_t e0 = (size_t)g * K;
  float M = -INFINITY;
  for (int j = 0; j < ns; j++) M = fmaxf(M, pm[e0 + j]);
  float L = 0.f;
  f4 o = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < ns; j++) {
    const float w = expf(pm[e0 + j] - M);
    L += pl[e0 + j] * w;
    o += w * *reinterpret_cast<const f4*>(po + (e0 + j) * HN + 4 * l16);
  }
  *reinterpret_cast<f4*>(y + ((size_t)b * T + t) * C + h * HN + 4 * l16) = o * (1.0f / L);
  if (l16 == 0) lse[g] = M + logf(L);
}

// D[bh][t] = dy . y (16 lanes per row).
__global__ __launch_bounds__(256) void sp_rowdot(int BHT, int T, int H, const float* __restrict__ y,
                                                 const float* __restrict__ dy, float* __restrict__ D) {
  const int g = blockIdx.x * 16 + (threadIdx.x >> 4), l16 = threadIdx.x & 15;
  if (g >= BHT) return;  // whole 16-lane groups exit together
  const int bh = g / T, t = g - bh * T, b = bh / H, h = bh - b * H, C = H * HN;
  const size_t e = ((size_t)b * T + t) * C + h * HN + 4 * l16;
  const f4 a = *reinterpret_cast<const f4*>(dy + e), c = *reinterpret_cast<const f4*>(y + e);
  const float d = sum16(a[0] * c[0] + a[1] * c[1] + a[2] * c[2] + a[3] * c[3]);
  if (l16 == 0) D[g] = d;
}

// Backward per chunk pair: grid (half the chunks, B H), 8 waves.  dk, dv of a chunk's
// keys; each listed query's dq share into pq[bh][t][j][64] (scaled).  Per
// block of 64 gathered queries, on the matrix cores: S^T = K Q^T and
// dP^T = V dY^T (wave w: keys of tile w%4, query tiles 2(w/4), 2(w/4)+1),
// P and dS = P (dP - D) to LDS as [key][query], then dV += P^T dY and
// dK += dS^T Q (keys of tile w%4, head dims of tiles 2(w/4)..) and the dq
// shares dS K (queries of tile w%4).
__global__ __launch_bounds__(512) void sp_bwd(int T, int H, int nc, int K, const float* __restrict__ q,
                                              const float* __restrict__ k, const float* __restrict__ v,
                                              const float* __restrict__ lse, const float* __restrict__ Din,
                                              const uint64_t* __restrict__ sel, const float* __restrict__ dy,
                                              const int* __restrict__ list, const int* __restrict__ cnt,
                                              float* __restrict__ dk, float* __restrict__ dv,
                                              float* __restrict__ pq) {
  __shared__ __attribute__((aligned(16))) float kR[TS][LP], vR[TS][LP], qR[TS][LP], doR[TS][LP];
  __shared__ __attribute__((aligned(16))) float pT[TS][LP], dsT[TS][LP];
  __shared__ int idx[TS];
  __shared__ float Ls[TS], Ds[TS];
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H, C = H * HN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, fr = lane & 15, fg = lane >> 4;
  const int rt = w & 3, cp = w >> 2;  // row tile, pair of column tiles
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  // chunks x and nc-1-x (as in sp_fwd)
  for (int pass = 0; pass < 2; pass++) {
  const int c = pass == 0 ? blockIdx.x : nc - 1 - blockIdx.x;
  if (pass == 1 && c == blockIdx.x) break;
  const int n_all = cnt[(size_t)bh * nc + c];
  const int* lst = list + ((size_t)bh * nc + c) * T;
  __syncthreads();  // the previous chunk's readers are done
  load_rows<512>(kR, k, b, T, C, h, c * TS);
  load_rows<512>(vR, v, b, T, C, h, c * TS);
  // adk[u][vv] = dK[key 16rt + 4fg + vv][d 16(2cp + u) + fr] (adv the same for dV)
  f4 adk[2] = {z, z}, adv[2] = {z, z};
  // Block b0's list entries, their lse and D, and its gathered q and dy rows
  // are fetched into registers while block b0 - 64 runs (thread: list
  // entry tid; rows tid/16 and tid/16 + 32, 4 columns at 4 (tid%16)).
  int pt = 0;
  float pL = 0.f, pD = 0.f;
  f4 pq4[2], pd4[2];
  auto fetch = [&](int b0) {
    const int n = min(TS, n_all - b0);
    if (tid < TS) {
      pt = tid < n ? lst[b0 + tid] : 0;
      pL = tid < n ? lse[(size_t)bh * T + pt] : 0.f;
      pD = tid < n ? Din[(size_t)bh * T + pt] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int row = (tid >> 4) + 32 * j, cc = (tid & 15) * 4;
      pq4[j] = pd4[j] = z;
      if (row < n) {
        const size_t o = ((size_t)b * T + lst[b0 + row]) * C + h * HN + cc;
        pq4[j] = *reinterpret_cast<const f4*>(q + o);
        pd4[j] = *reinterpret_cast<const f4*>(dy + o);
      }
    }
  };
  if (n_all > 0) fetch(0);
  for (int b0 = 0; b0 < n_all; b0 += TS) {
    const int n = min(TS, n_all - b0);
    __syncthreads();  // the previous block's readers are done
    if (tid < TS) {
      idx[tid] = pt;
      Ls[tid] = pL;
      Ds[tid] = pD;
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int row = (tid >> 4) + 32 * j, cc = (tid & 15) * 4;
      *reinterpret_cast<f4*>(&qR[row][cc]) = pq4[j];
      *reinterpret_cast<f4*>(&doR[row][cc]) = pd4[j];
    }
    __syncthreads();
    if (b0 + TS < n_all) fetch(b0 + TS);
    // s[u][vv] = S^T[key 16rt + 4fg + vv][query 16(2cp + u) + fr]; dp likewise
    f4 s[2] = {z, z}, dp[2] = {z, z};
#pragma unroll
    for (int kg = 0; kg < 4; kg++) {
      const f4 ak = ldf4(&kR[16 * rt + fr][16 * kg + 4 * fg]);
      const f4 av = ldf4(&vR[16 * rt + fr][16 * kg + 4 * fg]);
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int qr = 16 * (2 * cp + u) + fr;
        s[u] = mma16(ak, ldf4(&qR[qr][16 * kg + 4 * fg]), s[u]);
        dp[u] = mma16(av, ldf4(&doR[qr][16 * kg + 4 * fg]), dp[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int qi = 16 * (2 * cp + u) + fr;
      const int t = qi < n ? idx[qi] : -1;
      const float L = Ls[qi], D = Ds[qi];
#pragma unroll
      for (int vv = 0; vv < 4; vv++) {
        const int kl = 16 * rt + 4 * fg + vv, key = c * TS + kl;
        const float p = (t >= 0 && key <= t) ? expf(s[u][vv] * SCALE - L) : 0.f;
        pT[kl][qi] = p;
        dsT[kl][qi] = p * (dp[u][vv] - D);
      }
    }
    __syncthreads();
    // dV[key][d] += sum_q P^T[key][q] dY[q][d];  dK[key][d] += sum_q dS^T[key][q] Q[q][d]
#pragma unroll
    for (int kg = 0; kg < 4; kg++) {
      const f4 ap = ldf4(&pT[16 * rt + fr][16 * kg + 4 * fg]);
      const f4 ad = ldf4(&dsT[16 * rt + fr][16 * kg + 4 * fg]);
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int dcol = 16 * (2 * cp + u) + fr;
        adv[u] = mma16(ap, colf4(doR, 16 * kg, fg, dcol), adv[u]);
        adk[u] = mma16(ad, colf4(qR, 16 * kg, fg, dcol), adk[u]);
      }
    }
    // dq share[q][d] = sum_key dS[q][key] K[key][d]: queries of tile rt
    f4 aq[2] = {z, z};
#pragma unroll
    for (int kg = 0; kg < 4; kg++) {
      const f4 a = {dsT[16 * kg + 4 * fg][16 * rt + fr], dsT[16 * kg + 4 * fg + 1][16 * rt + fr],
                    dsT[16 * kg + 4 * fg + 2][16 * rt + fr], dsT[16 * kg + 4 * fg + 3][16 * rt + fr]};
#pragma unroll
      for (int u = 0; u < 2; u++) aq[u] = mma16(a, colf4(kR, 16 * kg, fg, 16 * (2 * cp + u) + fr), aq[u]);
    }
#pragma unroll
    for (int vv = 0; vv < 4; vv++) {
      const int r = 16 * rt + 4 * fg + vv;
      if (r >= n) continue;
      const int t = idx[r];
      const int j = slot_of(sel[(size_t)bh * T + t], c);
      if (j >= K) continue;  // as in sp_fwd
      float* dst = pq + (((size_t)bh * T + t) * K + j) * HN;
#pragma unroll
      for (int u = 0; u < 2; u++) dst[16 * (2 * cp + u) + fr] = aq[u][vv] * SCALE;
    }
  }
#pragma unroll
  for (int vv = 0; vv < 4; vv++) {
    const int key = c * TS + 16 * rt + 4 * fg + vv;
    if (key >= T) continue;
    const size_t e = ((size_t)b * T + key) * C + h * HN;
#pragma unroll
    for (int u = 0; u < 2; u++) {
      dk[e + 16 * (2 * cp + u) + fr] = adk[u][vv] * SCALE;
      dv[e + 16 * (2 * cp + u) + fr] = adv[u][vv];
    }
  }
  }
}

// dq = sum over the query's slots in chunk order (16 lanes per row).
__global__ __launch_bounds__(256) void sp_dq(int BHT, int T, int H, int K, const uint64_t* __restrict__ sel,
                                             const float* __restrict__ pq, float* __restrict__ dq) {
  const int g = blockIdx.x * 16 + (threadIdx.x >> 4), l16 = threadIdx.x & 15;
  if (g >= BHT) return;
  const int bh = g / T, t = g - bh * T, b = bh / H, h = bh - b * H, C = H * HN;
  const int ns = min(__popcll(sel[g]), K);
  f4 a = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < ns; j++) a += *reinterpret_cast<const f4*>(pq + ((size_t)g * K + j) * HN + 4 * l16);
  *reinterpret_cast<f4*>(dq + ((size_t)b * T + t) * C + h * HN + 4 * l16) = a;
}

}  // namespace mobak

int moba_num_chunks(int T, int chunk) { return (T + chunk - 1) / chunk; }

namespace {
// Workspace layout (both directions): chunk means, the row sums D, and for
// chunks of 64 the query lists, their counts and the per-slot partials.
struct MobaWs {
  float *kbar, *D, *part, *pm, *pl;
  int *list, *cnt;
  size_t bytes;
};
MobaWs moba_carve(void* base, int B, int T, int H, int chunk, int topk) {
  const int nc = moba_num_chunks(T, chunk), K = std::min(topk, nc);
  const size_t BH = (size_t)B * H, rows = BH * T;
  MobaWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    off = (off + 255) & ~(size_t)255;
    char* p = base ? (char*)base + off : nullptr;
    off += bytes;
    return p;
  };
  w.kbar = (float*)take(BH * nc * mobak::HN * sizeof(float));
  w.D = (float*)take(rows * sizeof(float));
  if (chunk == mobak::TS) {
    w.list = (int*)take(BH * nc * T * sizeof(int));
    w.cnt = (int*)take(BH * nc * sizeof(int));
    w.part = (float*)take(rows * K * mobak::HN * sizeof(float));
    w.pm = (float*)take(rows * K * sizeof(float));
    w.pl = (float*)take(rows * K * sizeof(float));
  }
  w.bytes = off;
  return w;
}
}  // namespace

size_t moba_ws_bytes(int B, int T, int H, int chunk, int topk) {
  return moba_carve(nullptr, B, T, H, chunk, topk).bytes;
}

hipError_t moba_launch_forward(int B, int T, int H, int chunk, int topk, const float* q, const float* k,
                               const float* v, float* y, float* lse, uint64_t* sel, void* ws,
                               hipStream_t st) {
  const int nc = moba_num_chunks(T, chunk);
  const MobaWs w = moba_carve(ws, B, T, H, chunk, topk);
  hipLaunchKernelGGL(mobak::kbar, dim3(nc, B * H), dim3(64), 0, st, T, H, chunk, k, w.kbar);
  const size_t waves = (size_t)B * T * H;
  hipLaunchKernelGGL(mobak::select, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, B, T, H, chunk, nc,
                     topk, q, w.kbar, sel);
  const int nqt = (T + mobak::TS - 1) / mobak::TS;
  if (chunk != mobak::TS) {
    hipLaunchKernelGGL(mobak::fwd, dim3(nqt, B * H), dim3(256), 0, st, T, H, chunk, nc, q, k, v, sel, y, lse);
    return hipGetLastError();
  }
  const int K = std::min(topk, nc), BHT = B * H * T;
  hipLaunchKernelGGL(mobak::sp_list, dim3(nc, B * H), dim3(256), 0, st, T, nc, sel, w.list, w.cnt);
  hipLaunchKernelGGL(mobak::sp_fwd, dim3((nc + 1) / 2, B * H), dim3(256), 0, st, T, H, nc, K, q, k, v, sel, w.list,
                     w.cnt, w.part, w.pm, w.pl);
  hipLaunchKernelGGL(mobak::sp_merge, dim3((BHT + 15) / 16), dim3(256), 0, st, BHT, T, H, K, sel, w.part,
                     w.pm, w.pl, y, lse);
  return hipGetLastError();
}

hipError_t moba_launch_backward(int B, int T, int H, int chunk, int topk, const float* q, const float* k,
                                const float* v, const float* y, const float* lse, const uint64_t* sel,
                                const float* dy, float* dq, float* dk, float* dv, void* ws,
                                hipStream_t st) {
  const int nc = moba_num_chunks(T, chunk);
  const int nt = (T + mobak::TS - 1) / mobak::TS;
  const MobaWs w = moba_carve(ws, B, T, H, chunk, topk);
  if (chunk != mobak::TS) {
    hipLaunchKernelGGL(mobak::bwd_dq, dim3(nt, B * H), dim3(256), 0, st, T, H, chunk, nc, q, k, v, y, lse,
                       sel, dy, dq, w.D);
    hipLaunchKernelGGL(mobak::bwd_dkv, dim3(nt, B * H), dim3(256), 0, st, T, H, chunk, nc, q, k, v, lse, w.D,
                       sel, dy, dk, dv);
    return hipGetLastError();
  }
  const int K = std::min(topk, nc), BHT = B * H * T;
  hipLaunchKernelGGL(mobak::sp_list, dim3(nc, B * H), dim3(256), 0, st, T, nc, sel, w.list, w.cnt);
  hipLaunchKernelGGL(mobak::sp_rowdot, dim3((BHT + 15) / 16), dim3(256), 0, st, BHT, T, H, y, dy, w.D);
  hipLaunchKernelGGL(mobak::sp_bwd, dim3((nc + 1) / 2, B * H), dim3(512), 0, st, T, H, nc, K, q, k, v, lse, w.D, sel,
                     dy, w.list, w.cnt, dk, dv, w.part);
  hipLaunchKernelGGL(mobak::sp_dq, dim3((BHT + 15) / 16), dim3(256), 0, st, BHT, T, H, K, sel, w.part, dq);
  return hipGetLastError();
}
