// GatedDeltaNet layer on gfx950, forward and through-gradient backward
// ("cortiq_engine/fcd_ops.rs", GatedDeltaNet through-backward section).
//
// Per window of T positions from a fresh state:
//   pre = causal depthwise conv(raw), cq = silu(pre)   [c_dim = 2 nk dk + nv dv]
//   q^ = q / (sqrt(|q|^2 + 1e-6) sqrt(dk)), k^ = k / sqrt(|k|^2 + 1e-6)
//   g = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b)
//   per v-head: S <- g S; kv = S^T k^; S <- S + k^ (beta (v - kv))^T; o = S^T q^
//   out = o / sqrt(mean(o^2) + eps) * norm * silu(z)
//
// S is [dk][dv].  In the forward every value column j of S evolves on its
// own (kv[j], the update of column j and o[j] only touch column j), so a
// workgroup owns 16 columns of one (batch, head): 16 lanes per column (one
// DPP row), each lane dk/16 key rows, and the column sums kv and o are
// 16-lane DPP sums.  The per-token inputs are staged through LDS in blocks
// of 16 tokens, and the state is checkpointed at every block start.  The
// backward walks the blocks in reverse, recomputes each block's states from
// its checkpoint, and runs the reverse step per column; the sums that cross
// columns (dq^ and dk^ over the value index, dg and dbeta over columns) are
// reduced across the wave's four columns with permlane swaps, across the
// four waves through LDS, and across the column blocks through fp32
// partials summed in a fixed order by the chain kernel.

#include "common.hpp"
#include "gdn.hpp"

namespace gdnk {

constexpr int TT = 16;   // tokens per staging block = checkpoint interval
constexpr int CB = 16;   // value columns per workgroup
constexpr int RF = 8;    // backward: tokens per flush of the cross-column sums
constexpr float L2_EPS = 1e-6f;
constexpr float SP_CUT = 20.0f;

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ float silu(float x) { return x * sigm(x); }
__device__ __forceinline__ float silu_grad(float x) {
  const float s = sigm(x);
  return s * (1.0f + x * (1.0f - s));
}
__device__ __forceinline__ float softplus(float x) { return x > SP_CUT ? x : log1pf(expf(x)); }
__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }

// ----------------------------------------------------------- convolution --
// pre[b][t][c] = sum_j raw[b][t - (kk-1) + j][c] conv[c][j] (zero before the
// window), cq = silu(pre); four channels per thread.
__global__ __launch_bounds__(256) void conv_fwd(int BT, int T, int cdim, int kk,
                                                const float* __restrict__ raw,
                                                const float* __restrict__ conv,
                                                float* __restrict__ pre, float* __restrict__ cq) {
  const size_t n4 = (size_t)BT * cdim / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t e = i * 4;
    const size_t bt = e / cdim;
    const int c = (int)(e - bt * cdim);
    const int t = (int)(bt % T);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < kk; j++) {
      const int back = kk - 1 - j;
      if (t - back < 0) continue;
      const f4 x = ld4(raw + e - (size_t)back * cdim);
#pragma unroll
      for (int m = 0; m < 4; m++) acc[m] = fmaf(x[m], conv[(size_t)(c + m) * kk + j], acc[m]);
    }
    st4(pre + e, acc);
    f4 s;
#pragma unroll
    for (int m = 0; m < 4; m++) s[m] = silu(acc[m]);
    st4(cq + e, s);
  }
}

// draw[b][t][c] = sum_j dpre[b][t + (kk-1) - j][c] conv[c][j] over positions
// inside the window, dpre = dcq silu'(pre).
__global__ __launch_bounds__(256) void conv_bwd(int BT, int T, int cdim, int kk,
                                                const float* __restrict__ pre,
                                                const float* __restrict__ dcq,
                                                const float* __restrict__ conv,
                                                float* __restrict__ draw) {
  const size_t n4 = (size_t)BT * cdim / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t e = i * 4;
    const size_t bt = e / cdim;
    const int c = (int)(e - bt * cdim);
    const int t = (int)(bt % T);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < kk; j++) {
      const int fwd = kk - 1 - j;
      if (t + fwd >= T) continue;
      const size_t ef = e + (size_t)fwd * cdim;
      const f4 p = ld4(pre + ef), d = ld4(dcq + ef);
#pragma unroll
      for (int m = 0; m < 4; m++)
        acc[m] = fmaf(d[m] * silu_grad(p[m]), conv[(size_t)(c + m) * kk + j], acc[m]);
    }
    st4(draw + e, acc);
  }
}

// The same two convolutions for KK taps, a thread sliding over TBK
// consecutive tokens of one channel quad: its 4 x KK weights are read once,
// and each input row (forward) or dpre = dcq silu'(pre) (backward) is loaded
// or formed once for the TBK outputs that use it.  The sums run over the taps
// in the order above.
template <int KK, int TBK>
__global__ __launch_bounds__(256) void conv_fwd_t(int B, int T, int cdim,
                                                  const float* __restrict__ raw,
                                                  const float* __restrict__ conv,
                                                  float* __restrict__ pre, float* __restrict__ cq) {
  const int C4 = cdim / 4, ntb = (T + TBK - 1) / TBK;
  const size_t n = (size_t)B * ntb * C4;
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int c4 = (int)(i % C4);
    const size_t rest = i / C4;
    const int tb = (int)(rest % ntb);
    const size_t b = rest / ntb;
    const int c = 4 * c4, t0 = tb * TBK;
    float w[4][KK];
#pragma unroll
    for (int m = 0; m < 4; m++)
#pragma unroll
      for (int j = 0; j < KK; j++) w[m][j] = conv[(size_t)(c + m) * KK + j];
    // rows t0 - (KK-1) .. t0 + TBK - 1 (zero before the window)
    f4 x[TBK + KK - 1];
#pragma unroll
    for (int q = 0; q < TBK + KK - 1; q++) {
      const int t = t0 - (KK - 1) + q;
      x[q] = t >= 0 && t < T ? ld4(raw + (b * T + t) * cdim + c) : z;
    }
#pragma unroll
    for (int u = 0; u < TBK; u++) {
      if (t0 + u >= T) break;
      f4 acc = z;
#pragma unroll
      for (int j = 0; j < KK; j++)
#pragma unroll
        for (int m = 0; m < 4; m++) acc[m] = fmaf(x[u + j][m], w[m][j], acc[m]);
      const size_t e = (b * T + t0 + u) * cdim + c;
      st4(pre + e, acc);
      f4 sl;
#pragma unroll
      for (int m = 0; m < 4; m++) sl[m] = silu(acc[m]);
      st4(cq + e, sl);
    }
  }
}

template <int KK, int TBK>
__global__ __launch_bounds__(256) void conv_bwd_t(int B, int T, int cdim,
                                                  const float* __restrict__ pre,
                                                  const float* __restrict__ dcq,
                                                  const float* __restrict__ conv,
                                                  float* __restrict__ draw) {
  const int C4 = cdim / 4, ntb = (T + TBK - 1) / TBK;
  const size_t n = (size_t)B * ntb * C4;
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int c4 = (int)(i % C4);
    const size_t rest = i / C4;
    const int tb = (int)(rest % ntb);
    const size_t b = rest / ntb;
    const int c = 4 * c4, t0 = tb * TBK;
    float w[4][KK];
#pragma unroll
    for (int m = 0; m < 4; m++)
#pragma unroll
      for (int j = 0; j < KK; j++) w[m][j] = conv[(size_t)(c + m) * KK + j];
    // dpre of rows t0 .. t0 + TBK + KK - 2 (zero past the window)
    f4 dp[TBK + KK - 1];
#pragma unroll
    for (int q = 0; q < TBK + KK - 1; q++) {
      const int t = t0 + q;
      dp[q] = z;
      if (t < T) {
        const size_t e = (b * T + t) * cdim + c;
        const f4 pv = ld4(pre + e), dv = ld4(dcq + e);
#pragma unroll
        for (int m = 0; m < 4; m++) dp[q][m] = dv[m] * silu_grad(pv[m]);
      }
    }
#pragma unroll
    for (int u = 0; u < TBK; u++) {
      if (t0 + u >= T) break;
      f4 acc = z;
#pragma unroll
      for (int j = 0; j < KK; j++)
#pragma unroll
        for (int m = 0; m < 4; m++) acc[m] = fmaf(dp[u + KK - 1 - j][m], w[m][j], acc[m]);
      st4(draw + (b * T + t0 + u) * cdim + c, acc);
    }
  }
}

// --------------------------------------------------- normalised q/k, gates --
// One 16-lane group per (token, k-head): q^ and k^ (DK/16 values per lane);
// lanes l < rep also make g and beta of v-head ko * rep + l.
template <int DK>
__global__ __launch_bounds__(256) void prep(int BT, int nk, int nv, int cdim,
                                            const float* __restrict__ cq,
                                            const float* __restrict__ a,
                                            const float* __restrict__ bb,
                                            const float* __restrict__ A_log,
                                            const float* __restrict__ dt_bias,
                                            float* __restrict__ qh, float* __restrict__ kh,
                                            float* __restrict__ g, float* __restrict__ beta) {
  constexpr int R4 = DK / 64;  // float4 per lane
  const size_t gid = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  if (gid >= (size_t)BT * nk) return;
  const size_t bt = gid / nk;
  const int ko = (int)(gid - bt * nk);
  const int kd = nk * DK, rep = nv / nk;
  const float* qr = cq + bt * cdim + (size_t)ko * DK;
  const float* kr = qr + kd;
  f4 q[R4], k[R4];
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int m = 0; m < R4; m++) {
    q[m] = ld4(qr + l16 * 4 + 64 * m);
    k[m] = ld4(kr + l16 * 4 + 64 * m);
    sq += (q[m][0] * q[m][0] + q[m][1] * q[m][1]) + (q[m][2] * q[m][2] + q[m][3] * q[m][3]);
    sk += (k[m][0] * k[m][0] + k[m][1] * k[m][1]) + (k[m][2] * k[m][2] + k[m][3] * k[m][3]);
  }
  sq = rowsum16(sq) + L2_EPS;
  sk = rowsum16(sk) + L2_EPS;
  const float invq = 1.0f / (sqrtf(sq) * sqrtf((float)DK)), invk = 1.0f / sqrtf(sk);
  float* qo = qh + gid * DK;
  float* ko_ = kh + gid * DK;
#pragma unroll
  for (int m = 0; m < R4; m++) {
    st4(qo + l16 * 4 + 64 * m, q[m] * invq);
    st4(ko_ + l16 * 4 + 64 * m, k[m] * invk);
  }
  if (l16 < rep) {
    const int h = ko * rep + l16;
    const size_t i = bt * nv + h;
    g[i] = expf(-expf(A_log[h]) * softplus(a[i] + dt_bias[h]));
    beta[i] = sigm(bb[i]);
  }
}

// ------------------------------------------------------ gated RMSNorm --
// One 16-lane group per (token, v-head): out = o inv norm silu(z),
// inv = 1 / sqrt(mean(o^2) + eps).  dv = 64 * NV4.
template <int NV4>
__global__ __launch_bounds__(256) void rms_fwd(int BTH, int nv, float eps,
                                               const float* __restrict__ o,
                                               const float* __restrict__ z,
                                               const float* __restrict__ norm,
                                               float* __restrict__ out) {
  constexpr int DV = 64 * NV4;
  const size_t gid = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  if (gid >= (size_t)BTH) return;
  const size_t base = gid * DV;
  f4 ov[NV4];
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < NV4; m++) {
    ov[m] = ld4(o + base + l16 * 4 + 64 * m);
    s += (ov[m][0] * ov[m][0] + ov[m][1] * ov[m][1]) + (ov[m][2] * ov[m][2] + ov[m][3] * ov[m][3]);
  }
  const float inv = 1.0f / sqrtf(rowsum16(s) / DV + eps);
#pragma unroll
  for (int m = 0; m < NV4; m++) {
    const int j = l16 * 4 + 64 * m;
    const f4 zz = ld4(z + base + j), w = ld4(norm + j);
    f4 r;
#pragma unroll
    for (int c = 0; c < 4; c++) r[c] = ov[m][c] * inv * w[c] * silu(zz[c]);
    st4(out + base + j, r);
  }
}

// dz = dout o inv norm silu'(z);  do = inv w_eff dout - o inv^3 mean(dout w_eff o),
// w_eff = norm silu(z).
template <int NV4>
__global__ __launch_bounds__(256) void rms_bwd(int BTH, int nv, float eps,
                                               const float* __restrict__ o,
                                               const float* __restrict__ z,
                                               const float* __restrict__ norm,
                                               const float* __restrict__ dout,
                                               float* __restrict__ dz, float* __restrict__ dobuf) {
  constexpr int DV = 64 * NV4;
  const size_t gid = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  if (gid >= (size_t)BTH) return;
  const size_t base = gid * DV;
  f4 ov[NV4], dv4[NV4], zz[NV4];
  float s = 0.f, sd = 0.f;
#pragma unroll
  for (int m = 0; m < NV4; m++) {
    const int j = l16 * 4 + 64 * m;
    ov[m] = ld4(o + base + j);
    dv4[m] = ld4(dout + base + j);
    zz[m] = ld4(z + base + j);
    const f4 w = ld4(norm + j);
#pragma unroll
    for (int c = 0; c < 4; c++) {
      s += ov[m][c] * ov[m][c];
      sd += dv4[m][c] * w[c] * silu(zz[m][c]) * ov[m][c];
    }
  }
  const float inv = 1.0f / sqrtf(rowsum16(s) / DV + eps);
  const float coef = rowsum16(sd) / DV * inv * inv * inv;
#pragma unroll
  for (int m = 0; m < NV4; m++) {
    const int j = l16 * 4 + 64 * m;
    const f4 w = ld4(norm + j);
    f4 dzz, d;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      dzz[c] = dv4[m][c] * ov[m][c] * inv * w[c] * silu_grad(zz[m][c]);
      d[c] = inv * w[c] * silu(zz[m][c]) * dv4[m][c] - ov[m][c] * coef;
    }
    st4(dz + base + j, dzz);
    st4(dobuf + base + j, d);
  }
}

// ------------------------------------------------------------ recurrence --
// Workgroup (b, h, column block), 256 threads: column cl = tid / 16 of the
// block (one DPP row), row group rg = tid % 16 owning key rows
// rg * RPL .. rg * RPL + RPL - 1.  Block inputs staged in LDS; a partial
// last block is padded with identity tokens (g = 1, beta = 0, k^ = q^ = 0).
template <int DK>
struct Stage {
  float k[2][TT][DK];
  float q[2][TT][DK];
  float v[2][TT][CB];
  float d[2][TT][CB];  // do (backward only)
  float g[2][TT];
  float b[2][TT];
};

// The staging in two halves, so that a block's inputs can be fetched
// into registers while the block before it runs: load_stage issues every
// global load of the block (from clamped, always valid token indices, so all
// are in flight together), store_stage writes them (zeros, or the identity
// token past the end) to LDS buffer buf.
template <int DK>
struct StageRegs {
  static constexpr int NKQ = 2 * TT * DK / 4 / 256;  // float4 slots of k^, q^ per thread
  f4 kq[NKQ];
  float v, d, g, b;
};

template <int DK>
__device__ __forceinline__ void load_stage(StageRegs<DK>& o, int t0, int T, int nv, int dv,
                                           int cdim, int kvoff, size_t bT, int h, int ko,
                                           int col0, const float* qh, const float* kh,
                                           const float* cq, const float* gg, const float* be,
                                           const float* dob, bool with_do, int nk) {
  constexpr int NQ4 = TT * DK / 4;
  static_assert(2 * NQ4 % 256 == 0 && TT * CB == 256, "staging assumes 256 threads");
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < StageRegs<DK>::NKQ; q++) {
    const int f = tid + 256 * q;
    const int which = f / NQ4, r = f - which * NQ4, tok = r / (DK / 4), c4 = r - tok * (DK / 4);
    const int t = min(t0 + tok, T - 1);
    o.kq[q] = ld4((which ? qh : kh) + ((bT + t) * nk + ko) * DK + c4 * 4);
  }
  {
    const int tok = tid / CB, c = tid - tok * CB, t = min(t0 + tok, T - 1);
    o.v = cq[(bT + t) * cdim + kvoff + (size_t)h * dv + col0 + c];
    o.d = with_do ? dob[((bT + t) * nv + h) * dv + col0 + c] : 0.f;
  }
  {
    const int t = min(t0 + (tid & (TT - 1)), T - 1);
    o.g = gg[(bT + t) * nv + h];
    o.b = be[(bT + t) * nv + h];
  }
}

template <int DK>
__device__ __forceinline__ void store_stage(Stage<DK>& st, const StageRegs<DK>& o, int buf, int t0,
                                            int T, bool with_do) {
  constexpr int NQ4 = TT * DK / 4;
  const int tid = threadIdx.x;
  const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < StageRegs<DK>::NKQ; q++) {
    const int f = tid + 256 * q;
    const int which = f / NQ4, r = f - which * NQ4, tok = r / (DK / 4), c4 = r - tok * (DK / 4);
    st4(which ? &st.q[buf][tok][c4 * 4] : &st.k[buf][tok][c4 * 4], t0 + tok < T ? o.kq[q] : z);
  }
  {
    const int tok = tid / CB, c = tid - tok * CB;
    const bool ok = t0 + tok < T;
    st.v[buf][tok][c] = ok ? o.v : 0.f;
    if (with_do) st.d[buf][tok][c] = ok ? o.d : 0.f;
  }
  if (tid < TT) {
    const bool ok = t0 + tid < T;
    st.g[buf][tid] = ok ? o.g : 1.f;
    st.b[buf][tid] = ok ? o.b : 0.f;
  }
}

template <int DK>
__global__ __launch_bounds__(256) void fwd_seq(int B, int T, int nk, int nv, int dv, int cdim,
                                               const float* __restrict__ qh,
                                               const float* __restrict__ kh,
                                               const float* __restrict__ cq,
                                               const float* __restrict__ gg,
                                               const float* __restrict__ be,
                                               float* __restrict__ o, float* __restrict__ ckpt,
                                               float* __restrict__ kvo) {
  constexpr int RPL = DK / 16;
  __shared__ __attribute__((aligned(16))) Stage<DK> st;
  const int ncb = dv / CB;
  const int g_ = blockIdx.x;
  const int bh = g_ / ncb, cb = g_ - bh * ncb;
  const int b = bh / nv, h = bh - b * nv, ko = h / (nv / nk);
  const int tid = threadIdx.x, rg = tid & 15, cl = tid >> 4;
  const int col0 = cb * CB, col = col0 + cl;
  const size_t bT = (size_t)b * T;
  const int kvoff = 2 * nk * DK;
  const int nblk = (T + TT - 1) / TT;
  float s[RPL];
#pragma unroll
  for (int i = 0; i < RPL; i++) s[i] = 0.f;
  StageRegs<DK> nx;
  load_stage<DK>(nx, 0, T, nv, dv, cdim, kvoff, bT, h, ko, col0, qh, kh, cq, gg, be, nullptr, false,
                 nk);
  store_stage<DK>(st, nx, 0, 0, T, false);
  __syncthreads();
  int buf = 0;
  for (int blk = 0; blk < nblk; blk++, buf ^= 1) {
    const int t0 = blk * TT;
    const bool more = blk + 1 < nblk;
    if (more)  // in flight while this block runs
      load_stage<DK>(nx, t0 + TT, T, nv, dv, cdim, kvoff, bT, h, ko, col0, qh, kh, cq, gg, be,
                     nullptr, false, nk);
    if (ckpt) {
      float* cp = ckpt + (((size_t)bh * nblk + blk) * dv + col) * DK + rg * RPL;
#pragma unroll
      for (int i = 0; i < RPL; i += 4) st4(cp + i, f4{s[i], s[i + 1], s[i + 2], s[i + 3]});
    }
    float ob = 0.f, kb = 0.f;
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
      const float gt = st.g[buf][tt], bt_ = st.b[buf][tt], vt = st.v[buf][tt][cl];
      float kr[RPL], qr[RPL];
#pragma unroll
      for (int i = 0; i < RPL; i += 4) {
        const f4 x = ld4(&st.k[buf][tt][rg * RPL + i]), y = ld4(&st.q[buf][tt][rg * RPL + i]);
        kr[i] = x[0]; kr[i + 1] = x[1]; kr[i + 2] = x[2]; kr[i + 3] = x[3];
        qr[i] = y[0]; qr[i + 1] = y[1]; qr[i + 2] = y[2]; qr[i + 3] = y[3];
      }
      float kv = 0.f;
#pragma unroll
      for (int i = 0; i < RPL; i++) {
        s[i] *= gt;
        kv = fmaf(s[i], kr[i], kv);
      }
      kv = rowsum16(kv);
      kb = rg == tt ? kv : kb;
      const float u = bt_ * (vt - kv);
      float ov = 0.f;
#pragma unroll
      for (int i = 0; i < RPL; i++) {
        s[i] = fmaf(kr[i], u, s[i]);
        ov = fmaf(s[i], qr[i], ov);
      }
      ov = rowsum16(ov);
      ob = rg == tt ? ov : ob;
    }
    if (t0 + rg < T) {
      o[((bT + t0 + rg) * nv + h) * dv + col] = ob;
      if (kvo) kvo[((bT + t0 + rg) * nv + h) * dv + col] = kb;
    }
    // the other buffer was last read in the block before, behind the
    // previous barrier
    if (more) store_stage<DK>(st, nx, buf ^ 1, t0 + TT, T, false);
    lds_barrier();
  }
}

// Partials per (column block, b, t, h): [0, DK) dq^, [DK, 2 DK) dk^, 2 DK
// g dg (the gradient of log g), 2 DK + 1 dbeta (sums over the block's 16
// columns).
template <int DK>
__global__ __launch_bounds__(256) void bwd_seq(int B, int T, int nk, int nv, int dv, int cdim,
                                               const float* __restrict__ qh,
                                               const float* __restrict__ kh,
                                               const float* __restrict__ cq,
                                               const float* __restrict__ gg,
                                               const float* __restrict__ be,
                                               const float* __restrict__ dob,
                                               const float* __restrict__ ckpt,
                                               float* __restrict__ part, float* __restrict__ dcq) {
  constexpr int RPL = DK / 16, PW = 2 * DK + 2;
  __shared__ __attribute__((aligned(16))) Stage<DK> st;
  // cross-column sums of RF tokens (flushed to the partials every RF tokens,
  // so the LDS of two workgroups fits one CU)
  __shared__ __attribute__((aligned(16))) float red[4][RF][PW];
  const int ncb = dv / CB;
  const int g_ = blockIdx.x;
  const int bh = g_ / ncb, cb = g_ - bh * ncb;
  const int b = bh / nv, h = bh - b * nv, ko = h / (nv / nk);
  const int tid = threadIdx.x, rg = tid & 15, cl = tid >> 4, lane = tid & 63, wave = tid >> 6;
  const int col0 = cb * CB, col = col0 + cl;
  const size_t bT = (size_t)b * T;
  const int kvoff = 2 * nk * DK;
  const int nblk = (T + TT - 1) / TT;
  const size_t pstride = (size_t)B * T * nv * PW;  // one column block's partials

  float G[RPL];
#pragma unroll
  for (int i = 0; i < RPL; i++) G[i] = 0.f;
  int buf = 0;
  StageRegs<DK> nx;
  load_stage<DK>(nx, (nblk - 1) * TT, T, nv, dv, cdim, kvoff, bT, h, ko, col0, qh, kh, cq, gg, be,
                 dob, true, nk);
  store_stage<DK>(st, nx, 0, (nblk - 1) * TT, T, true);
  // this lane's checkpoint rows of the current block, then of the one before
  auto ck_rows = [&](int blk_, f4 (&o)[RPL / 4]) {
    const float* cp = ckpt + (((size_t)bh * nblk + blk_) * dv + col) * DK + rg * RPL;
#pragma unroll
    for (int i = 0; i < RPL; i += 4) o[i / 4] = ld4(cp + i);
  };
  f4 ckc[RPL / 4], ckn[RPL / 4];
  ck_rows(nblk - 1, ckc);
  __syncthreads();
  for (int blk = nblk - 1; blk >= 0; blk--, buf ^= 1) {
    const int t0 = blk * TT;
    if (blk > 0) {  // in flight while this block runs
      load_stage<DK>(nx, t0 - TT, T, nv, dv, cdim, kvoff, bT, h, ko, col0, qh, kh, cq, gg, be, dob,
                     true, nk);
      ck_rows(blk - 1, ckn);
    }
    // recompute: Sh[tt] = state before token tt, kvh[tt] = S_pre^T k^ (this column)
    float Sh[TT + 1][RPL], kvh[TT];
#pragma unroll
    for (int i = 0; i < RPL; i += 4) {
      const f4 x = ckc[i / 4];
      Sh[0][i] = x[0]; Sh[0][i + 1] = x[1]; Sh[0][i + 2] = x[2]; Sh[0][i + 3] = x[3];
    }
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
      const float gt = st.g[buf][tt], bt_ = st.b[buf][tt], vt = st.v[buf][tt][cl];
      float kv = 0.f;
#pragma unroll
      for (int i = 0; i < RPL; i++) kv = fmaf(Sh[tt][i] * gt, st.k[buf][tt][rg * RPL + i], kv);
      kv = rowsum16(kv);
      kvh[tt] = kv;
      const float u = bt_ * (vt - kv);
#pragma unroll
      for (int i = 0; i < RPL; i++) Sh[tt + 1][i] = fmaf(st.k[buf][tt][rg * RPL + i], u, Sh[tt][i] * gt);
    }
    float dvb = 0.f;
#pragma unroll
    for (int tt = TT - 1; tt >= 0; tt--) {
      const float gt = st.g[buf][tt], bt_ = st.b[buf][tt], vt = st.v[buf][tt][cl];
      const float dot = st.d[buf][tt][cl];
      float kr[RPL], qr[RPL];
#pragma unroll
      for (int i = 0; i < RPL; i += 4) {
        const f4 x = ld4(&st.k[buf][tt][rg * RPL + i]), y = ld4(&st.q[buf][tt][rg * RPL + i]);
        kr[i] = x[0]; kr[i + 1] = x[1]; kr[i + 2] = x[2]; kr[i + 3] = x[3];
        qr[i] = y[0]; qr[i + 1] = y[1]; qr[i + 2] = y[2]; qr[i + 3] = y[3];
      }
      // o = S_t^T q^: G += q^ do; dq^ += S_t do
      float pq[RPL], pk[RPL];
      float du = 0.f;
#pragma unroll
      for (int i = 0; i < RPL; i++) {
        G[i] = fmaf(qr[i], dot, G[i]);
        pq[i] = Sh[tt + 1][i] * dot;
        du = fmaf(G[i], kr[i], du);
      }
      du = rowsum16(du);
      // S_t = S_pre + k^ u^T, u = beta (v - kv)
      const float vmk = vt - kvh[tt];
      const float u = bt_ * vmk;
      const float dkv = -bt_ * du;
      dvb = rg == tt ? bt_ * du : dvb;
      float dgp = 0.f;
#pragma unroll
      for (int i = 0; i < RPL; i++) {
        const float dsp = fmaf(kr[i], dkv, G[i]);                 // dS_pre
        pk[i] = fmaf(gt * Sh[tt][i], dkv, G[i] * u);               // dS u + S_pre dkv
        dgp = fmaf(dsp, Sh[tt][i], dgp);
        G[i] = gt * dsp;
      }
      dgp = rowsum16(dgp);
      // sums over the wave's four columns (lanes l, l^16, l^32, l^48) as a
      // reduce-scatter: the 2 RPL values (dq^ then dk^ shares of this lane's
      // key rows) are split in four quarters of RPL / 2, and lane l ends with
      // quarter l / 16 summed over the four columns
      constexpr int NQ = RPL / 2;
      float x[2 * RPL];
#pragma unroll
      for (int i = 0; i < RPL; i++) {
        x[i] = pq[i];
        x[RPL + i] = pk[i];
      }
      rows4_reduce_scatter<NQ>(x);
      const float sg = rows4sum(dgp), sb = rows4sum(du * vmk);
      const int slot = tt % RF;
      {
        const int qtr = lane >> 4;  // quarter: 0, 1 = dq^ rows, 2, 3 = dk^ rows
        float* dst = &red[wave][slot][(qtr >> 1) * DK + rg * RPL + (qtr & 1) * NQ];
        if constexpr (NQ % 4 == 0) {
#pragma unroll
          for (int i = 0; i < NQ; i += 4) st4(dst + i, f4{x[i], x[i + 1], x[i + 2], x[i + 3]});
        } else {
#pragma unroll
          for (int i = 0; i < NQ; i++) dst[i] = x[i];
        }
        if (lane == 0) {
          red[wave][slot][2 * DK] = sg * gt;  // g dg: the gradient of log g
          red[wave][slot][2 * DK + 1] = sb;
        }
      }
      if (slot == 0) {  // tokens tt .. tt + RF - 1 complete: sum the four waves
        lds_barrier();
        for (int f = tid; f < RF * PW; f += 256) {
          const int k = f / PW, c = f - k * PW, t = t0 + tt + k;
          if (t < T) {
            const float v = (red[0][k][c] + red[1][k][c]) + (red[2][k][c] + red[3][k][c]);
            part[cb * pstride + ((bT + t) * nv + h) * PW + c] = v;
          }
        }
        lds_barrier();  // red consumed before the next tokens write it
      }
    }
    if (t0 + rg < T) dcq[(bT + t0 + rg) * cdim + kvoff + (size_t)h * dv + col] = dvb;
    if (blk > 0) {
      store_stage<DK>(st, nx, buf ^ 1, t0 - TT, T, true);
#pragma unroll
      for (int i = 0; i < RPL / 4; i++) ckc[i] = ckn[i];
    }
    lds_barrier();  // red consumed; the next block's staging visible
  }
}


// ------------------------------------------------------ two-pass backward --
// For dk = dv.  With G_t the gradient of the state after token t including
// that token's read-out (G_t = dS_t + q^_t do_t^T), the reverse step is
// G_{t-1} = q^_{t-1} do_{t-1}^T + g_t (G_t - beta_t k^_t du_t^T), du_t =
// G_t^T k^_t: every value column of G evolves on its own, so the scan (pass 1)
// runs without the states.  Pass 2 then gives, per 16-token block from the
// checkpoint S0 and the gradient Ge entering the block's last token from later
// tokens, with u_t = beta_t (v_t - kv_t) and the decay products
// P(a, b) = g_{a+1} ... g_b, E_t = g_0 ... g_t (block-local tokens):
//   dq^_t = S_t do_t = E_t S0 do_t + sum_{tau <= t} P(tau, t) k^_tau (u_tau . do_t)
//   dk^_t = G_t u_t - beta_t g_t S_{t-1} du_t
//         = P(t, 15) Ge u_t + sum_{tau >= t} P(t, tau) q^_tau (do_tau . u_t)
//           - sum_{tau > t} P(t, tau) beta_tau k^_tau (du_tau . u_t)
//           - beta_t [E_t S0 du_t + sum_{tau < t} P(tau, t) k^_tau (u_tau . du_t)]
//   dbeta_t = du_t . (v_t - kv_t),  dv_t = beta_t du_t
//   g_t dg_t = g_t <G_t - beta_t k^_t du_t^T, S_{t-1}> = Phi_t - beta_t du_t . v_t
// with Phi_t = <G_t, S_t> carried backward from the block end,
// Phi_{t-1} = Phi_t - beta_t du_t . v_t + o_{t-1} . do_{t-1}, and
// Phi_{L-1} = <Ge, S_{L-1}> + o_{L-1} . do_{L-1} (S_{L-1} = the next checkpoint).
// Every decay factor is a product of decays in (0, 1], so any g in that range
// is taken without overflow, and no step divides by g.

// Pass 1, workgroup and lane layout of bwd_seq.  Writes per block the
// gradient entering its last token (gend, [bh][blk][dv][dk] like the
// checkpoints) and that gradient's inner product with the state after the
// block, by value column (anc [bh][blk][dv]); per token du and dv = beta du
// (into dcq).
template <int DK>
__global__ __launch_bounds__(256) void bwd_scan(int B, int T, int nk, int nv, int dv, int cdim,
                                                const float* __restrict__ qh,
                                                const float* __restrict__ kh,
                                                const float* __restrict__ cq,
                                                const float* __restrict__ gg,
                                                const float* __restrict__ be,
                                                const float* __restrict__ dob,
                                                const float* __restrict__ ckpt,
                                                float* __restrict__ gend, float* __restrict__ du_out,
                                                float* __restrict__ anc, float* __restrict__ dcq) {
  constexpr int RPL = DK / 16;
  __shared__ __attribute__((aligned(16))) Stage<DK> st;
  const int ncb = dv / CB;
  const int bh = blockIdx.x / ncb, cb = blockIdx.x - bh * ncb;
  const int b = bh / nv, h = bh - b * nv, ko = h / (nv / nk);
  const int tid = threadIdx.x, rg = tid & 15, cl = tid >> 4;
  const int col0 = cb * CB, col = col0 + cl;
  const size_t bT = (size_t)b * T;
  const int kvoff = 2 * nk * DK;
  const int nblk = (T + TT - 1) / TT;
  float G[RPL];
#pragma unroll
  for (int i = 0; i < RPL; i++) G[i] = 0.f;
  int buf = 0;
  StageRegs<DK> nx;
  load_stage<DK>(nx, (nblk - 1) * TT, T, nv, dv, cdim, kvoff, bT, h, ko, col0, qh, kh, cq, gg, be,
                 dob, true, nk);
  store_stage<DK>(st, nx, 0, (nblk - 1) * TT, T, true);
  __syncthreads();
  for (int blk = nblk - 1; blk >= 0; blk--, buf ^= 1) {
    const int t0 = blk * TT;
    if (blk > 0)  // in flight while this block runs
      load_stage<DK>(nx, t0 - TT, T, nv, dv, cdim, kvoff, bT, h, ko, col0, qh, kh, cq, gg, be, dob,
                     true, nk);
    {  // the gradient entering this block's last token, and its anchor
      const size_t so = (((size_t)bh * nblk + blk) * dv + col) * DK + rg * RPL;
      float an = 0.f;
      const float* sn = blk + 1 < nblk ? ckpt + so + (size_t)dv * DK : nullptr;
#pragma unroll
      for (int i = 0; i < RPL; i += 4) {
        st4(gend + so + i, f4{G[i], G[i + 1], G[i + 2], G[i + 3]});
        if (sn) {
          const f4 x = ld4(sn + i);
          an = fmaf(G[i], x[0], fmaf(G[i + 1], x[1], fmaf(G[i + 2], x[2], fmaf(G[i + 3], x[3], an))));
        }
      }
      an = rowsum16(an);
      if (rg == 0) anc[((size_t)bh * nblk + blk) * dv + col] = an;
    }
    float dub = 0.f;
#pragma unroll
    for (int tt = TT - 1; tt >= 0; tt--) {
      const float gt = st.g[buf][tt], bt_ = st.b[buf][tt], dot = st.d[buf][tt][cl];
      float kr[RPL], qr[RPL];
#pragma unroll
      for (int i = 0; i < RPL; i += 4) {
        const f4 x = ld4(&st.k[buf][tt][rg * RPL + i]), y = ld4(&st.q[buf][tt][rg * RPL + i]);
        kr[i] = x[0]; kr[i + 1] = x[1]; kr[i + 2] = x[2]; kr[i + 3] = x[3];
        qr[i] = y[0]; qr[i + 1] = y[1]; qr[i + 2] = y[2]; qr[i + 3] = y[3];
      }
      float du = 0.f;
#pragma unroll
      for (int i = 0; i < RPL; i++) {
        G[i] = fmaf(qr[i], dot, G[i]);
        du = fmaf(G[i], kr[i], du);
      }
      du = rowsum16(du);
      dub = rg == tt ? du : dub;
      const float c = -bt_ * du;
#pragma unroll
      for (int i = 0; i < RPL; i++) G[i] = gt * fmaf(kr[i], c, G[i]);
    }
    if (t0 + rg < T) {
      const size_t t = bT + t0 + rg;
      du_out[(t * nv + h) * dv + col] = dub;
      dcq[t * cdim + kvoff + (size_t)h * dv + col] = st.b[buf][rg] * dub;
    }
    if (blk > 0) store_stage<DK>(st, nx, buf ^ 1, t0 - TT, T, true);
    lds_barrier();
  }
}

__device__ __forceinline__ f4 mma16(f4 a, f4 b, f4 c) {
#pragma unroll
  for (int s = 0; s < 4; s++) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

// Pass 2: one workgroup per (b, v-head, 16-token block), D / 16 waves; wave w
// owns key columns 16w..16w+15 of dq^ and dk^.  MFMA lane layout (16x16x4 f32
// steps over a group of 16 k): A fragment lane l holds A[l%16][4(l/16)+s], B
// fragment B[4(l/16)+s][l%16], result element v = C[4(l/16)+v][l%16].
template <int D>
__global__ __launch_bounds__(64 * (D / 16)) void bwd_blk(int B, int T, int nk, int nv, int cdim,
                                                        const float* __restrict__ qh,
                                                        const float* __restrict__ kh,
                                                        const float* __restrict__ cq,
                                                        const float* __restrict__ gg,
                                                        const float* __restrict__ be,
                                                        const float* __restrict__ o,
                                                        const float* __restrict__ dob,
                                                        const float* __restrict__ ckpt,
                                                        const float* __restrict__ gend,
                                                        const float* __restrict__ du_in,
                                                        const float* __restrict__ kvi,
                                                        const float* __restrict__ anc,
                                                        float* __restrict__ part) {
  constexpr int NW = D / 16, NT = 64 * NW, RS = D + 4, XS = TT + 4, PW = 2 * D + 2;
  constexpr int SLOTS = TT * D / 4;  // float4 slots of one [TT][D] block
  static_assert(SLOTS % NT == 0, "staging assumes whole passes");
  __shared__ __attribute__((aligned(16))) float sDO[TT][RS];
  __shared__ __attribute__((aligned(16))) float sDU[TT][RS];
  __shared__ __attribute__((aligned(16))) float sU[TT][RS];
  __shared__ __attribute__((aligned(16))) float sQ[TT][RS];   // q^_t
  __shared__ __attribute__((aligned(16))) float sKB[TT][RS];  // beta_t k^_t
  __shared__ __attribute__((aligned(16))) float sK[TT][RS];   // k^_t
  // the Gram terms times their decay products
  __shared__ __attribute__((aligned(16))) float xA1[TT][XS];  // P(tau, t) do_t . u_tau, tau <= t
  __shared__ __attribute__((aligned(16))) float xB1[TT][XS];  // P(t, tau) u_t . do_tau, tau >= t
  __shared__ __attribute__((aligned(16))) float xB2[TT][XS];  // P(t, tau) u_t . du_tau, tau > t
  __shared__ __attribute__((aligned(16))) float xC2[TT][XS];  // P(tau, t) du_t . u_tau, tau < t
  __shared__ float sP[TT][TT + 1];                            // P(a, b), a <= b
  __shared__ float sE[TT], sG[TT], sBe[TT];
  __shared__ float sDb[TT], sOd[TT], sDvb[TT];  // dbeta, o . do, beta du . v per token
  __shared__ float sAnc;

  const int nblk = (T + TT - 1) / TT;
  const int gi = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = gi / nblk, blk = gi - bh * nblk;
  const int b = bh / nv, h = bh - b * nv, ko = h / (nv / nk);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, fr = lane & 15, fg = lane >> 4;
  const int t0 = blk * TT, n = min(TT, T - t0);
  const size_t bT = (size_t)b * T;
  const int kvoff = 2 * nk * D;
  const f4 z = {0.f, 0.f, 0.f, 0.f};

  // state fragments (B operand): sf[kg][s] = S0[i][16 kg + 4 fg + s], i = 16 w + fr
  const int i_key = 16 * w + fr;
  const size_t sb = ((size_t)bh * nblk + blk) * D * D;
  f4 sf[NW], gf[NW];
#pragma unroll
  for (int kg = 0; kg < NW; kg++) {
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const size_t j = 16 * kg + 4 * fg + s;
      sf[kg][s] = ckpt[sb + j * D + i_key];
      gf[kg][s] = gend[sb + j * D + i_key];
    }
  }
  if (tid < TT) {  // tokens past the end: g = 1, beta = 0
    const bool ok = tid < n;
    const size_t i = (bT + t0 + (ok ? tid : 0)) * nv + h;
    sG[tid] = ok ? gg[i] : 1.f;
    sBe[tid] = ok ? be[i] : 0.f;
  }
  if (w == 1) {  // the anchor: sum of the block end's per-column inner products
    float a = 0.f;
    for (int c = lane; c < D; c += 64) a += anc[((size_t)bh * nblk + blk) * D + c];
    a = wavesum(a);
    if (lane == 0) sAnc = a;
  }
  __syncthreads();
  static_assert(TT * TT <= NT, "one thread per decay product");
  if (tid < TT * TT) {  // products over the block's tokens, multiplied in token order
    const int a0 = tid / TT, b0 = tid - a0 * TT;
    float pr = 1.f;
    for (int q = a0 + 1; q <= b0; q++) pr *= sG[q];
    sP[a0][b0] = pr;
    if (tid < TT) {
      float e = 1.f;
      for (int q = 0; q <= tid; q++) e *= sG[q];
      sE[tid] = e;
    }
  }
  // stage the block: thread -> (token, 4 columns); per-token dot products over
  // the D columns summed by the D / 4 threads of a token
  constexpr int TPT = D / 4;  // threads per token in one pass
#pragma unroll
  for (int pass = 0; pass < SLOTS / NT; pass++) {
    const int f = tid + NT * pass, t = f / TPT, c4 = (f - t * TPT) * 4;
    const bool ok = t < n;
    const size_t tg = bT + t0 + (ok ? t : 0);
    const size_t vi = (tg * nv + h) * D + c4;
    const size_t ki = (tg * nk + ko) * D + c4;
    const f4 xdo = ok ? ld4(dob + vi) : z, xdu = ok ? ld4(du_in + vi) : z;
    const f4 xv = ok ? ld4(cq + tg * cdim + kvoff + (size_t)h * D + c4) : z;
    const f4 xkv = ok ? ld4(kvi + vi) : z, xo = ok ? ld4(o + vi) : z;
    const f4 xq = ok ? ld4(qh + ki) : z, xk = ok ? ld4(kh + ki) : z;
    const float bt_ = sBe[t];
    const f4 vk = xv - xkv;
    const f4 u = bt_ * vk;
    *reinterpret_cast<f4*>(&sDO[t][c4]) = xdo;
    *reinterpret_cast<f4*>(&sDU[t][c4]) = xdu;
    *reinterpret_cast<f4*>(&sU[t][c4]) = u;
    *reinterpret_cast<f4*>(&sQ[t][c4]) = xq;
    *reinterpret_cast<f4*>(&sKB[t][c4]) = bt_ * xk;
    *reinterpret_cast<f4*>(&sK[t][c4]) = xk;
    float pdb = 0.f, pod = 0.f, pdv = 0.f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      pdb = fmaf(xdu[c], vk[c], pdb);
      pod = fmaf(xo[c], xdo[c], pod);
      pdv = fmaf(xdu[c], xv[c], pdv);
    }
    // the TPT threads of token t are one aligned group of 16 or 32 lanes
    pdb = rowsum16(pdb);
    pod = rowsum16(pod);
    pdv = rowsum16(pdv);
    if (TPT == 32) {
      auto sw = [](float x) {
        auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(p[0]) + __uint_as_float(p[1]);
      };
      pdb = sw(pdb);
      pod = sw(pod);
      pdv = sw(pdv);
    }
    if (f - t * TPT == 0) {
      sDb[t] = pdb;
      sOd[t] = pod;
      sDvb[t] = bt_ * pdv;
    }
  }
  __syncthreads();
  // Gram matrices over the D values: wave 0 do.u, wave 1 u.du
  if (w < 2) {
    const float(*P)[RS] = w == 0 ? sDO : sU;
    const float(*Q)[RS] = w == 0 ? sU : sDU;
    f4 x = z;
#pragma unroll
    for (int kg = 0; kg < NW; kg++)
      x = mma16(*reinterpret_cast<const f4*>(&P[fr][16 * kg + 4 * fg]),
                *reinterpret_cast<const f4*>(&Q[fr][16 * kg + 4 * fg]), x);
    // x[v] = X[t = 4 fg + v][tau = fr]
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int t = 4 * fg + v;
      if (w == 0) {  // X = do . u^T
        const float y = x[v] * sP[fr][t];
        xA1[t][fr] = fr <= t ? y : 0.f;
        xB1[fr][t] = t >= fr ? y : 0.f;  // B1[t'][tau'] = X[tau'][t'], tau' >= t'
      } else {  // X = u . du^T
        const float y = x[v] * sP[t][fr];
        xB2[t][fr] = fr > t ? y : 0.f;
        xC2[fr][t] = t < fr ? y : 0.f;  // C2[t'][tau'] = X[tau'][t'], tau' < t'
      }
    }
  }
  __syncthreads();
  f4 aq = z, ab = z, ak = z;  // dq, the S_{t-1} du part, the G u part
#pragma unroll
  for (int kg = 0; kg < NW; kg++) {
    const f4 pdo = *reinterpret_cast<const f4*>(&sDO[fr][16 * kg + 4 * fg]);
    const f4 pdu = *reinterpret_cast<const f4*>(&sDU[fr][16 * kg + 4 * fg]);
    const f4 pu = *reinterpret_cast<const f4*>(&sU[fr][16 * kg + 4 * fg]);
    aq = mma16(pdo, sf[kg], aq);
    ab = mma16(pdu, sf[kg], ab);
    ak = mma16(pu, gf[kg], ak);
  }
  // lane holds tokens t = 4 fg + v at key i_key: the block-start terms take
  // their decays per token
#pragma unroll
  for (int v = 0; v < 4; v++) {
    const int t = 4 * fg + v;
    aq[v] *= sE[t];
    ab[v] *= sE[t];
    ak[v] *= sP[t][TT - 1];
  }
  f4 fk, fq, fkb;
#pragma unroll
  for (int s = 0; s < 4; s++) {
    fk[s] = sK[4 * fg + s][i_key];
    fq[s] = sQ[4 * fg + s][i_key];
    fkb[s] = -sKB[4 * fg + s][i_key];
  }
  aq = mma16(*reinterpret_cast<const f4*>(&xA1[fr][4 * fg]), fk, aq);
  ak = mma16(*reinterpret_cast<const f4*>(&xB1[fr][4 * fg]), fq, ak);
  ak = mma16(*reinterpret_cast<const f4*>(&xB2[fr][4 * fg]), fkb, ak);
  ab = mma16(*reinterpret_cast<const f4*>(&xC2[fr][4 * fg]), fk, ab);
#pragma unroll
  for (int v = 0; v < 4; v++) {
    const int t = 4 * fg + v;
    if (t < n) {
      float* pp = part + ((bT + t0 + t) * nv + h) * PW;
      pp[i_key] = aq[v];
      pp[D + i_key] = ak[v] - sBe[t] * ab[v];
    }
  }
  if (tid == 0) {  // g dg by the carried inner product, dbeta
    float phi = sAnc + sOd[n - 1];
    for (int t = n - 1; t >= 0; t--) {
      float* pp = part + ((bT + t0 + t) * nv + h) * PW;
      pp[2 * D] = phi - sDvb[t];
      pp[2 * D + 1] = sDb[t];
      if (t > 0) phi = phi - sDvb[t] + sOd[t - 1];
    }
  }
}

// Sums the partials (column blocks, then the rep v-heads of the k-head, in
// fixed order) and applies the chain rule of the normalisations and gates:
// one 16-lane group per (token, k-head).
//   dq = invq dq^ - q (dq^.q) invq / (|q|^2 + eps), likewise dk;
//   da = (g dg) (-exp(A_log)) sigmoid(a + dt_bias);  db = dbeta beta (1 - beta)
template <int DK>
__global__ __launch_bounds__(256) void chain(int B, int T, int nk, int nv, int ncb, int cdim,
                                             const float* __restrict__ part,
                                             const float* __restrict__ cq,
                                             const float* __restrict__ a,
                                             const float* __restrict__ A_log,
                                             const float* __restrict__ dt_bias,
                                             const float* __restrict__ be,
                                             float* __restrict__ dcq, float* __restrict__ da,
                                             float* __restrict__ db) {
  constexpr int R4 = DK / 64, PW = 2 * DK + 2;
  const size_t BT = (size_t)B * T;
  const size_t gid = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  if (gid >= BT * nk) return;
  const size_t bt = gid / nk;
  const int ko = (int)(gid - bt * nk);
  const int rep = nv / nk, kd = nk * DK;
  const size_t pstride = BT * nv * PW;
  f4 dq[R4], dk[R4];
#pragma unroll
  for (int m = 0; m < R4; m++) dq[m] = dk[m] = f4{0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < rep; r++) {
    const int h = ko * rep + r;
    float sgd = 0.f, sbd = 0.f;
    for (int c = 0; c < ncb; c++) {
      const float* p = part + c * pstride + (bt * nv + h) * PW;
#pragma unroll
      for (int m = 0; m < R4; m++) {
        dq[m] += ld4(p + l16 * 4 + 64 * m);
        dk[m] += ld4(p + DK + l16 * 4 + 64 * m);
      }
      sgd += p[2 * DK];
      sbd += p[2 * DK + 1];
    }
    if (l16 == 0) {
      const size_t i = bt * nv + h;
      const float bt_ = be[i];
      da[i] = sgd * (-expf(A_log[h])) * sigm(a[i] + dt_bias[h]);
      db[i] = sbd * bt_ * (1.0f - bt_);
    }
  }
  const float* qr = cq + bt * cdim + (size_t)ko * DK;
  const float* kr = qr + kd;
  f4 q[R4], k[R4];
  float sq = 0.f, sk = 0.f, pq = 0.f, pk = 0.f;
#pragma unroll
  for (int m = 0; m < R4; m++) {
    q[m] = ld4(qr + l16 * 4 + 64 * m);
    k[m] = ld4(kr + l16 * 4 + 64 * m);
#pragma unroll
    for (int c = 0; c < 4; c++) {
      sq += q[m][c] * q[m][c];
      sk += k[m][c] * k[m][c];
      pq += dq[m][c] * q[m][c];
      pk += dk[m][c] * k[m][c];
    }
  }
  const float nq2 = rowsum16(sq) + L2_EPS, nk2 = rowsum16(sk) + L2_EPS;
  pq = rowsum16(pq);
  pk = rowsum16(pk);
  const float invq = 1.0f / (sqrtf(nq2) * sqrtf((float)DK)), invk = 1.0f / sqrtf(nk2);
  const float cqf = pq * invq / nq2, ckf = pk * invk / nk2;
  float* dqo = dcq + bt * cdim + (size_t)ko * DK;
  float* dko = dqo + kd;
#pragma unroll
  for (int m = 0; m < R4; m++) {
    st4(dqo + l16 * 4 + 64 * m, invq * dq[m] - q[m] * cqf);
    st4(dko + l16 * 4 + 64 * m, invk * dk[m] - k[m] * ckf);
  }
}

}  // namespace gdnk

// ------------------------------------------------------------- launchers --
static unsigned grid4(size_t n4) {
  size_t b = (n4 + 255) / 256;
  return (unsigned)(b > 8192 ? 8192 : (b < 1 ? 1 : b));
}

bool gdn_two_pass(int dk, int dv) { return dk == dv && (dk == 64 || dk == 128); }

size_t gdn_ckpt_floats(int B, int T, int nv, int dk, int dv) {
  return (size_t)B * nv * ((T + gdnk::TT - 1) / gdnk::TT) * dv * dk;
}
size_t gdn_partial_floats(int B, int T, int nv, int dk, int dv) {
  const size_t ncb = gdn_two_pass(dk, dv) ? 1 : dv / gdnk::CB;
  return ncb * B * T * nv * (2 * dk + 2);
}

hipError_t gdn_launch_forward(const GdnArgs& p, hipStream_t st) {
  const int BT = p.B * p.T, cdim = 2 * p.nk * p.dk + p.nv * p.dv;
  if (p.kk == 4)
    hipLaunchKernelGGL((gdnk::conv_fwd_t<4, 8>),
                       dim3(grid4((size_t)p.B * ((p.T + 7) / 8) * cdim / 4)), dim3(256), 0, st,
                       p.B, p.T, cdim, p.raw, p.conv, p.pre, p.cq);
  else
    hipLaunchKernelGGL(gdnk::conv_fwd, dim3(grid4((size_t)BT * cdim / 4)), dim3(256), 0, st, BT,
                       p.T, cdim, p.kk, p.raw, p.conv, p.pre, p.cq);
  const unsigned gq = (unsigned)(((size_t)BT * p.nk + 15) / 16);
  if (p.dk == 128)
    hipLaunchKernelGGL(gdnk::prep<128>, dim3(gq), dim3(256), 0, st, BT, p.nk, p.nv, cdim, p.cq,
                       p.a, p.b, p.A_log, p.dt_bias, p.qh, p.kh, p.g, p.beta);
  else
    hipLaunchKernelGGL(gdnk::prep<64>, dim3(gq), dim3(256), 0, st, BT, p.nk, p.nv, cdim, p.cq, p.a,
                       p.b, p.A_log, p.dt_bias, p.qh, p.kh, p.g, p.beta);
  const dim3 gs(p.B * p.nv * (p.dv / gdnk::CB));
  if (p.dk == 128)
    hipLaunchKernelGGL(gdnk::fwd_seq<128>, gs, dim3(256), 0, st, p.B, p.T, p.nk, p.nv, p.dv, cdim,
                       p.qh, p.kh, p.cq, p.g, p.beta, p.o, p.ckpt, p.kv);
  else
    hipLaunchKernelGGL(gdnk::fwd_seq<64>, gs, dim3(256), 0, st, p.B, p.T, p.nk, p.nv, p.dv, cdim,
                       p.qh, p.kh, p.cq, p.g, p.beta, p.o, p.ckpt, p.kv);
  const int BTH = BT * p.nv;
  const unsigned gr = (unsigned)(((size_t)BTH + 15) / 16);
  if (p.dv == 128)
    hipLaunchKernelGGL(gdnk::rms_fwd<2>, dim3(gr), dim3(256), 0, st, BTH, p.nv, p.rms_eps, p.o,
                       p.z, p.norm, p.out);
  else
    hipLaunchKernelGGL(gdnk::rms_fwd<1>, dim3(gr), dim3(256), 0, st, BTH, p.nv, p.rms_eps, p.o,
                       p.z, p.norm, p.out);
  return hipGetLastError();
}

hipError_t gdn_launch_backward(const GdnArgs& p, hipStream_t st) {
  const int BT = p.B * p.T, cdim = 2 * p.nk * p.dk + p.nv * p.dv;
  const int BTH = BT * p.nv;
  const unsigned gr = (unsigned)(((size_t)BTH + 15) / 16);
  if (p.dv == 128)
    hipLaunchKernelGGL(gdnk::rms_bwd<2>, dim3(gr), dim3(256), 0, st, BTH, p.nv, p.rms_eps, p.o,
                       p.z, p.norm, p.dout, p.dz, p.dobuf);
  else
    hipLaunchKernelGGL(gdnk::rms_bwd<1>, dim3(gr), dim3(256), 0, st, BTH, p.nv, p.rms_eps, p.o,
                       p.z, p.norm, p.dout, p.dz, p.dobuf);
  const dim3 gs(p.B * p.nv * (p.dv / gdnk::CB));
  const int nblk = (p.T + gdnk::TT - 1) / gdnk::TT;
  int ncb = p.dv / gdnk::CB;  // partials per (token, head) summed by chain
  if (gdn_two_pass(p.dk, p.dv)) {
    ncb = 1;
    const dim3 gb(p.B * p.nv * nblk);
    if (p.dk == 128) {
      hipLaunchKernelGGL(gdnk::bwd_scan<128>, gs, dim3(256), 0, st, p.B, p.T, p.nk, p.nv, p.dv, cdim,
                         p.qh, p.kh, p.cq, p.g, p.beta, p.dobuf, p.ckpt, p.gend, p.du, p.anc,
                         p.dcq);
      hipLaunchKernelGGL(gdnk::bwd_blk<128>, gb, dim3(512), 0, st, p.B, p.T, p.nk, p.nv, cdim,
                         p.qh, p.kh, p.cq, p.g, p.beta, p.o, p.dobuf, p.ckpt, p.gend, p.du, p.kv,
                         p.anc, p.part);
    } else {
      hipLaunchKernelGGL(gdnk::bwd_scan<64>, gs, dim3(256), 0, st, p.B, p.T, p.nk, p.nv, p.dv, cdim,
                         p.qh, p.kh, p.cq, p.g, p.beta, p.dobuf, p.ckpt, p.gend, p.du, p.anc,
                         p.dcq);
      hipLaunchKernelGGL(gdnk::bwd_blk<64>, gb, dim3(256), 0, st, p.B, p.T, p.nk, p.nv, cdim,
                         p.qh, p.kh, p.cq, p.g, p.beta, p.o, p.dobuf, p.ckpt, p.gend, p.du, p.kv,
                         p.anc, p.part);
    }
  } else if (p.dk == 128) {
    hipLaunchKernelGGL(gdnk::bwd_seq<128>, gs, dim3(256), 0, st, p.B, p.T, p.nk, p.nv, p.dv, cdim,
                       p.qh, p.kh, p.cq, p.g, p.beta, p.dobuf, p.ckpt, p.part, p.dcq);
  } else {
    hipLaunchKernelGGL(gdnk::bwd_seq<64>, gs, dim3(256), 0, st, p.B, p.T, p.nk, p.nv, p.dv, cdim,
                       p.qh, p.kh, p.cq, p.g, p.beta, p.dobuf, p.ckpt, p.part, p.dcq);
  }
  const unsigned gq = (unsigned)(((size_t)BT * p.nk + 15) / 16);
  if (p.dk == 128)
    hipLaunchKernelGGL(gdnk::chain<128>, dim3(gq), dim3(256), 0, st, p.B, p.T, p.nk, p.nv, ncb,
                       cdim, p.part, p.cq, p.a, p.A_log, p.dt_bias, p.beta, p.dcq, p.da, p.db);
  else
    hipLaunchKernelGGL(gdnk::chain<64>, dim3(gq), dim3(256), 0, st, p.B, p.T, p.nk, p.nv, ncb, cdim,
                       p.part, p.cq, p.a, p.A_log, p.dt_bias, p.beta, p.dcq, p.da, p.db);
  if (p.kk == 4)
    hipLaunchKernelGGL((gdnk::conv_bwd_t<4, 8>),
                       dim3(grid4((size_t)p.B * ((p.T + 7) / 8) * cdim / 4)), dim3(256), 0, st,
                       p.B, p.T, cdim, p.pre, p.dcq, p.conv, p.draw);
  else
    hipLaunchKernelGGL(gdnk::conv_bwd, dim3(grid4((size_t)BT * cdim / 4)), dim3(256), 0, st, BT,
                       p.T, cdim, p.kk, p.pre, p.dcq, p.conv, p.draw);
  return hipGetLastError();
}
