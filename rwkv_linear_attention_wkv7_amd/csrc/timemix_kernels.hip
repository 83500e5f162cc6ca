// Fused elementwise / per-head kernels of the RWKV-7 time-mix block (gfx950).
//
// Formulas: "Foundry/cuda_kernels/timemix.cu" forward kernels k_tokenshift,
// k_decay, k_bias_sigmoid, k_tk, k_l2norm, k_keymod, k_vres0/k_vres,
// k_composites, k_groupnorm, k_bonus, k_mul and backward kernels k_split,
// k_bonus_bwd, k_groupnorm_bwd, k_p4_seed, k_comp_keymod, k_l2norm_bwd,
// k_tk_bwd, k_avec_bwd, k_wdecay_bwd, k_vvec0/k_vvec1, k_tokenshift_bwd.
// Here the per-token-and-head steps are fused into one pass each (pre-WKV,
// post-WKV and their backwards), a (token, head) pair is 16 lanes x float4
// (64 channels) with DPP row sums for its reductions, and the per-channel
// parameter gradients are summed deterministically: each workgroup reduces a
// fixed token block in registers and LDS and writes one partial row, and a
// second kernel adds the partial rows in a fixed order.

#include "common.hpp"
#include "timemix_kernels.hpp"

namespace tmk {

constexpr float DECAY = 0.606531f;  // exp(-0.606531 * sigmoid(.)) (timemix.cu RWDECAY_COEFF)
constexpr float GN_EPS = 64e-5f;    // group-norm epsilon
constexpr float L2_EPS = 1e-12f;    // added to the key norm
constexpr int N = WKV7_N;

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }
__device__ __forceinline__ float hsum4(f4 v) { return (v[0] + v[1]) + (v[2] + v[3]); }

// Partial-sum epilogue: every thread holds NV float4 partials for the 4
// channels ch0..ch0+3 of its 16-lane group; reduce over the 16 groups of the
// workgroup and write part[v][blk][C] for the workgroup's 64 channels.
template <int NV>
__device__ __forceinline__ void write_partials(const f4 (&p)[NV], float* part, int nblk, int blk,
                                               int C, int cbase) {
  __shared__ f4 red[NV][16][16];
  const int tid = threadIdx.x, l16 = tid & 15, grp = tid >> 4;
#pragma unroll
  for (int v = 0; v < NV; v++) red[v][grp][l16] = p[v];
  __syncthreads();
  for (int i = tid; i < NV * 16; i += 256) {
    const int v = i >> 4, c4 = i & 15;
    f4 s = red[v][0][c4];
#pragma unroll
    for (int gi = 1; gi < 16; gi++) s += red[v][gi][c4];
    st4(part + ((size_t)v * nblk + blk) * C + cbase + c4 * 4, s);
  }
}

// ------------------------------------------------------------- forward ----
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st16(__bf16* d, size_t e, f4 x) {
  *reinterpret_cast<bf16x4_t*>(d + e) = __builtin_convertvector(x, bf16x4_t);
}

// Token shift + lerp: xs_c = x + (prev - x) mu_c, prev = x[t-1] (x_prev or 0 at t=0).
__global__ __launch_bounds__(256) void shift_fwd(TmFwd p) {
  const size_t n4 = (size_t)p.BT * p.C / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t e = i * 4;
    const size_t bt = e / p.C;
    const int c = (int)(e - bt * p.C);
    const int t = (int)(bt % p.T);
    const f4 x = ld4(p.x + e);
    f4 prev = {0.f, 0.f, 0.f, 0.f};
    if (t > 0) prev = ld4(p.x + e - p.C);
    else if (p.x_prev) prev = ld4(p.x_prev + (bt / p.T) * p.C + c);
    const f4 d = prev - x;
    const f4 xr = x + d * ld4(p.mu_r + c), xk = x + d * ld4(p.mu_k + c), xv = x + d * ld4(p.mu_v + c);
    st4(p.xr + e, xr);
    st4(p.xw + e, x + d * ld4(p.mu_w + c));
    st4(p.xk + e, xk);
    st4(p.xv + e, xv);
    if (p.xr16) {
      st16(p.xr16, e, xr);
      st16(p.xk16, e, xk);
      st16(p.xv16, e, xv);
    }
    st4(p.xa + e, x + d * ld4(p.mu_a + c));
    st4(p.xg + e, x + d * ld4(p.mu_g + c));
    if (p.x_last && t == p.T - 1) st4(p.x_last + (bt / p.T) * p.C + c, x);
  }
}

// Pre-WKV, one 16-lane group per (token, head):
//   w = exp(-DECAY sigmoid(w0 + ow)); a = sigmoid(a0 + oa)
//   kk = l2norm(k k_k); k' = k (1 + (a-1) k_a); v' = v or v + (vf - v) sigmoid(v0 + ov)
//   A = -kk; Bv = kk a
__global__ __launch_bounds__(256) void pre_fwd(TmFwd p) {
  const size_t gidx = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  const int H = p.C / N;
  if (gidx >= (size_t)p.BT * H) return;
  const size_t bt = gidx / H;
  const int h = (int)(gidx - bt * H);
  const int c = h * N + l16 * 4;
  const size_t e = bt * p.C + c;
  const f4 k = ld4(p.k + e), v = ld4(p.v + e), ow = ld4(p.ow + e), oa = ld4(p.oa + e);
  const f4 w0 = ld4(p.w0 + c), a0 = ld4(p.a0 + c), kkw = ld4(p.k_k + c), ka = ld4(p.k_a + c);
  f4 w, a, tk;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    w[j] = expf(-DECAY * sigm(w0[j] + ow[j]));
    a[j] = sigm(a0[j] + oa[j]);
    tk[j] = k[j] * kkw[j];
  }
  const float nrm = sqrtf(rowsum16(hsum4(tk * tk)));
  const float inv = 1.0f / (nrm + L2_EPS);
  const f4 kk = tk * inv;
  f4 kmod, vmod;
#pragma unroll
  for (int j = 0; j < 4; j++) kmod[j] = k[j] * (1.0f + (a[j] - 1.0f) * ka[j]);
  if (p.layer_id == 0) {
    vmod = v;
    st4(p.v_first + e, v);
  } else {
    const f4 vf = ld4(p.v_first + e), ov = ld4(p.ov + e), v0 = ld4(p.v0 + c);
#pragma unroll
    for (int j = 0; j < 4; j++) vmod[j] = v[j] + (vf[j] - v[j]) * sigm(v0[j] + ov[j]);
  }
  st4(p.w + e, w);
  st4(p.a + e, a);
  st4(p.kk + e, kk);
  st4(p.kmod + e, kmod);
  st4(p.vmod + e, vmod);
  st4(p.A + e, -kk);
  st4(p.Bv + e, kk * a);
}

// Post-WKV, one 16-lane group per (token, head):
//   ygn = (y - mean) rstd ln_w + ln_b (biased variance, eps 64e-5)
//   alpha = sum_n r k' r_k ; tg = (ygn + alpha v') g
__global__ __launch_bounds__(256) void post_fwd(TmFwd p) {
  const size_t gidx = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  const int H = p.C / N;
  if (gidx >= (size_t)p.BT * H) return;
  const size_t bt = gidx / H;
  const int h = (int)(gidx - bt * H);
  const int c = h * N + l16 * 4;
  const size_t e = bt * p.C + c;
  const f4 y = ld4(p.y + e);
  const float mean = rowsum16(hsum4(y)) * (1.0f / N);
  const f4 d = y - mean;
  const float var = rowsum16(hsum4(d * d)) * (1.0f / N);
  const float rstd = 1.0f / sqrtf(var + GN_EPS);
  const f4 r = ld4(p.r + e), kmod = ld4(p.kmod + e), vmod = ld4(p.vmod + e), g = ld4(p.g + e);
  const float alpha = rowsum16(hsum4(r * kmod * ld4(p.r_k + c)));
  const f4 ygn = d * rstd * ld4(p.ln_w + c) + ld4(p.ln_b + c);
  st4(p.tg + e, (ygn + alpha * vmod) * g);
  if (p.tg16) st16(p.tg16, e, (ygn + alpha * vmod) * g);
  if (l16 == 0) {
    p.mean[gidx] = mean;
    p.rstd[gidx] = rstd;
    p.alpha[gidx] = alpha;
  }
}

// Decode (T = 1): pre-WKV, the WKV7 step with the state updated in place, and
// post-WKV in one workgroup per (b, h), the three steps above with the same
// lane layouts, so the results equal those of pre_fwd, the step kernel and
// post_fwd one after the other.  Lanes 0..15 form the head's pre-WKV vectors
// (channel 4 l16 .. 4 l16 + 3 each) and share them through LDS while every
// thread's state rows are in flight; thread (rg, cg) then owns state rows
// rg + 16m (m < 4) x columns 4cg..4cg+3 (the step kernel's layout); y goes
// back through LDS to lanes 0..15 for the group norm, the bonus and the gate.
// Only v_first (layer 0) and tg are written: decode keeps no backward cache.
__global__ __launch_bounds__(256) void step_fused(TmFwd p, float* __restrict__ state) {
  __shared__ f4 sv[6][16];  // w, k', A, Bv, r, v' by channel group
  __shared__ float sy[N];
  const int H = p.C / N;
  const int bh = xcd_remap(blockIdx.x, gridDim.x);
  const int bt = bh / H, h = bh - bt * H;  // token row = stream (T = 1)
  const int tid = threadIdx.x, cg = tid & 15, rg = tid >> 4;
  float* st = state + (size_t)bh * N * N;
  f4 S[4];
#pragma unroll
  for (int m = 0; m < 4; m++)
    S[m] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(st + (size_t)(rg + 16 * m) * N + cg * 4));

  const int c = h * N + cg * 4;
  const size_t e = (size_t)bt * p.C + c;
  f4 r, kmod, vmod, rk, lnw, lnb, gg;
  if (tid < 16) {
    const f4 k = ld4(p.k + e), v = ld4(p.v + e), ow = ld4(p.ow + e), oa = ld4(p.oa + e);
    const f4 w0 = ld4(p.w0 + c), a0 = ld4(p.a0 + c), kkw = ld4(p.k_k + c), ka = ld4(p.k_a + c);
    r = ld4(p.r + e);
    // the post-WKV inputs too, so no load waits after the state update
    rk = ld4(p.r_k + c);
    lnw = ld4(p.ln_w + c);
    lnb = ld4(p.ln_b + c);
    gg = ld4(p.g + e);
    f4 w, a, tk;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      w[j] = expf(-DECAY * sigm(w0[j] + ow[j]));
      a[j] = sigm(a0[j] + oa[j]);
      tk[j] = k[j] * kkw[j];
    }
    const float nrm = sqrtf(rowsum16(hsum4(tk * tk)));
    const float inv = 1.0f / (nrm + L2_EPS);
    const f4 kk = tk * inv;
#pragma unroll
    for (int j = 0; j < 4; j++) kmod[j] = k[j] * (1.0f + (a[j] - 1.0f) * ka[j]);
    if (p.layer_id == 0) {
      vmod = v;
      st4(p.v_first + e, v);
    } else {
      const f4 vf = ld4(p.v_first + e), ov = ld4(p.ov + e), v0 = ld4(p.v0 + c);
#pragma unroll
      for (int j = 0; j < 4; j++) vmod[j] = v[j] + (vf[j] - v[j]) * sigm(v0[j] + ov[j]);
    }
    sv[0][cg] = w;
    sv[1][cg] = kmod;
    sv[2][cg] = -kk;
    sv[3][cg] = kk * a;
    sv[4][cg] = r;
    sv[5][cg] = vmod;
  }
  __syncthreads();
  const f4 wv = sv[0][cg], kv = sv[1][cg], av = sv[2][cg], bb = sv[3][cg], rv = sv[4][cg];
  const float* vrow = reinterpret_cast<const float*>(sv[5]);
  float sa[4];
#pragma unroll
  for (int m = 0; m < 4; m++)
    sa[m] = fmaf(S[m][3], av[3], fmaf(S[m][2], av[2], fmaf(S[m][1], av[1], S[m][0] * av[0])));
#pragma unroll
  for (int m = 0; m < 4; m++) sa[m] = rowsum16(sa[m]);
  float yo[4];
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const float vv = vrow[rg + 16 * m];
#pragma unroll
    for (int q = 0; q < 4; q++) S[m][q] = fmaf(vv, kv[q], fmaf(sa[m], bb[q], S[m][q] * wv[q]));
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
    sy[rg + 16 * cg] = o;
  }
  __syncthreads();
  if (tid < 16) {
    const f4 y = ld4(&sy[4 * cg]);
    const float mean = rowsum16(hsum4(y)) * (1.0f / N);
    const f4 d = y - mean;
    const float var = rowsum16(hsum4(d * d)) * (1.0f / N);
    const float rstd = 1.0f / sqrtf(var + GN_EPS);
    const float alpha = rowsum16(hsum4(r * kmod * rk));
    const f4 ygn = d * rstd * lnw + lnb;
    st4(p.tg + e, (ygn + alpha * vmod) * gg);
  }
}

// ------------------------------------------------------------ backward ----
// Grid (H, token blocks); 16 groups x 16 lanes; group handles tokens
// blk*TB + grp + 16 i of head blockIdx.x.

// Post-WKV backward (k_split, k_bonus_bwd, k_groupnorm_bwd).  Partials: r_k, ln_w, ln_b.
__global__ __launch_bounds__(256) void post_bwd(TmBwd p) {
  const int h = blockIdx.x, blk = blockIdx.y, nblk = gridDim.y;
  const int l16 = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int H = p.C / N;
  const int c = h * N + l16 * 4;
  const f4 lnw = ld4(p.ln_w + c), lnb = ld4(p.ln_b + c), rk = ld4(p.r_k + c);
  f4 prk = {0.f, 0.f, 0.f, 0.f}, plw = prk, plb = prk;
  const size_t t_end = min((size_t)p.BT, (size_t)(blk + 1) * TB);
  for (size_t bt = (size_t)blk * TB + grp; bt < t_end; bt += 16) {
    const size_t e = bt * p.C + c, hi = bt * H + h;
    const f4 dtg = ld4(p.dtg + e), g = ld4(p.g + e), y = ld4(p.y + e);
    const f4 r = ld4(p.r + e), kmod = ld4(p.kmod + e), vmod = ld4(p.vmod + e);
    const float mean = p.mean[hi], rstd = p.rstd[hi], alpha = p.alpha[hi];
    const f4 nhat = (y - mean) * rstd;
    const f4 yb = nhat * lnw + lnb + alpha * vmod;
    const f4 dyb = dtg * g;
    st4(p.dg + e, dtg * yb);
    const float dalpha = rowsum16(hsum4(dyb * vmod));
    st4(p.dvmod + e, dyb * alpha);
    st4(p.dr + e, dalpha * kmod * rk);
    st4(p.dkmod + e, dalpha * r * rk);
    prk += dalpha * r * kmod;
    plw += dyb * nhat;
    plb += dyb;
    const f4 dn = dyb * lnw;
    const float m1 = rowsum16(hsum4(dn)) * (1.0f / N);
    const float m2 = rowsum16(hsum4(dn * nhat)) * (1.0f / N);
    st4(p.dy_wkv + e, rstd * (dn - m1 - nhat * m2));
  }
  const f4 parts[3] = {prk, plw, plb};
  write_partials<3>(parts, p.part_post, nblk, blk, p.C, h * N);
}

// Pre-WKV backward (k_p4_seed, k_comp_keymod, k_l2norm_bwd, k_tk_bwd,
// k_avec_bwd, k_wdecay_bwd, k_vvec0/1).  dr/dkmod/dvmod arrive holding the
// post-WKV contributions; the WKV gradients are added here.
// Partials: k_a, k_k, a0, w0, v0.
__global__ __launch_bounds__(256) void pre_bwd(TmBwd p) {
  const int h = blockIdx.x, blk = blockIdx.y, nblk = gridDim.y;
  const int l16 = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int c = h * N + l16 * 4;
  const f4 ka = ld4(p.k_a + c), kkw = ld4(p.k_k + c), w0 = ld4(p.w0 + c);
  const f4 v0 = p.layer_id > 0 ? ld4(p.v0 + c) : f4{0.f, 0.f, 0.f, 0.f};
  f4 pka = {0.f, 0.f, 0.f, 0.f}, pkk = pka, pa0 = pka, pw0 = pka, pv0 = pka;
  const size_t t_end = min((size_t)p.BT, (size_t)(blk + 1) * TB);
  for (size_t bt = (size_t)blk * TB + grp; bt < t_end; bt += 16) {
    const size_t e = bt * p.C + c;
    const f4 drn = ld4(p.dr + e) + ld4(p.gr + e);
    st4(p.dr + e, drn);
    if (p.dr16) st16(p.dr16, e, drn);
    const f4 dkmod = ld4(p.dkmod + e) + ld4(p.gk + e);
    const f4 dvmod = ld4(p.dvmod + e) + ld4(p.gv + e);
    const f4 a = ld4(p.a + e), kk = ld4(p.kk + e), k = ld4(p.k + e);
    const f4 dA = ld4(p.gA + e), dB = ld4(p.gB + e);
    const f4 dkk = dB * a - dA;
    const f4 da = dB * kk + dkmod * k * ka;
    f4 dk = dkmod * (1.0f + (a - 1.0f) * ka);
    pka += dkmod * k * (a - 1.0f);
    const f4 tk = k * kkw;
    const float nrm = sqrtf(rowsum16(hsum4(tk * tk)));
    const float inv = 1.0f / (nrm + L2_EPS);
    const float gdot = rowsum16(hsum4(dkk * tk));
    const float corr = nrm > 0.f ? inv * inv * gdot / nrm : 0.f;
    const f4 dtk = inv * dkk - corr * tk;
    dk += dtk * kkw;
    pkk += dtk * k;
    st4(p.dk + e, dk);
    if (p.dk16) st16(p.dk16, e, dk);
    const f4 dpa = da * a * (1.0f - a);
    pa0 += dpa;
    st4(p.dpre_a + e, dpa);
    const f4 w = ld4(p.w + e), ow = ld4(p.ow + e), dw = ld4(p.gw + e);
    f4 dpw;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float s = sigm(w0[j] + ow[j]);
      dpw[j] = dw[j] * w[j] * (-DECAY) * s * (1.0f - s);
    }
    pw0 += dpw;
    st4(p.dpre_w + e, dpw);
    if (p.layer_id == 0) {
      f4 dv = dvmod;
      if (p.dvf_in) dv += ld4(p.dvf_in + e);
      st4(p.dv + e, dv);
      if (p.dv16) st16(p.dv16, e, dv);
    } else {
      const f4 ov = ld4(p.ov + e), vf = ld4(p.v_first + e), v = ld4(p.v + e);
      f4 nu;
#pragma unroll
      for (int j = 0; j < 4; j++) nu[j] = sigm(v0[j] + ov[j]);
      st4(p.dv + e, dvmod * (1.0f - nu));
      if (p.dv16) st16(p.dv16, e, dvmod * (1.0f - nu));
      if (p.dvf_out) st4(p.dvf_out + e, p.dvf_accum ? ld4(p.dvf_out + e) + dvmod * nu : dvmod * nu);
      const f4 dpv = dvmod * (vf - v) * nu * (1.0f - nu);
      pv0 += dpv;
      st4(p.dpre_v + e, dpv);
    }
  }
  const f4 parts[5] = {pka, pkk, pa0, pw0, pv0};
  write_partials<5>(parts, p.part_pre, nblk, blk, p.C, h * N);
}

// Token-shift backward (k_tokenshift_bwd).  Grid (C/64, token blocks).
// Partials: mu_r, mu_w, mu_k, mu_v, mu_a, mu_g.
__global__ __launch_bounds__(256) void shift_bwd(TmBwd p) {
  const int cb = blockIdx.x, blk = blockIdx.y, nblk = gridDim.y;
  const int l16 = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int c = cb * N + l16 * 4;
  const f4 mr = ld4(p.mu_r + c), mw = ld4(p.mu_w + c), mk = ld4(p.mu_k + c);
  const f4 mv = ld4(p.mu_v + c), ma = ld4(p.mu_a + c), mg = ld4(p.mu_g + c);
  f4 q[6];
#pragma unroll
  for (int i = 0; i < 6; i++) q[i] = f4{0.f, 0.f, 0.f, 0.f};
  const size_t t_end = min((size_t)p.BT, (size_t)(blk + 1) * TB);
  for (size_t bt = (size_t)blk * TB + grp; bt < t_end; bt += 16) {
    const size_t e = bt * p.C + c;
    const int t = (int)(bt % p.T);
    const f4 x = ld4(p.x + e);
    f4 prev = {0.f, 0.f, 0.f, 0.f};
    if (t > 0) prev = ld4(p.x + e - p.C);
    else if (p.x_prev) prev = ld4(p.x_prev + (bt / p.T) * p.C + c);
    const f4 dr = ld4(p.dxr + e), dw = ld4(p.dxw + e), dk = ld4(p.dxk + e);
    const f4 dv = ld4(p.dxv + e), da = ld4(p.dxa + e), dg = ld4(p.dxg + e);
    const f4 pmx = prev - x;
    q[0] += dr * pmx; q[1] += dw * pmx; q[2] += dk * pmx;
    q[3] += dv * pmx; q[4] += da * pmx; q[5] += dg * pmx;
    f4 dx = dr * (1.0f - mr) + dw * (1.0f - mw) + dk * (1.0f - mk) + dv * (1.0f - mv) +
            da * (1.0f - ma) + dg * (1.0f - mg);
    if (t < p.T - 1) {
      const size_t en = e + p.C;
      dx += ld4(p.dxr + en) * mr + ld4(p.dxw + en) * mw + ld4(p.dxk + en) * mk +
            ld4(p.dxv + en) * mv + ld4(p.dxa + en) * ma + ld4(p.dxg + en) * mg;
    }
    st4(p.dx + e, dx);
    if (t == 0 && p.dx_prev)
      st4(p.dx_prev + (bt / p.T) * p.C + c, dr * mr + dw * mw + dk * mk + dv * mv + da * ma + dg * mg);
  }
  write_partials<6>(q, p.part_shift, nblk, blk, p.C, cb * N);
}

// out[v][c] = sum_blk part[v][blk][c], fixed order.  A workgroup owns 16
// columns of one vector and splits the rows over 64 row groups (lane l of
// wave w: column l % 16, group 4 w + l / 16; group g sums rows g, g + 64, ...
// with eight loads in flight into four accumulators); thread c < 16 then
// adds the 64 group sums in group order.  Narrow workgroups spread a sum of
// a few MB over enough CUs that per-CU load latency does not set its time.
constexpr int RP_WAVES = 16, RP_COLS = 16, RP_GROUPS = RP_WAVES * 64 / RP_COLS;
__global__ __launch_bounds__(64 * RP_WAVES) void reduce_partials(const float* __restrict__ part,
                                                                 int nblk, int C, VecOut outs) {
  const int v = blockIdx.y, tid = threadIdx.x;
  float* o = outs.p[v];
  if (!o) return;
  const int cl = tid % RP_COLS, grp = tid / RP_COLS;
  const int c = blockIdx.x * RP_COLS + cl;
  const int cc = c < C ? c : C - 1;
  const float* src = part + (size_t)v * nblk * C + cc;
  float sa[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;  // loads in flight per lane
  int b = grp;
  for (; b + (U - 1) * RP_GROUPS < nblk; b += U * RP_GROUPS) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; u++) x[u] = src[(size_t)(b + u * RP_GROUPS) * C];
#pragma unroll
    for (int u = 0; u < U; u++) sa[u & 3] += x[u];
  }
  for (; b < nblk; b += RP_GROUPS) sa[0] += src[(size_t)b * C];
  __shared__ float red[RP_GROUPS][RP_COLS];
  red[grp][cl] = (sa[0] + sa[1]) + (sa[2] + sa[3]);
  __syncthreads();
  if (tid < RP_COLS && c < C) {
    float sum = 0.f;
    for (int i = 0; i < RP_GROUPS; i++) sum += red[i][tid];
    o[c] = sum;
  }
}

}  // namespace tmk

// ------------------------------------------------------------ launchers ----
hipError_t tm_launch_shift_fwd(const TmFwd& p, hipStream_t st) {
  const size_t n4 = (size_t)p.BT * p.C / 4;
  int blocks = (int)((n4 + 255) / 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(tmk::shift_fwd, dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}
hipError_t tm_launch_pre_fwd(const TmFwd& p, hipStream_t st) {
  const size_t groups = (size_t)p.BT * (p.C / WKV7_N);
  hipLaunchKernelGGL(tmk::pre_fwd, dim3((unsigned)((groups + 15) / 16)), dim3(256), 0, st, p);
  return hipGetLastError();
}
hipError_t tm_launch_post_fwd(const TmFwd& p, hipStream_t st) {
  const size_t groups = (size_t)p.BT * (p.C / WKV7_N);
  hipLaunchKernelGGL(tmk::post_fwd, dim3((unsigned)((groups + 15) / 16)), dim3(256), 0, st, p);
  return hipGetLastError();
}
hipError_t tm_launch_step_fused(const TmFwd& p, float* state, hipStream_t st) {
  hipLaunchKernelGGL(tmk::step_fused, dim3((unsigned)((size_t)p.BT * (p.C / WKV7_N))), dim3(256), 0, st,
                     p, state);
  return hipGetLastError();
}
int tm_num_token_blocks(int BT) { return (BT + TB - 1) / TB; }
hipError_t tm_launch_post_bwd(const TmBwd& p, hipStream_t st) {
  hipLaunchKernelGGL(tmk::post_bwd, dim3(p.C / WKV7_N, tm_num_token_blocks(p.BT)), dim3(256), 0, st, p);
  return hipGetLastError();
}
hipError_t tm_launch_pre_bwd(const TmBwd& p, hipStream_t st) {
  hipLaunchKernelGGL(tmk::pre_bwd, dim3(p.C / WKV7_N, tm_num_token_blocks(p.BT)), dim3(256), 0, st, p);
  return hipGetLastError();
}
hipError_t tm_launch_shift_bwd(const TmBwd& p, hipStream_t st) {
  hipLaunchKernelGGL(tmk::shift_bwd, dim3(p.C / WKV7_N, tm_num_token_blocks(p.BT)), dim3(256), 0, st, p);
  return hipGetLastError();
}
hipError_t tm_launch_reduce(const float* part, int nvec, int nblk, int C, const VecOut& outs,
                            hipStream_t st) {
  if (nvec < 1 || nvec > 8 || C < 1 || nblk < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tmk::reduce_partials, dim3((C + tmk::RP_COLS - 1) / tmk::RP_COLS, nvec),
                     dim3(64 * tmk::RP_WAVES), 0, st, part, nblk, C, outs);
  return hipGetLastError();
}
