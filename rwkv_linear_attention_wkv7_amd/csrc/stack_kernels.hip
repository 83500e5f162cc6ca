// Kernels around the time-mix block in an RWKV-7 stack (gfx950): embedding
// gather, LayerNorm, channel-mix token shift.
//
// Pages: "Foundry/cuda_kernels/fullmodel.cu" (fm_k_emb_fwd: out[t] =
// emb[token[t]]; LayerNorm before each mix and at the output; fm_cm_fwd:
// token shift, sh @ Wk, relu^2, @ Wv) and "infotheory .../rwkv7/model.rs"
// (LayerNorm eps 1e-5; the channel-mix shift state ffn_x_prev).

#include "common.hpp"
#include "stack_kernels.hpp"

namespace stk {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr float LN_EPS = 1e-5f;
constexpr int MAXC4_LIMIT = 16;  // LayerNorm keeps a row in registers: C <= 64 * 4 * 16

// out[r] = emb[tok[r]] (float4 per thread); an id outside [0, V) gives a zero row
__global__ __launch_bounds__(256) void emb_gather(int R, int C, int V, const int* __restrict__ tok,
                                                  const float* __restrict__ emb,
                                                  float* __restrict__ out) {
  const size_t n4 = (size_t)R * C / 4;
  const int C4 = C / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t row = i / C4;
    const int c4 = (int)(i - row * C4);
    const int id = tok[row];
    reinterpret_cast<f4*>(out)[i] = (unsigned)id < (unsigned)V
                                        ? reinterpret_cast<const f4*>(emb + (size_t)id * C)[c4]
                                        : f4{0.f, 0.f, 0.f, 0.f};
  }
}

// y = (x - mean) / sqrt(var + eps) * w + b per row; one wave per row, the row
// held in registers (in-place safe).  mean/rstd are optional outputs.
template <int MAXC4>
__global__ __launch_bounds__(256) void layernorm_fwd(int R, int C, const float* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ b, float* y,
                                                     float* __restrict__ mean_out,
                                                     float* __restrict__ rstd_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= R) return;
  const int C4 = C / 4;
  const f4* xr = reinterpret_cast<const f4*>(x + (size_t)row * C);
  f4 v[MAXC4];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    const int c4 = lane + 64 * j;
    v[j] = c4 < C4 ? xr[c4] : f4{0.f, 0.f, 0.f, 0.f};
    s += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
  }
  const float mean = wavesum(s) / C;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    const int c4 = lane + 64 * j;
    if (c4 < C4) {
      const f4 d = v[j] - mean;
      q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
  }
  const float rstd = 1.0f / sqrtf(wavesum(q) / C + LN_EPS);
  f4* yr = reinterpret_cast<f4*>(y + (size_t)row * C);
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    const int c4 = lane + 64 * j;
    if (c4 < C4)
      yr[c4] = (v[j] - mean) * rstd * reinterpret_cast<const f4*>(w)[c4] +
               reinterpret_cast<const f4*>(b)[c4];
  }
  if (lane == 0) {
    if (mean_out) mean_out[row] = mean;
    if (rstd_out) rstd_out[row] = rstd;
  }
}

// sh = x + (prev - x) mu, prev = x[t-1] (x_prev or 0 at t = 0); x_last = x[T-1].
// x_last may alias x_prev only when T == 1 (same thread reads then writes).
__global__ __launch_bounds__(256) void cm_shift(int BT, int T, int C, const float* __restrict__ x,
                                                const float* x_prev, const float* __restrict__ mu,
                                                float* __restrict__ sh, float* x_last,
                                                __bf16* __restrict__ sh16) {
  const size_t n4 = (size_t)BT * C / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t e = i * 4;
    const size_t bt = e / C;
    const int c = (int)(e - bt * C);
    const int t = (int)(bt % T);
    const f4 xv = *reinterpret_cast<const f4*>(x + e);
    f4 prev = {0.f, 0.f, 0.f, 0.f};
    if (t > 0) prev = *reinterpret_cast<const f4*>(x + e - C);
    else if (x_prev) prev = *reinterpret_cast<const f4*>(x_prev + (bt / T) * C + c);
    const f4 shv = xv + (prev - xv) * *reinterpret_cast<const f4*>(mu + c);
    *reinterpret_cast<f4*>(sh + e) = shv;
    if (sh16) *reinterpret_cast<bf16x4_t*>(sh16 + e) = __builtin_convertvector(shv, bf16x4_t);
    if (x_last && t == T - 1) *reinterpret_cast<f4*>(x_last + (bt / T) * C + c) = xv;
  }
}

// One token per stream (T = 1): LayerNorm of each row fused with the token
// shift lerps that consume it (and, optionally, with the residual add of a
// split-K product before it: x += sum of its partials, written back).
// h = LN(x); out_m = h + (prev - h) mu_m for
// each mix m, prev = the previous token's LN output (x_prev, or 0); x_last
// receives h (it may be x_prev: each lane reads its prev before writing).
// One wave per row, the row in registers as in layernorm_fwd.
template <int MAXC4>
__global__ __launch_bounds__(256) void ln_mix(LnMix p) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.R) return;
  const int C = p.C, C4 = C / 4;
  const f4* xr = reinterpret_cast<const f4*>(p.x + (size_t)row * C);
  f4 v[MAXC4];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    const int c4 = lane + 64 * j;
    v[j] = c4 < C4 ? xr[c4] : f4{0.f, 0.f, 0.f, 0.f};
  }
  if (p.nparts > 0) {  // x + (sum of the partials in slice order)
    const size_t plane = (size_t)p.R * C;
#pragma unroll
    for (int j = 0; j < MAXC4; j++) {
      const int c4 = lane + 64 * j;
      if (c4 < C4) {
        const f4* pr = reinterpret_cast<const f4*>(p.part + (size_t)row * C) + c4;
        f4 ps = pr[0];
        for (int z = 1; z < p.nparts; z++) ps += pr[z * plane / 4];
        v[j] = ps + v[j];
        reinterpret_cast<f4*>(p.x_sum + (size_t)row * C)[c4] = v[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MAXC4; j++) s += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
  const float mean = wavesum(s) / C;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    const int c4 = lane + 64 * j;
    if (c4 < C4) {
      const f4 d = v[j] - mean;
      q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
  }
  const float rstd = 1.0f / sqrtf(wavesum(q) / C + LN_EPS);
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    const int c4 = lane + 64 * j;
    if (c4 < C4) {
      const size_t e = (size_t)row * C + 4 * c4;
      const f4 h = (v[j] - mean) * rstd * reinterpret_cast<const f4*>(p.w)[c4] +
                   reinterpret_cast<const f4*>(p.b)[c4];
      const f4 prev = p.x_prev ? *reinterpret_cast<const f4*>(p.x_prev + e) : f4{0.f, 0.f, 0.f, 0.f};
      if (p.x_last) *reinterpret_cast<f4*>(p.x_last + e) = h;
      const f4 d = prev - h;
      for (int m = 0; m < p.nmix; m++)
        *reinterpret_cast<f4*>(p.out[m] + e) = h + d * reinterpret_cast<const f4*>(p.mu[m])[c4];
    }
  }
}

}  // namespace stk

static unsigned grid_for(size_t n4) {
  size_t b = (n4 + 255) / 256;
  return (unsigned)(b > 8192 ? 8192 : (b < 1 ? 1 : b));
}

hipError_t stk_launch_emb_gather(int R, int C, int V, const int* tok, const float* emb, float* out,
                                 hipStream_t st) {
  hipLaunchKernelGGL(stk::emb_gather, dim3(grid_for((size_t)R * C / 4)), dim3(256), 0, st, R, C, V,
                     tok, emb, out);
  return hipGetLastError();
}
// float4 chunks per lane for a row of C floats: 1, 2, 4, 8 or 16
static int ln_chunks(int C) {
  const int need = (C / 4 + 63) / 64;
  int j = 1;
  while (j < need) j *= 2;
  return j;
}
hipError_t stk_launch_layernorm(int R, int C, const float* x, const float* w, const float* b,
                                float* y, float* mean, float* rstd, hipStream_t st) {
  const dim3 g((R + 3) / 4), t(256);
  switch (ln_chunks(C)) {
    case 1: hipLaunchKernelGGL(stk::layernorm_fwd<1>, g, t, 0, st, R, C, x, w, b, y, mean, rstd); break;
    case 2: hipLaunchKernelGGL(stk::layernorm_fwd<2>, g, t, 0, st, R, C, x, w, b, y, mean, rstd); break;
    case 4: hipLaunchKernelGGL(stk::layernorm_fwd<4>, g, t, 0, st, R, C, x, w, b, y, mean, rstd); break;
    case 8: hipLaunchKernelGGL(stk::layernorm_fwd<8>, g, t, 0, st, R, C, x, w, b, y, mean, rstd); break;
    default: hipLaunchKernelGGL(stk::layernorm_fwd<16>, g, t, 0, st, R, C, x, w, b, y, mean, rstd); break;
  }
  return hipGetLastError();
}
hipError_t stk_launch_cm_shift(int BT, int T, int C, const float* x, const float* x_prev,
                               const float* mu, float* sh, float* x_last, hipStream_t st,
                               __bf16* sh16) {
  hipLaunchKernelGGL(stk::cm_shift, dim3(grid_for((size_t)BT * C / 4)), dim3(256), 0, st, BT, T, C,
                     x, x_prev, mu, sh, x_last, sh16);
  return hipGetLastError();
}
int stk_max_layernorm_width() { return 64 * 4 * stk::MAXC4_LIMIT; }

hipError_t stk_launch_ln_mix(const LnMix& p, hipStream_t st) {
  const dim3 g((p.R + 3) / 4), t(256);
  switch (ln_chunks(p.C)) {
    case 1: hipLaunchKernelGGL(stk::ln_mix<1>, g, t, 0, st, p); break;
    case 2: hipLaunchKernelGGL(stk::ln_mix<2>, g, t, 0, st, p); break;
    case 4: hipLaunchKernelGGL(stk::ln_mix<4>, g, t, 0, st, p); break;
    case 8: hipLaunchKernelGGL(stk::ln_mix<8>, g, t, 0, st, p); break;
    default: hipLaunchKernelGGL(stk::ln_mix<16>, g, t, 0, st, p); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------ training kernels --
namespace stk {

// zero n 4-byte words (a kernel, not a memset: safe inside captured graphs)
__global__ __launch_bounds__(256) void fill_zero(size_t n, float* __restrict__ p) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0.f;
}

constexpr int LN_ROWS = 8;  // rows per workgroup in the LayerNorm backward (partial sums)

// LayerNorm backward, one wave per row (row in registers), 4 waves x 2 rows
// per workgroup.  dx = rstd (dn - mean(dn) - nhat mean(dn nhat)) + dres,
// dn = dy w; per-channel partials of dw = sum dy nhat and db = sum dy are
// written as part[0|1][blk][C] (summed later in a fixed order).
template <int MAXC4>
__global__ __launch_bounds__(256) void layernorm_bwd(int R, int C, const float* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ dy,
                                                     const float* dres, float* dx,
                                                     float* __restrict__ part,
                                                     __bf16* __restrict__ dx16) {
  __shared__ f4 red[2][4][MAXC4][64];
  const int blk = blockIdx.x, nblk = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int C4 = C / 4;
  f4 pw[MAXC4], pb[MAXC4];
#pragma unroll
  for (int j = 0; j < MAXC4; j++) pw[j] = pb[j] = f4{0.f, 0.f, 0.f, 0.f};
  const int r_end = min(R, (blk + 1) * LN_ROWS);
  for (int row = blk * LN_ROWS + wave; row < r_end; row += 4) {
    const f4* xr = reinterpret_cast<const f4*>(x + (size_t)row * C);
    const f4* gr = reinterpret_cast<const f4*>(dy + (size_t)row * C);
    const f4* rr = dres ? reinterpret_cast<const f4*>(dres + (size_t)row * C) : nullptr;
    f4 xv[MAXC4], gv[MAXC4], rv[MAXC4];
    float s = 0.f;
    // the row's x, dy and residual gradient are all requested up front
#pragma unroll
    for (int j = 0; j < MAXC4; j++) {
      const int c4 = lane + 64 * j;
      xv[j] = c4 < C4 ? xr[c4] : f4{0.f, 0.f, 0.f, 0.f};
      gv[j] = c4 < C4 ? gr[c4] : f4{0.f, 0.f, 0.f, 0.f};
      rv[j] = (rr && c4 < C4) ? rr[c4] : f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < MAXC4; j++) s += (xv[j][0] + xv[j][1]) + (xv[j][2] + xv[j][3]);
    const float mean = wavesum(s) / C;
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < MAXC4; j++) {
      if (lane + 64 * j < C4) {
        const f4 d = xv[j] - mean;
        q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
      }
    }
    const float rstd = 1.0f / sqrtf(wavesum(q) / C + LN_EPS);
    float m1 = 0.f, m2 = 0.f;
#pragma unroll
    for (int j = 0; j < MAXC4; j++) {
      const int c4 = lane + 64 * j;
      if (c4 < C4) {
        const f4 nh = (xv[j] - mean) * rstd;
        const f4 dn = gv[j] * reinterpret_cast<const f4*>(w)[c4];
        m1 += (dn[0] + dn[1]) + (dn[2] + dn[3]);
        const f4 t = dn * nh;
        m2 += (t[0] + t[1]) + (t[2] + t[3]);
        pw[j] += gv[j] * nh;
        pb[j] += gv[j];
        xv[j] = nh;  // keep nhat
        gv[j] = dn;  // keep dn
      }
    }
    m1 = wavesum(m1) / C;
    m2 = wavesum(m2) / C;
    f4* dxr = reinterpret_cast<f4*>(dx + (size_t)row * C);
#pragma unroll
    for (int j = 0; j < MAXC4; j++) {
      const int c4 = lane + 64 * j;
      if (c4 < C4) {
        f4 o = rstd * (gv[j] - m1 - xv[j] * m2) + rv[j];
        dxr[c4] = o;
        if (dx16) *reinterpret_cast<bf16x4_t*>(dx16 + (size_t)row * C + 4 * c4) = __builtin_convertvector(o, bf16x4_t);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MAXC4; j++) {
    red[0][wave][j][lane] = pw[j];
    red[1][wave][j][lane] = pb[j];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * C4; i += 256) {
    const int v = i / C4, c4 = i - v * C4, j = c4 >> 6, l = c4 & 63;
    f4 t = red[v][0][j][l];
#pragma unroll
    for (int wv = 1; wv < 4; wv++) t += red[v][wv][j][l];
    reinterpret_cast<f4*>(part + ((size_t)v * nblk + blk) * C)[c4] = t;
  }
}

constexpr int SB_TOK = 8;  // consecutive tokens per thread in the shift backward

// Float4 columns a thread group covers, and groups per workgroup, for width C:
// up to 256 columns side by side; narrower rows stack 256 / (C/4) token
// groups in one workgroup.
__host__ __device__ inline int sb_lanes(int C) { return C / 4 < 256 ? C / 4 : 256; }
__host__ __device__ inline int sb_groups(int C) { return 256 / sb_lanes(C); }

// Channel-mix token-shift backward: dx = dsh (1 - mu) + dsh[t+1] mu,
// dx_prev (t = 0) = dsh mu, partial dmu = sum dsh (prev - x).
// Grid (channel blocks of 256 float4 columns, token blocks).  A thread owns
// one float4 column and SB_TOK consecutive tokens: it loads x of those tokens
// and the one before, and dsh of those tokens and the one after, all at once
// (so their latencies overlap), then computes; x, dsh and dx cross HBM once
// and every wave touches 1 KB of one row per access.  Each workgroup writes
// one partial row of dmu (its groups summed through LDS).
__global__ __launch_bounds__(256) void cm_shift_bwd(int BT, int T, int C, const float* __restrict__ x,
                                                    const float* __restrict__ x_prev,
                                                    const float* __restrict__ mu,
                                                    const float* __restrict__ dsh,
                                                    float* __restrict__ dx, float* __restrict__ dx_prev,
                                                    float* __restrict__ part) {
  __shared__ f4 red[256];
  const int C4 = C / 4, lanes = sb_lanes(C), G = sb_groups(C);
  const int grp = threadIdx.x / lanes, l = threadIdx.x - grp * lanes;
  const int c4 = blockIdx.x * 256 + l;
  const f4* X = reinterpret_cast<const f4*>(x);
  const f4* D = reinterpret_cast<const f4*>(dsh);
  f4* DX = reinterpret_cast<f4*>(dx);
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  f4 pm = zero;
  const int bt0 = (blockIdx.y * G + grp) * SB_TOK;
  if (grp < G && c4 < C4 && bt0 < BT) {
    const f4 m = reinterpret_cast<const f4*>(mu)[c4];
    // xs[i]: x of token bt0 - 1 + i; ds[i]: dsh of token bt0 + i (zeros outside [0, BT))
    f4 xs[SB_TOK + 1], ds[SB_TOK + 1];
#pragma unroll
    for (int i = 0; i <= SB_TOK; i++) {
      const int tx_ = bt0 - 1 + i, td = bt0 + i;
      xs[i] = (tx_ >= 0 && tx_ < BT) ? X[(size_t)tx_ * C4 + c4] : zero;
      ds[i] = td < BT ? D[(size_t)td * C4 + c4] : zero;
    }
    const int t0 = bt0 % T, b0 = bt0 / T;
#pragma unroll
    for (int i = 0; i < SB_TOK; i++) {
      const int bt = bt0 + i;
      if (bt >= BT) break;
      int t = t0 + i, b = b0;
      while (t >= T) {  // at most a few wraps (T >= 1)
        t -= T;
        b++;
      }
      const f4 prev = t > 0 ? xs[i] : (x_prev ? reinterpret_cast<const f4*>(x_prev)[(size_t)b * C4 + c4] : zero);
      const f4 g = ds[i];
      const f4 gn = t < T - 1 ? ds[i + 1] : zero;  // the next token of the same sequence
      pm += g * (prev - xs[i + 1]);
      DX[(size_t)bt * C4 + c4] = g * (1.0f - m) + gn * m;
      if (t == 0 && dx_prev) reinterpret_cast<f4*>(dx_prev)[(size_t)b * C4 + c4] = g * m;
    }
  }
  red[threadIdx.x] = pm;
  __syncthreads();
  if (grp == 0 && c4 < C4) {
    f4 s = red[l];
    for (int gi = 1; gi < G; gi++) s += red[gi * lanes + l];
    reinterpret_cast<f4*>(part + (size_t)blockIdx.y * C)[c4] = s;
  }
}

// Number of targets in [0, V) (the counted tokens; one workgroup).
__global__ __launch_bounds__(256) void count_valid(int R, int V, const int* __restrict__ targets,
                                                   int* __restrict__ n_valid) {
  __shared__ int sm[4];
  int c = 0;
  for (int i = threadIdx.x; i < R; i += 256) c += (unsigned)targets[i] < (unsigned)V;
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) n_valid[0] = (sm[0] + sm[1]) + (sm[2] + sm[3]);
}

// Fused log-softmax cross-entropy, one workgroup per row, in place:
// loss_row[r] = lse - z[target];  z <- (softmax(z) - onehot(target)) / n_valid.
// A target outside [0, V) is ignored: zero row, zero loss term.  The maximum
// is exact; each exp(z - max) is an fp32 term in (0, 1], and their sum, its
// log and so lse are in double (the fullmodel page's fm_k_ce_bwd keeps the
// normaliser in double).
// d16 (optional): a bf16 copy of dlogits (dense [R][V], rounded to nearest
// even) for a later bf16 matrix product.
__device__ __forceinline__ void st16(__bf16* d16, size_t e, f4 x) {
  *reinterpret_cast<bf16x4_t*>(d16 + e) = __builtin_convertvector(x, bf16x4_t);
}
__global__ __launch_bounds__(256) void ce_fwd_bwd(int R, int V, float* __restrict__ z,
                                                  const int* __restrict__ targets,
                                                  const int* __restrict__ n_valid,
                                                  float* __restrict__ loss_row,
                                                  __bf16* __restrict__ d16) {
  __shared__ float smx[4];
  __shared__ double ssum[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  f4* zr = reinterpret_cast<f4*>(z + (size_t)row * V);
  const int V4 = V / 4;
  const int tgt = targets[row];
  if ((unsigned)tgt >= (unsigned)V) {  // ignored row (uniform per workgroup)
    for (int i = tid; i < V4; i += 256) {
      zr[i] = f4{0.f, 0.f, 0.f, 0.f};
      if (d16) st16(d16, (size_t)row * V + 4 * i, f4{0.f, 0.f, 0.f, 0.f});
    }
    if (tid == 0) loss_row[row] = 0.f;
    return;
  }
  const int nv = n_valid[0];
  const float inv_n = (float)(1.0 / (double)nv);  // nv >= 1 here
  float mx = -INFINITY;
  for (int i = tid; i < V4; i += 256) {
    const f4 v = zr[i];
    mx = fmaxf(mx, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  }
  // wave max via the sum machinery on exp-free values: use shuffles
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) smx[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(smx[0], smx[1]), fmaxf(smx[2], smx[3]));
  double s = 0.0;
  for (int i = tid; i < V4; i += 256) {
    const f4 v = zr[i];
    s += (double)((expf(v[0] - mx) + expf(v[1] - mx)) + (expf(v[2] - mx) + expf(v[3] - mx)));
  }
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) ssum[wave] = s;
  __syncthreads();
  s = (ssum[0] + ssum[1]) + (ssum[2] + ssum[3]);
  const double lse_d = (double)mx + log(s);
  const float lse = (float)lse_d;
  const float zt = z[(size_t)row * V + tgt];
  __syncthreads();  // every thread has read z[target] before it is overwritten
  for (int i = tid; i < V4; i += 256) {
    const f4 v = zr[i];
    f4 p;
#pragma unroll
    for (int c = 0; c < 4; c++) p[c] = expf(v[c] - lse) - ((4 * i + c) == tgt ? 1.0f : 0.0f);
    zr[i] = p * inv_n;
    if (d16) st16(d16, (size_t)row * V + 4 * i, p * inv_n);
  }
  if (tid == 0) loss_row[row] = (float)(lse_d - (double)zt);
}

// The same cross-entropy with the row held in registers: 1024 threads, NV4
// float4 per thread (V <= 4096 NV4), so the logits are read once and written
// once.  The arithmetic per float4 and the reductions' precisions are those
// of ce_fwd_bwd (fp32 max and terms, double sum and LSE).
template <int NV4>
__global__ __launch_bounds__(1024) void ce_fwd_bwd_reg(int R, int V, float* __restrict__ z,
                                                       const int* __restrict__ targets,
                                                       const int* __restrict__ n_valid,
                                                       float* __restrict__ loss_row,
                                                       __bf16* __restrict__ d16) {
  __shared__ float smx[16];
  __shared__ double ssum[16];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  f4* zr = reinterpret_cast<f4*>(z + (size_t)row * V);
  const int V4 = V / 4;
  const int tgt = targets[row];
  if ((unsigned)tgt >= (unsigned)V) {  // ignored row (uniform per workgroup)
    for (int i = tid; i < V4; i += 1024) {
      zr[i] = f4{0.f, 0.f, 0.f, 0.f};
      if (d16) st16(d16, (size_t)row * V + 4 * i, f4{0.f, 0.f, 0.f, 0.f});
    }
    if (tid == 0) loss_row[row] = 0.f;
    return;
  }
  const float zt = tid == 0 ? z[(size_t)row * V + tgt] : 0.f;  // read before any write (barriers below)
  f4 v[NV4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV4; i++) {
    const int idx = tid + i * 1024;
    v[i] = idx < V4 ? zr[idx] : f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    mx = fmaxf(mx, fmaxf(fmaxf(v[i][0], v[i][1]), fmaxf(v[i][2], v[i][3])));
  }
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) smx[wave] = mx;
  __syncthreads();
  mx = smx[0];
  for (int w = 1; w < 16; w++) mx = fmaxf(mx, smx[w]);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < NV4; i++)
    if (tid + i * 1024 < V4)
      s += (double)((expf(v[i][0] - mx) + expf(v[i][1] - mx)) + (expf(v[i][2] - mx) + expf(v[i][3] - mx)));
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) ssum[wave] = s;
  __syncthreads();
  s = 0.0;
  for (int w = 0; w < 16; w++) s += ssum[w];
  const double lse_d = (double)mx + log(s);
  const float lse = (float)lse_d;
  const float inv_n = (float)(1.0 / (double)n_valid[0]);  // >= 1 here
#pragma unroll
  for (int i = 0; i < NV4; i++) {
    const int idx = tid + i * 1024;
    if (idx < V4) {
      f4 p;
#pragma unroll
      for (int c = 0; c < 4; c++) p[c] = expf(v[i][c] - lse) - ((4 * idx + c) == tgt ? 1.0f : 0.0f);
      zr[idx] = p * inv_n;
      if (d16) st16(d16, (size_t)row * V + 4 * idx, p * inv_n);
    }
  }
  if (tid == 0) loss_row[row] = (float)(lse_d - (double)zt);
}

// loss = sum_r loss_row[r] / n_valid (0 when no target is valid), fixed order
// (one workgroup)
__global__ __launch_bounds__(256) void sum_rows(int R, const float* __restrict__ v,
                                                const int* __restrict__ n_valid,
                                                float* __restrict__ out) {
  __shared__ float sm[256];
  float s = 0.f;
  for (int i = threadIdx.x; i < R; i += 256) s += v[i];
  sm[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) sm[threadIdx.x] += sm[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int nv = n_valid[0];
    out[0] = nv > 0 ? (float)((double)sm[0] / (double)nv) : 0.f;
  }
}

// Embedding backward without float atomics.
// 1) integer counts per vocabulary row
__global__ __launch_bounds__(256) void emb_count(int R, int V, const int* __restrict__ tok,
                                                 int* __restrict__ count) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p < R && (unsigned)tok[p] < (unsigned)V) atomicAdd(&count[tok[p]], 1);
}
// 2) exclusive scan of the counts (one workgroup of 1024 threads, each a
// contiguous range; with V a multiple of 4 and at most 64 per thread the
// range is held in registers, read and written as int4, all loads in flight
// together)
__global__ __launch_bounds__(1024) void emb_scan(int V, const int* __restrict__ count,
                                                 int* __restrict__ off) {
  __shared__ int sm[1024];
  constexpr int MAXQ = 16;  // int4 per thread in the register path
  const int per = (V + 1023) / 1024;
  const int b = threadIdx.x * per, e = min(V, b + per);
  const bool vec = V % 4 == 0 && per % 4 == 0 && per <= 4 * MAXQ;  // the same for every thread
  int4 cv[MAXQ];
  int s = 0;
  if (vec) {
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      const int i = b + 4 * q;
      cv[q] = 4 * q < per && i < e ? *reinterpret_cast<const int4*>(count + i) : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < MAXQ; q++) s += (cv[q].x + cv[q].y) + (cv[q].z + cv[q].w);
  } else {
    for (int i = b; i < e; i++) s += count[i];
  }
  sm[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    const int t = threadIdx.x >= o ? sm[threadIdx.x - o] : 0;
    __syncthreads();
    sm[threadIdx.x] += t;
    __syncthreads();
  }
  int run = sm[threadIdx.x] - s;  // exclusive prefix of this thread's range
  if (vec) {
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      const int i = b + 4 * q;
      if (4 * q < per && i < e) {
        int4 o;
        o.x = run; run += cv[q].x;
        o.y = run; run += cv[q].y;
        o.z = run; run += cv[q].z;
        o.w = run; run += cv[q].w;
        *reinterpret_cast<int4*>(off + i) = o;
      }
    }
  } else {
    for (int i = b; i < e; i++) {
      off[i] = run;
      run += count[i];
    }
  }
}
// 3) position p goes to slot off[tok[p]] + #{q < p : tok[q] == tok[p]} (stable);
// positions with an id outside [0, V) are not placed (no gradient row).  The
// earlier ids are staged through LDS 256 at a time and read as broadcasts:
// whole tiles before the workgroup's own count in full, the workgroup's own
// tile up to the position.
__global__ __launch_bounds__(256) void emb_place(int R, int V, const int* __restrict__ tok,
                                                 const int* __restrict__ off, int* __restrict__ perm) {
  __shared__ __attribute__((aligned(16))) int tile[256];
  const int p0 = blockIdx.x * 256, tid = threadIdx.x, p = p0 + tid;
  const int v = p < R ? tok[p] : -1;
  int rank = 0;
  for (int q0 = 0; q0 <= p0; q0 += 256) {  // the same trip count for the whole workgroup
    __syncthreads();                        // the previous tile consumed
    tile[tid] = q0 + tid < R ? tok[q0 + tid] : -1;
    __syncthreads();
    if (q0 < p0) {
#pragma unroll 8
      for (int i = 0; i < 256; i += 4) {
        const int4 x = *reinterpret_cast<const int4*>(&tile[i]);
        rank += (x.x == v) + (x.y == v) + (x.z == v) + (x.w == v);
      }
    } else {
      for (int i = 0; i < tid; i++) rank += tile[i] == v;
    }
  }
  if (p < R && (unsigned)v < (unsigned)V) perm[off[v] + rank] = p;
}
// 4) demb[v] = sum of dx rows of its positions in position order; one wave per row
__global__ __launch_bounds__(256) void emb_rows(int V, int C, const int* __restrict__ count,
                                                const int* __restrict__ off,
                                                const int* __restrict__ perm,
                                                const float* __restrict__ dx,
                                                float* __restrict__ demb) {
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (v >= V) return;
  const int C4 = C / 4, n = count[v], o = off[v];
  for (int c4 = lane; c4 < C4; c4 += 64) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n; i++) acc += reinterpret_cast<const f4*>(dx + (size_t)perm[o + i] * C)[c4];
    reinterpret_cast<f4*>(demb + (size_t)v * C)[c4] = acc;
  }
}

}  // namespace stk

hipError_t stk_launch_fill_zero(float* p, size_t n, hipStream_t st) {
  hipLaunchKernelGGL(stk::fill_zero, dim3(grid_for(n)), dim3(256), 0, st, n, p);
  return hipGetLastError();
}
int stk_num_ln_blocks(int R) { return (R + stk::LN_ROWS - 1) / stk::LN_ROWS; }
int stk_num_shift_blocks(int BT, int C) {
  const int per = stk::sb_groups(C) * stk::SB_TOK;
  return (BT + per - 1) / per;
}

hipError_t stk_launch_layernorm_bwd(int R, int C, const float* x, const float* w, const float* dy,
                                    const float* dres, float* dx, float* part, hipStream_t st,
                                    __bf16* dx16) {
  const dim3 g(stk_num_ln_blocks(R)), t(256);
  switch (ln_chunks(C)) {
    case 1: hipLaunchKernelGGL(stk::layernorm_bwd<1>, g, t, 0, st, R, C, x, w, dy, dres, dx, part, dx16); break;
    case 2: hipLaunchKernelGGL(stk::layernorm_bwd<2>, g, t, 0, st, R, C, x, w, dy, dres, dx, part, dx16); break;
    case 4: hipLaunchKernelGGL(stk::layernorm_bwd<4>, g, t, 0, st, R, C, x, w, dy, dres, dx, part, dx16); break;
    case 8: hipLaunchKernelGGL(stk::layernorm_bwd<8>, g, t, 0, st, R, C, x, w, dy, dres, dx, part, dx16); break;
    default: hipLaunchKernelGGL(stk::layernorm_bwd<16>, g, t, 0, st, R, C, x, w, dy, dres, dx, part, dx16); break;
  }
  return hipGetLastError();
}
hipError_t stk_launch_cm_shift_bwd(int BT, int T, int C, const float* x, const float* x_prev,
                                   const float* mu, const float* dsh, float* dx, float* dx_prev,
                                   float* part, hipStream_t st) {
  hipLaunchKernelGGL(stk::cm_shift_bwd, dim3((C / 4 + 255) / 256, stk_num_shift_blocks(BT, C)), dim3(256), 0, st,
                     BT, T, C, x, x_prev, mu, dsh, dx, dx_prev, part);
  return hipGetLastError();
}
hipError_t stk_launch_ce(int R, int V, float* z, const int* targets, float* loss_row, float* loss,
                         int* n_valid, hipStream_t st, __bf16* d16) {
  hipLaunchKernelGGL(stk::count_valid, dim3(1), dim3(256), 0, st, R, V, targets, n_valid);
  const int V4 = V / 4;
  if (V4 >= 1024 && V4 <= 16 * 1024) {  // the row fits in the registers of 1024 threads
    const dim3 g(R), t(1024);
    if (V4 <= 1024) hipLaunchKernelGGL(stk::ce_fwd_bwd_reg<1>, g, t, 0, st, R, V, z, targets, n_valid, loss_row, d16);
    else if (V4 <= 2048) hipLaunchKernelGGL(stk::ce_fwd_bwd_reg<2>, g, t, 0, st, R, V, z, targets, n_valid, loss_row, d16);
    else if (V4 <= 4096) hipLaunchKernelGGL(stk::ce_fwd_bwd_reg<4>, g, t, 0, st, R, V, z, targets, n_valid, loss_row, d16);
    else if (V4 <= 8192) hipLaunchKernelGGL(stk::ce_fwd_bwd_reg<8>, g, t, 0, st, R, V, z, targets, n_valid, loss_row, d16);
    else hipLaunchKernelGGL(stk::ce_fwd_bwd_reg<16>, g, t, 0, st, R, V, z, targets, n_valid, loss_row, d16);
  } else {
    hipLaunchKernelGGL(stk::ce_fwd_bwd, dim3(R), dim3(256), 0, st, R, V, z, targets, n_valid,
                       loss_row, d16);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stk::sum_rows, dim3(1), dim3(256), 0, st, R, loss_row, n_valid, loss);
  return hipGetLastError();
}
hipError_t stk_launch_emb_bwd(int R, int V, int C, const int* tok, const float* dx, int* count,
                              int* off, int* perm, float* demb, hipStream_t st) {
  hipError_t e = stk_launch_fill_zero((float*)count, (size_t)V, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stk::emb_count, dim3((R + 255) / 256), dim3(256), 0, st, R, V, tok, count);
  hipLaunchKernelGGL(stk::emb_scan, dim3(1), dim3(1024), 0, st, V, count, off);
  hipLaunchKernelGGL(stk::emb_place, dim3((R + 255) / 256), dim3(256), 0, st, R, V, tok, off, perm);
  hipLaunchKernelGGL(stk::emb_rows, dim3((V + 3) / 4), dim3(256), 0, st, V, C, count, off, perm, dx,
                     demb);
  return hipGetLastError();
}
