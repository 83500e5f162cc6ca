// Argument blocks of the fused time-mix kernels (passed by value).
#pragma once
#include <hip/hip_runtime.h>

#include "gemm.hpp"

constexpr int TB = 128;  // tokens per workgroup in the backward partial-sum kernels

struct TmFwd {
  int BT, T, C, layer_id;
  const float *x, *x_prev;
  const float *mu_r, *mu_w, *mu_k, *mu_v, *mu_a, *mu_g;
  float *xr, *xw, *xk, *xv, *xa, *xg, *x_last;
  // optional bf16 copies of xr, xk, xv (dense [BT][C], rounded to nearest
  // even) for the r/k/v products' A operands
  __bf16 *xr16, *xk16, *xv16;
  // pre-WKV
  const float *k, *v, *ow, *oa, *ov, *w0, *a0, *v0, *k_k, *k_a;
  float* v_first;  // written on layer 0, read otherwise
  float *w, *a, *kk, *kmod, *vmod, *A, *Bv;
  // post-WKV
  const float *y, *r, *g, *r_k, *ln_w, *ln_b;
  float *tg, *mean, *rstd, *alpha;
  __bf16* tg16;  // optional bf16 copy of tg (post_fwd), the output product's A
};

struct TmBwd {
  int BT, T, C, layer_id;
  // post-WKV backward
  const float *dtg, *g, *y, *r, *kmod, *vmod, *mean, *rstd, *alpha, *r_k, *ln_w, *ln_b;
  float *dg, *dy_wkv, *dr, *dkmod, *dvmod, *part_post;
  // pre-WKV backward
  const float *gr, *gk, *gv, *gw, *gA, *gB;  // WKV7 gradients
  const float *a, *kk, *k, *w, *ow, *ov, *v, *v_first, *k_a, *k_k, *w0, *v0, *dvf_in;
  float *dk, *dv, *dpre_a, *dpre_w, *dpre_v, *dvf_out, *part_pre;
  // optional bf16 copies of the final dr, dk, dv (dense [BT][C], rounded to
  // nearest even) for the input-gradient products' A operands
  __bf16 *dr16, *dk16, *dv16;
  int dvf_accum;  // dvf_out += instead of =
  // token shift backward
  const float *x, *x_prev, *mu_r, *mu_w, *mu_k, *mu_v, *mu_a, *mu_g;
  const float *dxr, *dxw, *dxk, *dxv, *dxa, *dxg;
  float *dx, *dx_prev, *part_shift;
};

struct VecOut {
  float* p[8];
};

hipError_t tm_launch_shift_fwd(const TmFwd& p, hipStream_t st);
hipError_t tm_launch_pre_fwd(const TmFwd& p, hipStream_t st);
hipError_t tm_launch_post_fwd(const TmFwd& p, hipStream_t st);
// T = 1 (p.BT streams): pre-WKV, the WKV7 step on state [BT][H][N][N] in
// place, post-WKV; writes p.tg (and p.v_first on layer 0) only
hipError_t tm_launch_step_fused(const TmFwd& p, float* state, hipStream_t st);
int tm_num_token_blocks(int BT);
hipError_t tm_launch_post_bwd(const TmBwd& p, hipStream_t st);
hipError_t tm_launch_pre_bwd(const TmBwd& p, hipStream_t st);
hipError_t tm_launch_shift_bwd(const TmBwd& p, hipStream_t st);
hipError_t tm_launch_reduce(const float* part, int nvec, int nblk, int C, const VecOut& outs,
                            hipStream_t st);

// wkv7_seq.hip
hipError_t wkv7_launch_forward(int dtype, int B, int T, int H, const void* r, const void* w,
                               const void* k, const void* v, const void* a, const void* b,
                               const float* s0, void* y, float* sT, float* ckpt, float* chunk_ws, hipStream_t st);
// fp32 workspace of the chunked forward (records of every (b, h, chunk)); the
// forward takes the chunked kernels when it is given one and
// wkv7_use_chunked(T) (T of at least two chunks).
size_t wkv7_chunk_ws_floats(int B, int T, int H);
bool wkv7_use_chunked(int T);
hipError_t wkv7_launch_backward(int dtype, int B, int T, int H, const void* r, const void* w,
                                const void* k, const void* v, const void* a, const void* b,
                                const void* dy, const float* ckpt, const float* dsT, void* dr,
                                void* dw, void* dk, void* dv, void* da, void* db, float* ds0,
                                float* part, const int* gate, hipStream_t st);
size_t wkv7_bwd_partial_floats(int B, int T, int H);
// wkv7_bwd.hip: the two-pass backward (reverse scan of the state gradient,
// then per-chunk matrix-core products).  ckpt holds the forward's states and
// per-token sa (wkv7_ckpt_sa).  ws: wkv7_bwd2_ws_floats() fp32.  gate: NULL
// when every decay is known to lie in [1/8, 1] (the time-mix decay does);
// otherwise a zeroed int that the scan sets when some decay does not, after
// which the products return at once and the single-pass kernels, launched
// with the same gate, produce the results.
size_t wkv7_bwd2_ws_floats(int B, int T, int H);
hipError_t wkv7_launch_backward2(int dtype, int B, int T, int H, const void* r, const void* w,
                                 const void* k, const void* v, const void* a, const void* b,
                                 const void* dy, const float* ckpt, const float* dsT, void* dr,
                                 void* dw, void* dk, void* dv, void* da, void* db, float* ds0,
                                 float* ws, int* gate, hipStream_t st);
hipError_t wkv7_launch_step(int dtype, int B, int H, const void* r, const void* w, const void* k,
                            const void* v, const void* a, const void* b, float* state, void* y,
                            hipStream_t st);
int wkv7_ckpt_interval_const();
