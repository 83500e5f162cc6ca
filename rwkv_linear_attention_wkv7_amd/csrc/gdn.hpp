// Launch arguments of the GatedDeltaNet kernels (gdn.hip).
#pragma once
#include <hip/hip_runtime.h>

struct GdnArgs {
  int B, T, nk, nv, dk, dv, kk;
  float rms_eps;
  // inputs and frozen weights
  const float *raw, *z, *a, *b, *conv, *A_log, *dt_bias, *norm;
  // forward activations (the cache): pre and cq [B][T][c_dim], qh and kh
  // [B][T][nk][dk], g and beta [B][T][nv], o [B][T][nv][dv], ckpt
  // [B][nv][ceil(T/16)][dv][dk]
  float *pre, *cq, *qh, *kh, *g, *beta, *o, *ckpt;
  float* kv;   // [B][T][nv][dv]: (g S)^T k^ of each token (the two-pass backward's input)
  float* out;  // [B][T][nv][dv]
  // backward
  const float* dout;
  float *dz, *dobuf, *dcq, *part, *draw, *da, *db;
  // two-pass backward (dk = dv = 64 or 128): the gradient entering each
  // block's last token [B][nv][blocks][dv][dk], du [B][T][nv][dv], the block
  // ends' inner products by column [B][nv][blocks][dv]
  float *gend, *du, *anc;
};

// whether the two-pass backward applies to this shape
bool gdn_two_pass(int dk, int dv);

size_t gdn_ckpt_floats(int B, int T, int nv, int dk, int dv);
size_t gdn_partial_floats(int B, int T, int nv, int dk, int dv);
hipError_t gdn_launch_forward(const GdnArgs& p, hipStream_t st);
hipError_t gdn_launch_backward(const GdnArgs& p, hipStream_t st);
