// Launchers of the stack kernels (stack_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>

hipError_t stk_launch_emb_gather(int R, int C, int V, const int* tok, const float* emb, float* out,
                                 hipStream_t st);
hipError_t stk_launch_layernorm(int R, int C, const float* x, const float* w, const float* b,
                                float* y, float* mean, float* rstd, hipStream_t st);
// sh16: NULL or a bf16 copy of sh (dense [BT][C]) for the key product's A
hipError_t stk_launch_cm_shift(int BT, int T, int C, const float* x, const float* x_prev,
                               const float* mu, float* sh, float* x_last, hipStream_t st,
                               __bf16* sh16 = nullptr);

// LayerNorm fused with up to six token-shift lerps, one token per row (T = 1).
struct LnMix {
  int R, C, nmix;
  const float *x, *w, *b;
  const float* x_prev;  // previous token's LN output per row, or NULL (zeros)
  float* x_last;        // receives this token's LN output (may equal x_prev)
  const float* mu[6];
  float* out[6];
  // optional split-K partials of a product to add to x first: x_sum = x +
  // (part[0] + ... + part[nparts-1]) ([nparts][R][C]), written to x_sum
  // (which may be x) and normalised in place of x
  const float* part;
  int nparts;
  float* x_sum;
};
hipError_t stk_launch_ln_mix(const LnMix& p, hipStream_t st);
int stk_max_layernorm_width();
int stk_num_ln_blocks(int R);
// partial rows of the channel-mix shift backward (one per workgroup of tokens)
int stk_num_shift_blocks(int BT, int C);
// dx16: NULL or a bf16 copy of dx (dense [R][C]) for a later product's A
hipError_t stk_launch_layernorm_bwd(int R, int C, const float* x, const float* w, const float* dy,
                                    const float* dres, float* dx, float* part, hipStream_t st,
                                    __bf16* dx16 = nullptr);
hipError_t stk_launch_cm_shift_bwd(int BT, int T, int C, const float* x, const float* x_prev,
                                   const float* mu, const float* dsh, float* dx, float* dx_prev,
                                   float* part, hipStream_t st);
// Fused CE over R rows of V logits (in place: dlogits); n_valid: one int of
// scratch (the count of targets in [0, V)); d16: NULL or a bf16 copy of
// dlogits (dense [R][V], V a multiple of 4) for a later bf16 product.
hipError_t stk_launch_ce(int R, int V, float* z, const int* targets, float* loss_row, float* loss,
                         int* n_valid, hipStream_t st, __bf16* d16 = nullptr);
hipError_t stk_launch_emb_bwd(int R, int V, int C, const int* tok, const float* dx, int* count,
                              int* off, int* perm, float* demb, hipStream_t st);
hipError_t stk_launch_fill_zero(float* p, size_t n, hipStream_t st);
