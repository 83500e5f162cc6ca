/*
 * wkv7.h -- C-ABI of the MI355X (gfx950) RWKV-7 WKV7 / time-mix library.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains caller memory; scratch comes from the
 *    caller's workspace argument where a call needs one.
 *  - Work is enqueued on `stream` (NULL = the default stream) with no host
 *    synchronisation; results are valid once the stream has reached them.
 *  - Token tensors are [B][T][H][N] row-major (equivalently [B][T][C] with
 *    C = H*N, channel c = h*N + n).  States are [B][H][N][N] fp32 with
 *    S[i][j]: i the value index (row), j the key index (column).
 *  - Return value: 0 on success, or a negative wkv7_status.  Arguments are
 *    validated before anything is enqueued; on error nothing is enqueued and
 *    wkv7_last_error() describes the first problem found.
 *  - N must be 64.  Pointers must be 16-byte aligned (8-byte for bf16 data).
 *  - Aliasing: no tensor a call writes may overlap any other tensor of the
 *    call (read or written), including the workspace; tensors that are only
 *    read may overlap each other.  The exceptions are the in-place updates
 *    each call names (sT == s0, the decode state); anything else returns
 *    WKV7_EINVAL naming the two tensors.
 *  - The library keeps no state between calls beyond its loaded code (and
 *    the fixed device scratch of wkv7_backward_noalloc): calls are
 *    re-entrant, from any thread, on any stream.
 */
#ifndef WKV7_H
#define WKV7_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum wkv7_status {
  WKV7_OK = 0,
  WKV7_EINVAL = -1, /* bad shape, NULL required pointer, misalignment, overlapping tensors */
  WKV7_EHIP = -2,   /* a HIP launch or runtime error */
  WKV7_ENOSPC = -3  /* workspace smaller than the size query returned */
};

enum wkv7_dtype {
  WKV7_F32 = 0,  /* fp32 token tensors */
  WKV7_BF16 = 1  /* bf16 token tensors (state and accumulation stay fp32) */
};

/* Thread-local description of the last error (empty string if none). */
const char *wkv7_last_error(void);

/*
 * Optional second stream for the calls that overlap independent work on it
 * (wkv7_backward, timemix_backward, rwkv7_decode_step, rwkv7_train_step; each
 * says what it puts there).  Owned by the caller: a default-priority stream
 * and four events created with hipEventDisableTiming (or made by
 * wkv7_side_create).  A call forks the side stream from `stream` with these
 * events and joins it back to `stream` before returning, so everything stays
 * ordered on `stream` and a graph capture of `stream` records the side work
 * too.  The library retains nothing; one wkv7_side must not be used by two
 * calls at the same time (they would share its events).  NULL, or a side
 * whose stream is `stream` itself, runs everything on `stream`.
 */
typedef struct {
  hipStream_t stream;
  hipEvent_t ev[4];
} wkv7_side;
/* Create / destroy a wkv7_side (stream with hipStreamNonBlocking, events with
 * hipEventDisableTiming).  destroy accepts a zeroed or partly created side. */
int wkv7_side_create(wkv7_side *side);
int wkv7_side_destroy(wkv7_side *side);

/* Checkpoint interval L used by wkv7_forward / wkv7_backward (tokens). */
int wkv7_checkpoint_interval(void);

/* Number of fp32 elements of the checkpoint buffer:
 * B*H*ceil(T/L)*N*N (states) + B*T*H*N (the forward's sa per token). */
size_t wkv7_checkpoint_floats(int B, int T, int H, int N);

/*
 * WKV7 forward.  Per (b,h), starting from S = s0 (NULL = zero), for t = 0..T-1
 *     sa  = S a_t                                   (old state)
 *     S   = S diag(w_t) + sa b_t^T + v_t k_t^T
 *     y_t = S r_t                                   (updated state)
 * Pages: "Foundry/cuda_kernels/timemix.cu" (forward driver, k_composites: the
 * WKV7 kernel receives r, w, k', v', a = -kk, b = kk*a) and the per-head WKV
 * state-backward block of "infotheory .../rwkv7/model.rs" (read-out from the
 * updated state, rank-1 term from the old one).
 *
 * r,w,k,v,a,b: [B][T][H][N] of `dtype`.  y: [B][T][H][N] of `dtype` (written).
 * s0: [B][H][N][N] fp32 or NULL.  sT: [B][H][N][N] fp32 or NULL (written;
 * may equal s0 for an in-place state update).  ckpt: NULL, or
 * wkv7_checkpoint_floats() fp32: [B][H][ceil(T/L)][N][N], where checkpoint c
 * is the state after c*L tokens (c = 0 holds s0), then sa_t = S_{t-1} a_t of
 * every token, [B][T][H][N]; it is what wkv7_backward works from.
 * T >= 1, B >= 1, H >= 1.
 *
 * ws / ws_bytes: NULL, or device scratch of at least
 * wkv7_forward_workspace_bytes() bytes (16-byte aligned; contents
 * undefined before and after; owned by the caller, not retained).  The
 * query is nonzero exactly when T >= 2L; a workspace given for such a shape
 * selects the chunked matrix-core kernels (the recurrence unrolled over
 * chunks of L tokens, intra-chunk products on MFMA, a per-head state scan;
 * chunks whose cumulative decay leaves the fp32 exponent range of the
 * unrolled form run token by token).  ws NULL, or T < 2L, runs the
 * token-sequential kernel, which spreads each head over four workgroups; on
 * MI355X it is the faster of the two at every shape measured (B*H from 16
 * to 512, T up to 8192), and it is what every other call of this library
 * uses internally.  Both compute the same recurrence in fp32 and agree to
 * rounding.  A ws smaller than a nonzero query returns WKV7_ENOSPC.
 */
size_t wkv7_forward_workspace_bytes(int B, int T, int H, int N);
int wkv7_forward(int B, int T, int H, int N, int dtype,
                 const void *r, const void *w, const void *k, const void *v,
                 const void *a, const void *b, const float *s0,
                 void *y, float *sT, float *ckpt, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes wkv7_backward needs: one fp32 region shared by its two
 * paths (the two-pass path's dsa per token, state gradient every L tokens and
 * per-column sums; or the single-pass path's column partials), a flag, plus,
 * when have_ckpt is 0, the checkpoints
 * (recomputed by the token-sequential forward). */
size_t wkv7_backward_workspace_bytes(int B, int T, int H, int N, int have_ckpt);

/*
 * WKV7 backward: gradients of L = <dy, y> + <dsT, S_T> for the forward above
 * (reverse recurrence; with G = dL/dS_t, step t back:
 *     G += dy_t r_t^T;  dr_t = S_t^T dy_t;  dv_t = G k_t;  dk_t = G^T v_t;
 *     db_t = G^T sa_t;  dsa = G b_t;  dw_t = colsum(G .* S_{t-1});
 *     da_t = S_{t-1}^T dsa;  G = G diag(w_t) + dsa a_t^T ).
 * Same pages as wkv7_forward; the model.rs block gives these local terms.
 *
 * Computed in two passes when every decay lies in [1/8, 1] and the call
 * spans more than 512 (b, h, L-token chunk) triples: a reverse scan of G
 * alone (it never reads S), then per-chunk matrix-core products that give
 * the column sums from the checkpoints, the forward's sa and the scan's
 * boundary gradients; dw from a running sum of r dr - b db - k dk + a da.
 * Otherwise (a smaller call, or the scan finds a decay outside that range)
 * the single-pass kernel runs the step above token by token from the
 * checkpoints; both agree with the recurrence to fp32 rounding.
 *
 * ckpt: the forward's checkpoints, or NULL (then they are recomputed into the
 * workspace).  dy: [B][T][H][N] `dtype`.  dsT, s0: fp32 [B][H][N][N] or NULL.
 * dr,dw,dk,dv,da,db: [B][T][H][N] `dtype` (written).  ds0: fp32 or NULL.
 * ws: at least wkv7_backward_workspace_bytes() bytes (16-byte aligned;
 * contents undefined before and after).
 * side: NULL or a wkv7_side (checked, not used: every launch of this call
 * runs on `stream`).
 */
int wkv7_backward(int B, int T, int H, int N, int dtype,
                  const void *r, const void *w, const void *k, const void *v,
                  const void *a, const void *b, const float *s0, const float *ckpt,
                  const void *dy, const float *dsT,
                  void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                  float *ds0, void *ws, size_t ws_bytes, const wkv7_side *side,
                  hipStream_t stream);

/*
 * wkv7_backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, arguments, results and errors, with no workspace
 * argument.  Its scratch (wkv7_backward_workspace_bytes(B, T, H, N,
 * ckpt != NULL) bytes) comes from a fixed 64 MiB device array that each
 * device holds until the process ends; a shape needing more returns
 * WKV7_ENOSPC before anything is enqueued.  The call allocates nothing.  Every
 * call on one device shares that device's array, so calls that overlap on
 * one device (two streams, or two threads) race and must be serialised by
 * the caller.
 */
int wkv7_backward_noalloc(int B, int T, int H, int N, int dtype,
                          const void *r, const void *w, const void *k, const void *v,
                          const void *a, const void *b, const float *s0, const float *ckpt,
                          const void *dy, const float *dsT,
                          void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                          float *ds0, const wkv7_side *side, hipStream_t stream);

/*
 * Single-token streaming decode: the T = 1 forward with the state updated in
 * place.  Pages: the recurrence as for wkv7_forward; the per-layer streaming
 * state of "infotheory .../rwkv7/model.rs" (LayerState.att_state, [H][N][N]).
 * r,w,k,v,a,b,y: [B][H][N] `dtype`; state: [B][H][N][N] fp32 (read and
 * written in place; y must not overlap it or the inputs).
 */
int wkv7_step(int B, int H, int N, int dtype,
              const void *r, const void *w, const void *k, const void *v,
              const void *a, const void *b, float *state, void *y,
              hipStream_t stream);

/* ------------------------------------------------------------ time-mix -- */

/* Block geometry.  C = H*N, N = 64; LoRA ranks Dw, Da, Dv, Dg; layer_id 0
 * is the first block (publishes v_first, has no value-residual LoRA). */
typedef struct {
  int C, H, N, Dw, Da, Dv, Dg, layer_id;
} tm_shape;

/* fp32 weights, row-major [in][out] (y = x W), as on the timemix.cu page.
 * v0/V1/V2 are ignored (may be NULL) when layer_id == 0. */
typedef struct {
  const float *mu_r, *mu_w, *mu_k, *mu_v, *mu_a, *mu_g; /* [C] token-shift lerp */
  const float *Wr, *Wk, *Wv, *Wo;                       /* [C][C] */
  const float *w0, *W1, *W2;                            /* [C], [C][Dw], [Dw][C] */
  const float *a0, *A1, *A2;                            /* [C], [C][Da], [Da][C] */
  const float *v0, *V1, *V2;                            /* [C], [C][Dv], [Dv][C] */
  const float *G1, *G2;                                 /* [C][Dg], [Dg][C] */
  const float *k_k, *k_a, *r_k;                         /* [C] */
  const float *ln_w, *ln_b;                             /* [C] group-norm affine */
} tm_weights;

/* Gradients, same fields and shapes; every field is written (=, not +=). */
typedef struct {
  float *mu_r, *mu_w, *mu_k, *mu_v, *mu_a, *mu_g;
  float *Wr, *Wk, *Wv, *Wo;
  float *w0, *W1, *W2;
  float *a0, *A1, *A2;
  float *v0, *V1, *V2;
  float *G1, *G2;
  float *k_k, *k_a, *r_k;
  float *ln_w, *ln_b;
} tm_grads;

/* Bytes of the activation cache timemix_forward can leave for the backward. */
size_t timemix_cache_bytes(const tm_shape *s, int B, int T);
/* Workspace bytes for timemix_forward / timemix_backward. */
size_t timemix_forward_workspace_bytes(const tm_shape *s, int B, int T);
size_t timemix_backward_workspace_bytes(const tm_shape *s, int B, int T);

/*
 * Time-mix forward (no residual; the block adds it).  Pages:
 * "Foundry/cuda_kernels/timemix.cu" forward driver and kernels k_tokenshift
 * .. k_mul; LoRA formulas from the AttentionWeights of "infotheory
 * .../rwkv7/model.rs":
 *   xs_c = x + (x_prev_shift - x) mu_c  for c in r,w,k,v,a,g
 *   r = xs_r Wr; k = xs_k Wk; v = xs_v Wv
 *   w = exp(-0.606531 sigmoid(w0 + tanh(xs_w W1) W2))
 *   a = sigmoid(a0 + (xs_a A1) A2);  g = sigmoid(xs_g G1) G2
 *   kk = l2norm_head(k * k_k);  k' = k (1 + (a - 1) k_a)
 *   v' = v (layer 0, v_first := v)  or  v + (v_first - v) sigmoid(v0 + (xs_v V1) V2)
 *   y  = WKV7(r, w, k', v', -kk, kk * a; s0)
 *   out = ((groupnorm_head(y) * ln_w + ln_b) + (sum_head r k' r_k) v') * g  Wo
 * x: [B][T][C]; x_prev: [B][C] or NULL (zeros) -- the token before x[:,0];
 * v_first: [B][T][C], written on layer 0, read otherwise; s0/sT: fp32
 * [B][H][N][N] or NULL (sT may equal s0: in-place update); out: [B][T][C]
 * (written); x_last: [B][C] or NULL (written with x[:, T-1], the next call's
 * x_prev; it may equal x_prev when T == 1); cache: NULL or
 * timemix_cache_bytes() bytes kept for timemix_backward (then ws is unused).
 */
int timemix_forward(const tm_shape *s, const tm_weights *W, int B, int T,
                    const float *x, const float *x_prev, float *v_first,
                    const float *s0, float *sT, float *out, float *x_last,
                    void *cache, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Time-mix backward: gradients of L = <dout, out> + <dsT, S_T>
 * (+ <dv_first_in, v_first> on layer 0).  Pages: "Foundry/cuda_kernels/
 * timemix.cu" backward driver (phase order) and kernels k_split ..
 * k_tokenshift_bwd.  cache: the forward's cache for the same inputs, or NULL
 * (the forward is recomputed into the workspace).  G: every field written.
 * dx: [B][T][C]; dx_prev: [B][C] or NULL; dv_first_in: layer 0 only, [B][T][C]
 * or NULL; dv_first_out: layer > 0 only, [B][T][C] or NULL; ds0: fp32 or NULL.
 * side: NULL, or a wkv7_side on which the weight gradients (the X^T dY
 * products) run, overlapping the input-gradient chain on `stream`.
 */
int timemix_backward(const tm_shape *s, const tm_weights *W, int B, int T,
                     const float *x, const float *x_prev, const float *v_first,
                     const float *s0, const float *dout, const float *dsT,
                     const void *cache, tm_grads *G, float *dx, float *dx_prev,
                     const float *dv_first_in, float *dv_first_out, float *ds0,
                     void *ws, size_t ws_bytes, const wkv7_side *side, hipStream_t stream);


/* ------------------------------------------------------ decode stack -- */

/* RWKV-7 stack geometry: n_layer blocks of width C = H*N (N = 64), channel-mix
 * width F, vocabulary V, time-mix LoRA ranks, and whether layer 0 applies the
 * pre-norm ln0 to the embedding.  gemm_dtype selects the precision of the
 * products in every projection, LoRA, channel-mix and head GEMM: WKV7_F32
 * (fp32 operands) or WKV7_BF16 (operands rounded to bf16 to nearest even,
 * fp32 accumulation, as wkv7_gemm_bf16).  Tensors stay fp32 in memory either
 * way; the WKV7 recurrence and every elementwise step are fp32.
 * train_recompute (rwkv7_train_step only): 0 keeps every block's forward
 * activations in the workspace for its backward (about 1.1 GB per block at
 * B=4, T=2048, C=1024, F=4096); 1 keeps only the block inputs and recomputes
 * each block's forward in the backward (workspace for one block, one more
 * forward pass per step).  Results are identical. */
typedef struct {
  int n_layer, C, H, N, F, V, Dw, Da, Dv, Dg, use_ln0;
  int gemm_dtype;
  int train_recompute;
  /* Hybrid stack (rwkv7_train_step only; 0 elsewhere): n_attn MoBA attention
   * blocks interleaved with the n_layer RWKV-7 blocks as the fullmodel page's
   * fm_build does: after every n_layer / n_attn RWKV-7 blocks one attention
   * block, then the remaining RWKV-7 blocks.  moba_chunk and moba_topk are
   * the attention's chunk length and chunk count (moba_forward). */
  int n_attn, moba_chunk, moba_topk;
} rwkv7_config;

/* One block: LayerNorms, time-mix weights (layer_id = block index) and the
 * channel-mix (token-shift lerp mu_k [C], Wk [C][F], Wv [F][C]). */
typedef struct {
  const float *ln1_w, *ln1_b, *ln2_w, *ln2_b; /* [C] */
  tm_weights tm;
  const float *cm_mu_k, *cm_Wk, *cm_Wv;
} rwkv7_block;

/* One MoBA attention block of a hybrid stack.  Page: "Foundry/cuda_kernels/
 * fullmodel.cu", fm_attn_fwd / fm_attn_bwd: h1 = LN1(x); q, k, v = h1 Wq,
 * h1 Wk, h1 Wv (heads of 64, [in][out] weights); y = the MoBA core
 * (moba_forward); x1 = x + y Wo; h2 = LN2(x1); out = x1 + channel-mix(h2),
 * the channel-mix as in rwkv7_block. */
typedef struct {
  const float *ln1_w, *ln1_b, *ln2_w, *ln2_b; /* [C] */
  const float *Wq, *Wk, *Wv, *Wo;             /* [C][C] */
  const float *cm_mu_k, *cm_Wk, *cm_Wv;
} rwkv7_attn_block;

/* Whole model.  blocks is a HOST array of n_layer rwkv7_block (the pointers
 * inside are device pointers); ln0_w/b may be NULL when use_ln0 == 0; attn
 * a HOST array of n_attn rwkv7_attn_block (NULL when n_attn == 0). */
typedef struct {
  const float *emb;            /* [V][C] */
  const float *ln0_w, *ln0_b;  /* [C] */
  const float *ln_out_w, *ln_out_b;
  const float *head;           /* [C][V] (not tied to emb) */
  const rwkv7_block *blocks;
  const rwkv7_attn_block *attn;
} rwkv7_model;

size_t rwkv7_decode_workspace_bytes(const rwkv7_config *cfg, int B);

/*
 * One streaming-decode token for B independent streams through the stack.
 * Pages: block and model forward of "Foundry/cuda_kernels/fullmodel.cu"
 * (fm_rwkv_fwd: h1 = LN1(x), x1 = x + TM(h1), h2 = LN2(x1), out = x1 +
 * CM(h2); fm_cm_fwd; fm_forward: x0 = emb[token], ln_out, logits = h head)
 * and the streaming state of "infotheory .../rwkv7/model.rs" (LayerState:
 * att_x_prev, att_state, ffn_x_prev; layer-0 pre-norm; LayerNorm eps 1e-5).
 * tokens: [B] int32; an id outside [0, V) embeds as a zero row.  State
 * tensors are read and updated in place: att_x_prev, ffn_x_prev
 * [n_layer][B][C] (the previous token's LN1 / LN2 outputs), att_state
 * [n_layer][B][H][N][N] fp32.  logits: [B][V] fp32 (written).
 * side: NULL, or a wkv7_side; with one, from B = 512 on the streams are
 * advanced as two groups at once, the first on `stream` and the second on
 * the side stream (every kernel of the step is either bound by HBM over the
 * whole batch or a small latency-bound GEMM or row kernel, so the two chains
 * overlap).  Without one the groups run one after the other on `stream`.
 */
int rwkv7_decode_step(const rwkv7_config *cfg, const rwkv7_model *model, int B,
                      const int *tokens, float *att_x_prev, float *att_state,
                      float *ffn_x_prev, float *logits, void *ws, size_t ws_bytes,
                      const wkv7_side *side, hipStream_t stream);

/* --------------------------------------------------- training step -- */

/* Gradients of one block / of the model; same fields and shapes as
 * rwkv7_block / rwkv7_model, every field written (=).  blocks is a HOST array. */
typedef struct {
  float *ln1_w, *ln1_b, *ln2_w, *ln2_b;
  tm_grads tm;
  float *cm_mu_k, *cm_Wk, *cm_Wv;
} rwkv7_block_grads;

typedef struct {
  float *ln1_w, *ln1_b, *ln2_w, *ln2_b;
  float *Wq, *Wk, *Wv, *Wo;
  float *cm_mu_k, *cm_Wk, *cm_Wv;
} rwkv7_attn_grads;

typedef struct {
  float *emb, *ln0_w, *ln0_b, *ln_out_w, *ln_out_b, *head;
  rwkv7_block_grads *blocks;
  rwkv7_attn_grads *attn; /* HOST array of n_attn (NULL when n_attn == 0) */
} rwkv7_model_grads;

size_t rwkv7_train_workspace_bytes(const rwkv7_config *cfg, int B, int T);

/*
 * One training step of next-token cross-entropy over B sequences of T tokens
 * (zero initial state): loss = mean over the counted tokens of
 * log-sum-exp(logits) - logit[target]; every parameter gradient written.
 * Pages: whole-model forward/backward of "Foundry/cuda_kernels/fullmodel.cu"
 * (fm_forward, fm_backward: embedding gather / scatter-add, blocks walked in
 * reverse, fused log-softmax CE fm_k_ce_bwd with a double-precision
 * normaliser and dlogits = (softmax - onehot) / n_valid, rows of ignored
 * targets zero, head not tied; layer 0 receives the v_first gradient of the
 * later layers).  Differs from the page: every sum over tokens (parameter and
 * embedding gradients, the loss) is done in a fixed order, so the step is
 * bitwise reproducible.  The GEMMs run on the matrix cores in the precision
 * cfg->gemm_dtype names (fp32, or bf16 operands with fp32 accumulation); the
 * WKV7 state, its accumulation and every elementwise step are fp32.
 * tokens, targets: [B][T] int32 device.  A token id outside [0, V) embeds as
 * a zero row (and receives no embedding gradient); a target outside [0, V)
 * is ignored, like the page's ignore_index: its row of dlogits is zero, it
 * adds nothing to the loss and is not counted in n_valid (loss 0 when no
 * target is valid).  loss: one fp32 device value (written).
 * side: NULL, or a wkv7_side on which the weight gradients of the head, the
 * channel-mixes and the time-mixes run (as in timemix_backward), joined back
 * to `stream` within every block.
 * Hybrid stack (cfg->n_attn > 0): the attention blocks (model->attn, their
 * gradients grads->attn) sit in fm_build's interleave; their core is
 * moba_forward / moba_backward with cfg->moba_chunk and cfg->moba_topk (at
 * most 64 chunks per sequence), the backward holding the selection fixed as
 * the page does; the RWKV-7 blocks keep their layer indices 0 .. n_layer-1
 * (layer 0 publishes v_first).
 */
int rwkv7_train_step(const rwkv7_config *cfg, const rwkv7_model *model,
                     rwkv7_model_grads *grads, int B, int T, const int *tokens,
                     const int *targets, float *loss, void *ws, size_t ws_bytes,
                     const wkv7_side *side, hipStream_t stream);

/* --------------------------------------------- online TBPTT training -- */

/* Optimiser of rwkv7_online_segment.  optimizer 0: SGD, p -= lr clip(g);
 * 1: Adam (b1 = 0.9, b2 = 0.999, eps = 1e-8), m = b1 m + (1 - b1) clip(g),
 * v = b2 v + (1 - b2) clip(g)^2, p -= lr (m / (1 - b1^step)) /
 * (sqrt(v / (1 - b2^step)) + eps), with step the index of this update (1 for
 * the first).  clip > 0 clamps every gradient element to [-clip, clip];
 * clip = 0 leaves them. */
typedef struct {
  int optimizer;
  float lr, clip;
  int step;
} rwkv7_optim;

size_t rwkv7_online_workspace_bytes(const rwkv7_config *cfg, int B, int S);

/*
 * One online training segment for B streams of S (token, target) steps
 * starting from the streams' live decode state.  Page: "infotheory
 * .../rwkvzip/rwkv7/model.rs", online_train_segment_tbptt (checkpointed
 * forward, reverse replay carrying the recurrent gradient, update, live-state
 * replay) and apply_full_gradients (SGD / Adam, AdamStep constants):
 *   1. loss and gradients of the mean next-token cross-entropy over the B*S
 *      steps, backpropagated through the segment and truncated at its start
 *      (the start state is an input); written into `grads`;
 *   2. every parameter updated in place (the weights the model's pointers
 *      address are written, though the struct declares them const) with the
 *      optimiser `opt`; Adam reads and writes the moment mirrors adam_m and
 *      adam_v (zero before the first update; NULL for SGD);
 *   3. the segment replayed from the start state with the updated weights;
 *      att_x_prev, att_state, ffn_x_prev (layout of rwkv7_decode_step) hold
 *      the start state on entry and the new live state on return.
 * The page replays its checkpointed chunks one at a time to bound memory;
 * the gradient is the same, and here the whole segment's activations live in
 * the workspace.  Token ids and targets as in rwkv7_train_step.
 * side: as in rwkv7_train_step.
 */
int rwkv7_online_segment(const rwkv7_config *cfg, const rwkv7_model *model,
                         rwkv7_model_grads *grads, rwkv7_model_grads *adam_m,
                         rwkv7_model_grads *adam_v, const rwkv7_optim *opt, int B, int S,
                         const int *tokens, const int *targets, float *att_x_prev,
                         float *att_state, float *ffn_x_prev, float *loss, void *ws,
                         size_t ws_bytes, const wkv7_side *side, hipStream_t stream);

/* -------------------------------------------------- GatedDeltaNet layer -- */

/* Geometry of one GatedDeltaNet layer: nk key heads of size dk, nv value
 * heads of size dv (nv a multiple of nk, at most 16 value heads per key
 * head, grouped-query sharing), kk causal convolution taps (1..8), RMSNorm
 * epsilon.  The HIP kernels take dk and dv in {64, 128}.
 * c_dim = 2 nk dk + nv dv projection channels (q | k | v). */
typedef struct {
  int nk, nv, dk, dv, kk;
  float rms_eps;
} gdn_shape;

/* Frozen fp32 weights: conv [c_dim][kk] (tap kk-1 multiplies the current
 * position), A_log [nv], dt_bias [nv], norm [dv]. */
typedef struct {
  const float *conv, *A_log, *dt_bias, *norm;
} gdn_weights;

/* Bytes of the activations gdn_forward keeps for gdn_backward. */
size_t gdn_cache_bytes(const gdn_shape *s, int B, int T);
/* Workspace bytes of gdn_backward (plus the cache when have_cache is 0). */
size_t gdn_backward_workspace_bytes(const gdn_shape *s, int B, int T, int have_cache);

/*
 * GatedDeltaNet forward over B independent windows of T positions, each from
 * a fresh (zero) state.  Page: "cortiq_engine/fcd_ops.rs", GatedDeltaNet
 * section (gdn_conv_fwd, gdn_group_fwd, gdn_seq_fwd):
 *   pre = causal depthwise conv(raw), cq = silu(pre)
 *   q^ = q / (sqrt(|q|^2 + 1e-6) sqrt(dk)), k^ = k / sqrt(|k|^2 + 1e-6)
 *   g = exp(-exp(A_log) softplus(a + dt_bias)) (softplus(x) = x above 20),
 *   beta = sigmoid(b); per value head, S [dk][dv] from zero:
 *     S = g S;  kv = S^T k^;  S = S + k^ (beta (v - kv))^T;  o = S^T q^
 *   out = o / sqrt(mean(o^2) + rms_eps) * norm * silu(z)   (norm before gate)
 * raw: [B][T][c_dim]; z, out: [B][T][nv][dv]; a, b: [B][T][nv]; all fp32.
 * cache: NULL, or gdn_cache_bytes() bytes that receive the activations the
 * backward reuses (with NULL the call needs ws of gdn_cache_bytes() bytes).
 */
int gdn_forward(const gdn_shape *s, const gdn_weights *W, int B, int T, const float *raw,
                const float *z, const float *a, const float *b, float *out, void *cache,
                void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Gradients of <dout, out> with respect to raw, z, a and b (every weight
 * frozen: the page's through-backward gdn_seq_bwd).  cache: the forward's
 * cache for the same inputs, or NULL (the forward is recomputed into ws).
 * draw [B][T][c_dim], dz [B][T][nv][dv], da, db [B][T][nv] (written).
 */
int gdn_backward(const gdn_shape *s, const gdn_weights *W, int B, int T, const float *raw,
                 const float *z, const float *a, const float *b, const float *dout,
                 const void *cache, float *draw, float *dz, float *da, float *db, void *ws,
                 size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------ MoBA sparse attention --
 * The attention core of the hybrid stack's attention blocks.  Page:
 * "Foundry/cuda_kernels/fullmodel.cu", fm_attn_core_fwd and the attention
 * part of fm_attn_bwd (the selection kernel itself is not on the page; the
 * reading below is MoBA's gating).  Per (batch, head), head size N = 64,
 * scale 1/8: keys form chunks of `chunk` positions; query t (chunk
 * cur = t / chunk) attends to its own chunk up to itself and to the
 * (topk - 1) earlier chunks with the highest q_t . mean(k over the chunk)
 * (ties: the lower chunk index); y_t = softmax over those keys of
 * q_t . k / 8, times v.  With topk >= the number of chunks this is causal
 * softmax attention.
 * q, k, v, y, dy, dq, dk, dv: [B][T][H][N] fp32 (16-byte aligned).
 * lse: [B][H][T] fp32, the row log-sum-exp; sel: [B][H][T] 64-bit masks of
 * the attended chunks (bit c: chunk c).  At most 64 chunks per sequence;
 * 1 <= topk <= 64.  ws: moba_workspace_bytes() bytes (both calls, the same
 * chunk and topk).  With chunks of 64 keys only the selected (query, chunk)
 * pairs are computed: per chunk the queries that selected it are gathered,
 * their per-chunk softmax partials merged per query; other chunk lengths
 * walk 64-query tiles over the 64-key tiles any of their queries selected.
 * Every output is written, summed in a fixed order (no atomics).
 */
size_t moba_workspace_bytes(int B, int T, int H, int N, int chunk, int topk);
int moba_forward(int B, int T, int H, int N, int chunk, int topk, const float *q, const float *k,
                 const float *v, float *y, float *lse, uint64_t *sel, void *ws, size_t ws_bytes,
                 hipStream_t stream);
/* Gradients of <dy, y> with the selection sel held fixed (as the page's
 * backward does): needs the forward's y, lse and sel for the same q, k, v. */
int moba_backward(int B, int T, int H, int N, int chunk, int topk, const float *q, const float *k,
                  const float *v, const float *y, const float *lse, const uint64_t *sel,
                  const float *dy, float *dq, float *dk, float *dv, void *ws, size_t ws_bytes,
                  hipStream_t stream);

/* ------------------------------------------------------------- helpers -- */

/*
 * fp32 GEMM on the matrix cores: C = op(A) op(B) + beta C, row-major, where
 * op(A) is A [M][K] (lda) or, with transA, A^T for A stored [K][M]; op(B) is
 * B [K][N] (ldb) or, with transB, B^T for B stored [N][K].  This is the
 * contraction behind every projection and LoRA product of the time-mix
 * block ("Foundry/cuda_kernels/timemix.cu", rm_gemm: all matmuls as SGEMM over
 * the [B*T, *] token batch).  The dimensions read contiguously (K of A, N of
 * B, M of a transposed A, K of a transposed B) must be multiples of 4 and the
 * pointers 16-byte aligned.  No split-K (the time-mix backward splits its
 * weight gradients internally).
 */
int wkv7_gemm_f32(int transA, int transB, int M, int N, int K, const float *A, int lda,
                  const float *B, int ldb, float *C, int ldc, float beta, hipStream_t stream);

/*
 * Same contraction, layouts, requirements and errors as wkv7_gemm_f32, with
 * the operands rounded to bf16 (round to nearest even) and the products
 * accumulated in fp32 on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16 for
 * whole 256-row tiles, v_mfma_f32_16x16x32_bf16 otherwise).  A, B and C stay
 * fp32 in memory.  C must not overlap A, B or ws.  This is the bf16-GEMM
 * precision the full training-step configuration names for the projections;
 * the pages' own GEMMs are fp32 SGEMM.
 *
 * ws (optional, 256-byte aligned, ws_bytes >= the query when not NULL):
 * with it, a product on whole 256 x 128 tiles with K a multiple of 64 and
 * A not transposed first rounds A and B once into ws as bf16, stored
 * k-contiguous, and the matrix cores read those copies with no conversion in
 * the loop; without it (NULL) the operands are rounded as they are read from
 * LDS.  Both give the same bits.  The query returns 0 for shapes that do
 * not use it.  ENOSPC when ws is given and smaller than the query.
 */
size_t wkv7_gemm_bf16_workspace_bytes(int transA, int transB, int M, int N, int K);
int wkv7_gemm_bf16(int transA, int transB, int M, int N, int K, const float *A, int lda,
                   const float *B, int ldb, float *C, int ldc, float beta, void *ws,
                   size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* WKV7_H */
