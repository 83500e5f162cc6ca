"""RWKV-7 stack oracle: LayerNorm, channel-mix, embedding/head, decode step.

TEST INFRASTRUCTURE ONLY (see the package header).  numpy f64.

Block structure follows the block forward of "Foundry/cuda_kernels/
fullmodel.cu" (fm_rwkv_fwd: h1 = LN1(x); x1 = x + TM(h1); h2 = LN2(x1);
out = x1 + CM(h2)) and its whole-model forward (fm_forward: x0 = emb[token],
blocks, ln_out, logits = h @ head, head not tied to the embedding).  The
channel-mix is that page's fm_cm_fwd (shift, sh @ Wk, relu^2, @ Wv).  The
streaming-decode state and the layer-0 pre-norm follow "infotheory
.../rwkv7/model.rs" (LayerState: att_x_prev, att_state, ffn_x_prev;
BlockWeights.pre_norm on layer 0; Config: LayerNorm eps 1e-5).  In decode the
token-shift source of each mix is the previous token's LN output, which is
exactly what the sequence forward shifts.

A model is a dict:
  emb [V][C], head [C][V], ln_out_w/b [C], ln0_w/b [C] (or None),
  blocks: list of dicts with ln1_w/b, ln2_w/b [C], tm (time-mix params, see
  oracle.timemix), cm_mu_k [C], cm_Wk [C][F], cm_Wv [F][C]
and cfg = dict(C, H, F, V, n_layer).
"""
import numpy as np

from . import timemix as tm

LN_EPS = 1e-5


def layernorm(x, w, b, eps=LN_EPS):
    """(x - mean) / sqrt(var + eps) * w + b over the last axis (biased variance)."""
    x = np.asarray(x, np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * w + b


def channel_mix(mu_k, Wk, Wv, x, x_prev=None):
    """sh = x + (shift(x) - x) mu_k;  out = relu(sh @ Wk)^2 @ Wv."""
    x = np.asarray(x, np.float64)
    B, T, C = x.shape
    first = np.zeros((B, 1, C)) if x_prev is None else np.asarray(x_prev, np.float64)[:, None, :]
    prev = np.concatenate([first, x[:, :-1]], axis=1)
    sh = x + (prev - x) * mu_k
    ka = np.maximum(sh @ Wk, 0.0) ** 2
    return ka @ Wv


def _f64(m):
    out = {}
    for k, v in m.items():
        if k == "blocks":
            out[k] = [_f64(b) for b in v]
        elif k == "tm":
            out[k] = {kk: np.asarray(vv, np.float64) for kk, vv in v.items()}
        else:
            out[k] = None if v is None else np.asarray(v, np.float64)
    return out


def init_state(cfg, B):
    C, H, L = cfg["C"], cfg["H"], cfg["n_layer"]
    N = C // H
    return dict(att_x_prev=np.zeros((L, B, C)), att_state=np.zeros((L, B, H, N, N)),
                ffn_x_prev=np.zeros((L, B, C)))


def forward(model, cfg, tokens, state=None):
    """Logits [B][T][V] for int token ids [B][T], from `state` (None = zeros).

    Returns (logits, new_state).  Every layer carries its time-mix token shift
    (att_x_prev), its WKV state (att_state) and its channel-mix shift
    (ffn_x_prev) from one call to the next.
    """
    m = _f64(model)
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    H = cfg["H"]
    st = init_state(cfg, B) if state is None else {k: np.array(v, np.float64) for k, v in state.items()}
    x = m["emb"][tokens]
    if m.get("ln0_w") is not None:
        x = layernorm(x, m["ln0_w"], m["ln0_b"])
    v_first = None
    for l, bp in enumerate(m["blocks"]):
        h1 = layernorm(x, bp["ln1_w"], bp["ln1_b"])
        out, c = tm.forward(bp["tm"], h1, H, l, x_prev=st["att_x_prev"][l], v_first=v_first,
                            s0=st["att_state"][l])
        if l == 0:
            v_first = c["v_first"]
        st["att_x_prev"][l] = h1[:, -1]
        st["att_state"][l] = c["sT"]
        x = x + out
        h2 = layernorm(x, bp["ln2_w"], bp["ln2_b"])
        x = x + channel_mix(bp["cm_mu_k"], bp["cm_Wk"], bp["cm_Wv"], h2, x_prev=st["ffn_x_prev"][l])
        st["ffn_x_prev"][l] = h2[:, -1]
    h = layernorm(x, m["ln_out_w"], m["ln_out_b"])
    return h @ m["head"], st


def decode_step(model, cfg, tokens, state):
    """One streaming token per stream: tokens [B] -> logits [B][V], new state."""
    logits, st = forward(model, cfg, np.asarray(tokens)[:, None], state)
    return logits[:, 0], st
