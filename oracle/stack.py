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
from .precision import mm

LN_EPS = 1e-5


def layernorm(x, w, b, eps=LN_EPS):
    """(x - mean) / sqrt(var + eps) * w + b over the last axis (biased variance)."""
    x = np.asarray(x, np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * w + b


def channel_mix(mu_k, Wk, Wv, x, x_prev=None, gemm="f64"):
    """sh = x + (shift(x) - x) mu_k;  out = relu(sh Wk)^2 Wv (products per `gemm`)."""
    x = np.asarray(x, np.float64)
    B, T, C = x.shape
    first = np.zeros((B, 1, C)) if x_prev is None else np.asarray(x_prev, np.float64)[:, None, :]
    prev = np.concatenate([first, x[:, :-1]], axis=1)
    sh = x + (prev - x) * mu_k
    ka = np.maximum(mm(sh, Wk, gemm), 0.0) ** 2
    return mm(ka, Wv, gemm)


def embed(emb, tokens):
    """Rows emb[id] for each id; an id outside [0, V) gives a zero row (the
    reading of an id the table does not hold)."""
    tokens = np.asarray(tokens)
    V = emb.shape[0]
    ok = (tokens >= 0) & (tokens < V)
    return np.where(ok[..., None], emb[np.where(ok, tokens, 0)], 0.0)


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
    x = embed(m["emb"], tokens)
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


# ------------------------------------------------------------ training step --
# Whole-model forward+backward for next-token cross-entropy, following the
# fullmodel page's fm_forward / fm_backward: per-token CE with the
# log-sum-exp, loss = mean over the tokens, dlogits = (softmax - onehot) / n
# (fm_k_ce_bwd), head and embedding gradients (fm_k_emb_bwd adds each token's
# gradient into its embedding row), and blocks walked in reverse; layer 0
# receives the v_first gradient accumulated over the later layers.

def layernorm_backward(x, w, dy, eps=LN_EPS):
    """Gradients of y = LN(x) * w + b: returns dx, dw, db (dw, db summed over rows)."""
    x = np.asarray(x, np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    nhat = (x - mean) * rstd
    dn = dy * w
    dx = rstd * (dn - dn.mean(axis=-1, keepdims=True) - nhat * (dn * nhat).mean(axis=-1, keepdims=True))
    C = x.shape[-1]
    return dx, (dy * nhat).reshape(-1, C).sum(0), dy.reshape(-1, C).sum(0)


def channel_mix_backward(mu_k, Wk, Wv, x, dout, x_prev=None, gemm="f64"):
    """Gradients of channel_mix: returns dx, dx_prev, dmu_k, dWk, dWv."""
    x = np.asarray(x, np.float64)
    B, T, C = x.shape
    first = np.zeros((B, 1, C)) if x_prev is None else np.asarray(x_prev, np.float64)[:, None, :]
    prev = np.concatenate([first, x[:, :-1]], axis=1)
    sh = x + (prev - x) * mu_k
    fk = mm(sh, Wk, gemm)
    ka = np.maximum(fk, 0.0) ** 2
    dka = mm(dout, Wv.T, gemm)
    dWv = mm(ka.reshape(-1, ka.shape[-1]).T, dout.reshape(-1, C), gemm)
    dfk = dka * 2.0 * np.maximum(fk, 0.0)
    dsh = mm(dfk, Wk.T, gemm)
    dWk = mm(sh.reshape(-1, C).T, dfk.reshape(-1, dfk.shape[-1]), gemm)
    dmu = (dsh * (prev - x)).reshape(-1, C).sum(0)
    dx = dsh * (1.0 - mu_k)
    dprev = dsh * mu_k
    dx[:, :-1] += dprev[:, 1:]
    return dx, dprev[:, 0], dmu, dWk, dWv


def cross_entropy(logits, targets):
    """Mean CE over the counted tokens and dlogits = (softmax - onehot) / n_valid.

    As the fullmodel page's fm_k_ce_bwd does for its ignore_index, a target
    outside [0, V) is ignored: its dlogits row is zero, it adds nothing to the
    loss and is not counted in n_valid (loss 0 when nothing is counted)."""
    z = np.asarray(logits, np.float64)
    targets = np.asarray(targets)
    V = z.shape[-1]
    ok = (targets >= 0) & (targets < V)
    n = int(ok.sum())
    m = z.max(axis=-1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True))
    ti = np.where(ok, targets, 0)[..., None]
    per = lse[..., 0] - np.take_along_axis(z, ti, axis=-1)[..., 0]
    loss = float(np.sum(np.where(ok, per, 0.0)) / n) if n else 0.0
    p = np.exp(z - lse)
    np.put_along_axis(p, ti, np.take_along_axis(p, ti, axis=-1) - 1.0, axis=-1)
    p = np.where(ok[..., None], p, 0.0)
    return loss, (p / n if n else p)


def train_step(model, cfg, tokens, targets, gemm="f64", state=None):
    """Loss and gradients of every parameter for one batch.

    Returns (loss, grads) with grads mirroring the model dict (blocks[l]['tm']
    holds the time-mix gradients).  gemm: operand precision of every
    projection, LoRA, channel-mix and head product ("f64" or "bf16", see
    oracle.precision).  state: None (zero initial state) or a streaming state
    (init_state layout) the batch starts from; the gradients stop at it
    (truncated backpropagation through time: the state is an input, not a
    function of the parameters).
    """
    m = _f64(model)
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    H = cfg["H"]
    st = None if state is None else {k: np.asarray(v, np.float64) for k, v in state.items()}
    xp_tm = lambda l: None if st is None else st["att_x_prev"][l]
    s0_tm = lambda l: None if st is None else st["att_state"][l]
    xp_cm = lambda l: None if st is None else st["ffn_x_prev"][l]
    x = embed(m["emb"], tokens)
    use_ln0 = m.get("ln0_w") is not None
    x_emb = x
    if use_ln0:
        x = layernorm(x, m["ln0_w"], m["ln0_b"])
    xs, caches = [x], []
    v_first = None
    for l, bp in enumerate(m["blocks"]):
        h1 = layernorm(x, bp["ln1_w"], bp["ln1_b"])
        out, c = tm.forward(bp["tm"], h1, H, l, x_prev=xp_tm(l), v_first=v_first, s0=s0_tm(l),
                            gemm=gemm)
        if l == 0:
            v_first = c["v_first"]
        x1 = x + out
        h2 = layernorm(x1, bp["ln2_w"], bp["ln2_b"])
        x = x1 + channel_mix(bp["cm_mu_k"], bp["cm_Wk"], bp["cm_Wv"], h2, x_prev=xp_cm(l),
                             gemm=gemm)
        caches.append(dict(h1=h1, c=c, x1=x1, h2=h2))
        xs.append(x)
    hN = layernorm(x, m["ln_out_w"], m["ln_out_b"])
    loss, dlog = cross_entropy(mm(hN, m["head"], gemm), targets)

    G = {"head": mm(hN.reshape(-1, hN.shape[-1]).T, dlog.reshape(-1, dlog.shape[-1]), gemm)}
    dx, G["ln_out_w"], G["ln_out_b"] = layernorm_backward(x, m["ln_out_w"], mm(dlog, m["head"].T, gemm))
    G["blocks"] = [None] * len(m["blocks"])
    dvf = np.zeros_like(x)
    for l in range(len(m["blocks"]) - 1, -1, -1):
        bp, cc = m["blocks"][l], caches[l]
        gb = {}
        dh2, _, gb["cm_mu_k"], gb["cm_Wk"], gb["cm_Wv"] = channel_mix_backward(
            bp["cm_mu_k"], bp["cm_Wk"], bp["cm_Wv"], cc["h2"], dx, x_prev=xp_cm(l), gemm=gemm)
        d1, gb["ln2_w"], gb["ln2_b"] = layernorm_backward(cc["x1"], bp["ln2_w"], dh2)
        dx1 = dx + d1
        gt, dh1, _, dvf_out, _ = tm.backward(bp["tm"], cc["c"], dx1,
                                             dv_first_in=dvf if l == 0 else None)
        if l > 0:
            dvf = dvf + dvf_out
        gb["tm"] = gt
        d0, gb["ln1_w"], gb["ln1_b"] = layernorm_backward(xs[l], bp["ln1_w"], dh1)
        dx = dx1 + d0
        G["blocks"][l] = gb
    if use_ln0:
        dx, G["ln0_w"], G["ln0_b"] = layernorm_backward(x_emb, m["ln0_w"], dx)
    demb = np.zeros_like(m["emb"])
    ids = tokens.reshape(-1)
    ok = (ids >= 0) & (ids < demb.shape[0])
    np.add.at(demb, ids[ok], dx.reshape(-1, dx.shape[-1])[ok])
    G["emb"] = demb
    return loss, G
