"""GatedDeltaNet layer oracle (through-gradients only): numpy f64.

TEST INFRASTRUCTURE ONLY (see the package header).

Follows the GatedDeltaNet section of "cortiq_engine/fcd_ops.rs" (the
through-backward of gdn_step: gdn_conv_fwd / gdn_conv_bwd, gdn_group_fwd /
gdn_group_bwd, gdn_seq_fwd / gdn_seq_bwd).  Per window of T positions from a
fresh state (zeros):

  1. Depthwise causal convolution + SiLU over the c_dim = 2 nk dk + nv dv
     projection channels: pre[t][c] = sum_j raw[t - (kk-1) + j][c] conv[c][j]
     (positions before 0 are zero), cq = silu(pre).
  2. Per v-head h (k-head ko = h / (nv / nk), grouped-query sharing):
       q = cq[t][ko dk : (ko+1) dk], k = cq[t][nk dk + ko dk : ...],
       v = cq[t][2 nk dk + h dv : ...];
       q^ = q / (sqrt(|q|^2 + 1e-6) sqrt(dk)),  k^ = k / sqrt(|k|^2 + 1e-6);
       g = exp(-exp(A_log[h]) softplus(a[t][h] + dt_bias[h])) (softplus(x) = x
       for x > 20), beta = sigmoid(b[t][h]);
       S <- g S;  kv = S^T k^;  S <- S + k^ (beta (v - kv))^T;  o = S^T q^
     with S [dk][dv] (S[i][j]: i the key index, j the value index).
  3. Gated per-head RMSNorm, norm before gate:
       out[t][h dv + j] = o[j] / sqrt(mean(o^2) + rms_eps) norm[j] silu(z[t][h dv + j]).

The backward returns the gradients of L = <dout, out> with respect to the
four inputs raw, z, a, b (every weight frozen, as on the page).

Shapes: raw [T][c_dim], z [T][nv dv], a and b [T][nv], dout [T][nv dv];
conv [c_dim][kk] (tap kk-1 multiplies the current position), A_log, dt_bias
[nv], norm [dv].
"""
import numpy as np

L2_EPS = 1e-6       # added to |q|^2 and |k|^2 before the square root
SOFTPLUS_CUT = 20.0  # softplus(x) = x above this argument


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _silu_grad(x):
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def _softplus(x):
    return np.where(x > SOFTPLUS_CUT, x, np.log1p(np.exp(np.minimum(x, SOFTPLUS_CUT))))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def conv_forward(raw, conv):
    """Causal depthwise convolution: pre [T][c_dim]."""
    raw = np.asarray(raw, np.float64)
    T, c = raw.shape
    kk = conv.shape[1]
    pre = np.zeros((T, c))
    for j in range(kk):
        shift = kk - 1 - j           # tap j reads position t - shift
        if shift >= T:
            continue
        pre[shift:] += raw[:T - shift] * conv[:, j]
    return pre


def _heads(cq, nk, nv, dk, dv):
    T = cq.shape[0]
    kd = nk * dk
    q = cq[:, :kd].reshape(T, nk, dk)
    k = cq[:, kd:2 * kd].reshape(T, nk, dk)
    v = cq[:, 2 * kd:].reshape(T, nv, dv)
    return q, k, v


def forward(raw, z, a, b, cfg):
    """out [T][nv dv] and a cache of the intermediates (f64).

    cfg: dict nk, nv, dk, dv, rms_eps and arrays conv, A_log, dt_bias, norm.
    """
    nk, nv, dk, dv = cfg["nk"], cfg["nv"], cfg["dk"], cfg["dv"]
    rep = nv // nk
    conv = np.asarray(cfg["conv"], np.float64)
    raw = np.asarray(raw, np.float64)
    z = np.asarray(z, np.float64)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    T = raw.shape[0]
    pre = conv_forward(raw, conv)
    cq = _silu(pre)
    q, k, v = _heads(cq, nk, nv, dk, dv)
    nq2 = np.sum(q * q, axis=-1) + L2_EPS                 # [T][nk]
    nk2 = np.sum(k * k, axis=-1) + L2_EPS
    invq = 1.0 / (np.sqrt(nq2) * np.sqrt(dk))
    invk = 1.0 / np.sqrt(nk2)
    qh = q * invq[..., None]
    kh = k * invk[..., None]
    A_log = np.asarray(cfg["A_log"], np.float64)
    dt_bias = np.asarray(cfg["dt_bias"], np.float64)
    arg = a + dt_bias                                      # [T][nv]
    g = np.exp(-np.exp(A_log) * _softplus(arg))
    beta = _sigmoid(b)
    S_hist = np.zeros((nv, T + 1, dk, dv))           # S_0 = 0 (fresh state)
    kv = np.zeros((T, nv, dv))
    o = np.zeros((T, nv, dv))
    for h in range(nv):
        ko = h // rep
        S = S_hist[h, 0].copy()
        for t in range(T):
            S = g[t, h] * S
            kv[t, h] = S.T @ kh[t, ko]
            S = S + np.outer(kh[t, ko], beta[t, h] * (v[t, h] - kv[t, h]))
            o[t, h] = S.T @ qh[t, ko]
            S_hist[h, t + 1] = S
    norm = np.asarray(cfg["norm"], np.float64)
    ms = np.mean(o * o, axis=-1) + cfg["rms_eps"]            # [T][nv]
    inv = 1.0 / np.sqrt(ms)
    zz = z.reshape(T, nv, dv)
    out = o * inv[..., None] * norm * _silu(zz)
    cache = dict(raw=raw, z=z, a=a, b=b, pre=pre, cq=cq, q=q, k=k, v=v, nq2=nq2, nk2=nk2,
                 invq=invq, invk=invk, qh=qh, kh=kh, arg=arg, g=g, beta=beta, S_hist=S_hist,
                 kv=kv, o=o, inv=inv, cfg=cfg)
    return out.reshape(T, nv * dv), cache


def backward(cache, dout):
    """Gradients of <dout, out>: dict draw, dz, da, db (through-gradients)."""
    c = cache
    cfg = c["cfg"]
    nk, nv, dk, dv = cfg["nk"], cfg["nv"], cfg["dk"], cfg["dv"]
    rep = nv // nk
    T = c["raw"].shape[0]
    norm = np.asarray(cfg["norm"], np.float64)
    dout = np.asarray(dout, np.float64).reshape(T, nv, dv)
    o, inv = c["o"], c["inv"]
    zz = c["z"].reshape(T, nv, dv)
    # gated RMSNorm: out = o inv w silu(z)
    weff = norm * _silu(zz)
    dz = (dout * o * inv[..., None] * norm * _silu_grad(zz)).reshape(T, nv * dv)
    sdot = np.sum(dout * weff * o, axis=-1)                  # [T][nv]
    do = inv[..., None] * weff * dout - o * (sdot / dv * inv ** 3)[..., None]
    # recurrence, reverse
    qh, kh, v, kv, g, beta = c["qh"], c["kh"], c["v"], c["kv"], c["g"], c["beta"]
    dqh = np.zeros_like(qh)
    dkh = np.zeros_like(kh)
    dv_ = np.zeros_like(v)
    dg = np.zeros((T, nv))
    dbeta = np.zeros((T, nv))
    for h in range(nv):
        ko = h // rep
        dS = np.zeros((dk, dv))
        for t in range(T - 1, -1, -1):
            S_t = c["S_hist"][h, t + 1]
            S_prev = c["S_hist"][h, t]
            # o = S_t^T q^
            dS = dS + np.outer(qh[t, ko], do[t, h])
            dqh[t, ko] += S_t @ do[t, h]
            # S_t = S_pre + k^ u^T, u = beta (v - kv)
            u = beta[t, h] * (v[t, h] - kv[t, h])
            du = dS.T @ kh[t, ko]
            dkh[t, ko] += dS @ u
            dbeta[t, h] = du @ (v[t, h] - kv[t, h])
            dv_[t, h] = beta[t, h] * du
            dkv = -beta[t, h] * du
            # kv = S_pre^T k^ with S_pre = g S_prev
            dS_pre = dS + np.outer(kh[t, ko], dkv)
            dkh[t, ko] += (g[t, h] * S_prev) @ dkv
            dg[t, h] = np.sum(dS_pre * S_prev)
            dS = g[t, h] * dS_pre
    # gates: d softplus / d arg = sigmoid(arg) (the page uses it on both sides of
    # the cut, where it differs from 1 by at most sigmoid(-20) = 2e-9)
    A_log = np.asarray(cfg["A_log"], np.float64)
    sig = _sigmoid(c["arg"])
    da = dg * g * (-np.exp(A_log)) * sig
    db = dbeta * beta * (1.0 - beta)
    # l2 normalisations: q^ = q invq, invq = 1 / (sqrt(|q|^2 + eps) sqrt(dk))
    q, k = c["q"], c["k"]
    invq, invk, nq2, nk2 = c["invq"], c["invk"], c["nq2"], c["nk2"]
    qdot = np.sum(dqh * q, axis=-1)
    kdot = np.sum(dkh * k, axis=-1)
    dq = invq[..., None] * dqh - q * (qdot * invq / nq2)[..., None]
    dk = invk[..., None] * dkh - k * (kdot * invk / nk2)[..., None]
    dcq = np.concatenate([dq.reshape(T, -1), dk.reshape(T, -1), dv_.reshape(T, -1)], axis=1)
    # conv + SiLU
    dpre = dcq * _silu_grad(c["pre"])
    conv = np.asarray(cfg["conv"], np.float64)
    kk = conv.shape[1]
    draw = np.zeros_like(dpre)
    for j in range(kk):
        shift = kk - 1 - j
        if shift >= T:
            continue
        draw[:T - shift] += dpre[shift:] * conv[:, j]
    return dict(draw=draw, dz=dz, da=da, db=db)
