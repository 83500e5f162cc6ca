"""RWKV-7 time-mix block oracle: forward and hand-derived backward, numpy f64.

TEST INFRASTRUCTURE ONLY (see the package header).

Forward order and ops follow "Foundry/cuda_kernels/timemix.cu" (forward driver
tm_fwd_device and its elementwise kernels k_tokenshift ... k_mul); the LoRA
formulas follow the AttentionWeights comments of "infotheory
.../rwkv7/model.rs".  Local backward formulas follow the backward kernels of
the same timemix.cu page (k_split ... k_tokenshift_bwd) and its backward
driver's phase order; every one is the chain rule of the forward line it
undoes.

Weights are row-major [in][out] (y = x @ W), as on the timemix.cu page.
Token tensors are [B][T][C] with channel c = h*N + n.

Parameter names (dict keys):
  mu_r mu_w mu_k mu_v mu_a mu_g   [C]     token-shift lerp factors
  Wr Wk Wv Wo                     [C][C]
  w0 [C], W1 [C][Dw], W2 [Dw][C]          decay LoRA
  a0 [C], A1 [C][Da], A2 [Da][C]          in-context learning-rate LoRA
  v0 [C], V1 [C][Dv], V2 [Dv][C]          value-residual LoRA (layer > 0)
  G1 [C][Dg], G2 [Dg][C]                  gate LoRA
  k_k k_a r_k ln_w ln_b           [C]
"""
import numpy as np

from . import wkv7
from .precision import mm

# Decay coefficient exp(-0.606531 * sigmoid(.)) as written on the timemix.cu
# page (RWDECAY_COEFF); the model.rs page uses 1/sqrt(e), 3.4e-7 away.
DECAY = 0.606531
GN_EPS = 64e-5   # group-norm epsilon (timemix.cu k_groupnorm; model.rs Config)
L2_EPS = 1e-12   # key l2-norm epsilon, added to the norm (timemix.cu k_l2norm)

MIX = ("r", "w", "k", "v", "a", "g")


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _f64(p):
    return {k: (None if v is None else np.asarray(v, dtype=np.float64)) for k, v in p.items()}


def _prev(x, x_prev):
    """Token-shift source: x[t-1], with x_prev (or 0) at t = 0."""
    B, T, C = x.shape
    first = np.zeros((B, 1, C)) if x_prev is None else np.asarray(x_prev, np.float64)[:, None, :]
    return np.concatenate([first, x[:, :-1, :]], axis=1)


def forward(p, x, H, layer_id, x_prev=None, v_first=None, s0=None, gemm="f64"):
    """Time-mix forward.  Returns (out [B][T][C], cache).

    gemm: operand precision of the projections and LoRA products ("f64" or
    "bf16", see oracle.precision); the backward of this cache uses the same.

    cache holds every intermediate (f64) plus 'v_first' (the published value
    for layer 0, the input otherwise) and 'sT' (final WKV state).
    """
    p = _f64(p)
    x = np.asarray(x, np.float64)
    B, T, C = x.shape
    N = C // H
    assert H * N == C
    prev = _prev(x, x_prev)
    d = prev - x
    xs = {c: x + d * p["mu_" + c] for c in MIX}                      # k_tokenshift

    r = mm(xs["r"], p["Wr"], gemm)
    k = mm(xs["k"], p["Wk"], gemm)
    v = mm(xs["v"], p["Wv"], gemm)
    lw = mm(xs["w"], p["W1"], gemm)
    tw = np.tanh(lw)                                                 # k_tanh
    ow = mm(tw, p["W2"], gemm)
    sigw = sigmoid(p["w0"] + ow)                                     # k_decay
    w = np.exp(-DECAY * sigw)
    la = mm(xs["a"], p["A1"], gemm)
    a = sigmoid(p["a0"] + mm(la, p["A2"], gemm))                     # k_bias_sigmoid
    lg = mm(xs["g"], p["G1"], gemm)
    sg = sigmoid(lg)                                                 # k_sigmoid
    g = mm(sg, p["G2"], gemm)

    tk = (k * p["k_k"]).reshape(B, T, H, N)                          # k_tk
    nrm = np.sqrt(np.sum(tk * tk, axis=-1, keepdims=True))
    kk = tk / (nrm + L2_EPS)                                         # k_l2norm
    kmod = k * (1.0 + (a - 1.0) * p["k_a"])                          # k_keymod

    if layer_id == 0:                                                # k_vres0
        vmod = v
        vf = v
        lv = nu = None
    else:                                                            # k_vres
        vf = np.asarray(v_first, np.float64)
        lv = mm(xs["v"], p["V1"], gemm)
        nu = sigmoid(p["v0"] + mm(lv, p["V2"], gemm))
        vmod = v + (vf - v) * nu

    kk_c = kk.reshape(B, T, C)
    A = -kk_c                                                        # k_composites
    Bv = kk_c * a
    hv = lambda z: z.reshape(B, T, H, N)
    y, sT = wkv7.forward(hv(r), hv(w), hv(kmod), hv(vmod), hv(A), hv(Bv), s0=s0)

    mean = y.mean(axis=-1, keepdims=True)                            # k_groupnorm
    var = ((y - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + GN_EPS)
    nhat = (y - mean) * rstd
    ygn = nhat.reshape(B, T, C) * p["ln_w"] + p["ln_b"]
    alpha = np.sum(hv(r) * hv(kmod) * p["r_k"].reshape(H, N), axis=-1)   # k_bonus
    yb = ygn + (alpha[..., None] * hv(vmod)).reshape(B, T, C)
    tg = yb * g                                                      # k_mul
    out = mm(tg, p["Wo"], gemm)

    cache = dict(x=x, prev=prev, xs=xs, r=r, k=k, v=v, lw=lw, tw=tw, sigw=sigw, w=w,
                 la=la, a=a, sg=sg, g=g, tk=tk, nrm=nrm, kk=kk, kmod=kmod, vmod=vmod,
                 lv=lv, nu=nu, v_first=vf, A=A, Bv=Bv, y=y, sT=sT, nhat=nhat, rstd=rstd,
                 alpha=alpha, yb=yb, tg=tg, s0=s0, H=H, N=N, layer_id=layer_id, gemm=gemm)
    return out, cache


def _colsum(z):
    """Sum over every axis but the last (a per-channel parameter gradient)."""
    return z.reshape(-1, z.shape[-1]).sum(axis=0)


def _wgrad(xin, dout, gemm):
    """dW = x^T dy over all tokens, for y = x W."""
    return mm(xin.reshape(-1, xin.shape[-1]).T, dout.reshape(-1, dout.shape[-1]), gemm)


def backward(p, cache, dout, dsT=None, dv_first_in=None):
    """Gradients of L = <dout, out> + <dsT, S_T> for the forward that made cache.

    dv_first_in (layer 0 only): dL/dv_first accumulated by later layers; it
    flows into v because layer 0 publishes v_first = v.

    Returns (grads, dx, dx_prev, dv_first_out, ds0); grads has one entry per
    parameter (v0/V1/V2 only for layer > 0); dv_first_out is None on layer 0.
    """
    p = _f64(p)
    c = cache
    gemm = c.get("gemm", "f64")
    B, T, C = c["x"].shape
    H, N, L = c["H"], c["N"], c["layer_id"]
    hv = lambda z: z.reshape(B, T, H, N)
    dout = np.asarray(dout, np.float64)
    G = {}

    # out = tg @ Wo
    dtg = mm(dout, p["Wo"].T, gemm)
    G["Wo"] = _wgrad(c["tg"], dout, gemm)
    # tg = yb * g                                                     (k_split)
    dyb = dtg * c["g"]
    dg = dtg * c["yb"]
    # yb = ygn + alpha * vmod; alpha = sum_n r kmod r_k                (k_bonus_bwd)
    dalpha = np.sum(hv(dyb) * hv(c["vmod"]), axis=-1)
    dvmod = (hv(dyb) * c["alpha"][..., None]).reshape(B, T, C)
    rk = p["r_k"].reshape(H, N)
    dr = (dalpha[..., None] * hv(c["kmod"]) * rk).reshape(B, T, C)
    dkmod = (dalpha[..., None] * hv(c["r"]) * rk).reshape(B, T, C)
    G["r_k"] = _colsum((dalpha[..., None] * hv(c["r"]) * hv(c["kmod"])).reshape(B, T, C))
    # ygn = nhat * ln_w + ln_b; nhat = (y - mean) * rstd               (k_groupnorm_bwd)
    nhat = c["nhat"]
    G["ln_w"] = _colsum(dyb * nhat.reshape(B, T, C))
    G["ln_b"] = _colsum(dyb)
    dn = hv(dyb) * p["ln_w"].reshape(H, N)
    dy_wkv = c["rstd"] * (dn - dn.mean(axis=-1, keepdims=True)
                          - nhat * (dn * nhat).mean(axis=-1, keepdims=True))

    # WKV7
    gw = wkv7.backward(hv(c["r"]), hv(c["w"]), hv(c["kmod"]), hv(c["vmod"]), hv(c["A"]),
                       hv(c["Bv"]), dy_wkv, s0=c["s0"], dsT=dsT)
    flat = lambda z: z.reshape(B, T, C)
    dr = dr + flat(gw["dr"])                                         # k_p4_seed
    dkmod = dkmod + flat(gw["dk"])
    dvmod = dvmod + flat(gw["dv"])
    dw = flat(gw["dw"])
    dA = flat(gw["da"])
    dB = flat(gw["db"])

    a, k, kk = c["a"], c["k"], c["kk"].reshape(B, T, C)
    # A = -kk; Bv = kk * a; kmod = k (1 + (a - 1) k_a)                 (k_comp_keymod)
    dkk = -dA + dB * a
    da = dB * kk + dkmod * k * p["k_a"]
    dk = dkmod * (1.0 + (a - 1.0) * p["k_a"])
    G["k_a"] = _colsum(dkmod * k * (a - 1.0))
    # kk = tk / (|tk| + eps), per head                                 (k_l2norm_bwd)
    tk, nrm = c["tk"], c["nrm"]
    inv = 1.0 / (nrm + L2_EPS)
    dkk_h = hv(dkk)
    gdot = np.sum(dkk_h * tk, axis=-1, keepdims=True)
    safe = np.where(nrm > 0, nrm, 1.0)
    dtk = inv * dkk_h - np.where(nrm > 0, inv * inv * gdot * tk / safe, 0.0)
    dtk = dtk.reshape(B, T, C)
    # tk = k * k_k                                                     (k_tk_bwd)
    dk = dk + dtk * p["k_k"]
    G["k_k"] = _colsum(dtk * k)

    # value residual                                                   (k_vvec0 / k_vvec1)
    dxv_extra = 0.0
    dv_first_out = None
    if L == 0:
        dv = dvmod if dv_first_in is None else dvmod + np.asarray(dv_first_in, np.float64)
    else:
        nu, vf, v = c["nu"], c["v_first"], c["v"]
        dv = dvmod * (1.0 - nu)
        dv_first_out = dvmod * nu
        dpre = dvmod * (vf - v) * nu * (1.0 - nu)
        G["v0"] = _colsum(dpre)
        dlv = mm(dpre, p["V2"].T, gemm)
        G["V2"] = _wgrad(c["lv"], dpre, gemm)
        dxv_extra = mm(dlv, p["V1"].T, gemm)
        G["V1"] = _wgrad(c["xs"]["v"], dlv, gemm)

    # a = sigmoid(a0 + (xa @ A1) @ A2)                                 (k_avec_bwd)
    dpre_a = da * a * (1.0 - a)
    G["a0"] = _colsum(dpre_a)
    dla = mm(dpre_a, p["A2"].T, gemm)
    G["A2"] = _wgrad(c["la"], dpre_a, gemm)
    dxa = mm(dla, p["A1"].T, gemm)
    G["A1"] = _wgrad(c["xs"]["a"], dla, gemm)

    # w = exp(-DECAY * sigmoid(w0 + tanh(xw @ W1) @ W2))               (k_wdecay_bwd)
    sigw = c["sigw"]
    dpre_w = dw * c["w"] * (-DECAY) * sigw * (1.0 - sigw)
    G["w0"] = _colsum(dpre_w)
    dtw = mm(dpre_w, p["W2"].T, gemm)
    G["W2"] = _wgrad(c["tw"], dpre_w, gemm)
    dlw = dtw * (1.0 - c["tw"] ** 2)                                 # k_tanhderiv
    dxw = mm(dlw, p["W1"].T, gemm)
    G["W1"] = _wgrad(c["xs"]["w"], dlw, gemm)

    # g = sigmoid(xg @ G1) @ G2
    dsg = mm(dg, p["G2"].T, gemm)
    G["G2"] = _wgrad(c["sg"], dg, gemm)
    dlg = dsg * c["sg"] * (1.0 - c["sg"])                            # k_sigderiv
    dxg = mm(dlg, p["G1"].T, gemm)
    G["G1"] = _wgrad(c["xs"]["g"], dlg, gemm)

    # r, k, v projections
    dxr = mm(dr, p["Wr"].T, gemm)
    G["Wr"] = _wgrad(c["xs"]["r"], dr, gemm)
    dxk = mm(dk, p["Wk"].T, gemm)
    G["Wk"] = _wgrad(c["xs"]["k"], dk, gemm)
    dxv = mm(dv, p["Wv"].T, gemm) + dxv_extra
    G["Wv"] = _wgrad(c["xs"]["v"], dv, gemm)

    # token shift: xs_c = x (1 - mu_c) + prev mu_c                     (k_tokenshift_bwd)
    dxs = dict(r=dxr, w=dxw, k=dxk, v=dxv, a=dxa, g=dxg)
    x, prev = c["x"], c["prev"]
    dx = np.zeros_like(x)
    dprev = np.zeros_like(x)
    for ch in MIX:
        mu = p["mu_" + ch]
        G["mu_" + ch] = _colsum(dxs[ch] * (prev - x))
        dx += dxs[ch] * (1.0 - mu)
        dprev += dxs[ch] * mu
    dx[:, :-1, :] += dprev[:, 1:, :]
    dx_prev = dprev[:, 0, :]
    return G, dx, dx_prev, dv_first_out, gw["ds0"]
