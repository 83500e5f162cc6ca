"""Seeded synthetic inputs for the WKV7 / time-mix workloads.

This module only draws random numbers and casts them; both the HIP path and
the CPU oracle consume what it returns, and neither is imported here.

Every tensor gets its own PCG64 stream keyed by (seed, tensor name), so adding
a tensor never changes the others.  Floating point draws are made in f64 and
rounded once to the storage type (fp32, or bf16 by round-to-nearest-even of
the fp32 value).

Input recipes (WKV7 alone):
  r, k, v ~ N(0, 1);  w = exp(-0.606531 * sigmoid(u)), u ~ N(0, 1)
  kk = (k * k_k) / |k * k_k| per head, k_k ~ U(0.5, 1.5) per channel
  a = -kk;  b = kk * sigmoid(z), z ~ N(0, 1);  dy ~ N(0, 1)
This reproduces the value distribution the time-mix block feeds the WKV7
recurrence (decay in (0.545, 1), a rank-1 removal along a unit key).

Weights for the time-mix block and the stack (random init, std 0.02):
  every matrix ~ N(0, 0.02^2); mu_* = 0.5 + U(-0.02, 0.02); k_k = k_a = r_k = 1;
  norm weights 1, biases 0; w0 = a0 = v0 = 0.  The "perturbed" variant adds
  N(0, 0.1^2) to every per-channel vector so that no path is degenerate.
"""
import zlib

import numpy as np

DECAY_COEFF = 0.606531


def rng(seed: int, name: str) -> np.random.Generator:
    """Independent PCG64 stream for tensor `name` under `seed`."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), zlib.crc32(name.encode())])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 array holding exactly the bf16-rounded values of x."""
    return bf16_bits_to_f32(to_bf16_bits(x))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def wkv7_inputs(B, T, H, N, seed=0, bf16=False, with_state=False):
    """r, w, k, v, a, b, dy as fp32 [B][T][H][N] arrays (bf16-rounded if bf16).

    with_state adds s0 and dsT ~ N(0, 1) [B][H][N][N] (fp32).
    """
    shp = (B, T, H, N)
    r = rng(seed, "r").standard_normal(shp)
    k = rng(seed, "k").standard_normal(shp)
    v = rng(seed, "v").standard_normal(shp)
    u = rng(seed, "u").standard_normal(shp)
    w = np.exp(-DECAY_COEFF * _sigmoid(u))
    k_k = rng(seed, "k_k").uniform(0.5, 1.5, size=(H, N))
    kt = k * k_k
    kk = kt / np.sqrt(np.sum(kt * kt, axis=-1, keepdims=True))
    z = rng(seed, "z").standard_normal(shp)
    a = -kk
    b = kk * _sigmoid(z)
    dy = rng(seed, "dy").standard_normal(shp)
    out = dict(r=r, w=w, k=k, v=v, a=a, b=b, dy=dy)
    if with_state:
        out["s0"] = rng(seed, "s0").standard_normal((B, H, N, N))
        out["dsT"] = rng(seed, "dsT").standard_normal((B, H, N, N))
    for name in list(out):
        f = out[name].astype(np.float32)
        if bf16 and name in ("r", "w", "k", "v", "a", "b", "dy"):
            f = round_bf16(f)
        out[name] = f
    return out


def timemix_params(C, H, Dw, Da, Dv, Dg, layer_id, seed=0, perturbed=False, std=0.02):
    """fp32 time-mix weights, row-major [in][out]; v0/V1/V2 only for layer > 0."""
    def mat(name, shape):
        return (std * rng(seed, name).standard_normal(shape)).astype(np.float32)

    p = {}
    for c in ("r", "w", "k", "v", "a", "g"):
        p["mu_" + c] = 0.5 + rng(seed, "mu_" + c).uniform(-0.02, 0.02, size=C)
    for nm in ("Wr", "Wk", "Wv", "Wo"):
        p[nm] = mat(nm, (C, C))
    p["W1"], p["W2"] = mat("W1", (C, Dw)), mat("W2", (Dw, C))
    p["A1"], p["A2"] = mat("A1", (C, Da)), mat("A2", (Da, C))
    p["G1"], p["G2"] = mat("G1", (C, Dg)), mat("G2", (Dg, C))
    p["w0"] = np.zeros(C)
    p["a0"] = np.zeros(C)
    p["k_k"] = np.ones(C)
    p["k_a"] = np.ones(C)
    p["r_k"] = np.ones(C)
    p["ln_w"] = np.ones(C)
    p["ln_b"] = np.zeros(C)
    vec = ["mu_r", "mu_w", "mu_k", "mu_v", "mu_a", "mu_g", "w0", "a0", "k_k", "k_a", "r_k",
           "ln_w", "ln_b"]
    if layer_id > 0:
        p["V1"], p["V2"] = mat("V1", (C, Dv)), mat("V2", (Dv, C))
        p["v0"] = np.zeros(C)
        vec.append("v0")
    if perturbed:
        for nm in vec:
            p[nm] = p[nm] + 0.1 * rng(seed, "perturb_" + nm).standard_normal(C)
    return {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in p.items()}


def timemix_inputs(B, T, C, seed=0, with_state=False, H=None):
    """x, v_first, dout ~ N(0, 1) [B][T][C]; x_prev [B][C]; optional s0/dsT."""
    out = dict(
        x=rng(seed, "x").standard_normal((B, T, C)),
        v_first=rng(seed, "v_first").standard_normal((B, T, C)),
        dout=rng(seed, "dout").standard_normal((B, T, C)),
        x_prev=rng(seed, "x_prev").standard_normal((B, C)),
    )
    if with_state:
        N = C // H
        out["s0"] = rng(seed, "s0").standard_normal((B, H, N, N))
        out["dsT"] = rng(seed, "dsT").standard_normal((B, H, N, N))
    return {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in out.items()}


def stack_model(C, H, F, V, n_layer, ranks, seed=0, use_ln0=True, perturbed=False, std=0.02):
    """Random-init RWKV-7 stack (fp32): embedding, blocks, ln_out, head.

    ranks = (Dw, Da, Dv, Dg).  LayerNorm weights 1 / biases 0 (perturbed:
    1 + N(0, 0.1^2) / N(0, 0.1^2)); channel-mix mu_k = 0.5 + U(-0.02, 0.02).
    """
    def mat(name, shape):
        return (std * rng(seed, name).standard_normal(shape)).astype(np.float32)

    def ln(name):
        w, b = np.ones(C), np.zeros(C)
        if perturbed:
            w = w + 0.1 * rng(seed, name + "_w").standard_normal(C)
            b = b + 0.1 * rng(seed, name + "_b").standard_normal(C)
        return w.astype(np.float32), b.astype(np.float32)

    m = {"emb": mat("emb", (V, C)), "head": mat("head", (C, V))}
    m["ln_out_w"], m["ln_out_b"] = ln("ln_out")
    if use_ln0:
        m["ln0_w"], m["ln0_b"] = ln("ln0")
    else:
        m["ln0_w"] = m["ln0_b"] = None
    blocks = []
    for l in range(n_layer):
        bp = {}
        bp["ln1_w"], bp["ln1_b"] = ln(f"ln1_{l}")
        bp["ln2_w"], bp["ln2_b"] = ln(f"ln2_{l}")
        bp["tm"] = timemix_params(C, H, *ranks, layer_id=l, seed=seed * 1000 + l + 1,
                                  perturbed=perturbed, std=std)
        bp["cm_mu_k"] = (0.5 + rng(seed, f"cm_mu_{l}").uniform(-0.02, 0.02, size=C)).astype(np.float32)
        bp["cm_Wk"] = mat(f"cm_Wk_{l}", (C, F))
        bp["cm_Wv"] = mat(f"cm_Wv_{l}", (F, C))
        blocks.append(bp)
    m["blocks"] = blocks
    return m


def attn_blocks(C, F, n_attn, seed=0, perturbed=False, std=0.02):
    """Random-init attention blocks of a hybrid stack (fp32): LayerNorms as
    stack_model, Wq, Wk, Wv, Wo [C][C] and channel-mix Wk [C][F], Wv [F][C]
    ~ N(0, std^2), mu_k = 0.5 + U(-0.02, 0.02)."""
    def mat(name, shape):
        return (std * rng(seed, name).standard_normal(shape)).astype(np.float32)

    def ln(name):
        w, b = np.ones(C), np.zeros(C)
        if perturbed:
            w = w + 0.1 * rng(seed, name + "_w").standard_normal(C)
            b = b + 0.1 * rng(seed, name + "_b").standard_normal(C)
        return w.astype(np.float32), b.astype(np.float32)

    out = []
    for a in range(n_attn):
        ab = {}
        ab["ln1_w"], ab["ln1_b"] = ln(f"attn_ln1_{a}")
        ab["ln2_w"], ab["ln2_b"] = ln(f"attn_ln2_{a}")
        for w in ("Wq", "Wk", "Wv", "Wo"):
            ab[w] = mat(f"attn_{w}_{a}", (C, C))
        ab["cm_mu_k"] = (0.5 + rng(seed, f"attn_cm_mu_{a}").uniform(-0.02, 0.02, size=C)).astype(np.float32)
        ab["cm_Wk"] = mat(f"attn_cm_Wk_{a}", (C, F))
        ab["cm_Wv"] = mat(f"attn_cm_Wv_{a}", (F, C))
        out.append(ab)
    return out


def token_ids(B, T, V, seed=0, name="tokens"):
    """Uniform int32 token ids [B][T] in [0, V)."""
    return rng(seed, name).integers(0, V, size=(B, T)).astype(np.int32)


def gdn_config(nk, nv, dk, dv, kk=4, seed=0, rms_eps=1e-6):
    """Frozen GatedDeltaNet weights: conv taps ~ N(0, 1/kk) [c_dim][kk],
    A_log ~ U(-2, 1) (decay rates e^A_log in (0.14, 2.7)), dt_bias ~ N(0, 0.5^2),
    norm ~ 1 + N(0, 0.1^2) [dv]."""
    c_dim = 2 * nk * dk + nv * dv
    return dict(nk=nk, nv=nv, dk=dk, dv=dv, kk=kk, rms_eps=rms_eps,
                conv=(rng(seed, "gdn_conv").standard_normal((c_dim, kk)) / np.sqrt(kk)).astype(np.float32),
                A_log=rng(seed, "gdn_A_log").uniform(-2.0, 1.0, size=nv).astype(np.float32),
                dt_bias=(0.5 * rng(seed, "gdn_dt_bias").standard_normal(nv)).astype(np.float32),
                norm=(1.0 + 0.1 * rng(seed, "gdn_norm").standard_normal(dv)).astype(np.float32))


def gdn_inputs(B, T, cfg, seed=0):
    """raw [B][T][c_dim], z [B][T][nv dv], a, b [B][T][nv], dout [B][T][nv dv],
    all ~ N(0, 1) (fp32): the projections feeding one GatedDeltaNet layer."""
    nk, nv, dk, dv = cfg["nk"], cfg["nv"], cfg["dk"], cfg["dv"]
    c_dim = 2 * nk * dk + nv * dv
    out = dict(raw=rng(seed, "gdn_raw").standard_normal((B, T, c_dim)),
               z=rng(seed, "gdn_z").standard_normal((B, T, nv * dv)),
               a=rng(seed, "gdn_a").standard_normal((B, T, nv)),
               b=rng(seed, "gdn_b").standard_normal((B, T, nv)),
               dout=rng(seed, "gdn_dout").standard_normal((B, T, nv * dv)))
    return {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in out.items()}
