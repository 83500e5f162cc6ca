"""MoBA sparse attention and the hybrid RWKV-7 / attention stack: numpy f64.

TEST INFRASTRUCTURE ONLY (see the package header).

Follows "Foundry/cuda_kernels/fullmodel.cu": the attention block
(fm_attn_fwd / fm_attn_bwd: h1 = LN1(x); q, k, v = h1 Wq, h1 Wk, h1 Wv; y =
MoBA core; x1 = x + y Wo; h2 = LN2(x1); out = x1 + channel-mix(h2)), the MoBA
core (fm_attn_core_fwd: per head, softmax of scale q k^T over the keys the
selection allows, times v, scale = 1/sqrt(N); its backward with the
selection held fixed: dP = dy v^T, dv = P^T dy, dS = softmax backward of
(P, dP) times scale, dq = dS k, dk = dS^T q) and the block interleave of
fm_build (after every n_rwkv / n_attn RWKV-7 blocks one attention block,
then the remaining RWKV-7 blocks).

The selection kernel itself (moba_scores_softmax) is not on the page.  Its
reading here is the plainest one the rest supports, MoBA's gating:
  - keys form chunks of `chunk` consecutive positions;
  - a query at position t in chunk cur = t // chunk always attends to the
    keys of its own chunk up to itself (causal);
  - each earlier chunk c < cur is scored by q_t . mean(k over chunk c), and
    the top (topk - 1) scores are selected (ties: the lower chunk index), so
    that topk chunks are attended in all, the current one included;
  - chunks after the current one are never attended.
With topk >= the number of chunks this is plain causal softmax attention.
"""
import numpy as np

from . import stack
from . import timemix as tm
from .precision import mm


def block_order(n_rwkv, n_attn):
    """[("rwkv", i) | ("attn", a)] in stack order (fm_build's interleave)."""
    if n_attn == 0:
        return [("rwkv", i) for i in range(n_rwkv)]
    interval = n_rwkv // n_attn
    order = []
    for a in range(n_attn):
        order += [("rwkv", j) for j in range(a * interval, (a + 1) * interval)]
        order.append(("attn", a))
    order += [("rwkv", j) for j in range(n_attn * interval, n_rwkv)]
    return order


def select(q, k, chunk, topk):
    """Selected chunks sel[t][c] (bool) for one head: q, k [T][N]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    T = q.shape[0]
    nc = (T + chunk - 1) // chunk
    kbar = np.stack([k[c * chunk:(c + 1) * chunk].mean(axis=0) for c in range(nc)])
    sel = np.zeros((T, nc), dtype=bool)
    for t in range(T):
        cur = t // chunk
        sel[t, cur] = True
        if cur == 0 or topk <= 1:
            continue
        scores = kbar[:cur] @ q[t]
        ranked = sorted(range(cur), key=lambda c: (-scores[c], c))
        sel[t, ranked[:topk - 1]] = True
    return sel


def allowed(sel, chunk):
    """mask[t][tau]: key tau is attended by query t (selected chunk, causal)."""
    T = sel.shape[0]
    tau = np.arange(T)
    mask = sel[:, tau // chunk]
    return mask & (tau[None, :] <= np.arange(T)[:, None])


def core_forward(q, k, v, H, chunk, topk, sel=None):
    """MoBA core over [B][T][C] q, k, v (C = H N): y [B][T][C] and a cache
    (P, the key mask, the row log-sum-exp lse [B][H][T] and the selection).

    sel: None (select here), or the selection to use, bool [B][H][T][chunks]:
    the selection is a discrete decision taken on floating-point scores, so a
    comparison with another implementation checks the two selections on
    their own and then evaluates the attention for the same one."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, T, C = q.shape
    N = C // H
    nc = (T + chunk - 1) // chunk
    scale = 1.0 / np.sqrt(N)
    y = np.zeros_like(q)
    P = np.zeros((B, H, T, T))
    masks = np.zeros((B, H, T, T), dtype=bool)
    lse = np.zeros((B, H, T))
    sels = np.zeros((B, H, T, nc), dtype=bool)
    for b in range(B):
        for h in range(H):
            sl = slice(h * N, (h + 1) * N)
            qh, kh, vh = q[b, :, sl], k[b, :, sl], v[b, :, sl]
            sels[b, h] = select(qh, kh, chunk, topk) if sel is None else sel[b, h]
            mask = allowed(sels[b, h], chunk)
            s = np.where(mask, scale * (qh @ kh.T), -np.inf)
            mx = s.max(axis=1, keepdims=True)
            e = np.where(mask, np.exp(s - mx), 0.0)
            z = e.sum(axis=1, keepdims=True)
            p = e / z
            y[b, :, sl] = p @ vh
            P[b, h], masks[b, h] = p, mask
            lse[b, h] = (mx + np.log(z))[:, 0]
    return y, dict(q=q, k=k, v=v, P=P, mask=masks, lse=lse, sel=sels, H=H, scale=scale)


def chunk_scores(q, k, chunk):
    """Gating scores [T][chunks] of one head: q_t . mean(k over chunk c)
    (the selection ranks the earlier chunks by these)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    T = q.shape[0]
    nc = (T + chunk - 1) // chunk
    kbar = np.stack([k[c * chunk:(c + 1) * chunk].mean(axis=0) for c in range(nc)])
    return q @ kbar.T


def core_backward(cache, dy):
    """dq, dk, dv of <dy, y> with the selection held fixed."""
    q, k, v, P, H, scale = (cache[n] for n in ("q", "k", "v", "P", "H", "scale"))
    dy = np.asarray(dy, np.float64)
    B, T, C = q.shape
    N = C // H
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            sl = slice(h * N, (h + 1) * N)
            p, dyh = P[b, h], dy[b, :, sl]
            dv[b, :, sl] = p.T @ dyh
            dp = dyh @ v[b, :, sl].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True)) * scale
            dq[b, :, sl] = ds @ k[b, :, sl]
            dk[b, :, sl] = ds.T @ q[b, :, sl]
    return dq, dk, dv


def attn_block_forward(ab, x, H, chunk, topk, gemm="f64"):
    """One attention block: out [B][T][C] and its cache."""
    h1 = stack.layernorm(x, ab["ln1_w"], ab["ln1_b"])
    q, k, v = (mm(h1, ab[w], gemm) for w in ("Wq", "Wk", "Wv"))
    y, core = core_forward(q, k, v, H, chunk, topk)
    x1 = x + mm(y, ab["Wo"], gemm)
    h2 = stack.layernorm(x1, ab["ln2_w"], ab["ln2_b"])
    out = x1 + stack.channel_mix(ab["cm_mu_k"], ab["cm_Wk"], ab["cm_Wv"], h2, gemm=gemm)
    return out, dict(x=x, h1=h1, y=y, core=core, x1=x1, h2=h2)


def attn_block_backward(ab, c, dout, gemm="f64"):
    """dx and the block's parameter gradients from dout."""
    g = {}
    C = c["x"].shape[-1]
    dh2, _, g["cm_mu_k"], g["cm_Wk"], g["cm_Wv"] = stack.channel_mix_backward(
        ab["cm_mu_k"], ab["cm_Wk"], ab["cm_Wv"], c["h2"], dout, gemm=gemm)
    d1, g["ln2_w"], g["ln2_b"] = stack.layernorm_backward(c["x1"], ab["ln2_w"], dh2)
    dx1 = dout + d1
    flat = lambda a: a.reshape(-1, a.shape[-1])
    g["Wo"] = mm(flat(c["y"]).T, flat(dx1), gemm)
    dy = mm(dx1, ab["Wo"].T, gemm)
    dq, dk, dv = core_backward(c["core"], dy)
    dh1 = np.zeros_like(c["h1"])
    for w, d in (("Wq", dq), ("Wk", dk), ("Wv", dv)):
        g[w] = mm(flat(c["h1"]).T, flat(d), gemm)
        dh1 = dh1 + mm(d, ab[w].T, gemm)
    d0, g["ln1_w"], g["ln1_b"] = stack.layernorm_backward(c["x"], ab["ln1_w"], dh1)
    assert d0.shape[-1] == C
    return dx1 + d0, g


def forward(model, cfg, tokens):
    """Logits [B][T][V] of the hybrid stack (zero initial state)."""
    loss, _, logits = _run(model, cfg, tokens, None, "f64", want_grads=False)
    return logits


def train_step(model, cfg, tokens, targets, gemm="f64"):
    """Loss and gradients of every parameter of the hybrid stack.

    model: as oracle.stack (blocks = the RWKV-7 blocks, time-mix layer index =
    the block's index among them) plus attn: list of attention-block dicts
    (ln1_w/b, ln2_w/b, Wq, Wk, Wv, Wo [C][C], cm_mu_k, cm_Wk, cm_Wv);
    cfg: C, H, F, V, n_layer (RWKV-7 blocks), n_attn, chunk, topk.
    Returns (loss, grads) with grads mirroring the model (attn included)."""
    loss, G, _ = _run(model, cfg, tokens, targets, gemm, want_grads=True)
    return loss, G


def _run(model, cfg, tokens, targets, gemm, want_grads):
    m = stack._f64({k: v for k, v in model.items() if k != "attn"})
    m["attn"] = [{k: np.asarray(v, np.float64) for k, v in ab.items()} for ab in model["attn"]]
    tokens = np.asarray(tokens)
    H, chunk, topk = cfg["H"], cfg["chunk"], cfg["topk"]
    order = block_order(cfg["n_layer"], cfg["n_attn"])
    x = stack.embed(m["emb"], tokens)
    use_ln0 = m.get("ln0_w") is not None
    x_emb = x
    if use_ln0:
        x = stack.layernorm(x, m["ln0_w"], m["ln0_b"])
    xs, caches, v_first = [x], [], None
    for kind, i in order:
        if kind == "attn":
            x, c = attn_block_forward(m["attn"][i], x, H, chunk, topk, gemm)
        else:
            bp = m["blocks"][i]
            h1 = stack.layernorm(x, bp["ln1_w"], bp["ln1_b"])
            out, tc = tm.forward(bp["tm"], h1, H, i, v_first=v_first, gemm=gemm)
            if i == 0:
                v_first = tc["v_first"]
            x1 = x + out
            h2 = stack.layernorm(x1, bp["ln2_w"], bp["ln2_b"])
            x = x1 + stack.channel_mix(bp["cm_mu_k"], bp["cm_Wk"], bp["cm_Wv"], h2, gemm=gemm)
            c = dict(h1=h1, c=tc, x1=x1, h2=h2)
        caches.append(c)
        xs.append(x)
    hN = stack.layernorm(x, m["ln_out_w"], m["ln_out_b"])
    logits = mm(hN, m["head"], gemm)
    if not want_grads:
        return None, None, logits
    loss, dlog = stack.cross_entropy(logits, targets)
    G = {"head": mm(hN.reshape(-1, hN.shape[-1]).T, dlog.reshape(-1, dlog.shape[-1]), gemm)}
    dx, G["ln_out_w"], G["ln_out_b"] = stack.layernorm_backward(x, m["ln_out_w"],
                                                                mm(dlog, m["head"].T, gemm))
    G["blocks"] = [None] * len(m["blocks"])
    G["attn"] = [None] * len(m["attn"])
    dvf = np.zeros_like(x)
    for pos in range(len(order) - 1, -1, -1):
        kind, i = order[pos]
        cc = caches[pos]
        if kind == "attn":
            dx, G["attn"][i] = attn_block_backward(m["attn"][i], cc, dx, gemm)
            continue
        bp, gb = m["blocks"][i], {}
        dh2, _, gb["cm_mu_k"], gb["cm_Wk"], gb["cm_Wv"] = stack.channel_mix_backward(
            bp["cm_mu_k"], bp["cm_Wk"], bp["cm_Wv"], cc["h2"], dx, gemm=gemm)
        d1, gb["ln2_w"], gb["ln2_b"] = stack.layernorm_backward(cc["x1"], bp["ln2_w"], dh2)
        dx1 = dx + d1
        gt, dh1, _, dvf_out, _ = tm.backward(bp["tm"], cc["c"], dx1,
                                             dv_first_in=dvf if i == 0 else None)
        if i > 0:
            dvf = dvf + dvf_out
        gb["tm"] = gt
        d0, gb["ln1_w"], gb["ln1_b"] = stack.layernorm_backward(xs[pos], bp["ln1_w"], dh1)
        dx = dx1 + d0
        G["blocks"][i] = gb
    if use_ln0:
        dx, G["ln0_w"], G["ln0_b"] = stack.layernorm_backward(x_emb, m["ln0_w"], dx)
    demb = np.zeros_like(m["emb"])
    ids = tokens.reshape(-1)
    ok = (ids >= 0) & (ids < demb.shape[0])
    np.add.at(demb, ids[ok], dx.reshape(-1, dx.shape[-1])[ok])
    G["emb"] = demb
    return loss, G, logits
