"""Pins for the MoBA attention and hybrid-stack oracle (CPU only).

- With top-k covering every chunk the core is causal softmax attention,
  written out here with explicit loops.
- chunk 1, top-k 1: each query attends to itself only, y_t = v_t.
- The selection on a hand-built case: chunk means and a query chosen so the
  scores, the tie and the attended keys are known, and y written out.
- The core backward (selection held fixed) against central differences.
- The block interleave of the fullmodel page's fm_build on several counts.
- The hybrid training step: loss and every attention-block parameter, the
  embedding, head and a sample of RWKV-7 parameters against central
  differences of the loss.
Page: "Foundry/cuda_kernels/fullmodel.cu" (fm_build interleave,
fm_attn_core_fwd, fm_attn_fwd, fm_attn_bwd).
"""
import math

import numpy as np
import pytest

from oracle import moba
from rwkv_linear_attention_wkv7_amd import synth


def test_full_topk_is_causal_softmax_attention():
    rng = np.random.default_rng(0)
    B, T, H, N = 2, 9, 2, 4
    q, k, v = (rng.standard_normal((B, T, H * N)) for _ in range(3))
    y, _ = moba.core_forward(q, k, v, H, chunk=2, topk=5)   # 5 chunks cover T = 9
    for b in range(B):
        for h in range(H):
            for t in range(T):
                sl = slice(h * N, (h + 1) * N)
                w = [math.exp(sum(q[b, t, sl] * k[b, s, sl]) / math.sqrt(N)) for s in range(t + 1)]
                want = sum(w[s] * v[b, s, sl] for s in range(t + 1)) / sum(w)
                np.testing.assert_allclose(y[b, t, sl], want, rtol=1e-12, atol=1e-13)


def test_chunk_one_topk_one_attends_to_itself():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((1, 7, 8)) for _ in range(3))
    y, _ = moba.core_forward(q, k, v, H=2, chunk=1, topk=1)
    np.testing.assert_allclose(y, v, rtol=1e-14)


def test_selection_by_hand():
    """T = 8, chunk 2, N = 2, one head, top-k 3 (the current chunk + 2).
    Keys: chunk 0 = (1,0),(1,0) (mean (1,0)); chunk 1 = (0,2),(0,0) (mean
    (0,1)); chunk 2 = (-1,0),(-1,0) (mean (-1,0)); chunk 3 = (0,0),(3,3).
    Query t = 6 (chunk 3) is (0,1): scores 0, 1, 0 for chunks 0, 1, 2; chunk 1
    wins, the tie between 0 and 2 goes to the lower index.  So t = 6 attends
    to keys 0, 1, 2, 3 and 6 (not 7: causal)."""
    k = np.array([[1, 0], [1, 0], [0, 2], [0, 0], [-1, 0], [-1, 0], [0, 0], [3, 3]], float)
    q = np.zeros((8, 2))
    q[6] = [0, 1]
    v = np.arange(16, dtype=float).reshape(8, 2)
    sel = moba.select(q, k, 2, 3)
    assert sel[6].tolist() == [True, True, False, True]
    y, c = moba.core_forward(q[None], k[None], v[None], H=1, chunk=2, topk=3)
    s = {tau: (q[6] @ k[tau]) / math.sqrt(2) for tau in (0, 1, 2, 3, 6)}
    z = sum(math.exp(x) for x in s.values())
    want = sum(math.exp(s[tau]) / z * v[tau] for tau in s)
    np.testing.assert_allclose(y[0, 6], want, rtol=1e-13)
    assert c["mask"][0, 0, 6].tolist() == [True, True, True, True, False, False, True, False]
    # t = 1 (chunk 0): only keys 0, 1; t = 3 (chunk 1, one earlier chunk): keys 0..3
    assert c["mask"][0, 0, 1].tolist() == [True, True] + [False] * 6
    assert c["mask"][0, 0, 3].tolist() == [True] * 4 + [False] * 4


def _fd(fn, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        lp = fn()
        x[i] = old - eps
        lm = fn()
        x[i] = old
        g[i] = (lp - lm) / (2 * eps)
    return g


def test_core_backward_central_fd():
    rng = np.random.default_rng(3)
    B, T, H, N = 1, 7, 2, 3
    q, k, v, dy = (rng.standard_normal((B, T, H * N)) for _ in range(4))
    y, c = moba.core_forward(q, k, v, H, chunk=2, topk=2)
    dq, dk, dv = moba.core_backward(c, dy)
    sel0 = [moba.select(q[0, :, h * N:(h + 1) * N], k[0, :, h * N:(h + 1) * N], 2, 2) for h in range(H)]
    fn = lambda: float(np.sum(dy * moba.core_forward(q, k, v, H, 2, 2)[0]))
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = _fd(fn, x)
        err = np.max(np.abs(g - fd)) / np.max(np.abs(fd))
        assert err < 1e-6, (name, err)
    # the perturbations left the selection as it was (no score near a tie)
    for h in range(H):
        assert (moba.select(q[0, :, h * N:(h + 1) * N], k[0, :, h * N:(h + 1) * N], 2, 2) == sel0[h]).all()


@pytest.mark.parametrize("n_rwkv,n_attn,want", [
    (6, 2, "r0 r1 r2 a0 r3 r4 r5 a1"),
    (5, 2, "r0 r1 a0 r2 r3 a1 r4"),
    (3, 0, "r0 r1 r2"),
    (1, 2, "a0 a1 r0"),
    (4, 1, "r0 r1 r2 r3 a0"),
])
def test_block_interleave(n_rwkv, n_attn, want):
    got = " ".join(("r" if kind == "rwkv" else "a") + str(i) for kind, i in moba.block_order(n_rwkv, n_attn))
    assert got == want


def _hybrid(seed=4):
    C, H, F, V, L = 8, 2, 12, 11, 2
    m = synth.stack_model(C, H, F, V, L, (4, 4, 4, 4), seed=seed, perturbed=True, std=0.4,
                          use_ln0=True)
    m = {k: v for k, v in m.items()}
    m["attn"] = synth.attn_blocks(C, F, 1, seed=seed, perturbed=True, std=0.4)
    m = _to64(m)
    cfg = dict(C=C, H=H, F=F, V=V, n_layer=L, n_attn=1, chunk=2, topk=2)
    tok = synth.token_ids(2, 6, V, seed=seed + 1)
    tgt = synth.token_ids(2, 6, V, seed=seed + 2)
    return m, cfg, tok, tgt


def _to64(m):
    out = {}
    for k, v in m.items():
        if k == "blocks":
            out[k] = [{kk: ({k3: np.asarray(v3, np.float64) for k3, v3 in vv.items()} if kk == "tm"
                            else np.asarray(vv, np.float64)) for kk, vv in b.items()} for b in v]
        elif k == "attn":
            out[k] = [{kk: np.asarray(vv, np.float64) for kk, vv in a.items()} for a in v]
        else:
            out[k] = None if v is None else np.asarray(v, np.float64)
    return out


def test_hybrid_train_step_central_fd():
    m, cfg, tok, tgt = _hybrid()
    loss, G = moba.train_step(m, cfg, tok, tgt)
    fn = lambda: moba.train_step(m, cfg, tok, tgt)[0]
    checks = [(m["attn"][0][n], G["attn"][0][n], f"attn.{n}") for n in m["attn"][0]]
    checks += [(m["emb"], G["emb"], "emb"), (m["head"], G["head"], "head"),
               (m["ln0_w"], G["ln0_w"], "ln0_w")]
    for l in range(cfg["n_layer"]):
        checks += [(m["blocks"][l]["tm"]["Wv"], G["blocks"][l]["tm"]["Wv"], f"tm.Wv[{l}]"),
                   (m["blocks"][l]["cm_Wk"], G["blocks"][l]["cm_Wk"], f"cm_Wk[{l}]")]
    for x, g, name in checks:
        fd = _fd(fn, x, eps=1e-6)
        err = np.max(np.abs(g - fd)) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-5, (name, err)


def test_hybrid_without_attention_is_the_rwkv_stack():
    from oracle import stack
    m, cfg, tok, tgt = _hybrid()
    m["attn"] = []
    cfg = dict(cfg, n_attn=0)
    l1, G1 = moba.train_step(m, cfg, tok, tgt)
    l2, G2 = stack.train_step({k: v for k, v in m.items() if k != "attn"}, cfg, tok, tgt)
    assert l1 == l2
    np.testing.assert_array_equal(G1["emb"], G2["emb"])
