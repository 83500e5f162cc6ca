"""Hand-derived cases for the time-mix block and stack assembly of the oracle
(CPU only).

The expected values below are worked out by hand (in the comments) from the
definitions on the pages, for weights chosen so that every intermediate is a
small closed form: a one-hot input picks one row of every projection, LoRA
products reduce to sigma(+-ln 3) in {1/4, 3/4} or sigma(0) = 1/2, and the WKV
state has a known start.  None of the expected numbers is produced by the
oracle's own code.  Together they pin the composition lines of the time-mix
forward (decay, a-gate, g-LoRA, key scaling, key-mod, value residual,
composites a = -kk and b = kk*a, bonus and its placement, gate multiply, the
[in][out] orientation of every weight) and the stack assembly (ln0, residual
adds, LayerNorm with zero weight, channel-mix relu^2, ln_out and the head).

Pages: "Foundry/cuda_kernels/timemix.cu" (forward driver and k_tokenshift ..
k_mul), "infotheory .../rwkv7/model.rs" (AttentionWeights LoRA formulas),
"Foundry/cuda_kernels/fullmodel.cu" (block and model forward).

The group norm and LayerNorm appear below only in their textbook form
((y - mean) / sqrt(biased var + eps) * w + b over a head or row), whose own
properties are pinned separately (test_oracle_timemix, test_oracle_stack).
"""
import math

import numpy as np
import pytest

from oracle import stack
from oracle import timemix as tm

LN3 = math.log(3.0)
H, N = 2, 4
C = H * N
GN_EPS = 64e-5   # group-norm epsilon of the time-mix block (timemix.cu k_groupnorm)
LN_EPS = 1e-5    # LayerNorm epsilon (model.rs Config)


def _textbook_norm(y, w, b, eps):
    m = y.mean()
    var = ((y - m) ** 2).mean()
    return (y - m) / math.sqrt(var + eps) * w + b


def hand_params(layer_id, rng, v_row=(1, 2, 3, 4, 1, -1, 1, -1)):
    """Time-mix weights of the hand cases.  With x = e_0 every product x W is
    row 0 of W; the other rows are random so that a transposed weight (W x)
    would be seen.  Ranks Dw = Da = Dv = 4, Dg = C."""
    D = 4
    rnd = lambda *s: rng.standard_normal(s)
    p = {f"mu_{c}": np.zeros(C) for c in "rwkvag"}
    p["Wr"], p["Wk"], p["Wv"] = rnd(C, C), rnd(C, C), rnd(C, C)
    p["Wr"][0] = [1, 1, 0, 0, 0, 0, 2, 0]          # r: head 0 (1,1,0,0), head 1 (0,0,2,0)
    p["Wk"][0] = [3, 4, 0, 0, 0, 0, 1, 0]          # k: head 0 (3,4,0,0), head 1 (0,0,1,0)
    p["Wv"][0] = v_row                             # v
    p["Wo"] = np.eye(C)
    p["Wo"][0, 7] = 1.0                            # out[7] = tg[7] + tg[0]
    # decay: tw = tanh(x W1) = (tanh 1, 0, 0, 0); ow = tw W2 = +-ln 3 (head 0 / head 1)
    p["W1"] = rnd(C, D)
    p["W1"][0] = [1, 0, 0, 0]
    p["W2"] = rnd(D, C)
    p["W2"][0] = np.r_[np.full(N, LN3), np.full(N, -LN3)] / math.tanh(1.0)
    p["w0"] = np.zeros(C)
    # a-gate: la = x A1 = (1, 0, 0, 0); a = sigmoid(0 + la A2) = 3/4 (head 0), 1/4 (head 1)
    p["A1"] = rnd(C, D)
    p["A1"][0] = [1, 0, 0, 0]
    p["A2"] = rnd(D, C)
    p["A2"][0] = np.r_[np.full(N, LN3), np.full(N, -LN3)]
    p["a0"] = np.zeros(C)
    # gate: sigmoid(x G1) = 1/2 everywhere, G2 = diag(2,2,2,2,6,6,6,6): g = 1 / 3
    p["G1"] = np.zeros((C, C))
    p["G2"] = np.diag(np.r_[np.full(N, 2.0), np.full(N, 6.0)])
    p["k_k"] = np.array([1, 0.75, 1, 1, 1, 1, 0.5, 1.0])   # tk head 0 = (3,3,0,0)
    p["k_a"] = np.r_[np.ones(N), np.full(N, 0.5)]
    p["r_k"] = np.array([0, 1, 0, 0, 0, 0, 1, 0.0])
    p["ln_w"] = np.full(C, 2.0)
    p["ln_b"] = np.full(C, 0.1)
    if layer_id > 0:
        # value residual: nu = sigmoid(0 + (x V1) V2) = 1/4 (head 0), 3/4 (head 1)
        p["V1"] = rnd(C, D)
        p["V1"][0] = [1, 0, 0, 0]
        p["V2"] = rnd(D, C)
        p["V2"][0] = np.r_[np.full(N, -LN3), np.full(N, LN3)]
        p["v0"] = np.zeros(C)
    return p


# Per-head quantities of the hand cases, derived once here:
#   head 0: r = (1,1,0,0), k = (3,4,0,0), a = 3/4, k_k -> tk = (3,3,0,0),
#           kk = (1,1,0,0)/sqrt2, k' = k (1 + (a - 1) * 1) = (2.25, 3, 0, 0),
#           b = kk a, so b.r = (3/4) sqrt2 and kk (b.r) = (3/4, 3/4, 0, 0),
#           k'.r = 5.25, bonus alpha = r[1] k'[1] = 3, w = exp(-0.606531 * 3/4)
#   head 1: r = (0,0,2,0), k = (0,0,1,0), a = 1/4, kk = (0,0,1,0),
#           k' = k (1 + (1/4 - 1) * 1/2) = (0, 0, 0.625, 0), b.r = 1/2,
#           kk (b.r) = (0,0,1/2,0), k'.r = 1.25, alpha = r[2] k'[2] = 1.25,
#           w = exp(-0.606531 * 1/4)
W0 = math.exp(-0.606531 * 0.75)
W1_ = math.exp(-0.606531 * 0.25)
ALPHA = (3.0, 1.25)
GATE = (1.0, 3.0)
KR = (5.25, 1.25)


def expected_out(vprime, s0_identity):
    """out of the hand case for per-head v' (2 x 4).

    From a zero state, y = v' (k'.r).  From s0 = I, y = I diag(w) r + (I a_vec)
    (b.r) + v' (k'.r) = w r - kk (b.r) + v' (k'.r)."""
    y = [KR[h] * np.asarray(vprime[h], float) for h in range(H)]
    if s0_identity:
        y[0] = y[0] + W0 * np.array([1, 1, 0, 0]) - np.array([0.75, 0.75, 0, 0])
        y[1] = y[1] + W1_ * np.array([0, 0, 2, 0]) - np.array([0, 0, 0.5, 0])
    tg = []
    for h in range(H):
        ygn = _textbook_norm(y[h], 2.0, 0.1, GN_EPS)
        yb = ygn + ALPHA[h] * np.asarray(vprime[h], float)
        tg.append(yb * GATE[h])
    tg = np.concatenate(tg)
    out = tg.copy()
    out[7] += tg[0]
    return out, y


def _run(p, layer_id, s0_identity, v_first=None):
    x = np.zeros((1, 1, C))
    x[0, 0, 0] = 1.0
    s0 = np.broadcast_to(np.eye(N), (1, H, N, N)).copy() if s0_identity else None
    vf = None if v_first is None else np.asarray(v_first, float).reshape(1, 1, C)
    return tm.forward(p, x, H, layer_id, v_first=vf, s0=s0)


@pytest.mark.parametrize("s0_identity", [False, True])
def test_timemix_hand_case_layer0(s0_identity):
    p = hand_params(0, np.random.default_rng(11))
    out, c = _run(p, 0, s0_identity)
    vprime = [(1, 2, 3, 4), (1, -1, 1, -1)]       # layer 0: v' = v
    ref, y = expected_out(vprime, s0_identity)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-10, atol=1e-10)
    # the intermediates named on the pages, by hand
    np.testing.assert_allclose(c["w"][0, 0], np.r_[np.full(N, W0), np.full(N, W1_)], rtol=1e-13)
    np.testing.assert_allclose(c["a"][0, 0], np.r_[np.full(N, 0.75), np.full(N, 0.25)], rtol=1e-13)
    np.testing.assert_allclose(c["g"][0, 0], np.r_[np.full(N, 1.0), np.full(N, 3.0)], rtol=1e-13)
    s2 = 1 / math.sqrt(2)
    np.testing.assert_allclose(c["kmod"][0, 0], [2.25, 3, 0, 0, 0, 0, 0.625, 0], atol=1e-13)
    np.testing.assert_allclose(c["A"][0, 0], [-s2, -s2, 0, 0, 0, 0, -1, 0], atol=1e-13)
    np.testing.assert_allclose(c["Bv"][0, 0], [0.75 * s2, 0.75 * s2, 0, 0, 0, 0, 0.25, 0], atol=1e-13)
    np.testing.assert_allclose(c["alpha"][0, 0], ALPHA, rtol=1e-13)
    np.testing.assert_allclose(c["y"][0, 0], np.stack(y), rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(c["v_first"], c["v"])


@pytest.mark.parametrize("s0_identity", [False, True])
def test_timemix_hand_case_value_residual(s0_identity):
    p = hand_params(1, np.random.default_rng(12))
    vf = [5, 6, 7, 8, -1, 1, -1, 1]
    out, c = _run(p, 1, s0_identity, v_first=vf)
    # v' = v + (v_first - v) nu, nu = 1/4 (head 0), 3/4 (head 1):
    #   head 0: (1,2,3,4) + (4,4,4,4)/4 = (2,3,4,5)
    #   head 1: (1,-1,1,-1) + (-2,2,-2,2) * 3/4 = (-0.5, 0.5, -0.5, 0.5)
    vprime = [(2, 3, 4, 5), (-0.5, 0.5, -0.5, 0.5)]
    ref, _ = expected_out(vprime, s0_identity)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(c["vmod"][0, 0], np.concatenate(vprime), atol=1e-13)
    np.testing.assert_allclose(c["nu"][0, 0], np.r_[np.full(N, 0.25), np.full(N, 0.75)], rtol=1e-13)


def test_timemix_token_shift_lerp_by_hand():
    """xs_c = x + (x_prev - x) mu_c with distinct mu per mix: x = e_0 and
    x_prev = e_1 give xs_c = (1 - mu_c) e_0 + mu_c e_1."""
    p = hand_params(0, np.random.default_rng(13))
    mus = dict(r=0.1, w=0.2, k=0.3, v=0.4, a=0.6, g=0.7)
    for ch, m in mus.items():
        p["mu_" + ch] = np.full(C, m)
    x = np.zeros((1, 1, C))
    x[0, 0, 0] = 1.0
    xp = np.zeros((1, C))
    xp[0, 1] = 1.0
    _, c = tm.forward(p, x, H, 0, x_prev=xp)
    for ch, m in mus.items():
        want = np.zeros(C)
        want[0], want[1] = 1 - m, m
        np.testing.assert_allclose(c["xs"][ch][0, 0], want, rtol=1e-14, err_msg=ch)
    # r = xs_r Wr: rows 0 and 1 of Wr, weighted
    np.testing.assert_allclose(c["r"][0, 0], 0.9 * p["Wr"][0] + 0.1 * p["Wr"][1], rtol=1e-13)


def _hand_stack(n_layer, use_ln0, rng):
    """A stack whose LayerNorms feeding each block have weight 0 and a one-hot
    bias, so every block sees a known input whatever the residual stream holds:
    LN1 gives e_0 (the time-mix hand case, zero state), LN2 gives e_0 too.
    Channel-mix (F = 4): sh = e_0 (1 - 1/2); fk = sh Wk = (1, -1, 2, 0);
    relu(fk)^2 = (1, 0, 4, 0); out = Wv[0] + 4 Wv[2]."""
    V, F = 5, 4
    m = {"emb": rng.standard_normal((V, C)), "head": rng.standard_normal((C, V)),
         "ln_out_w": 1 + 0.3 * rng.standard_normal(C), "ln_out_b": 0.3 * rng.standard_normal(C)}
    if use_ln0:
        m["ln0_w"], m["ln0_b"] = np.full(C, 1.5), np.full(C, -0.2)
    else:
        m["ln0_w"] = m["ln0_b"] = None
    e0 = np.zeros(C)
    e0[0] = 1.0
    blocks = []
    v_rows = [(1, 2, 3, 4, 1, -1, 1, -1), (5, 6, 7, 8, -1, 1, -1, 1)]
    for l in range(n_layer):
        bp = dict(ln1_w=np.zeros(C), ln1_b=e0.copy(), ln2_w=np.zeros(C), ln2_b=e0.copy())
        bp["tm"] = hand_params(l, rng, v_row=v_rows[l])
        bp["cm_mu_k"] = np.full(C, 0.5)
        bp["cm_Wk"] = rng.standard_normal((C, F))
        bp["cm_Wk"][0] = [2, -2, 4, 0]
        bp["cm_Wv"] = rng.standard_normal((F, C))
        blocks.append(bp)
    m["blocks"] = blocks
    return m, dict(C=C, H=H, F=F, V=V, n_layer=n_layer)


@pytest.mark.parametrize("n_layer,use_ln0", [(1, True), (1, False), (2, True)])
def test_stack_assembly_by_hand(n_layer, use_ln0):
    m, cfg = _hand_stack(n_layer, use_ln0, np.random.default_rng(20 + n_layer))
    tok = np.array([[3]])
    logits, st = stack.forward(m, cfg, tok)
    # x0 = emb[3], through ln0 when present
    x = m["emb"][3].copy()
    if use_ln0:
        x = _textbook_norm(x, 1.5, -0.2, LN_EPS)
    # layer 0: time-mix hand case from a zero state (v' = v); layer 1 uses
    # v_first = layer 0's v: v' head 0 = (5,6,7,8) + ((1,2,3,4) - (5,6,7,8))/4
    # = (4,5,6,7), head 1 = (-1,1,-1,1) + (2,-2,2,-2) * 3/4 = (0.5,-0.5,0.5,-0.5)
    vprimes = [[(1, 2, 3, 4), (1, -1, 1, -1)], [(4, 5, 6, 7), (0.5, -0.5, 0.5, -0.5)]]
    for l in range(n_layer):
        tm_out, _ = expected_out(vprimes[l], s0_identity=False)
        x = x + tm_out
        Wv = m["blocks"][l]["cm_Wv"]
        x = x + Wv[0] + 4.0 * Wv[2]
    h = _textbook_norm(x, m["ln_out_w"], m["ln_out_b"], LN_EPS)
    want = np.array([sum(h[c] * m["head"][c, j] for c in range(C)) for j in range(cfg["V"])])
    np.testing.assert_allclose(logits[0, 0], want, rtol=1e-11, atol=1e-12)
    # the streaming state keeps the LN outputs (e_0) as the next token's shift source
    for l in range(n_layer):
        np.testing.assert_allclose(st["att_x_prev"][l, 0], np.eye(C)[0])
        np.testing.assert_allclose(st["ffn_x_prev"][l, 0], np.eye(C)[0])


def test_train_step_loss_by_hand():
    """The training step's loss on the hand stack: mean over tokens of
    logsumexp(logits) - logit[target], logits as in the assembly case."""
    from oracle import stack as st_
    m, cfg = _hand_stack(1, False, np.random.default_rng(31))
    tok, tgt = np.array([[3]]), np.array([[1]])
    loss, _ = st_.train_step(m, cfg, tok, tgt)
    logits, _ = stack.forward(m, cfg, tok)
    z = logits[0, 0]
    want = math.log(sum(math.exp(v) for v in z)) - z[1]
    assert abs(loss - want) < 1e-12 * max(1.0, abs(want))
