"""Pins for the stack oracle (CPU only): LayerNorm's textbook properties, the
channel-mix token shift, and step-by-step decode equal to the sequence
forward (the streaming state carries exactly what the sequence shifts)."""
import numpy as np

from oracle import stack
from rwkv_linear_attention_wkv7_amd import synth


def _model(perturbed=True, L=3, C=128, H=2, F=256, V=64):
    cfg = dict(C=C, H=H, F=F, V=V, n_layer=L)
    m = synth.stack_model(C, H, F, V, L, (16, 16, 16, 32), seed=4, perturbed=perturbed, std=0.2)
    return m, cfg


def test_layernorm_textbook():
    x = np.random.default_rng(0).standard_normal((5, 7, 96)) * 3 + 1
    y = stack.layernorm(x, np.ones(96), np.zeros(96))
    var = x.var(axis=-1)
    np.testing.assert_allclose(y.mean(axis=-1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=-1), var / (var + stack.LN_EPS), rtol=1e-12)
    w, b = np.arange(96) * 0.1, np.ones(96)
    np.testing.assert_allclose(stack.layernorm(x, w, b), y * w + b, rtol=1e-12)


def test_channel_mix_shift_and_square_relu():
    g = np.random.default_rng(1)
    C, F = 16, 24
    mu, Wk, Wv = g.uniform(0, 1, C), g.standard_normal((C, F)), g.standard_normal((F, C))
    x = g.standard_normal((2, 3, C))
    out = stack.channel_mix(mu, Wk, Wv, x, x_prev=None)
    # position 1 alone, with x_prev = x[:, 0], equals position 1 of the sequence
    o1 = stack.channel_mix(mu, Wk, Wv, x[:, 1:2], x_prev=x[:, 0])
    np.testing.assert_allclose(o1[:, 0], out[:, 1], rtol=1e-13)
    # first position with no previous token: sh = x (1 - mu)
    sh = x[:, 0] * (1 - mu)
    np.testing.assert_allclose(out[:, 0], np.maximum(sh @ Wk, 0) ** 2 @ Wv, rtol=1e-13)


def test_decode_steps_equal_sequence_forward():
    m, cfg = _model()
    B, T = 3, 6
    tok = synth.token_ids(B, T, cfg["V"], seed=2)
    logits_seq, st_seq = stack.forward(m, cfg, tok)
    st = stack.init_state(cfg, B)
    for t in range(T):
        lg, st = stack.decode_step(m, cfg, tok[:, t], st)
        np.testing.assert_allclose(lg, logits_seq[:, t], rtol=1e-10, atol=1e-12)
    for k in st:
        np.testing.assert_allclose(st[k], st_seq[k], rtol=1e-10, atol=1e-12)


def test_stream_independence():
    """Streams do not interact: a stream's logits do not depend on the others."""
    m, cfg = _model(L=2)
    tok = synth.token_ids(4, 3, cfg["V"], seed=3)
    full, _ = stack.forward(m, cfg, tok)
    one, _ = stack.forward(m, cfg, tok[2:3])
    np.testing.assert_allclose(one[0], full[2], rtol=1e-12, atol=1e-14)


def test_cross_entropy_textbook():
    z = np.random.default_rng(3).standard_normal((4, 5, 9))
    t = np.random.default_rng(4).integers(0, 9, size=(4, 5))
    loss, d = stack.cross_entropy(z, t)
    p = np.exp(z) / np.exp(z).sum(-1, keepdims=True)
    ref = -np.mean(np.log(np.take_along_axis(p, t[..., None], -1)))
    np.testing.assert_allclose(loss, ref, rtol=1e-13)
    np.testing.assert_allclose(d.sum(-1), 0.0, atol=1e-15)        # each row sums to 0
    np.testing.assert_allclose((d * 20).sum(-1), 0.0, atol=1e-13)


def test_cross_entropy_ignored_targets():
    """Targets outside [0, V) are ignored (the fullmodel page's ignore_index):
    the loss is the textbook mean over the counted tokens only, ignored rows
    of dlogits are zero and the others are scaled by 1 / n_valid."""
    z = np.random.default_rng(5).standard_normal((3, 4, 7))
    t = np.random.default_rng(6).integers(0, 7, size=(3, 4))
    t[0, 1], t[2, 3], t[1, 0] = -1, 7, 100
    loss, d = stack.cross_entropy(z, t)
    ok = (t >= 0) & (t < 7)
    p = np.exp(z) / np.exp(z).sum(-1, keepdims=True)
    lp = np.log(np.take_along_axis(p, np.where(ok, t, 0)[..., None], -1))[..., 0]
    np.testing.assert_allclose(loss, -lp[ok].mean(), rtol=1e-13)
    assert np.all(d[~ok] == 0.0)
    one = np.zeros_like(z)
    np.put_along_axis(one, np.where(ok, t, 0)[..., None], 1.0, -1)
    np.testing.assert_allclose(d[ok], (p - one)[ok] / ok.sum(), rtol=1e-12, atol=1e-15)
    # nothing counted: zero loss and zero gradient
    loss0, d0 = stack.cross_entropy(z, np.full((3, 4), -1))
    assert loss0 == 0.0 and np.all(d0 == 0.0)


def test_embedding_out_of_range_ids_are_zero_rows():
    emb = np.random.default_rng(7).standard_normal((5, 3))
    x = stack.embed(emb, np.array([[0, 4, -1, 5, 2]]))
    np.testing.assert_array_equal(x[0, [0, 1, 4]], emb[[0, 4, 2]])
    assert np.all(x[0, [2, 3]] == 0.0)


def _fd(fn, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        mi = it.multi_index
        old = x[mi]
        x[mi] = old + eps
        lp = fn()
        x[mi] = old - eps
        lm = fn()
        x[mi] = old
        g[mi] = (lp - lm) / (2 * eps)
    return g


def test_train_step_central_fd():
    """Every parameter of a tiny 2-layer model against central differences of the loss."""
    C, H, F, V, L = 8, 2, 12, 11, 2
    cfg = dict(C=C, H=H, F=F, V=V, n_layer=L)
    N = C // H
    for use_ln0 in (False, True):
        m = synth.stack_model(C, H, F, V, L, (4, 4, 4, 4), seed=6, perturbed=True, std=0.4,
                              use_ln0=use_ln0)
        m = stack._f64(m)
        # tiny head size: the oracle's recurrence is N-generic
        tok = synth.token_ids(2, 3, V, seed=1)
        tgt = synth.token_ids(2, 3, V, seed=2)
        # one out-of-range id (zero row, no gradient) and one ignored target
        tok[1, 1], tgt[0, 2] = V + 3, -1
        loss, G = stack.train_step(m, cfg, tok, tgt)
        fn = lambda: stack.train_step(m, cfg, tok, tgt)[0]
        checks = [("emb", m["emb"], G["emb"]), ("head", m["head"], G["head"]),
                  ("ln_out_w", m["ln_out_w"], G["ln_out_w"]), ("ln_out_b", m["ln_out_b"], G["ln_out_b"])]
        if use_ln0:
            checks += [("ln0_w", m["ln0_w"], G["ln0_w"]), ("ln0_b", m["ln0_b"], G["ln0_b"])]
        for l in range(L):
            bp, gb = m["blocks"][l], G["blocks"][l]
            for k in ("ln1_w", "ln1_b", "ln2_w", "ln2_b", "cm_mu_k", "cm_Wk", "cm_Wv"):
                checks.append((f"{k}[{l}]", bp[k], gb[k]))
            for k in bp["tm"]:
                checks.append((f"tm.{k}[{l}]", bp["tm"][k], gb["tm"][k]))
        for name, p, g in checks:
            fd = _fd(fn, p)
            err = np.max(np.abs(fd - g)) / max(np.max(np.abs(fd)), 1e-30)
            assert err < 1e-5, (use_ln0, name, err)
