"""Pins for the online TBPTT segment oracle (CPU only).

- Adam's first update from zero moments is lr g / (|g| + eps) in closed form
  (bias-corrected moments are g and g^2), and constant gradients keep the
  bias-corrected moments at g and g^2 on later steps.
- SGD with clipping: p - lr clamp(g, -clip, clip).
- lr = 0 leaves the weights and gives the plain forward's state.
- The gradient from a nonzero start state (truncated BPTT over the segment)
  against central finite differences of the segment loss.
Page: "infotheory .../rwkvzip/rwkv7/model.rs", online_train_segment_tbptt
and apply_full_gradients (AdamStep constants).
"""
import numpy as np
import pytest

from oracle import online, stack
from rwkv_linear_attention_wkv7_amd import synth


def _setup(seed=2, L=2, B=2, S=4):
    C, H, F, V = 8, 2, 12, 11
    cfg = dict(C=C, H=H, F=F, V=V, n_layer=L)
    m = stack._f64(synth.stack_model(C, H, F, V, L, (4, 4, 4, 4), seed=seed, perturbed=True,
                                     std=0.4, use_ln0=True))
    tok = synth.token_ids(B, S, V, seed=seed + 1)
    tgt = synth.token_ids(B, S, V, seed=seed + 2)
    # a live state from a few earlier tokens
    _, st = stack.forward(m, cfg, synth.token_ids(B, 3, V, seed=seed + 3))
    return m, cfg, tok, tgt, st


def test_adam_first_step_closed_form():
    m, cfg, tok, tgt, st = _setup()
    lr = 0.01
    loss, new, _, G, ad = online.train_segment(m, cfg, tok, tgt, st, "adam", lr=lr, t=1)
    for path, p in online._leaves(m):
        g = online._get(G, path)
        np.testing.assert_allclose(online._get(new, path), p - lr * g / (np.abs(g) + 1e-8),
                                   rtol=1e-12, atol=1e-15, err_msg=str(path))
        np.testing.assert_allclose(online._get(ad["m"], path), 0.1 * g, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(online._get(ad["v"], path), 0.001 * g * g, rtol=1e-12, atol=1e-300)


def test_adam_constant_gradient_moments():
    g = np.array([0.5, -2.0, 1e-3])
    p = np.zeros(3)
    mo, vo = np.zeros(3), np.zeros(3)
    for t in range(1, 6):
        p_new, mo, vo = online.adam_update(p, g, mo, vo, t, 0.1, 0.0)
        # m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2: bias-corrected g, g^2
        np.testing.assert_allclose(mo, (1 - 0.9 ** t) * g, rtol=1e-13)
        np.testing.assert_allclose(vo, (1 - 0.999 ** t) * g * g, rtol=1e-12)
        np.testing.assert_allclose(p_new - p, -0.1 * g / (np.abs(g) + 1e-8), rtol=1e-12)
        p = p_new


def test_sgd_with_clip():
    m, cfg, tok, tgt, st = _setup(seed=4)
    lr, clip = 0.5, 0.02
    _, new, _, G, _ = online.train_segment(m, cfg, tok, tgt, st, "sgd", lr=lr, clip=clip)
    n_clipped = 0
    for path, p in online._leaves(m):
        g = online._get(G, path)
        n_clipped += int(np.sum(np.abs(g) > clip))
        np.testing.assert_allclose(online._get(new, path), p - lr * np.clip(g, -clip, clip),
                                   rtol=1e-13, atol=1e-15)
    assert n_clipped > 0   # the case exercises the clamp


def test_zero_learning_rate_replays_the_forward():
    m, cfg, tok, tgt, st = _setup(seed=6)
    _, new, new_state, _, _ = online.train_segment(m, cfg, tok, tgt, st, "sgd", lr=0.0)
    for path, p in online._leaves(m):
        np.testing.assert_array_equal(online._get(new, path), p)
    # the live state is the streaming state after the segment's tokens
    state = {k: v.copy() for k, v in st.items()}
    for t in range(tok.shape[1]):
        _, state = stack.decode_step(m, cfg, tok[:, t], state)
    for k in state:
        np.testing.assert_allclose(new_state[k], state[k], rtol=1e-10, atol=1e-12)


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


def test_truncated_bptt_gradient_central_fd():
    """From a nonzero start state, every gradient the segment uses against
    central differences of its loss (the state held fixed)."""
    m, cfg, tok, tgt, st = _setup(seed=8, S=3)
    loss, G = stack.train_step(m, cfg, tok, tgt, state=st)
    fn = lambda: stack.train_step(m, cfg, tok, tgt, state=st)[0]
    checks = [("emb", m["emb"], G["emb"]), ("head", m["head"], G["head"])]
    for l in range(2):
        bp, gb = m["blocks"][l], G["blocks"][l]
        for k in ("ln1_w", "cm_mu_k", "cm_Wk"):
            checks.append((f"{k}[{l}]", bp[k], gb[k]))
        for k in ("mu_r", "mu_k", "Wr", "Wk", "w0", "W1", "k_k", "ln_w"):
            checks.append((f"tm.{k}[{l}]", bp["tm"][k], gb["tm"][k]))
    for name, p, g in checks:
        fd = _fd(fn, p)
        err = np.max(np.abs(fd - g)) / max(np.max(np.abs(fd)), 1e-30)
        assert err < 1e-5, (name, err)
