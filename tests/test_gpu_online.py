"""GPU parity of rwkv7_online_segment (online TBPTT segment: gradients from a
live state truncated at the segment start, SGD / Adam update, live-state
replay with the updated weights) against the f64 oracle (oracle/online.py).
Tolerances: loss 1e-4, gradients 1e-3 (fp32 gradients); the new weights
against the update rule applied to the GPU's gradient within two fp32 ulps
of the weight plus 1e-5 lr (fp32 update arithmetic); the live state 1e-4
(fp32 forward) against the oracle's forward with the updated weights.  Page:
"infotheory .../rwkvzip/rwkv7/model.rs", online_train_segment_tbptt."""
import numpy as np
import pytest
import torch

from oracle import online, stack
from rwkv_linear_attention_wkv7_amd import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu


def _dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _setup(hip, L=2, C=128, H=2, F=256, V=64, B=3, S=20, seed=11):
    from rwkv_linear_attention_wkv7_amd import binding
    ranks = (16, 16, 16, 32)
    m = synth.stack_model(C, H, F, V, L, ranks, seed=seed, perturbed=True, std=0.2)
    w = {k: _dev(v) for k, v in m.items() if k != "blocks"}
    w["blocks"] = [{k: ({kk: _dev(vv) for kk, vv in v.items()} if k == "tm" else _dev(v))
                    for k, v in b.items()} for b in m["blocks"]]
    dm = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=ranks, use_ln0=1), w)
    cfg = dict(C=C, H=H, F=F, V=V, n_layer=L)
    # a live state from a few decoded tokens
    pre = synth.token_ids(B, 5, V, seed=seed + 1)
    _, st = stack.forward(m, cfg, pre)
    tok = synth.token_ids(B, S, V, seed=seed + 2)
    tgt = synth.token_ids(B, S, V, seed=seed + 3)
    return m, cfg, dm, st, tok, tgt


def _flat(G):
    for k, v in G.items():
        if k == "blocks":
            for l, b in enumerate(v):
                for kk, vv in b.items():
                    if kk == "tm":
                        for k3, v3 in vv.items():
                            yield f"tm.{k3}[{l}]", v3
                    else:
                        yield f"{kk}[{l}]", vv
        elif v is not None:
            yield k, v


@pytest.mark.parametrize("optimizer,clip", [("adam", 0.0), ("sgd", 0.05), ("adam", 0.05)])
def test_online_segment_parity(hip, optimizer, clip):
    """Each stage against the oracle given the previous stage's GPU result:
    loss and gradients against the oracle's segment; the update against the
    oracle's update rule applied to the GPU's own gradient (Adam's first step
    is lr g / (|g| + eps) per element, so gradient elements below the
    gradient's rounding noise may move anywhere in [-lr, lr]; the rule itself
    is what is checked here); the live state against the oracle's forward
    with the GPU's updated weights from the same start state."""
    from rwkv_linear_attention_wkv7_amd import binding
    m, cfg, dm, st, tok, tgt = _setup(hip)
    lr = 1e-3 if optimizer == "adam" else 0.05
    old = {n: t.cpu().numpy().astype(np.float64) for n, t in _flat(dm.w)}
    grads = binding.TrainGrads(dm)
    am = binding.TrainGrads(dm, zero=True) if optimizer == "adam" else None
    av = binding.TrainGrads(dm, zero=True) if optimizer == "adam" else None
    state = {k: _dev(v.astype(np.float32)) for k, v in st.items()}
    st32 = {k: v.astype(np.float32).astype(np.float64) for k, v in st.items()}
    print(f"[online] {optimizer} clip={clip}", flush=True)
    loss = hip.rwkv7_online_segment(dm, grads, _dev(tok), _dev(tgt), state, optimizer=optimizer,
                                    lr=lr, clip=clip, step=1, adam_m=am, adam_v=av)
    torch.cuda.synchronize()
    # 1. loss and gradients of the segment from the live state
    ref_loss, G = stack.train_step(m, cfg, tok, tgt, state=st32)
    assert abs(float(loss.item()) - ref_loss) <= 1e-4 * abs(ref_loss)
    ref_g = dict(_flat(G))
    g_gpu = {n: g.cpu().numpy().astype(np.float64) for n, g in _flat(grads.g)}
    for name, g in g_gpu.items():
        assert_close(f"grad {name}", g, ref_g[name], 1e-3)
    # 2. the update rule on the GPU's gradient.  Bound per tensor: the new
    # weight is stored in fp32 (one rounding, <= 2^-24 |p|, two ulps allowed)
    # and the update itself is computed in fp32 (relative 1e-5 of lr, which
    # covers 1 - b2 from the fp32 0.999)
    new_w = {n: p.cpu().numpy().astype(np.float64) for n, p in _flat(dm.w)}
    for name, g in g_gpu.items():
        if optimizer == "adam":
            want, mo, vo = online.adam_update(old[name], g, 0.0, 0.0, 1, lr, clip)
            # moments in fp32 arithmetic: 1 - b2 from the fp32 0.999 is 1.3e-5 away
            # from 0.001 (the page's AdamStep holds b1, b2 as f32 too)
            assert_close(f"adam m {name}", dict(_flat(am.g))[name].cpu().numpy(), mo, 1e-4)
            assert_close(f"adam v {name}", dict(_flat(av.g))[name].cpu().numpy(), vo, 1e-4)
        else:
            want = online.sgd_update(old[name], g, lr, clip)
        err = float(np.max(np.abs(new_w[name] - want)))
        bound = 2.0 ** -23 * float(np.max(np.abs(want))) + 1e-5 * lr
        assert err <= bound, f"update {name}: |p_new - rule| {err:.3e} > {bound:.3e}"
    # 3. the live state: the segment replayed with the updated weights
    m_new = {k: v for k, v in m.items() if k != "blocks"}
    for k in list(m_new):
        if new_w.get(k) is not None:
            m_new[k] = new_w[k]
    m_new["blocks"] = []
    for l, b in enumerate(m["blocks"]):
        nb = {k: new_w[f"{k}[{l}]"] for k in b if k != "tm"}
        nb["tm"] = {k: new_w[f"tm.{k}[{l}]"] for k in b["tm"]}
        m_new["blocks"].append(nb)
    _, ref_state = stack.forward(m_new, cfg, tok, st32)
    for k in state:
        assert_close(f"state {k}", state[k].cpu().numpy(), ref_state[k], 1e-4)


def test_online_segment_zero_rate_state_matches_decode(hip):
    """lr = 0: the live state after the segment equals decoding its tokens one
    at a time with rwkv7_decode_step from the same start state."""
    from rwkv_linear_attention_wkv7_amd import binding
    m, cfg, dm, st, tok, tgt = _setup(hip, seed=21, S=17)
    grads = binding.TrainGrads(dm)
    s1 = {k: _dev(v.astype(np.float32)) for k, v in st.items()}
    s2 = {k: v.clone() for k, v in s1.items()}
    print("[online] zero rate vs decode", flush=True)
    hip.rwkv7_online_segment(dm, grads, _dev(tok), _dev(tgt), s1, optimizer="sgd", lr=0.0)
    for t in range(tok.shape[1]):
        hip.rwkv7_decode_step(dm, _dev(np.ascontiguousarray(tok[:, t])), s2)
    torch.cuda.synchronize()
    for k in s1:
        assert_close(k, s1[k].cpu().numpy(), s2[k].cpu().numpy().astype(np.float64), 1e-4)
