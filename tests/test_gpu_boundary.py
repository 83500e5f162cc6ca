"""GPU checks of the C-ABI's stated behaviour beyond the parity numbers: the
permitted in-place updates give the out-of-place results, the side stream
only moves work (results bitwise equal with and without it), and the
training step's handling of token ids and targets outside the vocabulary
matches the oracle (ignored targets as the fullmodel page's ignore_index)."""
import numpy as np
import pytest
import torch

from oracle import stack
from rwkv_linear_attention_wkv7_amd import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
NAMES = ("r", "w", "k", "v", "a", "b")


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def test_wkv7_forward_in_place_state(hip):
    d = synth.wkv7_inputs(2, 45, 3, 64, seed=31, with_state=True)
    ins = [_dev(d[n]) for n in NAMES]
    s0 = _dev(d["s0"])
    print("[boundary] wkv7_forward sT == s0, B=2 T=45 H=3", flush=True)
    y, sT, _ = hip.wkv7_forward(*ins, s0=s0)
    st = s0.clone()
    y2, sT2, _ = hip.wkv7_forward(*ins, s0=st, sT=st)
    torch.cuda.synchronize()
    assert sT2.data_ptr() == st.data_ptr()
    assert torch.equal(y, y2) and torch.equal(sT, st)


def test_wkv7_backward_side_stream_bitwise(hip):
    """T = 4200 with and without a side stream (accepted, every launch on the
    caller's stream): the same bits."""
    d = synth.wkv7_inputs(1, 4200, 2, 64, seed=32, with_state=True)
    ins = [_dev(d[n]) for n in NAMES]
    s0, dsT, dy = _dev(d["s0"]), _dev(d["dsT"]), _dev(d["dy"])
    print("[boundary] wkv7_backward side vs none, T=4200", flush=True)
    _, _, ck = hip.wkv7_forward(*ins, s0=s0, want_ckpt=True)
    g1 = hip.wkv7_backward(*ins, dy, s0=s0, ckpt=ck, dsT=dsT, side=True)
    g2 = hip.wkv7_backward(*ins, dy, s0=s0, ckpt=ck, dsT=dsT, side=False)
    torch.cuda.synchronize()
    for n in ("dr", "dw", "dk", "dv", "da", "db", "ds0"):
        assert torch.equal(g1[n], g2[n]), n


def test_timemix_side_stream_and_in_place(hip):
    B, T, C, H = 2, 33, 128, 2
    p = synth.timemix_params(C, H, 16, 16, 16, 32, 1, seed=33, perturbed=True)
    t = synth.timemix_inputs(B, T, C, seed=34, with_state=True, H=H)
    s = hip.tm_shape(C, H, 16, 16, 16, 32, 1)
    W = {k: _dev(v) for k, v in p.items()}
    x, dout, vf, s0 = (_dev(t[k]) for k in ("x", "dout", "v_first", "s0"))
    print("[boundary] timemix side vs none, in-place state", flush=True)
    f = hip.timemix_forward(s, W, x, v_first=vf, s0=s0, want_cache=True)
    b1 = hip.timemix_backward(s, W, x, dout, v_first=vf, s0=s0, cache=f["cache"], side=True)
    b2 = hip.timemix_backward(s, W, x, dout, v_first=vf, s0=s0, cache=f["cache"], side=False)
    torch.cuda.synchronize()
    for k in b1["grads"]:
        assert torch.equal(b1["grads"][k], b2["grads"][k]), k
    assert torch.equal(b1["dx"], b2["dx"]) and torch.equal(b1["ds0"], b2["ds0"])
    # the state updated in place: sT == s0 through the C-ABI
    from rwkv_linear_attention_wkv7_amd import binding
    import ctypes
    st = s0.clone()
    out = torch.empty_like(x)
    cw = binding._pack_weights(s, W)
    nbytes = binding.timemix_cache_bytes(s, B, T)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    binding._check(binding.lib().timemix_forward(
        ctypes.byref(s), ctypes.byref(cw), B, T, binding._p(x), None, binding._p(vf),
        binding._p(st), binding._p(st), binding._p(out), None, None, binding._p(ws), nbytes,
        binding._stream()))
    torch.cuda.synchronize()
    assert torch.equal(out, f["out"]) and torch.equal(st, f["sT"])


def test_decode_side_stream_bitwise(hip):
    """1540 streams: two stream groups, on two streams or one after the other."""
    from rwkv_linear_attention_wkv7_amd import binding
    L, C, H, F, V, B = 2, 128, 2, 256, 64, 1540
    m = synth.stack_model(C, H, F, V, L, (16, 16, 16, 32), seed=35, perturbed=True, std=0.2)
    d = lambda x: None if x is None else _dev(x)
    wm = {k: d(v) for k, v in m.items() if k != "blocks"}
    wm["blocks"] = [{k: ({kk: d(vv) for kk, vv in v.items()} if k == "tm" else d(v))
                     for k, v in b.items()} for b in m["blocks"]]
    dm = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=(16, 16, 16, 32)), wm)
    tok = _dev(synth.token_ids(B, 3, V, seed=36))
    print(f"[boundary] decode side vs none, B={B}", flush=True)
    s1, s2 = dm.new_state(B), dm.new_state(B)
    for t in range(3):
        cur = tok[:, t].contiguous()
        l1 = hip.rwkv7_decode_step(dm, cur, s1, side=True)
        l2 = hip.rwkv7_decode_step(dm, cur, s2, side=False)
        torch.cuda.synchronize()
        assert torch.equal(l1, l2), t
    for k in s1:
        assert torch.equal(s1[k], s2[k]), k


@pytest.mark.parametrize("use_ln0", [False, True])
def test_train_step_unknown_ids_and_ignored_targets(hip, use_ln0):
    """Token ids outside [0, V) embed as zero rows and get no embedding
    gradient; targets outside [0, V) are ignored (zero dlogits row, not
    counted in the mean); fp32 GEMMs against the f64 oracle at 1e-3."""
    from rwkv_linear_attention_wkv7_amd import binding
    L, C, H, F, V, B, T = 2, 128, 2, 256, 256, 2, 24
    ranks = (16, 16, 16, 32)
    m = synth.stack_model(C, H, F, V, L, ranks, seed=37, perturbed=True, std=0.2, use_ln0=use_ln0)
    d = lambda x: None if x is None else _dev(x)
    wm = {k: d(v) for k, v in m.items() if k != "blocks"}
    wm["blocks"] = [{k: ({kk: d(vv) for kk, vv in v.items()} if k == "tm" else d(v))
                     for k, v in b.items()} for b in m["blocks"]]
    dm = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=ranks, use_ln0=int(use_ln0)),
                             wm)
    grads = binding.TrainGrads(dm)
    x = synth.token_ids(B, T, V, seed=38)
    y = synth.token_ids(B, T, V, seed=39)
    x[0, 3], x[1, 10], x[1, 11] = -5, V, V + 100
    y[0, 0], y[1, 7], y[1, 23] = -1, V, -100
    print(f"[boundary] train step with unknown ids / ignored targets, ln0={use_ln0}", flush=True)
    loss = float(hip.rwkv7_train_step(dm, grads, _dev(x), _dev(y)).item())
    ref_loss, G = stack.train_step(m, dict(C=C, H=H, F=F, V=V, n_layer=L), x, y)
    assert abs(loss - ref_loss) <= 1e-4 * abs(ref_loss), (loss, ref_loss)
    g = grads.g
    assert_close("emb", g["emb"].cpu().numpy(), G["emb"], 1e-3)
    assert_close("head", g["head"].cpu().numpy(), G["head"], 1e-3)
    for l in range(L):
        for k in ("ln1_w", "cm_Wk", "cm_Wv"):
            assert_close(f"{k}[{l}]", g["blocks"][l][k].cpu().numpy(), G["blocks"][l][k], 1e-3)
        for k in ("Wr", "w0", "k_k"):
            assert_close(f"tm.{k}[{l}]", g["blocks"][l]["tm"][k].cpu().numpy(),
                         G["blocks"][l]["tm"][k], 1e-3)
    # every target ignored: loss 0, zero head gradient
    yall = np.full_like(y, -1)
    loss0 = float(hip.rwkv7_train_step(dm, grads, _dev(x), _dev(yall)).item())
    torch.cuda.synchronize()
    assert loss0 == 0.0 and not torch.any(grads.g["head"]).item()
