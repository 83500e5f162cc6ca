"""GPU parity of timemix_forward / timemix_backward against the f64 oracle.

Per tensor max|gpu - oracle| / max|oracle|: forward outputs <= 1e-4,
gradients <= 1e-3 (fp32 everywhere).
"""
import numpy as np
import pytest
import torch

from oracle import timemix as otm
from rwkv_linear_attention_wkv7_amd import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _case(hip, B, T, C, ranks, layer_id, with_state, seed, perturbed=True, use_cache=True,
          sample=None):
    from rwkv_linear_attention_wkv7_amd import binding
    H = C // 64
    Dw, Da, Dv, Dg = ranks
    p = synth.timemix_params(C, H, Dw, Da, Dv, Dg, layer_id, seed=seed, perturbed=perturbed)
    d = synth.timemix_inputs(B, T, C, seed=seed + 1, with_state=with_state, H=H)
    s = binding.tm_shape(C, H, Dw, Da, Dv, Dg, layer_id)
    W = {k: _dev(v) for k, v in p.items()}
    x, dout = _dev(d["x"]), _dev(d["dout"])
    x_prev = _dev(d["x_prev"])
    vf = _dev(d["v_first"]) if layer_id > 0 else None
    s0 = _dev(d["s0"]) if with_state else None
    dsT = _dev(d["dsT"]) if with_state else None
    dvf_in = _dev(d["v_first"] * 0.5) if layer_id == 0 else None
    print(f"[timemix] B={B} T={T} C={C} ranks={ranks} layer={layer_id} state={with_state}", flush=True)
    f = binding.timemix_forward(s, W, x, x_prev=x_prev, v_first=vf, s0=s0, want_cache=use_cache,
                                want_x_last=True)
    g = binding.timemix_backward(s, W, x, dout, x_prev=x_prev, v_first=vf, s0=s0, dsT=dsT,
                                 cache=f["cache"], dv_first_in=dvf_in)
    torch.cuda.synchronize()

    out_r, c = otm.forward(p, d["x"], H, layer_id, x_prev=d["x_prev"],
                           v_first=d["v_first"] if layer_id > 0 else None,
                           s0=d["s0"] if with_state else None)
    G, dx, dxp, dvf_out, ds0 = otm.backward(
        p, c, d["dout"], dsT=d["dsT"] if with_state else None,
        dv_first_in=(d["v_first"] * 0.5) if layer_id == 0 else None)
    np_ = lambda t: t.cpu().numpy()
    assert_close("out", np_(f["out"]), out_r, 1e-4)
    assert_close("sT", np_(f["sT"]), c["sT"], 1e-4)
    assert_close("x_last", np_(f["x_last"]), d["x"][:, -1], 0.0)
    if layer_id == 0:
        assert_close("v_first", np_(f["v_first"]), c["v_first"], 1e-4)
    errs = {}
    for n, ref in G.items():
        errs[n] = assert_close("d" + n, np_(g["grads"][n]), ref, 1e-3)
    assert set(G) == set(g["grads"])
    assert_close("dx", np_(g["dx"]), dx, 1e-3)
    assert_close("dx_prev", np_(g["dx_prev"]), dxp, 1e-3)
    assert_close("ds0", np_(g["ds0"]), ds0, 1e-3)
    if layer_id > 0:
        assert_close("dv_first", np_(g["dv_first_out"]), dvf_out, 1e-3)
    return errs


@pytest.mark.parametrize("layer_id", [0, 1])
def test_timemix_small(hip, layer_id):
    _case(hip, 2, 40, 256, (32, 32, 32, 64), layer_id, True, seed=20 + layer_id)


def test_timemix_no_cache_recompute(hip):
    _case(hip, 2, 19, 128, (16, 16, 16, 32), 1, True, seed=30, use_cache=False)


def test_timemix_single_token(hip):
    _case(hip, 3, 1, 256, (32, 32, 32, 64), 1, True, seed=40)


def test_timemix_default_init(hip):
    """The std-0.02 random-init weights of the benchmark (unperturbed vectors)."""
    _case(hip, 2, 33, 256, (32, 32, 32, 64), 1, False, seed=50, perturbed=False)


def test_timemix_full_size(hip):
    """B=8, T=1024, C=768 (H=12), ranks 64/64/32/128, layer > 0: the time-mix
    forward+backward configuration, every output element checked."""
    _case(hip, 8, 1024, 768, (64, 64, 32, 128), 1, False, seed=60, perturbed=False)
