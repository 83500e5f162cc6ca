"""GPU parity of the WKV7 kernels (through the C-ABI) against the f64 oracle.

Tolerances (per tensor, max|gpu - oracle| / max|oracle|): fp32 forward 1e-4,
fp32 gradients 1e-3, bf16 tensors 2e-2.  bf16 cases feed the oracle the same
bf16-rounded inputs widened exactly to f64.
"""
import numpy as np
import pytest
import torch

from oracle import wkv7 as ow
from rwkv_linear_attention_wkv7_amd import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
NAMES = ("r", "w", "k", "v", "a", "b")
GRADS = ("dr", "dw", "dk", "dv", "da", "db")


def _dev(x, dt=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dt).contiguous()


def _run(hip, d, dtype, with_state, chunked=True):
    ins = [_dev(d[n], dtype) for n in NAMES]
    s0 = _dev(d["s0"]) if with_state else None
    dsT = _dev(d["dsT"]) if with_state else None
    y, sT, ck = hip_forward(ins, s0, chunked)
    g = hip.wkv7_backward(*ins, _dev(d["dy"], dtype), s0=s0, ckpt=ck, dsT=dsT)
    torch.cuda.synchronize()
    return y, sT, g


def hip_forward(ins, s0, chunked=True):
    from rwkv_linear_attention_wkv7_amd import binding
    return binding.wkv7_forward(*ins, s0=s0, want_ckpt=True, chunked=chunked)


def _check(d, y, sT, g, with_state, ftol, gtol, sel=None):
    sel = sel or (slice(None), slice(None))
    pick = lambda x: np.asarray(x)[sel[0], :, sel[1]]
    ins = [pick(d[n]).astype(np.float64) for n in NAMES]
    s0 = d["s0"][sel].astype(np.float64) if with_state else None
    dsT = d["dsT"][sel].astype(np.float64) if with_state else None
    yr, sTr = ow.forward(*ins, s0=s0)
    gr = ow.backward(*ins, pick(d["dy"]).astype(np.float64), s0=s0, dsT=dsT)
    tofp = lambda t: t.float().cpu().numpy()
    assert_close("y", pick(tofp(y)), yr, ftol)
    assert_close("sT", tofp(sT)[sel], sTr, ftol)
    for n in GRADS:
        assert_close(n, pick(tofp(g[n])), gr[n], gtol)
    if with_state:
        assert_close("ds0", tofp(g["ds0"])[sel], gr["ds0"], gtol)


@pytest.mark.parametrize("B,T,H,with_state", [
    (1, 64, 4, False),     # the small fp32 configuration: B=1, T=64, H=4, N=64
    (2, 37, 3, True),      # ragged tail across checkpoint chunks, nonzero s0 / dsT
    (1, 1, 2, True),       # single token
    (3, 16, 1, False),     # exactly one checkpoint chunk
    (2, 130, 2, True),     # many chunks, ragged
    (6, 40, 24, True),     # 144 heads: 32-row forward workgroups, two backward slices
    (4, 130, 16, True),    # 576 (b, h, chunk) triples: the two-pass backward
])
@pytest.mark.parametrize("chunked", [True, False])
def test_wkv7_fp32_parity(hip, B, T, H, with_state, chunked):
    """chunked: the matrix-core chunked forward (T >= 32) or, False, the
    token-sequential forward; the backward recomputes from either's
    checkpoints."""
    d = synth.wkv7_inputs(B, T, H, 64, seed=B * 100 + T, with_state=with_state)
    print(f"[wkv7 fp32] B={B} T={T} H={H} state={with_state} chunked={chunked}", flush=True)
    y, sT, g = _run(hip, d, torch.float32, with_state, chunked)
    _check(d, y, sT, g, with_state, 1e-4, 1e-3)


@pytest.mark.parametrize("B,H", [(2, 2), (4, 24)])
def test_wkv7_extreme_decay(hip, B, H):
    """Decays far outside the time-mix range: chunks whose cumulative decay
    leaves the matrix-core path's exponent window (w = 1e-3 over a chunk, an
    exact w = 0) run token by token, others (w = 1: no decay at all) stay on
    the chunk path; forward and gradients against the oracle, fp32.  The
    backward of B=2 H=2 (28 chunk triples) runs the single-pass kernels
    directly; that of B=4 H=24 (672) starts the two-pass path, whose scan
    finds the decays outside [1/8, 1] and hands the call to them."""
    d = synth.wkv7_inputs(B, 100, H, 64, seed=21, with_state=True)
    w = d["w"].copy()
    w[:, 16:32] = 1e-3
    w[0, 40, 1, 5] = 0.0
    w[:, 64:80] = 1.0
    d["w"] = w
    print(f"[wkv7 extreme decay] B={B} T=100 H={H}", flush=True)
    y, sT, g = _run(hip, d, torch.float32, True)
    _check(d, y, sT, g, True, 1e-4, 1e-3)


@pytest.mark.parametrize("lo", [0.125, 0.2])
def test_wkv7_strong_decay_two_pass(hip, lo):
    """Decays spread over [lo, 1] (log-uniform), inside the range the two-pass
    backward serves (the decay of a 16-token chunk reaches 0.125^16, so its
    e^{+-g} factors span about e^{+-33}); ragged T, nonzero s0 and dsT; fp32
    forward and gradients against the oracle.  B=4 H=16 T=150: 640 (b, h,
    chunk) triples, above the size the single-pass kernels take directly."""
    d = synth.wkv7_inputs(4, 150, 16, 64, seed=41, with_state=True)
    g = np.random.default_rng(41)
    d["w"] = np.exp(np.log(lo) * g.random(d["w"].shape)).astype(np.float32)
    print(f"[wkv7 strong decay] B=4 T=150 H=16 w in [{lo}, 1]", flush=True)
    y, sT, gr = _run(hip, d, torch.float32, True, False)
    _check(d, y, sT, gr, True, 1e-4, 1e-3)


def test_wkv7_backward_without_checkpoints(hip):
    from rwkv_linear_attention_wkv7_amd import binding
    d = synth.wkv7_inputs(2, 40, 2, 64, seed=5, with_state=True)
    ins = [_dev(d[n]) for n in NAMES]
    s0, dsT, dy = _dev(d["s0"]), _dev(d["dsT"]), _dev(d["dy"])
    # the backward recomputes missing checkpoints with the token-sequential
    # forward, so it matches that forward's checkpoints bit for bit
    y, sT, ck = binding.wkv7_forward(*ins, s0=s0, want_ckpt=True, chunked=False)
    g1 = binding.wkv7_backward(*ins, dy, s0=s0, ckpt=ck, dsT=dsT)
    g2 = binding.wkv7_backward(*ins, dy, s0=s0, ckpt=None, dsT=dsT)
    torch.cuda.synchronize()
    for n in GRADS + ("ds0",):
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("chunked", [True, False])
def test_wkv7_bf16_parity(hip, chunked):
    d = synth.wkv7_inputs(2, 200, 3, 64, seed=7, bf16=True, with_state=True)
    y, sT, g = _run(hip, d, torch.bfloat16, True, chunked)
    _check(d, y, sT, g, True, 2e-2, 2e-2)


@pytest.mark.parametrize("chunked", [False, True])
def test_wkv7_bf16_long_context_full_size(hip, chunked):
    """B=4, T=8192, H=32 bf16 (the long-context configuration), checked on
    sampled (b, h) pairs: the recurrence of each (b, h) is independent.
    chunked=False is the token-sequential forward the benchmark times; True
    asks for the chunked matrix-core forward at the same size."""
    B, T, H = 4, 8192, 32
    d = synth.wkv7_inputs(B, T, H, 64, seed=3, bf16=True)
    print(f"[wkv7 long bf16] B={B} T={T} H={H} chunked={chunked}", flush=True)
    y, sT, g = _run(hip, d, torch.bfloat16, False, chunked)
    for (b, h) in ((0, 0), (3, 31), (1, 17), (2, 5)):
        _check(d, y, sT, g, False, 2e-2, 2e-2, sel=(slice(b, b + 1), slice(h, h + 1)))


def test_wkv7_backward_segments(hip):
    """T = 4200: the backward call runs its reverse pass as two launches (the
    state gradient handed from one to the next) with each segment's column
    reduction on a second stream; ragged last chunk, nonzero s0 and dsT,
    ds0 checked; fp32 against the oracle."""
    B, T, H = 1, 4200, 2
    d = synth.wkv7_inputs(B, T, H, 64, seed=21, with_state=True)
    print(f"[wkv7 segments] B={B} T={T} H={H}", flush=True)
    y, sT, g = _run(hip, d, torch.float32, True, False)
    _check(d, y, sT, g, True, 1e-4, 1e-3)


def test_wkv7_chunked_long_few_heads(hip):
    """B=1, T=4096, H=16: few (b, h) pairs and a long sequence through the
    chunked matrix-core forward (256 chunks per head, state carried across
    all of them); fp32, sampled heads against the oracle."""
    B, T, H = 1, 4096, 16
    d = synth.wkv7_inputs(B, T, H, 64, seed=13, with_state=True)
    print(f"[wkv7 chunked long] B={B} T={T} H={H}", flush=True)
    y, sT, g = _run(hip, d, torch.float32, True, True)
    for h in (0, 9, 15):
        _check(d, y, sT, g, True, 1e-4, 1e-3, sel=(slice(0, 1), slice(h, h + 1)))


def test_wkv7_state_passing_and_determinism(hip):
    from rwkv_linear_attention_wkv7_amd import binding
    d = synth.wkv7_inputs(2, 50, 2, 64, seed=9, with_state=True)
    ins = [_dev(d[n]) for n in NAMES]
    s0 = _dev(d["s0"])
    y, sT, _ = binding.wkv7_forward(*ins, s0=s0)
    y1, s1, _ = binding.wkv7_forward(*[x[:, :21].contiguous() for x in ins], s0=s0)
    y2, s2, _ = binding.wkv7_forward(*[x[:, 21:].contiguous() for x in ins], s0=s1)
    yb, sTb, _ = binding.wkv7_forward(*ins, s0=s0)
    torch.cuda.synchronize()
    assert torch.equal(y, yb) and torch.equal(sT, sTb)   # run-to-run bitwise
    assert torch.allclose(torch.cat([y1, y2], 1), y, rtol=1e-5, atol=1e-5)
    assert torch.allclose(s2, sT, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("dtype,tol", [(torch.float32, 1e-4), (torch.bfloat16, 2e-2)])
def test_wkv7_step_parity(hip, dtype, tol):
    from rwkv_linear_attention_wkv7_amd import binding
    B, H, T = 5, 3, 6
    d = synth.wkv7_inputs(B, T, H, 64, seed=11, bf16=dtype == torch.bfloat16, with_state=True)
    state = _dev(d["s0"])
    S = d["s0"].astype(np.float64)
    for t in range(T):
        ins = [_dev(d[n][:, t], dtype) for n in NAMES]
        y = binding.wkv7_step(*ins, state)
        yr, S = ow.step(*(d[n][:, t].astype(np.float64) for n in NAMES), state=S)
        torch.cuda.synchronize()
        assert_close(f"y[{t}]", y.float().cpu().numpy(), yr, tol)
    assert_close("state", state.cpu().numpy(), S, tol)


def test_wkv7_step_decode_size(hip):
    """2048 streams x 4 heads (the decode configuration's per-layer state)."""
    from rwkv_linear_attention_wkv7_amd import binding
    B, H = 2048, 4
    d = synth.wkv7_inputs(B, 1, H, 64, seed=12, with_state=True)
    state = _dev(d["s0"])
    ins = [_dev(d[n][:, 0]) for n in NAMES]
    y = binding.wkv7_step(*ins, state)
    torch.cuda.synchronize()
    idx = [0, 2047, 1000, 513]
    yr, Sr = ow.step(*(d[n][idx, 0].astype(np.float64) for n in NAMES), state=d["s0"][idx].astype(np.float64))
    assert_close("y", y.cpu().numpy()[idx], yr, 1e-4)
    assert_close("state", state.cpu().numpy()[idx], Sr, 1e-4)
