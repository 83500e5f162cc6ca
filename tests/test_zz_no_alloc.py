"""wkv7_backward_noalloc (fixed device scratch, no allocation) against
wkv7_backward with a caller workspace, through the C-ABI: two calls in a
row, the second with a smaller input (the scratch keeps the first call's
contents), each compared bitwise with the workspace call (same kernels, same
order of arithmetic) and the second also with the f64 oracle."""
import numpy as np
import pytest
import torch

from oracle import wkv7 as ow
from rwkv_linear_attention_wkv7_amd import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
NAMES = ("r", "w", "k", "v", "a", "b")
GRADS = ("dr", "dw", "dk", "dv", "da", "db", "ds0")


def _case(hip, B, T, H, seed, with_ckpt, dtype):
    d = synth.wkv7_inputs(B, T, H, 64, seed=seed, with_state=True, bf16=dtype == torch.bfloat16)
    dev = lambda x, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(dt)
    ins = [dev(d[n], dtype) for n in NAMES]
    s0, dsT, dy = dev(d["s0"]), dev(d["dsT"]), dev(d["dy"], dtype)
    ck = None
    if with_ckpt:
        _, _, ck = hip.wkv7_forward(*ins, s0=s0, want_ckpt=True)
    print(f"[no-alloc] B={B} T={T} H={H} ckpt={with_ckpt} dtype={dtype}", flush=True)
    ref = hip.wkv7_backward(*ins, dy, s0=s0, ckpt=ck, dsT=dsT)
    out = {n: torch.full_like(ref[n], float("nan")) for n in GRADS}
    got = hip.wkv7_backward_noalloc(*ins, dy, s0=s0, ckpt=ck, dsT=dsT, out=out)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(got[n], ref[n]), n
    return d, got


def test_backward_noalloc_two_calls(hip):
    # first: no checkpoints (recomputed into the fixed scratch), several chunks
    _case(hip, 2, 300, 3, seed=41, with_ckpt=False, dtype=torch.float32)
    # second, smaller: the scratch still holds the first call's data
    d, got = _case(hip, 1, 40, 2, seed=42, with_ckpt=True, dtype=torch.float32)
    ins = [d[n].astype(np.float64) for n in NAMES]
    gr = ow.backward(*ins, d["dy"].astype(np.float64), s0=d["s0"].astype(np.float64),
                     dsT=d["dsT"].astype(np.float64))
    for n in GRADS:
        assert_close(n, got[n].cpu().numpy(), gr[n], 1e-3)


def test_backward_noalloc_bf16_and_long(hip):
    """bf16 tensors, and T = 2100, from the same scratch."""
    _case(hip, 1, 2100, 2, seed=43, with_ckpt=True, dtype=torch.float32)
    _case(hip, 2, 77, 2, seed=44, with_ckpt=False, dtype=torch.bfloat16)
