"""C-ABI checks that run without a GPU.

The library must export every function declared in include/*.h, and every
argument error must be reported (with a message) before anything touches the
device, so the error paths are exercised here with host-side calls only.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    from rwkv_linear_attention_wkv7_amd import binding
    return binding.lib()


@pytest.fixture(scope="module")
def Lfake(L):
    """The library, for calls made with fake device addresses.  Every such
    call must fail validation; so that a check that wrongly passed could never
    launch a kernel on those addresses, these tests run only on a host that
    sees no GPU."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("calls with fake device addresses run only where no GPU is visible")
    return L


def test_header_declares_the_five_calls():
    names = _declared_functions()
    for n in ("wkv7_forward", "wkv7_backward", "wkv7_step", "timemix_forward", "timemix_backward"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/ but not exported"


def _err(L):
    return L.wkv7_last_error().decode()


A = ctypes.c_void_p(4096)      # aligned fake device address: never dereferenced here
MIS = ctypes.c_void_p(4100)    # misaligned


def _fwd(L, B=1, T=4, H=2, N=64, dtype=0, ptrs=None, s0=None):
    p = ptrs or [A] * 7
    return L.wkv7_forward(B, T, H, N, dtype, *p[:6], s0, p[6], None, None, None, 0, None)


def test_forward_rejects_bad_shapes(Lfake):
    L = Lfake
    assert _fwd(L, N=32) == -1 and "N=32" in _err(L)
    assert _fwd(L, T=0) == -1 and ">= 1" in _err(L)
    assert _fwd(L, B=0) == -1
    assert _fwd(L, H=0) == -1
    assert _fwd(L, dtype=7) == -1 and "dtype" in _err(L)


def test_forward_rejects_null_and_misaligned(Lfake):
    L = Lfake
    assert _fwd(L, ptrs=[A, A, None, A, A, A, A]) == -1 and "k is NULL" in _err(L)
    assert _fwd(L, ptrs=[A, A, A, A, A, A, None]) == -1 and "y is NULL" in _err(L)
    assert _fwd(L, ptrs=[A, MIS, A, A, A, A, A]) == -1 and "aligned" in _err(L)
    assert _fwd(L, s0=MIS) == -1 and "s0" in _err(L)
    # bf16 data only needs 8-byte alignment
    mis8 = ctypes.c_void_p(4104)
    rc = L.wkv7_forward(1, 4, 2, 64, 1, mis8, A, A, A, A, A, None, ctypes.c_void_p(4098), None, None,
                        None, 0, None)
    assert rc == -1 and "y is not 8-byte aligned" in _err(L)


def test_forward_workspace_size_and_check(Lfake):
    L = Lfake
    # short sequences run token by token: no workspace
    assert L.wkv7_forward_workspace_bytes(2, 31, 4, 64) == 0
    need = L.wkv7_forward_workspace_bytes(2, 64, 4, 64)
    assert need > 0 and need % 16 == 0
    assert L.wkv7_forward_workspace_bytes(2, 65, 4, 64) > need  # one more chunk
    # the chunked path can be asked for at any B*H once T spans two chunks
    assert L.wkv7_forward_workspace_bytes(4, 8192, 32, 64) > 0
    assert L.wkv7_forward_workspace_bytes(1, 8192, 63, 64) > 0
    p = [A] * 7
    rc = L.wkv7_forward(2, 64, 4, 64, 0, *p[:6], None, p[6], None, None, A, need - 4, None)
    assert rc == -3 and "workspace" in _err(L)


def test_backward_needs_workspace_without_checkpoints(Lfake):
    L = Lfake
    need = L.wkv7_backward_workspace_bytes(1, 64, 4, 64, 0)
    have = L.wkv7_backward_workspace_bytes(1, 64, 4, 64, 1)
    assert need >= have + L.wkv7_checkpoint_floats(1, 64, 4, 64) * 4
    assert have > 0   # column partials of the row-split reverse pass
    ptr13 = [A] * 13
    rc = L.wkv7_backward(1, 64, 4, 64, 0, *ptr13[:6], None, None, ptr13[6], None, *ptr13[7:13],
                         None, A, need - 1, None, None)
    assert rc == -3 and "workspace" in _err(L)


def test_step_rejects_null_state(Lfake):
    L = Lfake
    rc = L.wkv7_step(2, 4, 64, 0, A, A, A, A, A, A, None, A, None)
    assert rc == -1 and "state is NULL" in _err(L)
    assert L.wkv7_step(2, 4, 48, 0, A, A, A, A, A, A, A, A, None) == -1


def test_checkpoint_sizes(L):
    """Checkpoint buffer: the state every Lc tokens, then the forward's
    per-token sa (one N-vector per token and head)."""
    Lc = L.wkv7_checkpoint_interval()
    assert Lc >= 1
    for T in (1, Lc, Lc + 1, 8192):
        assert L.wkv7_checkpoint_floats(4, T, 32, 64) == 4 * 32 * (-(-T // Lc)) * 64 * 64 + 4 * T * 32 * 64
    assert L.wkv7_checkpoint_floats(4, 16, 32, 32) == 0


def _tm(C=256, H=4, Dw=32, Da=32, Dv=32, Dg=64, layer=1, N=64):
    from rwkv_linear_attention_wkv7_amd import binding
    return binding.TmShape(C, H, N, Dw, Da, Dv, Dg, layer)


def _weights(layer):
    from rwkv_linear_attention_wkv7_amd import binding
    w = binding.TmWeights()
    for n in binding.WEIGHT_FIELDS:
        setattr(w, n, None if (layer == 0 and n in ("v0", "V1", "V2")) else 4096)
    return w


def test_timemix_forward_validation(Lfake):
    L = Lfake
    w = _weights(1)
    s = _tm(C=250)
    rc = L.timemix_forward(ctypes.byref(s), ctypes.byref(w), 2, 8, A, None, A, None, None, A, None,
                           None, A, 1 << 30, None)
    assert rc == -1 and "C=250" in _err(L)
    s = _tm(Dw=30)
    rc = L.timemix_forward(ctypes.byref(s), ctypes.byref(w), 2, 8, A, None, A, None, None, A, None,
                           None, A, 1 << 30, None)
    assert rc == -1 and "multiples of 4" in _err(L)
    s = _tm()
    need = L.timemix_forward_workspace_bytes(ctypes.byref(s), 2, 8)
    rc = L.timemix_forward(ctypes.byref(s), ctypes.byref(w), 2, 8, A, None, A, None, None, A, None,
                           None, A, need - 1, None)
    assert rc == -3 and "workspace" in _err(L)
    w0 = _weights(0)  # layer > 0 needs the value-residual LoRA
    rc = L.timemix_forward(ctypes.byref(s), ctypes.byref(w0), 2, 8, A, None, A, None, None, A,
                           None, None, A, need, None)
    assert rc == -1 and "v0" in _err(L)


def test_timemix_backward_validation(Lfake):
    L = Lfake
    from rwkv_linear_attention_wkv7_amd import binding
    s = _tm(layer=0)
    w = _weights(0)
    g = binding.TmGrads()
    for n in binding.WEIGHT_FIELDS:
        setattr(g, n, 4096)
    g.Wk = None
    need = L.timemix_backward_workspace_bytes(ctypes.byref(s), 2, 8)
    assert need > L.timemix_cache_bytes(ctypes.byref(s), 2, 8)
    rc = L.timemix_backward(ctypes.byref(s), ctypes.byref(w), 2, 8, A, None, None, None, A, None,
                            None, ctypes.byref(g), A, None, None, None, None, A, need, None, None)
    assert rc == -1 and "gradient" in _err(L)
    g.Wk = 4096
    rc = L.timemix_backward(ctypes.byref(s), ctypes.byref(w), 2, 8, A, None, None, None, A, None,
                            None, ctypes.byref(g), A, None, None, None, None, A, need - 1, None, None)
    assert rc == -3


# ---------------------------------------------------------------- aliasing --
# Every call rejects a written tensor that overlaps another of its tensors.
# The fake addresses below are spaced 256 MiB apart, so only the overlaps a
# test creates on purpose exist; every case fails validation, so nothing is
# ever launched.
_SP = 1 << 28


def _addrs(n, base=1 << 32):
    return [ctypes.c_void_p(base + i * _SP) for i in range(n)]


def _fwd_alias(L, p, s0=None, sT=None, ckpt=None):
    return L.wkv7_forward(1, 64, 2, 64, 0, *p[:6], s0, p[6], sT, ckpt, None, 0, None)


def test_forward_rejects_overlapping_outputs(Lfake):
    L = Lfake
    p = _addrs(10)
    q = p[:6] + [p[0]]                       # y == r
    assert _fwd_alias(L, q) == -1 and "overlaps" in _err(L) and "y" in _err(L)
    q = p[:6] + [ctypes.c_void_p(p[3].value + 4096)]   # y inside v
    assert _fwd_alias(L, q) == -1 and "overlaps" in _err(L)
    # sT overlapping (not equal to) s0
    assert _fwd_alias(L, p[:7], s0=p[7], sT=ctypes.c_void_p(p[7].value + 64)) == -1
    assert "sT" in _err(L) and "s0" in _err(L)
    # checkpoints over an input
    assert _fwd_alias(L, p[:7], ckpt=p[2]) == -1 and "ckpt" in _err(L)


def test_backward_rejects_overlaps(Lfake):
    L = Lfake
    p = _addrs(20)
    need = L.wkv7_backward_workspace_bytes(1, 64, 2, 64, 1)

    def bwd(ptr13, s0=None, ckpt=p[14], dsT=None, ds0=None, ws=p[15]):
        return L.wkv7_backward(1, 64, 2, 64, 0, *ptr13[:6], s0, ckpt, ptr13[6], dsT, *ptr13[7:13],
                               ds0, ws, need, None, None)

    base = p[:13]
    q = list(base)
    q[7] = q[6]                               # dr == dy
    assert bwd(q) == -1 and "overlaps" in _err(L)
    assert bwd(base, ds0=ctypes.c_void_p(p[15].value + 1024)) == -1   # ds0 inside ws
    assert "ds0" in _err(L) or "ws" in _err(L)
    assert bwd(base, dsT=p[16], ds0=p[16]) == -1 and "ds0" in _err(L)  # no in-place state gradient
    q = list(base)
    q[12] = p[14]                             # db over the checkpoints
    assert bwd(q) == -1 and "ckpt" in _err(L)


def test_step_rejects_output_over_state(Lfake):
    L = Lfake
    p = _addrs(9)
    rc = L.wkv7_step(2, 4, 64, 0, *p[:6], p[7], ctypes.c_void_p(p[7].value + 256), None)
    assert rc == -1 and "overlaps" in _err(L)
    rc = L.wkv7_step(2, 4, 64, 0, *p[:6], p[7], p[1], None)   # y == w
    assert rc == -1 and "overlaps" in _err(L)


def _tm_weights_at(base, layer):
    from rwkv_linear_attention_wkv7_amd import binding
    w = binding.TmWeights()
    for i, n in enumerate(binding.WEIGHT_FIELDS):
        setattr(w, n, None if (layer == 0 and n in ("v0", "V1", "V2")) else base + i * _SP)
    return w


def test_timemix_rejects_overlaps(Lfake):
    L = Lfake
    from rwkv_linear_attention_wkv7_amd import binding
    s = _tm(layer=1)
    w = _tm_weights_at(1 << 40, 1)
    x, xp, vf, s0, sT, out, xl, ws = _addrs(8, base=1 << 44)
    need = L.timemix_forward_workspace_bytes(ctypes.byref(s), 2, 8)

    def fwd(**kw):
        a = dict(x=x, xp=xp, vf=vf, s0=s0, sT=sT, out=out, xl=xl, ws=ws)
        a.update(kw)
        return L.timemix_forward(ctypes.byref(s), ctypes.byref(w), 2, 8, a["x"], a["xp"], a["vf"],
                                 a["s0"], a["sT"], a["out"], a["xl"], None, a["ws"], need, None)

    assert fwd(out=x) == -1 and "overlaps" in _err(L)
    assert fwd(out=ctypes.c_void_p(w.Wo)) == -1 and "Wo" in _err(L)    # output over a weight
    assert fwd(xl=xp) == -1 and "x_last" in _err(L)   # in place only for one token
    assert fwd(ws=ctypes.c_void_p(out.value + 256)) == -1
    # backward: a gradient over a weight, dx over dout
    g = binding.TmGrads()
    for i, n in enumerate(binding.WEIGHT_FIELDS):
        setattr(g, n, (1 << 42) + i * _SP)
    nb = L.timemix_backward_workspace_bytes(ctypes.byref(s), 2, 8)
    dout, dx = _addrs(2, base=1 << 45)

    def bwd(dxp=dx):
        return L.timemix_backward(ctypes.byref(s), ctypes.byref(w), 2, 8, x, None, vf, None, dout,
                                  None, None, ctypes.byref(g), dxp, None, None, None, None, ws, nb,
                                  None, None)
    assert bwd(dxp=dout) == -1 and "overlaps" in _err(L)
    g.Wk = w.Wk
    assert bwd() == -1 and "Wk" in _err(L)


def test_gemm_rejects_output_over_operand(Lfake):
    L = Lfake
    a, b = _addrs(2)
    assert L.wkv7_gemm_f32(0, 0, 64, 64, 64, a, 64, b, 64, a, 64, 0.0, None) == -1
    assert "overlaps" in _err(L)
    c = ctypes.c_void_p(b.value + 64 * 63 * 4)   # C starts in B's last row
    assert L.wkv7_gemm_bf16(0, 0, 64, 64, 64, a, 64, b, 64, c, 64, 0.0, None, 0, None) == -1


def test_gemm_bf16_workspace(L, Lfake):
    """The bf16-copy workspace: (M + N) K bf16 values for whole 256 x 128
    tiles with K a multiple of 64 and A not transposed, else none; a given
    workspace smaller than that is ENOSPC, one overlapping C is EINVAL."""
    q = L.wkv7_gemm_bf16_workspace_bytes
    assert q(0, 0, 8192, 4096, 1024) == (8192 + 4096) * 1024 * 2
    assert q(0, 1, 8192, 1024, 4096) == (8192 + 1024) * 4096 * 2
    assert q(1, 0, 1024, 4096, 8192) == 0          # X^T dY reads fp32
    assert q(0, 0, 8192, 4096, 96) == 0            # K not a multiple of 64
    assert q(0, 0, 100, 4096, 1024) == 0           # M not a multiple of 256
    a, b, c, w = _addrs(4, base=1 << 40)
    need = q(0, 0, 256, 128, 64)
    assert L.wkv7_gemm_bf16(0, 0, 256, 128, 64, a, 64, b, 128, c, 128, 0.0, w, need - 1, None) == -3
    assert "needs" in _err(L)
    assert L.wkv7_gemm_bf16(0, 0, 256, 128, 64, a, 64, b, 128, c, 128, 0.0, c, need, None) == -1
    assert "overlaps" in _err(L)


def test_side_stream_validation(Lfake):
    L = Lfake
    from rwkv_linear_attention_wkv7_amd import binding
    p = _addrs(16)
    need = L.wkv7_backward_workspace_bytes(1, 64, 2, 64, 1)
    sd = binding.Wkv7Side()
    sd.stream = 12345
    for i in range(3):
        sd.ev[i] = 1000 + i       # ev[3] left NULL
    rc = L.wkv7_backward(1, 64, 2, 64, 0, *p[:6], None, p[14], p[6], None, *p[7:13], None, p[15],
                         need, ctypes.byref(sd), None)
    assert rc == -1 and "ev[3]" in _err(L)
    assert L.wkv7_side_destroy(None) == 0


def test_backward_noalloc_rejects_shapes_beyond_its_scratch(Lfake):
    """The fixed-scratch backward refuses, before any device call, a shape
    whose scratch exceeds its 64 MiB array."""
    L = Lfake
    p = _addrs(16)
    B, T, H = 4, 8192, 32
    assert L.wkv7_backward_workspace_bytes(B, T, H, 64, 1) > (64 << 20)
    rc = L.wkv7_backward_noalloc(B, T, H, 64, 0, *p[:6], None, p[14], p[6], None, *p[7:13], None,
                                 None, None)
    assert rc == -3 and "fixed scratch" in _err(L)
    q = list(p[:13])
    q[8] = q[6]   # dw == dy: overlap checks as wkv7_backward
    rc = L.wkv7_backward_noalloc(1, 64, 2, 64, 0, *q[:6], None, p[14], q[6], None, *q[7:13], None,
                                 None, None)
    assert rc == -1 and "overlaps" in _err(L)
