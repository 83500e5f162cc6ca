"""ctypes binding of the C-ABI in ``include/wkv7.h`` (argument marshalling only).

Each function has the name of the C call it wraps.  PyTorch supplies device
memory and the current HIP stream; every step of the computation runs in the
HIP library.  Output and workspace tensors are allocated here with
``torch.empty`` when the caller does not pass them.  If the library has not
been built this module raises instead of falling back to anything else.
"""
import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libwkv7_amd.so")

WKV7_F32, WKV7_BF16 = 0, 1
WEIGHT_FIELDS = ("mu_r", "mu_w", "mu_k", "mu_v", "mu_a", "mu_g", "Wr", "Wk", "Wv", "Wo",
                 "w0", "W1", "W2", "a0", "A1", "A2", "v0", "V1", "V2", "G1", "G2",
                 "k_k", "k_a", "r_k", "ln_w", "ln_b")


class TmShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("C", "H", "N", "Dw", "Da", "Dv", "Dg", "layer_id")]


class TmWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class TmGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class Rwkv7Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("n_layer", "C", "H", "N", "F", "V", "Dw", "Da", "Dv",
                                            "Dg", "use_ln0", "gemm_dtype", "train_recompute",
                                            "n_attn", "moba_chunk", "moba_topk")]


ATTN_FIELDS = ("ln1_w", "ln1_b", "ln2_w", "ln2_b", "Wq", "Wk", "Wv", "Wo", "cm_mu_k", "cm_Wk",
               "cm_Wv")


class Rwkv7AttnBlock(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ATTN_FIELDS]


class Rwkv7AttnGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ATTN_FIELDS]


class Rwkv7Block(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_void_p) for n in ("ln1_w", "ln1_b", "ln2_w", "ln2_b")] +
                [("tm", TmWeights)] +
                [(n, ctypes.c_void_p) for n in ("cm_mu_k", "cm_Wk", "cm_Wv")])


class Rwkv7Model(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("emb", "ln0_w", "ln0_b", "ln_out_w", "ln_out_b",
                                               "head")] + [("blocks", ctypes.POINTER(Rwkv7Block)),
                                                           ("attn", ctypes.POINTER(Rwkv7AttnBlock))]


class Rwkv7BlockGrads(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_void_p) for n in ("ln1_w", "ln1_b", "ln2_w", "ln2_b")] +
                [("tm", TmGrads)] +
                [(n, ctypes.c_void_p) for n in ("cm_mu_k", "cm_Wk", "cm_Wv")])


class Rwkv7ModelGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("emb", "ln0_w", "ln0_b", "ln_out_w", "ln_out_b",
                                               "head")] + [("blocks", ctypes.POINTER(Rwkv7BlockGrads)),
                                                           ("attn", ctypes.POINTER(Rwkv7AttnGrads))]


class GdnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("nk", "nv", "dk", "dv", "kk")] + [("rms_eps", ctypes.c_float)]


class GdnWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("conv", "A_log", "dt_bias", "norm")]


class Rwkv7Optim(ctypes.Structure):
    _fields_ = [("optimizer", ctypes.c_int), ("lr", ctypes.c_float), ("clip", ctypes.c_float),
                ("step", ctypes.c_int)]


class Wkv7Side(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("ev", ctypes.c_void_p * 4)]


class Wkv7Error(RuntimeError):
    pass


_lib = None
_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Wkv7Error(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.wkv7_last_error.restype = ctypes.c_char_p
        L.wkv7_checkpoint_interval.restype = _i
        L.wkv7_checkpoint_floats.argtypes = [_i] * 4
        L.wkv7_checkpoint_floats.restype = _sz
        L.wkv7_forward_workspace_bytes.argtypes = [_i] * 4
        L.wkv7_forward_workspace_bytes.restype = _sz
        L.wkv7_forward.argtypes = [_i] * 5 + [_vp] * 11 + [_sz, _vp]
        L.wkv7_forward.restype = _i
        L.wkv7_backward_workspace_bytes.argtypes = [_i] * 5
        L.wkv7_backward_workspace_bytes.restype = _sz
        L.wkv7_backward.argtypes = [_i] * 5 + [_vp] * 17 + [_vp, _sz, _vp, _vp]
        L.wkv7_backward.restype = _i
        L.wkv7_backward_noalloc.argtypes = [_i] * 5 + [_vp] * 17 + [_vp, _vp]
        L.wkv7_backward_noalloc.restype = _i
        L.wkv7_step.argtypes = [_i] * 4 + [_vp] * 9
        L.wkv7_step.restype = _i
        sp = ctypes.POINTER(TmShape)
        for fn in ("timemix_cache_bytes", "timemix_forward_workspace_bytes",
                   "timemix_backward_workspace_bytes"):
            getattr(L, fn).argtypes = [sp, _i, _i]
            getattr(L, fn).restype = _sz
        L.timemix_forward.argtypes = [sp, ctypes.POINTER(TmWeights), _i, _i] + [_vp] * 9 + [_sz, _vp]
        L.timemix_forward.restype = _i
        L.timemix_backward.argtypes = ([sp, ctypes.POINTER(TmWeights), _i, _i] + [_vp] * 6 +
                                       [_vp, ctypes.POINTER(TmGrads)] + [_vp] * 6 + [_sz, _vp, _vp])
        L.timemix_backward.restype = _i
        L.wkv7_gemm_f32.argtypes = [_i] * 5 + [_vp, _i, _vp, _i, _vp, _i, ctypes.c_float, _vp]
        L.wkv7_gemm_f32.restype = _i
        L.wkv7_gemm_bf16.argtypes = [_i] * 5 + [_vp, _i, _vp, _i, _vp, _i, ctypes.c_float, _vp, _sz, _vp]
        L.wkv7_gemm_bf16.restype = _i
        L.wkv7_gemm_bf16_workspace_bytes.argtypes = [_i] * 5
        L.wkv7_gemm_bf16_workspace_bytes.restype = _sz
        cp = ctypes.POINTER(Rwkv7Config)
        L.rwkv7_decode_workspace_bytes.argtypes = [cp, _i]
        L.rwkv7_decode_workspace_bytes.restype = _sz
        L.rwkv7_decode_step.argtypes = [cp, ctypes.POINTER(Rwkv7Model), _i] + [_vp] * 6 + [_sz, _vp, _vp]
        L.rwkv7_decode_step.restype = _i
        L.rwkv7_train_workspace_bytes.argtypes = [cp, _i, _i]
        L.rwkv7_train_workspace_bytes.restype = _sz
        L.rwkv7_train_step.argtypes = ([cp, ctypes.POINTER(Rwkv7Model), ctypes.POINTER(Rwkv7ModelGrads),
                                        _i, _i] + [_vp] * 4 + [_sz, _vp, _vp])
        L.rwkv7_train_step.restype = _i
        gp, gw = ctypes.POINTER(GdnShape), ctypes.POINTER(GdnWeights)
        L.gdn_cache_bytes.argtypes = [gp, _i, _i]
        L.gdn_cache_bytes.restype = _sz
        L.gdn_backward_workspace_bytes.argtypes = [gp, _i, _i, _i]
        L.gdn_backward_workspace_bytes.restype = _sz
        L.gdn_forward.argtypes = [gp, gw, _i, _i] + [_vp] * 7 + [_sz, _vp]
        L.gdn_forward.restype = _i
        L.gdn_backward.argtypes = [gp, gw, _i, _i] + [_vp] * 11 + [_sz, _vp]
        L.gdn_backward.restype = _i
        L.moba_workspace_bytes.argtypes = [_i] * 6
        L.moba_workspace_bytes.restype = _sz
        L.moba_forward.argtypes = [_i] * 6 + [_vp] * 7 + [_sz, _vp]
        L.moba_forward.restype = _i
        L.moba_backward.argtypes = [_i] * 6 + [_vp] * 11 + [_sz, _vp]
        L.moba_backward.restype = _i
        L.rwkv7_online_workspace_bytes.argtypes = [cp, _i, _i]
        L.rwkv7_online_workspace_bytes.restype = _sz
        mg = ctypes.POINTER(Rwkv7ModelGrads)
        L.rwkv7_online_segment.argtypes = ([cp, ctypes.POINTER(Rwkv7Model), mg, mg, mg,
                                            ctypes.POINTER(Rwkv7Optim), _i, _i] + [_vp] * 7 +
                                           [_sz, _vp, _vp])
        L.rwkv7_online_segment.restype = _i
        L.wkv7_side_create.argtypes = [ctypes.POINTER(Wkv7Side)]
        L.wkv7_side_create.restype = _i
        L.wkv7_side_destroy.argtypes = [ctypes.POINTER(Wkv7Side)]
        L.wkv7_side_destroy.restype = _i
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise Wkv7Error(f"status {rc}: {lib().wkv7_last_error().decode()}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# One side stream (wkv7_side) per device, created by the first call that
# wants it outside a graph capture and owned by this module; the lock keeps
# two threads from using its events at once.
_sides = {}
_side_lock = threading.Lock()


class _SideUse:
    """Context manager giving the side pointer for the current device (or
    None when side=False) and holding the lock while the call enqueues."""

    def __init__(self, use):
        self.use = use

    def __enter__(self):
        if not self.use:
            return None
        _side_lock.acquire()
        dev = torch.cuda.current_device()
        sd = _sides.get(dev)
        if sd is None and torch.cuda.is_current_stream_capturing():
            # no stream is created inside a capture: this call runs on one stream
            _side_lock.release()
            self.use = False
            return None
        if sd is None:
            sd = Wkv7Side()
            rc = lib().wkv7_side_create(ctypes.byref(sd))
            if rc != 0:
                _side_lock.release()
                _check(rc)
            _sides[dev] = sd
        return ctypes.byref(sd)

    def __exit__(self, *exc):
        if self.use:
            _side_lock.release()
        return False


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t


def _opt(t, shape, dtype, name):
    return None if t is None else _need(t, shape, dtype, name)


def _dt(x):
    if x.dtype == torch.float32:
        return WKV7_F32
    if x.dtype == torch.bfloat16:
        return WKV7_BF16
    raise ValueError(f"unsupported dtype {x.dtype}")


# ------------------------------------------------------------------ WKV7 --
def wkv7_checkpoint_interval():
    return lib().wkv7_checkpoint_interval()


def wkv7_checkpoint_floats(B, T, H, N=64):
    return lib().wkv7_checkpoint_floats(B, T, H, N)


def wkv7_forward(r, w, k, v, a, b, s0=None, y=None, sT=None, ckpt=None,
                 want_state=True, want_ckpt=False, chunked=False, ws=None):
    """y = WKV7(r, w, k, v, a, b; s0).  Returns (y, sT or None, ckpt or None).

    chunked: pass the workspace that selects the chunked matrix-core kernels
    (for T >= 32); False (the default, and the faster path on MI355X) runs the
    token-sequential kernel.  ws: a preallocated uint8 device workspace for
    the chunked path (allocated here when None)."""
    B, T, H, N = r.shape
    dt = r.dtype
    for n, t in zip("rwkvab", (r, w, k, v, a, b)):
        _need(t, (B, T, H, N), dt, n)
    _opt(s0, (B, H, N, N), torch.float32, "s0")
    y = _opt(y, (B, T, H, N), dt, "y") if y is not None else torch.empty_like(r)
    if sT is None and want_state:
        sT = torch.empty((B, H, N, N), device=r.device, dtype=torch.float32)
    _opt(sT, (B, H, N, N), torch.float32, "sT")
    if ckpt is None and want_ckpt:
        ckpt = torch.empty(wkv7_checkpoint_floats(B, T, H, N), device=r.device, dtype=torch.float32)
    _opt(ckpt, (wkv7_checkpoint_floats(B, T, H, N),), torch.float32, "ckpt")
    nws = lib().wkv7_forward_workspace_bytes(B, T, H, N) if chunked else 0
    if nws and ws is None:
        ws = torch.empty(nws, device=r.device, dtype=torch.uint8)
    if not nws:
        ws = None
    elif ws.numel() < nws:
        raise ValueError(f"ws holds {ws.numel()} bytes, {nws} needed")
    _check(lib().wkv7_forward(B, T, H, N, _dt(r), _p(r), _p(w), _p(k), _p(v), _p(a), _p(b),
                              _p(s0), _p(y), _p(sT), _p(ckpt), _p(ws), nws, _stream()))
    return y, sT, ckpt


def wkv7_backward(r, w, k, v, a, b, dy, s0=None, ckpt=None, dsT=None, want_ds0=True, side=True):
    """Gradients of <dy, y> + <dsT, S_T>.  Returns dict dr, dw, dk, dv, da, db, ds0.

    side: overlap the long-sequence reductions on this module's side stream."""
    B, T, H, N = r.shape
    dt = r.dtype
    for n, t in zip(("r", "w", "k", "v", "a", "b", "dy"), (r, w, k, v, a, b, dy)):
        _need(t, (B, T, H, N), dt, n)
    _opt(s0, (B, H, N, N), torch.float32, "s0")
    _opt(dsT, (B, H, N, N), torch.float32, "dsT")
    _opt(ckpt, (wkv7_checkpoint_floats(B, T, H, N),), torch.float32, "ckpt")
    out = {n: torch.empty_like(r) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    out["ds0"] = torch.empty((B, H, N, N), device=r.device, dtype=torch.float32) if want_ds0 else None
    nbytes = lib().wkv7_backward_workspace_bytes(B, T, H, N, int(ckpt is not None))
    ws = torch.empty(max(nbytes, 1), device=r.device, dtype=torch.uint8)
    with _SideUse(side) as sd:
        _check(lib().wkv7_backward(B, T, H, N, _dt(r), _p(r), _p(w), _p(k), _p(v), _p(a), _p(b),
                                   _p(s0), _p(ckpt), _p(dy), _p(dsT), _p(out["dr"]), _p(out["dw"]),
                                   _p(out["dk"]), _p(out["dv"]), _p(out["da"]), _p(out["db"]),
                                   _p(out["ds0"]), _p(ws), nbytes, sd, _stream()))
    return out


def wkv7_backward_noalloc(r, w, k, v, a, b, dy, s0=None, ckpt=None, dsT=None, out=None,
                          side=True):
    """wkv7_backward with the library's fixed device scratch instead of a
    workspace.  out: optional dict of preallocated gradient tensors (dr, dw,
    dk, dv, da, db, ds0), so that the call itself allocates nothing."""
    B, T, H, N = r.shape
    dt = r.dtype
    for n, t in zip(("r", "w", "k", "v", "a", "b", "dy"), (r, w, k, v, a, b, dy)):
        _need(t, (B, T, H, N), dt, n)
    _opt(s0, (B, H, N, N), torch.float32, "s0")
    _opt(dsT, (B, H, N, N), torch.float32, "dsT")
    _opt(ckpt, (wkv7_checkpoint_floats(B, T, H, N),), torch.float32, "ckpt")
    if out is None:
        out = {n: torch.empty_like(r) for n in ("dr", "dw", "dk", "dv", "da", "db")}
        out["ds0"] = torch.empty((B, H, N, N), device=r.device, dtype=torch.float32)
    for n in ("dr", "dw", "dk", "dv", "da", "db"):
        _need(out[n], (B, T, H, N), dt, n)
    _opt(out.get("ds0"), (B, H, N, N), torch.float32, "ds0")
    with _SideUse(side) as sd:
        _check(lib().wkv7_backward_noalloc(B, T, H, N, _dt(r), _p(r), _p(w), _p(k), _p(v), _p(a),
                                           _p(b), _p(s0), _p(ckpt), _p(dy), _p(dsT), _p(out["dr"]),
                                           _p(out["dw"]), _p(out["dk"]), _p(out["dv"]),
                                           _p(out["da"]), _p(out["db"]), _p(out.get("ds0")), sd,
                                           _stream()))
    return out


def wkv7_step(r, w, k, v, a, b, state, y=None):
    """One decode token; r..b are [B][H][N]; state [B][H][N][N] is updated in place."""
    B, H, N = r.shape
    dt = r.dtype
    for n, t in zip("rwkvab", (r, w, k, v, a, b)):
        _need(t, (B, H, N), dt, n)
    _need(state, (B, H, N, N), torch.float32, "state")
    y = _opt(y, (B, H, N), dt, "y") if y is not None else torch.empty_like(r)
    _check(lib().wkv7_step(B, H, N, _dt(r), _p(r), _p(w), _p(k), _p(v), _p(a), _p(b),
                           _p(state), _p(y), _stream()))
    return y


# -------------------------------------------------------------- time-mix --
def tm_shape(C, H, Dw, Da, Dv, Dg, layer_id, N=64):
    return TmShape(C, H, N, Dw, Da, Dv, Dg, layer_id)


def _weight_shapes(s):
    C = s.C
    shp = {n: (C,) for n in ("mu_r", "mu_w", "mu_k", "mu_v", "mu_a", "mu_g", "w0", "a0", "v0",
                             "k_k", "k_a", "r_k", "ln_w", "ln_b")}
    shp.update(Wr=(C, C), Wk=(C, C), Wv=(C, C), Wo=(C, C), W1=(C, s.Dw), W2=(s.Dw, C),
               A1=(C, s.Da), A2=(s.Da, C), V1=(C, s.Dv), V2=(s.Dv, C), G1=(C, s.Dg), G2=(s.Dg, C))
    return shp


def _pack_weights(s, W):
    shp = _weight_shapes(s)
    cw = TmWeights()
    for n in WEIGHT_FIELDS:
        if s.layer_id == 0 and n in ("v0", "V1", "V2"):
            setattr(cw, n, None)
            continue
        setattr(cw, n, _need(W[n], shp[n], torch.float32, n).data_ptr())
    return cw


def timemix_cache_bytes(s, B, T):
    return lib().timemix_cache_bytes(ctypes.byref(s), B, T)


def timemix_forward(s, W, x, x_prev=None, v_first=None, s0=None, want_state=True,
                    want_cache=False, want_x_last=False):
    """Returns dict out, sT, x_last, v_first, cache (None where not requested)."""
    B, T, C = x.shape
    H, N = s.H, s.N
    _need(x, (B, T, C), torch.float32, "x")
    _opt(x_prev, (B, C), torch.float32, "x_prev")
    _opt(s0, (B, H, N, N), torch.float32, "s0")
    if s.layer_id == 0:
        v_first = torch.empty_like(x)
    else:
        _need(v_first, (B, T, C), torch.float32, "v_first")
    cw = _pack_weights(s, W)
    out = torch.empty_like(x)
    sT = torch.empty((B, H, N, N), device=x.device, dtype=torch.float32) if want_state else None
    x_last = torch.empty((B, C), device=x.device, dtype=torch.float32) if want_x_last else None
    nbytes = timemix_cache_bytes(s, B, T)
    buf = torch.empty(nbytes, device=x.device, dtype=torch.uint8)
    cache = buf if want_cache else None
    ws = None if want_cache else buf
    _check(lib().timemix_forward(ctypes.byref(s), ctypes.byref(cw), B, T, _p(x), _p(x_prev),
                                 _p(v_first), _p(s0), _p(sT), _p(out), _p(x_last), _p(cache),
                                 _p(ws), 0 if ws is None else nbytes, _stream()))
    return dict(out=out, sT=sT, x_last=x_last, v_first=v_first, cache=cache)


def timemix_backward(s, W, x, dout, x_prev=None, v_first=None, s0=None, dsT=None, cache=None,
                     dv_first_in=None, want_dx_prev=True, want_ds0=True, want_dv_first=True,
                     side=True):
    """Returns dict grads (per weight), dx, dx_prev, dv_first_out, ds0."""
    B, T, C = x.shape
    H, N = s.H, s.N
    _need(x, (B, T, C), torch.float32, "x")
    _need(dout, (B, T, C), torch.float32, "dout")
    _opt(x_prev, (B, C), torch.float32, "x_prev")
    _opt(s0, (B, H, N, N), torch.float32, "s0")
    _opt(dsT, (B, H, N, N), torch.float32, "dsT")
    if s.layer_id > 0:
        _need(v_first, (B, T, C), torch.float32, "v_first")
    if cache is not None:
        _need(cache, (timemix_cache_bytes(s, B, T),), torch.uint8, "cache")
    if s.layer_id == 0:
        _opt(dv_first_in, (B, T, C), torch.float32, "dv_first_in")
    cw = _pack_weights(s, W)
    shp = _weight_shapes(s)
    grads = {}
    cg = TmGrads()
    for n in WEIGHT_FIELDS:
        if s.layer_id == 0 and n in ("v0", "V1", "V2"):
            setattr(cg, n, None)
            continue
        grads[n] = torch.empty(shp[n], device=x.device, dtype=torch.float32)
        setattr(cg, n, grads[n].data_ptr())
    dx = torch.empty_like(x)
    dx_prev = torch.empty((B, C), device=x.device, dtype=torch.float32) if want_dx_prev else None
    dvf_out = torch.empty_like(x) if (s.layer_id > 0 and want_dv_first) else None
    ds0 = torch.empty((B, H, N, N), device=x.device, dtype=torch.float32) if want_ds0 else None
    nbytes = lib().timemix_backward_workspace_bytes(ctypes.byref(s), B, T)
    ws = torch.empty(nbytes, device=x.device, dtype=torch.uint8)
    with _SideUse(side) as sd:
        _check(lib().timemix_backward(ctypes.byref(s), ctypes.byref(cw), B, T, _p(x), _p(x_prev),
                                      _p(v_first), _p(s0), _p(dout), _p(dsT), _p(cache),
                                      ctypes.byref(cg), _p(dx), _p(dx_prev),
                                      _p(dv_first_in if s.layer_id == 0 else None), _p(dvf_out),
                                      _p(ds0), _p(ws), nbytes, sd, _stream()))
    return dict(grads=grads, dx=dx, dx_prev=dx_prev, dv_first_out=dvf_out, ds0=ds0)


# ------------------------------------------------------------------ GEMM --
def _gemm(fn, A, B, C, transA, transB, beta, ws=False):
    """ws: False (the fp32 call, no workspace argument), None (bf16 without
    one), True (bf16 with a workspace allocated here) or a uint8 tensor."""
    M, K = (A.shape[1], A.shape[0]) if transA else tuple(A.shape)
    K2, N = (B.shape[1], B.shape[0]) if transB else tuple(B.shape)
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    for n, t in (("A", A), ("B", B)):
        _need(t, tuple(t.shape), torch.float32, n)
    if C is None:
        C = torch.empty((M, N), device=A.device, dtype=torch.float32)
    _need(C, (M, N), torch.float32, "C")
    args = [int(transA), int(transB), M, N, K, _p(A), A.shape[1], _p(B), B.shape[1], _p(C), N, beta]
    if ws is not False:
        if ws is True:
            n = lib().wkv7_gemm_bf16_workspace_bytes(int(transA), int(transB), M, N, K)
            ws = torch.empty(n, device=A.device, dtype=torch.uint8) if n else None
        args += [_p(ws), 0 if ws is None else ws.numel()]
    _check(fn(*args, _stream()))
    return C


def wkv7_gemm_f32(A, B, C=None, transA=False, transB=False, beta=0.0):
    """C = op(A) op(B) + beta C on the matrix cores (fp32, row-major)."""
    return _gemm(lib().wkv7_gemm_f32, A, B, C, transA, transB, beta)


def wkv7_gemm_bf16_workspace_bytes(M, N, K, transA=False, transB=False):
    return lib().wkv7_gemm_bf16_workspace_bytes(int(transA), int(transB), M, N, K)


def wkv7_gemm_bf16(A, B, C=None, transA=False, transB=False, beta=0.0, ws=True):
    """As wkv7_gemm_f32 with bf16-rounded operands and fp32 accumulation.
    ws: True allocates the bf16-copy workspace the shape asks for, None runs
    without one (operands rounded in LDS), or a uint8 device tensor."""
    return _gemm(lib().wkv7_gemm_bf16, A, B, C, transA, transB, beta, ws=ws)


# ---------------------------------------------------------- decode stack --
class DecodeModel:
    """Device-resident weights of an RWKV-7 stack plus the C structs that
    point at them (the structs hold raw pointers, so the tensors are kept)."""

    def __init__(self, cfg, weights):
        """cfg: dict n_layer, C, H, F, V, ranks=(Dw, Da, Dv, Dg), use_ln0,
        gemm_dtype ('f32' default, or 'bf16': bf16 operands, fp32 accumulation),
        train_recompute (0 default: keep every block's activations for the
        training step's backward; 1: recompute each block from its input),
        n_attn (0 default), moba_chunk, moba_topk: MoBA attention blocks of a
        hybrid stack (training step only).
        weights: dict of device tensors as laid out by synth.stack_model, plus
        "attn": the attention blocks (synth.attn_blocks) when n_attn > 0."""
        L, C, H, F, V = cfg["n_layer"], cfg["C"], cfg["H"], cfg["F"], cfg["V"]
        Dw, Da, Dv, Dg = cfg["ranks"]
        gd = cfg.get("gemm_dtype", "f32")
        if gd not in ("f32", "bf16"):
            raise ValueError(f"gemm_dtype must be 'f32' or 'bf16', not {gd!r}")
        NA = int(cfg.get("n_attn", 0))
        self.cfg = Rwkv7Config(L, C, H, 64, F, V, Dw, Da, Dv, Dg, int(cfg.get("use_ln0", 1)),
                               1 if gd == "bf16" else 0, int(cfg.get("train_recompute", 0)), NA,
                               int(cfg.get("moba_chunk", 0)), int(cfg.get("moba_topk", 0)))
        self.w = weights
        blocks = (Rwkv7Block * L)()
        for l, bw in enumerate(weights["blocks"]):
            b = blocks[l]
            for n in ("ln1_w", "ln1_b", "ln2_w", "ln2_b"):
                setattr(b, n, _need(bw[n], (C,), torch.float32, n).data_ptr())
            b.tm = _pack_weights(tm_shape(C, H, Dw, Da, Dv, Dg, l), bw["tm"])
            b.cm_mu_k = _need(bw["cm_mu_k"], (C,), torch.float32, "cm_mu_k").data_ptr()
            b.cm_Wk = _need(bw["cm_Wk"], (C, F), torch.float32, "cm_Wk").data_ptr()
            b.cm_Wv = _need(bw["cm_Wv"], (F, C), torch.float32, "cm_Wv").data_ptr()
        self._blocks = blocks
        m = Rwkv7Model()
        m.emb = _need(weights["emb"], (V, C), torch.float32, "emb").data_ptr()
        m.head = _need(weights["head"], (C, V), torch.float32, "head").data_ptr()
        for n in ("ln_out_w", "ln_out_b", "ln0_w", "ln0_b"):
            t = weights.get(n)
            setattr(m, n, None if t is None else _need(t, (C,), torch.float32, n).data_ptr())
        m.blocks = ctypes.cast(blocks, ctypes.POINTER(Rwkv7Block))
        if NA:
            attn = (Rwkv7AttnBlock * NA)()
            shapes = dict(Wq=(C, C), Wk=(C, C), Wv=(C, C), Wo=(C, C), cm_Wk=(C, F), cm_Wv=(F, C))
            for a, aw in enumerate(weights["attn"]):
                for n in ATTN_FIELDS:
                    setattr(attn[a], n, _need(aw[n], shapes.get(n, (C,)), torch.float32, n).data_ptr())
            self._attn = attn
            m.attn = ctypes.cast(attn, ctypes.POINTER(Rwkv7AttnBlock))
        self.model = m

    def new_state(self, B, device="cuda"):
        c = self.cfg
        z = lambda *s: torch.zeros(s, device=device, dtype=torch.float32)
        return dict(att_x_prev=z(c.n_layer, B, c.C), att_state=z(c.n_layer, B, c.H, 64, 64),
                    ffn_x_prev=z(c.n_layer, B, c.C))


def rwkv7_decode_workspace_bytes(dm, B):
    return lib().rwkv7_decode_workspace_bytes(ctypes.byref(dm.cfg), B)


def rwkv7_decode_step(dm, tokens, state, logits=None, ws=None, side=True):
    """One token per stream: tokens [B] int32 (device); state dict updated in place."""
    c = dm.cfg
    B = tokens.shape[0]
    _need(tokens, (B,), torch.int32, "tokens")
    _need(state["att_x_prev"], (c.n_layer, B, c.C), torch.float32, "att_x_prev")
    _need(state["att_state"], (c.n_layer, B, c.H, 64, 64), torch.float32, "att_state")
    _need(state["ffn_x_prev"], (c.n_layer, B, c.C), torch.float32, "ffn_x_prev")
    if logits is None:
        logits = torch.empty((B, c.V), device=tokens.device, dtype=torch.float32)
    _need(logits, (B, c.V), torch.float32, "logits")
    nbytes = rwkv7_decode_workspace_bytes(dm, B)
    if ws is None:
        ws = torch.empty(nbytes, device=tokens.device, dtype=torch.uint8)
    with _SideUse(side) as sd:
        _check(lib().rwkv7_decode_step(ctypes.byref(c), ctypes.byref(dm.model), B, _p(tokens),
                                       _p(state["att_x_prev"]), _p(state["att_state"]),
                                       _p(state["ffn_x_prev"]), _p(logits), _p(ws), ws.numel(),
                                       sd, _stream()))
    return logits


# ---------------------------------------------------------- training step --
class TrainGrads:
    """Device buffers mirroring a DecodeModel's weights (torch.empty, or zeros
    with zero=True: the Adam moments of rwkv7_online_segment)."""

    def __init__(self, dm, zero=False):
        c = dm.cfg
        dev = dm.w["emb"].device
        mk = torch.zeros_like if zero else torch.empty_like
        e = lambda t: None if t is None else mk(t)
        w = dm.w
        self.g = {k: e(w.get(k)) for k in ("emb", "head", "ln_out_w", "ln_out_b", "ln0_w", "ln0_b")}
        self.g["blocks"] = []
        blocks = (Rwkv7BlockGrads * c.n_layer)()
        for l, bw in enumerate(w["blocks"]):
            gb = {k: mk(bw[k]) for k in ("ln1_w", "ln1_b", "ln2_w", "ln2_b", "cm_mu_k",
                                          "cm_Wk", "cm_Wv")}
            gb["tm"] = {}
            b = blocks[l]
            for k in ("ln1_w", "ln1_b", "ln2_w", "ln2_b", "cm_mu_k", "cm_Wk", "cm_Wv"):
                setattr(b, k, gb[k].data_ptr())
            tg = TmGrads()
            for n in WEIGHT_FIELDS:
                if l == 0 and n in ("v0", "V1", "V2"):
                    setattr(tg, n, None)
                    continue
                gb["tm"][n] = mk(bw["tm"][n])
                setattr(tg, n, gb["tm"][n].data_ptr())
            b.tm = tg
            self.g["blocks"].append(gb)
        self._blocks = blocks
        mg = Rwkv7ModelGrads()
        for n in ("emb", "head", "ln_out_w", "ln_out_b", "ln0_w", "ln0_b"):
            t = self.g[n]
            setattr(mg, n, None if t is None else t.data_ptr())
        mg.blocks = ctypes.cast(blocks, ctypes.POINTER(Rwkv7BlockGrads))
        if c.n_attn:
            self.g["attn"] = []
            attn = (Rwkv7AttnGrads * c.n_attn)()
            for a, aw in enumerate(w["attn"]):
                ga = {n: mk(aw[n]) for n in ATTN_FIELDS}
                for n in ATTN_FIELDS:
                    setattr(attn[a], n, ga[n].data_ptr())
                self.g["attn"].append(ga)
            self._attn = attn
            mg.attn = ctypes.cast(attn, ctypes.POINTER(Rwkv7AttnGrads))
        self.struct = mg


def rwkv7_train_workspace_bytes(dm, B, T):
    return lib().rwkv7_train_workspace_bytes(ctypes.byref(dm.cfg), B, T)


def rwkv7_train_step(dm, grads, tokens, targets, loss=None, ws=None, side=True):
    """Loss (device scalar tensor) of one step; grads (TrainGrads) are written."""
    B, T = tokens.shape
    _need(tokens, (B, T), torch.int32, "tokens")
    _need(targets, (B, T), torch.int32, "targets")
    if loss is None:
        loss = torch.empty(1, device=tokens.device, dtype=torch.float32)
    nbytes = rwkv7_train_workspace_bytes(dm, B, T)
    if ws is None:
        ws = torch.empty(nbytes, device=tokens.device, dtype=torch.uint8)
    with _SideUse(side) as sd:
        _check(lib().rwkv7_train_step(ctypes.byref(dm.cfg), ctypes.byref(dm.model),
                                      ctypes.byref(grads.struct), B, T, _p(tokens), _p(targets),
                                      _p(loss), _p(ws), ws.numel(), sd, _stream()))
    return loss


# ------------------------------------------------------------ GatedDeltaNet --
class Gdn:
    """A GatedDeltaNet layer's geometry and frozen device weights (the C
    structs hold raw pointers, so the tensors are kept here)."""

    def __init__(self, nk, nv, dk, dv, kk, rms_eps, conv, A_log, dt_bias, norm):
        self.shape = GdnShape(nk, nv, dk, dv, kk, rms_eps)
        cdim = 2 * nk * dk + nv * dv
        self.cdim = cdim
        self.w = dict(conv=_need(conv, (cdim, kk), torch.float32, "conv"),
                      A_log=_need(A_log, (nv,), torch.float32, "A_log"),
                      dt_bias=_need(dt_bias, (nv,), torch.float32, "dt_bias"),
                      norm=_need(norm, (dv,), torch.float32, "norm"))
        self.weights = GdnWeights(*(self.w[k].data_ptr() for k in ("conv", "A_log", "dt_bias", "norm")))

    def _inputs(self, raw, z, a, b):
        s = self.shape
        B, T = raw.shape[:2]
        _need(raw, (B, T, self.cdim), torch.float32, "raw")
        _need(z, (B, T, s.nv * s.dv), torch.float32, "z")
        _need(a, (B, T, s.nv), torch.float32, "a")
        _need(b, (B, T, s.nv), torch.float32, "b")
        return B, T


def gdn_cache_bytes(layer, B, T):
    return lib().gdn_cache_bytes(ctypes.byref(layer.shape), B, T)


def gdn_forward(layer, raw, z, a, b, want_cache=True, out=None, cache=None):
    """out [B][T][nv dv]; returns (out, cache or None)."""
    B, T = layer._inputs(raw, z, a, b)
    s = layer.shape
    out = _opt(out, (B, T, s.nv * s.dv), torch.float32, "out") if out is not None else \
        torch.empty((B, T, s.nv * s.dv), device=raw.device, dtype=torch.float32)
    n = gdn_cache_bytes(layer, B, T)
    buf = cache if cache is not None else torch.empty(n, device=raw.device, dtype=torch.uint8)
    _check(lib().gdn_forward(ctypes.byref(s), ctypes.byref(layer.weights), B, T, _p(raw), _p(z),
                             _p(a), _p(b), _p(out), _p(buf if want_cache else None),
                             _p(None if want_cache else buf), 0 if want_cache else n, _stream()))
    return out, (buf if want_cache else None)


def gdn_backward(layer, raw, z, a, b, dout, cache=None, ws=None):
    """Gradients of <dout, out>: dict draw, dz, da, db."""
    B, T = layer._inputs(raw, z, a, b)
    s = layer.shape
    _need(dout, (B, T, s.nv * s.dv), torch.float32, "dout")
    g = dict(draw=torch.empty_like(raw), dz=torch.empty_like(z), da=torch.empty_like(a),
             db=torch.empty_like(b))
    n = lib().gdn_backward_workspace_bytes(ctypes.byref(s), B, T, int(cache is not None))
    if ws is None:
        ws = torch.empty(n, device=raw.device, dtype=torch.uint8)
    _check(lib().gdn_backward(ctypes.byref(s), ctypes.byref(layer.weights), B, T, _p(raw), _p(z),
                              _p(a), _p(b), _p(dout), _p(cache), _p(g["draw"]), _p(g["dz"]),
                              _p(g["da"]), _p(g["db"]), _p(ws), ws.numel(), _stream()))
    return g


# ------------------------------------------------------ online training --
def rwkv7_online_workspace_bytes(dm, B, S):
    return lib().rwkv7_online_workspace_bytes(ctypes.byref(dm.cfg), B, S)


def rwkv7_online_segment(dm, grads, tokens, targets, state, optimizer="adam", lr=1e-3, clip=0.0,
                         step=1, adam_m=None, adam_v=None, loss=None, ws=None, side=True):
    """One online TBPTT segment: grads written, dm's weights updated in place,
    state (dict as DecodeModel.new_state) advanced to the live state after
    replaying the segment with the new weights.  adam_m / adam_v: TrainGrads
    made with zero=True (Adam only).  Returns the segment's loss (device)."""
    c = dm.cfg
    B, S = tokens.shape
    _need(tokens, (B, S), torch.int32, "tokens")
    _need(targets, (B, S), torch.int32, "targets")
    _need(state["att_x_prev"], (c.n_layer, B, c.C), torch.float32, "att_x_prev")
    _need(state["att_state"], (c.n_layer, B, c.H, 64, 64), torch.float32, "att_state")
    _need(state["ffn_x_prev"], (c.n_layer, B, c.C), torch.float32, "ffn_x_prev")
    if optimizer not in ("sgd", "adam"):
        raise ValueError(f"optimizer must be 'sgd' or 'adam', not {optimizer!r}")
    adam = optimizer == "adam"
    opt = Rwkv7Optim(1 if adam else 0, lr, clip, step)
    if loss is None:
        loss = torch.empty(1, device=tokens.device, dtype=torch.float32)
    n = rwkv7_online_workspace_bytes(dm, B, S)
    if ws is None:
        ws = torch.empty(n, device=tokens.device, dtype=torch.uint8)
    mp = ctypes.byref(adam_m.struct) if adam else None
    vp = ctypes.byref(adam_v.struct) if adam else None
    with _SideUse(side) as sd:
        _check(lib().rwkv7_online_segment(ctypes.byref(c), ctypes.byref(dm.model),
                                          ctypes.byref(grads.struct), mp, vp, ctypes.byref(opt), B, S,
                                          _p(tokens), _p(targets), _p(state["att_x_prev"]),
                                          _p(state["att_state"]), _p(state["ffn_x_prev"]), _p(loss),
                                          _p(ws), ws.numel(), sd, _stream()))
    return loss


# ------------------------------------------------------ MoBA attention --
def moba_forward(q, k, v, H, chunk, topk, y=None, ws=None):
    """MoBA attention core: q, k, v [B][T][H*64] fp32 (device).  Returns
    (y, lse [B][H][T], sel [B][H][T] int64 masks of the attended chunks)."""
    B, T, C = q.shape
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need(t, (B, T, C), torch.float32, n)
    if y is None:
        y = torch.empty_like(q)
    lse = torch.empty((B, H, T), device=q.device, dtype=torch.float32)
    sel = torch.empty((B, H, T), device=q.device, dtype=torch.int64)
    n = lib().moba_workspace_bytes(B, T, H, C // H, chunk, topk)
    if ws is None:
        ws = torch.empty(max(n, 1), device=q.device, dtype=torch.uint8)
    _check(lib().moba_forward(B, T, H, C // H, chunk, topk, _p(q), _p(k), _p(v), _p(y), _p(lse),
                              _p(sel), _p(ws), ws.numel(), _stream()))
    return y, lse, sel


def moba_backward(q, k, v, y, lse, sel, dy, H, chunk, topk, ws=None):
    """Gradients (dq, dk, dv) of <dy, y> with the selection sel held fixed
    (chunk and topk as in the forward)."""
    B, T, C = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("y", y), ("dy", dy)):
        _need(t, (B, T, C), torch.float32, n)
    _need(lse, (B, H, T), torch.float32, "lse")
    _need(sel, (B, H, T), torch.int64, "sel")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    n = lib().moba_workspace_bytes(B, T, H, C // H, chunk, topk)
    if ws is None:
        ws = torch.empty(max(n, 1), device=q.device, dtype=torch.uint8)
    _check(lib().moba_backward(B, T, H, C // H, chunk, topk, _p(q), _p(k), _p(v), _p(y), _p(lse), _p(sel),
                               _p(dy), _p(dq), _p(dk), _p(dv), _p(ws), ws.numel(), _stream()))
    return dq, dk, dv
