"""Pins of the oracle's GEMM operand precision (oracle.precision).

round_bf16 is checked against hand-computed values of rounding to 8
significant bits (ties to even) and against an independent brute force over
IEEE bit patterns: the two bf16 neighbours of an fp32 value are its top 16
bits and that plus one unit in the last place; the nearer wins, ties go to the
even pattern.  The bf16 mode of the training-step oracle is checked against
the plain f64 oracle run with every matrix product intercepted (a numpy
subclass rounds the operands of each matmul it sees): equality means every
product, and nothing but products, is rounded.
"""
import types

import numpy as np
import pytest

from oracle import precision, stack, timemix
from rwkv_linear_attention_wkv7_amd import synth


@pytest.mark.parametrize("x,want", [
    (1.0, 1.0), (0.0, 0.0), (-2.5, -2.5),
    (1.0 + 2.0 ** -8, 1.0),                      # tie between 1 and 1 + 2^-7: even is 1
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),      # tie between mantissas 1 and 2: even is 2
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),
    (-(1.0 + 2.0 ** -8 + 2.0 ** -30), -(1.0 + 2.0 ** -7)),
    (np.pi, 3.140625),                            # 201/64
    (1e-3, 131 * 2.0 ** -17),                    # 0.00099945068359375
    (65504.0, 65536.0),                          # 255.875/256 rounds up a binade
])
def test_round_bf16_values(x, want):
    assert precision.round_bf16(np.float64(x)) == want


def _bf16_bruteforce(x32):
    bits = x32.view(np.uint32).astype(np.uint64)
    lo = (bits & 0xFFFF0000).astype(np.uint32)
    hi = (lo.astype(np.uint64) + 0x10000).astype(np.uint32)
    flo = lo.view(np.float32).astype(np.float64)
    fhi = hi.view(np.float32).astype(np.float64)
    x = x32.astype(np.float64)
    dlo, dhi = np.abs(x - flo), np.abs(fhi - x)
    even_lo = ((lo >> 16) & 1) == 0
    return np.where(dlo < dhi, flo, np.where(dhi < dlo, fhi, np.where(even_lo, flo, fhi)))


def test_round_bf16_bruteforce():
    g = np.random.default_rng(0)
    x = (g.standard_normal(200000) * np.exp(g.uniform(-20, 20, 200000))).astype(np.float32)
    # exact ties: bf16 values plus half a bf16 ulp
    base = (x[:5000].view(np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, base.astype(np.uint32).view(np.float32)])
    got = precision.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, _bf16_bruteforce(x))


def test_mm_modes():
    g = np.random.default_rng(1)
    a, b = g.standard_normal((5, 7)), g.standard_normal((7, 3))
    np.testing.assert_array_equal(precision.mm(a, b), a @ b)
    with pytest.raises(ValueError):
        precision.mm(a, b, "fp8")


class _BF(np.ndarray):
    """Rounds both operands of every matmul it takes part in (f64 result)."""

    def __array_ufunc__(self, uf, method, *inputs, **kw):
        ins = [np.asarray(i) if isinstance(i, _BF) else i for i in inputs]
        if "out" in kw:
            kw["out"] = tuple(np.asarray(o) if isinstance(o, _BF) else o for o in kw["out"])
        if uf is np.matmul and method == "__call__":
            ins = [precision.round_bf16(i) for i in ins]
        r = getattr(uf, method)(*ins, **kw)
        return r.view(_BF) if isinstance(r, np.ndarray) and r.dtype == np.float64 else r


def test_train_step_bf16_rounds_every_product(monkeypatch):
    L, C, H, F, V = 2, 128, 2, 256, 300
    m = synth.stack_model(C, H, F, V, L, (16, 16, 16, 32), seed=5, perturbed=True, std=0.1,
                          use_ln0=True)
    tok = synth.token_ids(2, 13, V, seed=6)
    x, y = tok[:, :-1], tok[:, 1:]
    cfg = dict(C=C, H=H, F=F, V=V, n_layer=L)
    loss_b, G_b = stack.train_step(m, cfg, x, y, gemm="bf16")

    # the plain oracle with intercepted products
    npx = types.SimpleNamespace(**{k: getattr(np, k) for k in dir(np) if not k.startswith("__")})
    npx.asarray = lambda v, dtype=None: np.asanyarray(v, dtype=dtype)
    monkeypatch.setattr(stack, "np", npx)
    monkeypatch.setattr(timemix, "np", npx)
    conv = lambda v: None if v is None else np.asarray(v, np.float64).view(_BF)
    mb = {k: ([{kk: ({a: conv(b) for a, b in vv.items()} if kk == "tm" else conv(vv))
                for kk, vv in blk.items()} for blk in v] if k == "blocks" else conv(v))
          for k, v in m.items()}
    loss_i, G_i = stack.train_step(mb, cfg, x, y)
    monkeypatch.undo()

    loss_f, G_f = stack.train_step(m, cfg, x, y)
    assert loss_b == pytest.approx(loss_i, rel=1e-13, abs=0)
    assert loss_b != loss_f  # the rounding is in effect
    pairs = [(G_b[k], G_i[k]) for k in ("emb", "head", "ln_out_w", "ln0_w")]
    for l in range(L):
        pairs += [(G_b["blocks"][l][k], G_i["blocks"][l][k]) for k in ("cm_Wk", "cm_Wv", "ln1_w")]
        pairs += [(G_b["blocks"][l]["tm"][k], G_i["blocks"][l]["tm"][k]) for k in G_b["blocks"][l]["tm"]]
    for a, b in pairs:
        a, b = np.asarray(a), np.asarray(b)
        assert np.max(np.abs(a - b)) <= 1e-12 * max(np.max(np.abs(b)), 1e-300)
