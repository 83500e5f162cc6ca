"""GPU parity of rwkv7_train_step (full RWKV-7 training step: embedding,
blocks, LM head, fused log-softmax CE, forward and backward) against the f64
oracle.  Loss and every gradient are compared (max|gpu - oracle| /
max|oracle|): loss <= 1e-4, gradients <= 1e-3 with fp32 GEMMs (fp32 end to
end) against the f64 oracle.  With bf16 GEMMs the oracle runs at that stated
precision (every matrix-product operand rounded to bf16, f64 elsewhere:
oracle.precision) and loss and gradients are held to 2e-2, the bf16
tolerance.  At the full model size the bf16 gradients are ill-conditioned
with respect to rounding: rounding the f64 oracle's own products to bf16
moves its embedding gradient by ~45% (random init, std 0.02), and merely
storing each product of the bf16 oracle as fp32 instead of f64 moves some of
its time-mix gradients by ~9% (a cascade of flipped bf16 roundings through 24
blocks).  So at the full model size (24 blocks) every bf16 gradient is held
to a bound calibrated by the oracle's own bf16 spread: err(gpu vs f64 oracle)
<= 2 err(bf16 oracle vs f64 oracle) + 1e-3, per tensor (scale-aware: every
spread is below 0.5, so a gradient off by a factor of 2 fails).  At the configuration's batch and
width with two blocks (B=4, T=2048, C=1024, vocab 65536), where the cascade
is short, loss and every gradient are held to 2e-2 against the bf16-operand
oracle, run one sequence at a time (the loss is a mean over tokens, so the
batch gradient is the mean of the per-sequence ones).  The complete
per-tensor 2e-2 comparison also runs on the small models, and the fp32-GEMM
run of the full-size step meets 1e-3 on every gradient."""
import math

import numpy as np
import pytest
import torch

from oracle import stack
from rwkv_linear_attention_wkv7_amd import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu


def _dev_model(m):
    d = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = {k: d(v) for k, v in m.items() if k != "blocks"}
    out["blocks"] = [{k: ({kk: d(vv) for kk, vv in v.items()} if k == "tm" else d(v))
                      for k, v in b.items()} for b in m["blocks"]]
    return out


def _run(hip, L, C, H, F, V, ranks, B, T, seed, perturbed, std, use_ln0, gemm="f32", recompute=0):
    from rwkv_linear_attention_wkv7_amd import binding
    m = synth.stack_model(C, H, F, V, L, ranks, seed=seed, perturbed=perturbed, std=std,
                          use_ln0=use_ln0)
    dm = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=ranks,
                                  use_ln0=int(use_ln0), gemm_dtype=gemm, train_recompute=recompute),
                             _dev_model(m))
    grads = binding.TrainGrads(dm)
    tok = synth.token_ids(B, T + 1, V, seed=seed + 100)
    x, y = np.ascontiguousarray(tok[:, :-1]), np.ascontiguousarray(tok[:, 1:])
    print(f"[train] L={L} C={C} F={F} V={V} B={B} T={T} gemm={gemm} recompute={recompute}", flush=True)
    loss = hip.rwkv7_train_step(dm, grads, torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    torch.cuda.synchronize()
    return m, dm, grads, x, y, float(loss.item())


def _pairs(g, G):
    """(name, gpu tensor, oracle array) for every gradient of the model."""
    for k in ("emb", "head", "ln_out_w", "ln_out_b", "ln0_w", "ln0_b"):
        if g.get(k) is not None:
            yield k, g[k], G[k]
    for l, gb in enumerate(g["blocks"]):
        for k in ("ln1_w", "ln1_b", "ln2_w", "ln2_b", "cm_mu_k", "cm_Wk", "cm_Wv"):
            yield f"{k}[{l}]", gb[k], G["blocks"][l][k]
        assert set(gb["tm"]) == set(G["blocks"][l]["tm"])
        for k, v in gb["tm"].items():
            yield f"tm.{k}[{l}]", v, G["blocks"][l]["tm"][k]


def _compare(m, grads, x, y, loss, cfg, gemm="f32"):
    """Every gradient at the tolerance against the oracle at the run's precision."""
    tl, tg = (1e-4, 1e-3) if gemm == "f32" else (2e-2, 2e-2)
    ref_loss, G = stack.train_step(m, cfg, x, y, gemm="f64" if gemm == "f32" else "bf16")
    assert abs(loss - ref_loss) <= tl * abs(ref_loss), (loss, ref_loss)
    worst = [0.0, ""]
    for name, got, ref in _pairs(grads.g, G):
        e = assert_close(name, got.cpu().numpy(), ref, tg)
        if e > worst[0]:
            worst[:] = [e, name]
    print(f"[train] gemm={gemm} loss {loss:.6f} oracle {ref_loss:.6f}; worst gradient "
          f"{worst[1]} rel err {worst[0]:.2e}", flush=True)


def _compare_calibrated(m, grads, x, y, loss, cfg):
    """bf16 GEMMs at the full model size: per tensor, err(gpu vs f64 oracle) <=
    2 err(bf16-operand oracle vs f64 oracle) + 1e-3; loss at 2e-2.  The GPU
    run and the bf16-operand oracle are two draws of the same rounding
    cascade (fp32 against f64 accumulation flips different bf16 roundings), so
    their distances to the f64 result differ by a random factor; every spread
    here is below 0.5, so a gradient off by a factor of 2 or of the wrong
    sign still fails."""
    from tests.parity import rel_err
    l64, G64 = stack.train_step(m, cfg, x, y, gemm="f64")
    l16, G16 = stack.train_step(m, cfg, x, y, gemm="bf16")
    assert abs(loss - l64) <= 2e-2 * abs(l64), (loss, l64)
    ref16 = dict((n, r) for n, _, r in _pairs(grads.g, G16))
    ratios = []
    for name, got, r64 in _pairs(grads.g, G64):
        spread = rel_err(ref16[name], r64)
        e = rel_err(got.cpu().numpy(), r64)
        ratios.append((e / (2.0 * spread + 1e-3), e, spread, name))
    ratios.sort(reverse=True)
    print(f"[train] bf16 full size: loss {loss:.6f} f64 oracle {l64:.6f}; {len(ratios)} tensors; "
          f"err / bound, highest: " + ", ".join(f"{n} {q:.3f} (err {e:.2e}, spread {s:.2e})"
                                               for q, e, s, n in ratios[:6]), flush=True)
    bad = [r for r in ratios if r[0] > 1.0]
    assert not bad, f"{len(bad)} tensors above 2 x oracle bf16 spread + 1e-3, e.g. {bad[:3]}"


@pytest.mark.parametrize("gemm", ["f32", "bf16"])
@pytest.mark.parametrize("use_ln0", [False, True])
def test_train_step_small(hip, use_ln0, gemm):
    L, C, H, F, V = 3, 128, 2, 256, 512
    m, dm, grads, x, y, loss = _run(hip, L, C, H, F, V, (16, 16, 16, 32), 2, 40, seed=3,
                                    perturbed=True, std=0.2, use_ln0=use_ln0, gemm=gemm)
    _compare(m, grads, x, y, loss, dict(C=C, H=H, F=F, V=V, n_layer=L), gemm)


@pytest.mark.parametrize("V", [6148, 65536])
def test_train_step_ragged_wide_vocab_ignored_targets(hip, V):
    """Sequences of 37 tokens (the channel-mix shift backward's per-thread
    token runs cross sequence boundaries), a vocabulary wide enough for the
    register-resident cross-entropy (6148: a partial last register slice),
    and targets outside [0, V) (-1 and V) that are ignored: zero dlogits rows,
    no loss term, the mean over the counted positions."""
    from rwkv_linear_attention_wkv7_amd import binding
    L, C, H, F, B, T = 1, 128, 2, 256, 3, 37
    ranks = (16, 16, 16, 32)
    m = synth.stack_model(C, H, F, V, L, ranks, seed=21, perturbed=True, std=0.2, use_ln0=False)
    dm = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=ranks, use_ln0=0),
                             _dev_model(m))
    grads = binding.TrainGrads(dm)
    tok = synth.token_ids(B, T + 1, V, seed=22)
    x, y = np.ascontiguousarray(tok[:, :-1]), np.ascontiguousarray(tok[:, 1:]).copy()
    y[0, 3], y[1, 0], y[2, T - 1], y[2, 10] = -1, V, -1, V + 7
    print(f"[train] ragged T={T} V={V} with ignored targets", flush=True)
    loss = hip.rwkv7_train_step(dm, grads, torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    torch.cuda.synchronize()
    _compare(m, grads, x, y, float(loss.item()), dict(C=C, H=H, F=F, V=V, n_layer=L))


@pytest.mark.parametrize("gemm", ["f32", "bf16"])
def test_train_step_full_model_short_batch(hip, gemm):
    """Full model size: 24 blocks, C=1024 (H=16), FFN 4096, vocab 65536, ranks
    64/64/32/128, std-0.02 random init; one sequence of 256 tokens so the f64
    oracle fits; every gradient compared."""
    L, C, H, F, V = 24, 1024, 16, 4096, 65536
    m, dm, grads, x, y, loss = _run(hip, L, C, H, F, V, (64, 64, 32, 128), 1, 256, seed=0,
                                    perturbed=False, std=0.02, use_ln0=False, gemm=gemm)
    cfg = dict(C=C, H=H, F=F, V=V, n_layer=L)
    if gemm == "f32":
        _compare(m, grads, x, y, loss, cfg, gemm)
    else:
        _compare_calibrated(m, grads, x, y, loss, cfg)


@pytest.mark.parametrize("gemm", ["f32", "bf16"])
def test_train_step_full_config_properties(hip, gemm):
    """B=4, T=2048 at the full model size, every block's activations kept, and
    the same step recomputing each block from its input.  At random init the LN output rows
    have unit variance and the head entries N(0, 0.02^2), so the logits are
    ~N(0, s2) with s2 = C 0.02^2 and the expected loss is
    E[logsumexp] - E[z_target] = ln(V) + s2/2 (log of the mean of e^z);
    every gradient is finite; two runs are bitwise identical (fixed-order
    reductions only)."""
    from rwkv_linear_attention_wkv7_amd import binding
    L, C, H, F, V = 24, 1024, 16, 4096, 65536
    m, dm, grads, x, y, loss = _run(hip, L, C, H, F, V, (64, 64, 32, 128), 4, 2048, seed=0,
                                    perturbed=False, std=0.02, use_ln0=False, gemm=gemm)
    expect = math.log(V) + C * 0.02 ** 2 / 2
    # the one-block workspace that recomputes each block gives the same bits
    dm_r = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=(64, 64, 32, 128), use_ln0=0,
                                    gemm_dtype=gemm, train_recompute=1), dm.w)
    gr = binding.TrainGrads(dm_r)
    loss_r = binding.rwkv7_train_step(dm_r, gr, torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    torch.cuda.synchronize()
    assert float(loss_r.item()) == loss
    assert torch.equal(gr.g["emb"], grads.g["emb"])
    assert torch.equal(gr.g["blocks"][0]["tm"]["Wr"], grads.g["blocks"][0]["tm"]["Wr"])
    assert torch.equal(gr.g["blocks"][23]["cm_Wk"], grads.g["blocks"][23]["cm_Wk"])
    del gr, dm_r
    assert abs(loss - expect) < 3e-2, (loss, expect)
    first = {"emb": grads.g["emb"].clone(), "head": grads.g["head"].clone(),
             "Wr0": grads.g["blocks"][0]["tm"]["Wr"].clone(),
             "cmk23": grads.g["blocks"][23]["cm_Wk"].clone()}
    for t in first.values():
        assert torch.isfinite(t).all()
    loss2 = binding.rwkv7_train_step(dm, grads, torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    torch.cuda.synchronize()
    assert float(loss2.item()) == loss
    assert torch.equal(first["emb"], grads.g["emb"])
    assert torch.equal(first["head"], grads.g["head"])
    assert torch.equal(first["Wr0"], grads.g["blocks"][0]["tm"]["Wr"])
    assert torch.equal(first["cmk23"], grads.g["blocks"][23]["cm_Wk"])


# ---- the configuration's batch and width (B=4, T=2048, C=1024, FFN 4096,
# vocab 65536, ranks 64/64/32/128, bf16 GEMMs) with two blocks: the GPU step
# runs once on the whole batch; the bf16-operand oracle runs one sequence per
# test and the per-sequence results are averaged, then compared.
_C4 = {}
_C4_B, _C4_T, _C4_L = 4, 2048, 2


def _flat(G):
    """name -> tensor/array for a nested gradient dict (GPU or oracle)."""
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


def _c4_gpu(hip):
    if "gpu" not in _C4:
        L, C, H, F, V = _C4_L, 1024, 16, 4096, 65536
        m, dm, grads, x, y, loss = _run(hip, L, C, H, F, V, (64, 64, 32, 128), _C4_B, _C4_T, seed=5,
                                        perturbed=False, std=0.02, use_ln0=False, gemm="bf16")
        g = {n: t.cpu().numpy() for n, t in _flat(grads.g)}
        _C4.update(gpu=g, loss=loss, m=m, x=x, y=y, cfg=dict(C=C, H=H, F=F, V=V, n_layer=L),
                   acc={}, acc_loss=0.0, done=set())
        del dm, grads
        torch.cuda.empty_cache()
    return _C4


@pytest.mark.parametrize("b", range(_C4_B))
def test_train_step_config_batch_two_blocks_sequence(hip, b):
    st = _c4_gpu(hip)
    print(f"[train c4 batch] oracle sequence {b}", flush=True)
    lb, Gb = stack.train_step(st["m"], st["cfg"], st["x"][b:b + 1], st["y"][b:b + 1], gemm="bf16")
    for name, r in _flat(Gb):
        st["acc"][name] = st["acc"].get(name, 0.0) + np.asarray(r) / _C4_B
    st["acc_loss"] += lb / _C4_B
    st["done"].add(b)


def test_train_step_config_batch_two_blocks_compare(hip):
    st = _c4_gpu(hip)
    if st["done"] != set(range(_C4_B)):
        pytest.skip("needs every per-sequence oracle test of this batch first")
    assert set(st["gpu"]) == set(st["acc"])
    assert abs(st["loss"] - st["acc_loss"]) <= 2e-2 * abs(st["acc_loss"]), (st["loss"], st["acc_loss"])
    worst = [0.0, ""]
    for name in sorted(st["gpu"]):
        e = assert_close(name, st["gpu"][name], st["acc"][name], 2e-2)
        if e > worst[0]:
            worst[:] = [e, name]
    print(f"[train c4 batch] loss {st['loss']:.6f} oracle {st['acc_loss']:.6f}; worst gradient "
          f"{worst[1]} rel err {worst[0]:.2e} over {len(st['gpu'])} tensors", flush=True)
    _C4.clear()
