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
blocks).  So at full size the bf16 run is held to 2e-2 on the loss and on the
head / ln_out gradients (well conditioned), and every other gradient must
point the same way as the oracle's (cosine >= 0.95); the complete per-tensor
2e-2 comparison runs on the small models, and the fp32-GEMM run of the same
full-size step meets 1e-3 on every gradient."""
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


def _compare(m, grads, x, y, loss, cfg, gemm="f32", only=None):
    """only: names checked at the tolerance; the rest get the cosine check."""
    tl, tg = (1e-4, 1e-3) if gemm == "f32" else (2e-2, 2e-2)
    ref_loss, G = stack.train_step(m, cfg, x, y, gemm="f64" if gemm == "f32" else "bf16")
    assert abs(loss - ref_loss) <= tl * abs(ref_loss), (loss, ref_loss)
    g = grads.g
    worst = [0.0, ""]
    cos_min = [1.0, ""]

    def chk(name, got, ref, tol):
        if only is not None and name not in only:
            a, b = np.asarray(got, np.float64).ravel(), np.asarray(ref, np.float64).ravel()
            c = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))
            if c < cos_min[0]:
                cos_min[:] = [c, name]
            assert c >= 0.95, f"{name}: cosine {c:.4f} < 0.95"
            return
        e = assert_close(name, got, ref, tol)
        if e > worst[0]:
            worst[:] = [e, name]
    np_ = lambda t: t.cpu().numpy()
    for k in ("emb", "head", "ln_out_w", "ln_out_b"):
        chk(k, np_(g[k]), G[k], tg)
    if g.get("ln0_w") is not None:
        chk("ln0_w", np_(g["ln0_w"]), G["ln0_w"], tg)
        chk("ln0_b", np_(g["ln0_b"]), G["ln0_b"], tg)
    for l, gb in enumerate(g["blocks"]):
        for k in ("ln1_w", "ln1_b", "ln2_w", "ln2_b", "cm_mu_k", "cm_Wk", "cm_Wv"):
            chk(f"{k}[{l}]", np_(gb[k]), G["blocks"][l][k], tg)
        assert set(gb["tm"]) == set(G["blocks"][l]["tm"])
        for k, v in gb["tm"].items():
            chk(f"tm.{k}[{l}]", np_(v), G["blocks"][l]["tm"][k], tg)
    print(f"[train] gemm={gemm} loss {loss:.6f} oracle {ref_loss:.6f}; worst gradient "
          f"{worst[1]} rel err {worst[0]:.2e}; lowest cosine {cos_min[1]} {cos_min[0]:.5f}",
          flush=True)


@pytest.mark.parametrize("gemm", ["f32", "bf16"])
@pytest.mark.parametrize("use_ln0", [False, True])
def test_train_step_small(hip, use_ln0, gemm):
    L, C, H, F, V = 3, 128, 2, 256, 512
    m, dm, grads, x, y, loss = _run(hip, L, C, H, F, V, (16, 16, 16, 32), 2, 40, seed=3,
                                    perturbed=True, std=0.2, use_ln0=use_ln0, gemm=gemm)
    _compare(m, grads, x, y, loss, dict(C=C, H=H, F=F, V=V, n_layer=L), gemm)


@pytest.mark.parametrize("gemm", ["f32", "bf16"])
def test_train_step_full_model_short_batch(hip, gemm):
    """Full model size: 24 blocks, C=1024 (H=16), FFN 4096, vocab 65536, ranks
    64/64/32/128, std-0.02 random init; one sequence of 256 tokens so the f64
    oracle fits; every gradient compared."""
    L, C, H, F, V = 24, 1024, 16, 4096, 65536
    m, dm, grads, x, y, loss = _run(hip, L, C, H, F, V, (64, 64, 32, 128), 1, 256, seed=0,
                                    perturbed=False, std=0.02, use_ln0=False, gemm=gemm)
    only = None if gemm == "f32" else ("head", "ln_out_w", "ln_out_b")
    _compare(m, grads, x, y, loss, dict(C=C, H=H, F=F, V=V, n_layer=L), gemm, only)


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
