"""GPU parity of the MoBA attention core (moba_forward / moba_backward)
against the f64 oracle (oracle/moba.py).

The chunk selection is a discrete decision the GPU takes on fp32 scores and
the oracle on f64 ones.  Per query the oracle's choice is unique unless the
(topk-1)-th and topk-th best scores of the earlier chunks lie within a
rounding margin: where it is unique the GPU mask must equal it; elsewhere
every chunk the GPU chose must score at least the boundary minus the margin
(a valid choice among near-ties), and the current chunk must be in and no
later chunk.  y, the row log-sum-exp and the gradients are then compared
with the oracle evaluated on the GPU's selection (max|gpu - oracle| /
max|oracle|): forward 1e-4, gradients 1e-3 (fp32 tolerances)."""
import numpy as np
import pytest
import torch

from oracle import moba as om
from tests.parity import assert_close

pytestmark = pytest.mark.gpu


def _bits(sel, nc):
    s = np.asarray(sel).astype(np.uint64)
    return ((s[..., None] >> np.arange(nc, dtype=np.uint64)) & np.uint64(1)).astype(bool)


def _check_selection(q, k, H, chunk, topk, sel_bool):
    B, T, C = q.shape
    N = C // H
    for b in range(B):
        for h in range(H):
            sl = slice(h * N, (h + 1) * N)
            sc = om.chunk_scores(q[b, :, sl], k[b, :, sl], chunk)
            want = om.select(q[b, :, sl], k[b, :, sl], chunk, topk)
            margin = 1e-5 * max(1.0, float(np.abs(sc).max()))
            for t in range(T):
                cur = t // chunk
                got = sel_bool[b, h, t]
                assert got[cur] and not got[cur + 1:].any(), (b, h, t)
                past = sc[t, :cur]
                if cur <= topk - 1:
                    assert got[:cur].all(), (b, h, t)
                    continue
                srt = np.sort(past)[::-1]
                edge, nxt = srt[topk - 2], srt[topk - 1]
                if edge - nxt > margin:
                    assert (got == want[t]).all(), (b, h, t)
                else:
                    chosen = np.nonzero(got[:cur])[0]
                    assert len(chosen) == topk - 1 and (past[chosen] >= edge - margin).all(), (b, h, t)


def _run(hip, B, T, H, chunk, topk, seed, heads=None):
    g = np.random.default_rng(seed)
    C = H * 64
    q, k, v, dy = (g.standard_normal((B, T, C)).astype(np.float32) for _ in range(4))
    print(f"[moba] B={B} T={T} H={H} chunk={chunk} topk={topk}", flush=True)
    d = lambda x: torch.from_numpy(x).cuda()
    y, lse, sel = hip.moba_forward(d(q), d(k), d(v), H, chunk, topk)
    dq, dk, dv = hip.moba_backward(d(q), d(k), d(v), y, lse, sel, d(dy), H, chunk, topk)
    torch.cuda.synchronize()
    nc = (T + chunk - 1) // chunk
    sb = _bits(sel.cpu().numpy(), nc)
    got = dict(y=y.cpu().numpy(), lse=lse.cpu().numpy(), dq=dq.cpu().numpy(), dk=dk.cpu().numpy(),
               dv=dv.cpu().numpy())
    for b, h in heads or [(b, h) for b in range(B) for h in range(H)]:
        sl = slice(h * 64, (h + 1) * 64)
        one = lambda x: x[b:b + 1, :, sl]
        _check_selection(one(q), one(k), 1, chunk, topk, sb[b:b + 1, h:h + 1])
        yo, c = om.core_forward(one(q), one(k), one(v), 1, chunk, topk, sel=sb[b:b + 1, h:h + 1])
        gq, gk, gv = om.core_backward(c, one(dy))
        tag = f"[b={b} h={h}]"
        assert_close("y" + tag, got["y"][b, :, sl], yo[0], 1e-4)
        assert_close("lse" + tag, got["lse"][b, h], c["lse"][0, 0], 1e-4)
        assert_close("dq" + tag, got["dq"][b, :, sl], gq[0], 1e-3)
        assert_close("dk" + tag, got["dk"][b, :, sl], gk[0], 1e-3)
        assert_close("dv" + tag, got["dv"][b, :, sl], gv[0], 1e-3)


@pytest.mark.parametrize("B,T,H,chunk,topk", [
    (2, 37, 2, 8, 3),      # ragged last query / key tile, 5 chunks
    (1, 200, 3, 16, 4),    # several tiles, partial last chunk
    (2, 256, 2, 64, 2),    # chunk = tile
    (1, 130, 1, 100, 2),   # chunk wider than a tile
    (1, 64, 2, 1, 64),     # one key per chunk, every chunk selected: causal attention
    (1, 300, 2, 5, 64),    # 60 chunks, all selected
    (1, 96, 2, 32, 1),     # current chunk only
    # chunks of 64 keys: the gathered (query, chunk) path
    (1, 70, 2, 64, 2),     # two chunks, the second partial
    (2, 300, 2, 64, 3),    # five chunks, partial last one
    (1, 320, 1, 64, 1),    # current chunk only
    (1, 512, 2, 64, 64),   # every chunk: causal attention
])
def test_moba_parity_small(hip, B, T, H, chunk, topk):
    _run(hip, B, T, H, chunk, topk, seed=T + chunk + topk)


def test_moba_full_size_sampled_heads(hip):
    """The hybrid stack's attention: B=4, T=2048, H=16 (C=1024), chunks of 64,
    top-4, on three sampled (batch, head) pairs (heads are independent)."""
    _run(hip, 4, 2048, 16, 64, 4, seed=7, heads=[(0, 0), (3, 15), (1, 7)])
