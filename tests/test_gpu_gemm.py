"""GPU parity of the matrix-core GEMMs (C-ABI wkv7_gemm_f32, wkv7_gemm_bf16)
against their definition C = op(A) op(B) (+ beta C), evaluated in f64 with
numpy.  Shapes cover every tile choice, ragged M, short and long K, and the
three layouts the time-mix block uses (X W, dY W^T, X^T dY) plus A^T B^T.
Tolerance: max|gpu - f64| / max|f64| <= 1e-5 (fp32 accumulation over K <=
1024).  The bf16 GEMM is held to the same 1e-5 against the f64 product of the
operands rounded to bf16 (round to nearest even, done on the host), which
pins its rounding and its fp32 accumulation, and to 2e-2 (the bf16
tolerance) against the unrounded product."""
import numpy as np
import pytest
import torch

from rwkv_linear_attention_wkv7_amd import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu


SHAPES = [(8192, 768, 768), (2048, 256, 256), (2048, 1024, 256),
          (2048, 256, 1024), (8192, 32, 768), (8192, 768, 64),
          (37, 64, 40), (1, 32, 4), (130, 128, 96)]
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("tA,tB", LAYOUTS)
def test_gemm_layouts(hip, M, N, K, tA, tB):
    g = np.random.default_rng(M * 7 + N * 3 + K)
    a = g.standard_normal((K, M) if tA else (M, K)).astype(np.float32)
    b = g.standard_normal((N, K) if tB else (K, N)).astype(np.float32)
    c0 = g.standard_normal((M, N)).astype(np.float32)
    A, Bm, C = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(c0.copy()).cuda()
    if tA and M % 4:
        # a transposed A is read along M in float4: rejected before any launch
        with pytest.raises(hip.Wkv7Error, match="multiples of 4"):
            hip.wkv7_gemm_f32(A, Bm, C, transA=tA, transB=tB, beta=0.5)
        return
    hip.wkv7_gemm_f32(A, Bm, C, transA=tA, transB=tB, beta=0.5)
    torch.cuda.synchronize()
    opa = a.astype(np.float64).T if tA else a.astype(np.float64)
    opb = b.astype(np.float64).T if tB else b.astype(np.float64)
    ref = opa @ opb + 0.5 * c0.astype(np.float64)
    assert_close("C", C.cpu().numpy(), ref, 1e-5)


@pytest.mark.parametrize("M,N,K", SHAPES + [(8192, 4096, 1024), (1024, 1024, 8192), (260, 36, 200)])
@pytest.mark.parametrize("tA,tB", LAYOUTS)
def test_gemm_bf16_layouts(hip, M, N, K, tA, tB):
    g = np.random.default_rng(M * 5 + N * 11 + K)
    a = g.standard_normal((K, M) if tA else (M, K)).astype(np.float32)
    b = g.standard_normal((N, K) if tB else (K, N)).astype(np.float32)
    c0 = g.standard_normal((M, N)).astype(np.float32)
    A, Bm, C = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(c0.copy()).cuda()
    if tA and M % 4:
        # a transposed A is read along M in float4: rejected before any launch
        with pytest.raises(hip.Wkv7Error, match="multiples of 4"):
            hip.wkv7_gemm_bf16(A, Bm, C, transA=tA, transB=tB, beta=0.5)
        return
    print(f"[gemm_bf16] M={M} N={N} K={K} tA={tA} tB={tB}", flush=True)
    hip.wkv7_gemm_bf16(A, Bm, C, transA=tA, transB=tB, beta=0.5)
    torch.cuda.synchronize()
    out = C.cpu().numpy()
    op = lambda x, t: x.T if t else x
    ar, br = synth.round_bf16(a).astype(np.float64), synth.round_bf16(b).astype(np.float64)
    ref_r = op(ar, tA) @ op(br, tB) + 0.5 * c0.astype(np.float64)
    assert_close("C (bf16 operands)", out, ref_r, 1e-5)
    ref = op(a.astype(np.float64), tA) @ op(b.astype(np.float64), tB) + 0.5 * c0.astype(np.float64)
    assert_close("C", out, ref, 2e-2)


@pytest.mark.parametrize("M,N,K,tB", [(8192, 4096, 1024, False), (8192, 1024, 4096, True),
                                      (2048, 2048, 256, False), (8192, 768, 768, True),
                                      (4096, 65536, 1024, False)])
def test_gemm_bf16_copies_give_the_same_bits(hip, M, N, K, tB):
    """With a workspace the operands are rounded to bf16 once into it
    (k-contiguous; B transposed when stored [K][N]) and multiplied without
    conversion; without one they are rounded as they are read from LDS.  The
    roundings and the order of the k steps are the same, so the results are
    bitwise equal; and they match the f64 product of the rounded operands."""
    g = np.random.default_rng(M + N + K)
    a = g.standard_normal((M, K)).astype(np.float32)
    b = g.standard_normal((N, K) if tB else (K, N)).astype(np.float32)
    A, Bm = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    assert hip.wkv7_gemm_bf16_workspace_bytes(M, N, K, transB=tB) == (M + N) * K * 2
    print(f"[gemm_bf16 copies] M={M} N={N} K={K} tB={tB}", flush=True)
    c1 = hip.wkv7_gemm_bf16(A, Bm, transB=tB, ws=None)
    c2 = hip.wkv7_gemm_bf16(A, Bm, transB=tB, ws=True)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    rows = np.random.default_rng(1).choice(M, 64, replace=False)
    ar, br = synth.round_bf16(a[rows]).astype(np.float64), synth.round_bf16(b).astype(np.float64)
    ref = ar @ (br.T if tB else br)
    assert_close("C rows (bf16 operands)", c2.cpu().numpy()[rows], ref, 1e-5)
