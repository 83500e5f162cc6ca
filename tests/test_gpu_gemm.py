"""GPU parity of the fp32 matrix-core GEMM (C-ABI wkv7_gemm_f32) against its
definition C = op(A) op(B) (+ beta C), evaluated in f64 with numpy.  Shapes
cover every tile choice, ragged M, short and long K, and the three layouts the
time-mix block uses (X W, dY W^T, X^T dY) plus A^T B^T.
Tolerance: max|gpu - f64| / max|f64| <= 1e-5 (fp32 accumulation over K <= 1024)."""
import numpy as np
import pytest
import torch

from tests.parity import assert_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(8192, 768, 768), (2048, 256, 256), (2048, 1024, 256),
                                   (2048, 256, 1024), (8192, 32, 768), (8192, 768, 64),
                                   (37, 64, 40), (1, 32, 4), (130, 128, 96)])
@pytest.mark.parametrize("tA,tB", [(False, False), (False, True), (True, False), (True, True)])
def test_gemm_layouts(hip, M, N, K, tA, tB):
    if tA and M % 4:
        pytest.skip("a transposed A is read along M in float4: M must be a multiple of 4")
    g = np.random.default_rng(M * 7 + N * 3 + K)
    a = g.standard_normal((K, M) if tA else (M, K)).astype(np.float32)
    b = g.standard_normal((N, K) if tB else (K, N)).astype(np.float32)
    c0 = g.standard_normal((M, N)).astype(np.float32)
    A, Bm, C = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(c0.copy()).cuda()
    hip.wkv7_gemm_f32(A, Bm, C, transA=tA, transB=tB, beta=0.5)
    torch.cuda.synchronize()
    opa = a.astype(np.float64).T if tA else a.astype(np.float64)
    opb = b.astype(np.float64).T if tB else b.astype(np.float64)
    ref = opa @ opb + 0.5 * c0.astype(np.float64)
    assert_close("C", C.cpu().numpy(), ref, 1e-5)
