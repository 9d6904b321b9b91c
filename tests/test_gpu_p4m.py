"""GPU parity of the p4m (dihedral D4) layer against its fp64 oracle.

The library runs p4m as the C_4 layer on 2C' x 2D' channels with a tied weight (see
include/eqlinear.h). Checked here through the C ABI and the torch layer:
- the tied weight, bit for bit, against the oracle's group law;
- y, dx and dw of EQLinearP4MFunction against oracle.p4m_oracle (relative Frobenius error
  <= 1e-5 for fp32, <= 3e-3 for fp16), through the training entry points and through the
  plain passes, on shapes whose C_4 view spans several tiles with ragged tails;
- equivariance of the GPU outputs under right translation by r and by s.
"""
import numpy as np
import pytest
import torch

import group_circulant_linear_p4_amd as eql
from group_circulant_linear_p4_amd.layer import EQLinearP4M, EQLinearP4MFunction
from oracle import p4m_oracle as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-5, "f16": 3e-3}
NP = {"f32": np.float32, "f16": np.float16}
TT = {"f32": torch.float32, "f16": torch.float16}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def inputs(N, Cp, Dp, dtype, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((N, Cp * 8), dtype=np.float32).astype(NP[dtype])
    w = (g.standard_normal((Dp, Cp, 8), dtype=np.float32) / np.sqrt(Cp * 8)).astype(NP[dtype])
    dy = g.standard_normal((N, Dp * 8), dtype=np.float32).astype(NP[dtype])
    return x, w, dy


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_p4m_expanded_weight_follows_the_group_law(dtype):
    Dp, Cp = 37, 11
    _, w, _ = inputs(1, Cp, Dp, dtype, 1)
    w4 = torch.empty((2 * Dp, 2 * Cp, 4), dtype=TT[dtype], device=DEV)
    eql.eqlinear_p4m_expand_weight(torch.from_numpy(w).to(DEV), w4, Dp, Cp, eql.EQL_F16 if dtype == "f16" else eql.EQL_F32)
    torch.cuda.synchronize()
    got = w4.cpu().numpy()
    ref = np.empty_like(got)
    for bo in range(2):
        for bi in range(2):
            for k in range(4):
                ref[bo::2, bi::2, k] = w[:, :, P.index(k if bo == 0 else -k, bo ^ bi)]
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))


CASES = [(300, 5, 7), (1000, 48, 40), (2049, 17, 130), (4100, 96, 64)]


@pytest.mark.parametrize("keep", [True, False], ids=["train", "plain"])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("shape", CASES, ids=lambda s: "N%d_C%d_D%d" % s)
def test_p4m_layer_matches_oracle(dtype, shape, keep):
    """keep: the training entry points (the weight gradient reads the spectra the forward
    and the input gradient left in the workspace); otherwise the plain passes."""
    N, Cp, Dp = shape
    print("case p4m layer %s N=%d C'=%d D'=%d keep_spectra=%s" % (dtype, N, Cp, Dp, keep), flush=True)
    x, w, dy = inputs(N, Cp, Dp, dtype, 10 + N)
    xt = torch.from_numpy(x).to(DEV).requires_grad_(True)
    wt = torch.from_numpy(w).to(DEV).requires_grad_(True)
    y = EQLinearP4MFunction.apply(xt, wt, keep)
    y.backward(torch.from_numpy(dy).to(DEV))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert rel_err(y.detach().cpu().numpy(), P.fwd(x, w)) <= tol
    assert rel_err(xt.grad.cpu().numpy(), P.bwd_x(dy, w)) <= tol
    assert rel_err(wt.grad.cpu().numpy(), P.bwd_w(x, dy)) <= tol


@pytest.mark.parametrize("a", [1, 4], ids=["r", "s"])
def test_p4m_gpu_outputs_are_equivariant(a):
    """Right translation of x by r (index 1) or s (index 4) translates the GPU's y the
    same way; the residual is bounded by the fp32 parity tolerance."""
    N, Cp, Dp = 777, 9, 13
    x, w, _ = inputs(N, Cp, Dp, "f32", 5)
    layer = EQLinearP4M(Cp, Dp, device=DEV, dtype=torch.float32)
    with torch.no_grad():
        layer.weight.copy_(torch.from_numpy(w))
        y = layer(torch.from_numpy(x).to(DEV)).cpu().numpy()
        y_t = layer(torch.from_numpy(P.right_translate(x, a).astype(np.float32)).to(DEV)).cpu().numpy()
    assert rel_err(y_t, P.right_translate(y, a)) <= TOL["f32"]
