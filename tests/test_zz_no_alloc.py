"""The no-allocation epilogue backward against the workspace entry point.

eqlinear_fused_epilogue_bwd_noalloc keeps the bias gradient's row-block partials in
the library's static per-device scratch instead of a caller workspace; it runs the
same kernels with the same launch plan, so dpre and dbias must equal
eqlinear_fused_epilogue_bwd's bit for bit.  Two calls in a row, the second on a
smaller input, show that what the first call left in the scratch does not leak into
the second; the small case is also held to the oracle's fp16 / fp32 bounds.
"""
import numpy as np
import pytest
import torch

import group_circulant_linear_p4_amd as eql
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-5, "f16": 3e-3}
DT = {"f32": eql.EQL_F32, "f16": eql.EQL_F16}
ACT = {"gelu": eql.EQL_ACT_GELU, "none": eql.EQL_ACT_NONE}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def inputs(T, N, Dp, dtype, seed):
    wl = W.Workload("t", "test", T, N, 8, Dp, dtype, ("fwd",), seed=seed)
    return W.make_dy(wl), W.make_residual(wl)


def with_workspace(dy_d, pre_d, N, Dp, T, dtype, act, bias):
    code = DT[dtype]
    nbytes = eql.eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, code)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    dpre = torch.empty_like(dy_d)
    db = torch.empty(Dp, dtype=dy_d.dtype, device=DEV) if bias else None
    eql.eqlinear_fused_epilogue_bwd(dy_d, pre_d, dpre, db, ws, nbytes, N, Dp, T, code, ACT[act])
    return dpre, db


def no_alloc(dy_d, pre_d, N, Dp, T, dtype, act, bias):
    dpre = torch.empty_like(dy_d)
    db = torch.empty(Dp, dtype=dy_d.dtype, device=DEV) if bias else None
    eql.eqlinear_fused_epilogue_bwd_noalloc(dy_d, pre_d, dpre, db, N, Dp, T, DT[dtype], ACT[act])
    return dpre, db


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("act", ["gelu", "none"])
def test_no_alloc_matches_workspace_entry_point(dtype, act):
    # First call: the benchmark layer's shape in fp16 (p4, N = 65536, D'T = 4096: 256
    # row blocks, 4 MiB of partials), a quarter of its rows in fp32; second: a smaller
    # ragged shape (T = 3, 1301 rows, D'T = 21, 82 row blocks of 16 rows).
    big = 65536 if dtype == "f16" else 16384
    for (T, N, Dp, seed) in ((4, big, 1024, 5), (3, 1301, 7, 6)):
        print("case no-alloc epilogue bwd %s %s T=%d N=%d D'=%d" % (dtype, act, T, N, Dp), flush=True)
        dy, pre = inputs(T, N, Dp, dtype, seed)
        dy_d = torch.from_numpy(dy).to(DEV)
        pre_d = torch.from_numpy(pre).to(DEV) if act == "gelu" else None
        ref_dpre, ref_db = with_workspace(dy_d, pre_d, N, Dp, T, dtype, act, True)
        got_dpre, got_db = no_alloc(dy_d, pre_d, N, Dp, T, dtype, act, True)
        torch.cuda.synchronize()
        assert torch.equal(got_dpre, ref_dpre)
        assert torch.equal(got_db, ref_db)
        if N < 10000:
            o_dpre, o_db = oracle.fused_epilogue_bwd(dy, pre, T, act=act)
            assert rel_err(got_dpre.cpu().numpy(), o_dpre) <= TOL[dtype]
            assert rel_err(got_db.cpu().numpy(), o_db) <= TOL[dtype]


def test_no_alloc_without_bias_and_empty():
    """Without dbias the scratch is unused; N = 0 writes a zero bias gradient."""
    dy, pre = inputs(4, 777, 33, "f16", 7)
    dy_d, pre_d = torch.from_numpy(dy).to(DEV), torch.from_numpy(pre).to(DEV)
    ref_dpre, _ = with_workspace(dy_d, pre_d, 777, 33, 4, "f16", "gelu", False)
    got_dpre, _ = no_alloc(dy_d, pre_d, 777, 33, 4, "f16", "gelu", False)
    empty = torch.empty((0, 40), dtype=torch.float32, device=DEV)
    db = torch.full((10,), 7.0, dtype=torch.float32, device=DEV)
    eql.eqlinear_fused_epilogue_bwd_noalloc(empty, None, empty, db, 0, 10, 4, eql.EQL_F32, eql.EQL_ACT_NONE)
    torch.cuda.synchronize()
    assert torch.equal(got_dpre, ref_dpre)
    assert torch.count_nonzero(db).item() == 0


def test_no_alloc_refuses_a_shape_beyond_its_scratch():
    """2^20 + 1024 rows of D'T = 4096 fp16 need more than the 16 MiB scratch: refused
    before anything is launched, the outputs untouched."""
    N, Dp, T = (1 << 20) + 1024, 1024, 4
    assert eql.eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, eql.EQL_F16) > eql.EQL_NOALLOC_SCRATCH_BYTES
    dy = torch.zeros((16, 16), dtype=torch.float16, device=DEV)   # never read
    db = torch.full((Dp,), 3.0, dtype=torch.float16, device=DEV)
    with pytest.raises(eql.EqlError) as e:
        eql.eqlinear_fused_epilogue_bwd_noalloc(dy, None, dy, db, N, Dp, T, eql.EQL_F16, eql.EQL_ACT_NONE)
    assert e.value.status == eql.EQL_ESCRATCH
    torch.cuda.synchronize()
    assert torch.all(db == 3.0).item()
