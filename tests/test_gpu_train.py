"""GPU parity of the training-step entry points (eqlinear_fwd_train,
eqlinear_bwd_x_train, eqlinear_bwd_w_train) through the C ABI:

  * y and dx bit-identical to eqlinear_fwd and eqlinear_bwd_x (the spectrum side
    output must not change the layer's outputs);
  * dw against the fp64 oracle, with the bounds of the other parity tests;
  * the spectra the forward kernel leaves in the workspace against those the weight
    gradient's own transform writes there (eqlinear_bwd_w on a second workspace):
    the Re/Im planes are the same single rounding of an exact difference, so they
    must match bit for bit; the two real planes take a second fp16 rounding in the
    forward's butterflies and must lie within one rounding of the partial sums.
Shapes cover both weight-gradient paths, every forward tile width, ragged rows and
channels, the shapes the forward kernel cannot serve (other T, fp32, rows that are not
16-byte aligned; the entry points then run the separate transform), one row and no
rows, and the two large workloads at full size.
"""
import numpy as np
import pytest
import torch

import group_circulant_linear_p4_amd as eql
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 3e-3}
DEV = "cuda:0"
DT = {"f32": eql.EQL_F32, "f16": eql.EQL_F16}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def ceil_div(a, b):
    return -(-a // b)


def align256(v):
    return ceil_div(v, 256) * 256


def tile_width(ch):
    return 256 if ceil_div(ch, 256) * 256 * 3 <= ch * 4 else 64


def bwdw_fused(N, Cp, Dp, T, elt):
    """The weight gradient's path rule as the header documents it."""
    if N == 0 or T not in (1, 2, 4) or (Dp * T * elt) % 16 or N * Dp * T * elt >= 2**32:
        return False
    planes = {1: 1, 2: 2, 4: 6}[T]
    return 2.0 * planes * N * Dp * Cp / (elt * T * N * (Cp + Dp)) < 400.0


def spectrum_sections(N, Cp, Dp, T, elt):
    """(offset, channel count, padded channel count) of dy's and x's operand units in the
    weight-gradient workspace, as the header documents the layout (dy's is None on the
    fused path)."""
    kg = ceil_div(N, 2 * (16 // elt))
    if bwdw_fused(N, Cp, Dp, T, elt):
        best, cpad = None, None
        for nb in (4, 3, 2):
            if (T * nb) % 4:
                continue
            padded = ceil_div(Cp, 32 * nb) * 32 * nb
            if best is None or padded < best:
                best, cpad = padded, padded
        return None, (0, Cp, cpad, kg)
    dpad = ceil_div(Dp, tile_width(Dp)) * tile_width(Dp)
    cpad = ceil_div(Cp, tile_width(Cp)) * tile_width(Cp)
    dyh = align256(kg * T * 2 * dpad * 16)
    return (0, Dp, dpad, kg), (dyh, Cp, cpad, kg)


def planes_of(ws, section, N, T, dtype):
    """The valid part of one spectrum section as [T][N][channels] values."""
    off, ch, kpad, kg = section
    nd = np.float16 if dtype == "f16" else np.float32
    g = 16 // np.dtype(nd).itemsize
    raw = ws[off:off + kg * T * 2 * kpad * 16].cpu().numpy().view(nd)
    u = raw.reshape(kg, T, 2, kpad, g)                  # unit (kg, p, half, k), row offset e
    u = u.transpose(1, 0, 2, 4, 3).reshape(T, kg * 2 * g, kpad)
    return u[:, :N, :ch].astype(np.float64)


def check_spectra(got, ref, src, T, dtype, what):
    """got/ref: [T][N][ch] planes; src: the [N][ch*T] matrix they transform."""
    assert np.isfinite(got).all(), what
    if dtype == "f16" and T == 4:
        # Re / Im: one rounding of an exact difference on both sides.
        if not np.array_equal(got[2:], ref[2:]):
            bad = np.argwhere(got[2:] != ref[2:])
            print("%s: %d Re/Im values differ; first (plane-2, row, channel): %s" % (what, len(bad), bad[:8].tolist()))
            for p, r, c in bad[:8]:
                print("   got %r ref %r" % (got[2 + p, r, c], ref[2 + p, r, c]))
            raise AssertionError("%s: Re/Im planes differ" % what)
        # X0, X2: the forward rounds (x0 + x2) and (x1 + x3) first; within one fp16
        # rounding (2^-11 relative) of those partial sums, plus one of the result.
        g = src.reshape(src.shape[0], -1, 4).astype(np.float64)
        bound = 2.0**-11 * (np.abs(g[..., 0] + g[..., 2]) + np.abs(g[..., 1] + g[..., 3]))
        for p in (0, 1):
            d = np.abs(got[p] - ref[p])
            assert (d <= bound + 2.0**-11 * np.abs(ref[p]) + 1e-30).all(), "%s: plane %d off" % (what, p)
    else:
        assert np.array_equal(got, ref), "%s: the separate transform must be reproduced exactly" % what


def run_case(T, dtype, N, Cp, Dp, seed=0, spectra=True, wl=None):
    code = DT[dtype]
    if wl is None:
        wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd", "bwd_x", "bwd_w"), seed=seed)
    x, w, dy = W.make_x(wl), W.make_w(wl), W.make_dy(wl)
    xd, wd, dyd = (torch.from_numpy(a).to(DEV) for a in (x, w, dy))
    packs = []
    for mode, (o, i) in ((eql.EQL_PACK_FWD, (Dp, Cp)), (eql.EQL_PACK_BWDX, (Cp, Dp))):
        buf = torch.empty(eql.eqlinear_packed_weight_bytes(o, i, T, code), dtype=torch.uint8, device=DEV)
        eql.eqlinear_pack_weight(wd, buf, Dp, Cp, T, code, mode)
        packs.append(buf)
    wp, wpb = packs
    nbytes = eql.eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, code)
    ws = torch.full((max(nbytes, 16),), 0xFF, dtype=torch.uint8, device=DEV)  # NaN-filled
    ws_ref = torch.empty_like(ws)
    mk = lambda r, c: torch.empty((r, c), dtype=xd.dtype, device=DEV)
    y, dx, y0, dx0 = mk(N, Dp * T), mk(N, Cp * T), mk(N, Dp * T), mk(N, Cp * T)
    dw = torch.empty((Dp, Cp, T), dtype=xd.dtype, device=DEV)
    dw0 = torch.empty_like(dw)
    print("case T=%d %s N=%d C'=%d D'=%d fused=%s" % (T, dtype, N, Cp, Dp,
                                                      bwdw_fused(N, Cp, Dp, T, xd.element_size())), flush=True)
    eql.eqlinear_fwd_train(xd, wp, y, ws, nbytes, N, Cp, Dp, T, code)
    eql.eqlinear_bwd_x_train(dyd, wpb, dx, ws, nbytes, N, Cp, Dp, T, code)
    if spectra:
        ws_after = ws.clone()
    eql.eqlinear_bwd_w_train(dyd, dw, ws, nbytes, N, Cp, Dp, T, code)
    eql.eqlinear_fwd(xd, wp, y0, N, Cp, Dp, T, code)
    eql.eqlinear_bwd_x(dyd, wpb, dx0, N, Cp, Dp, T, code)
    eql.eqlinear_bwd_w(xd, dyd, dw0, ws_ref, nbytes, N, Cp, Dp, T, code)
    torch.cuda.synchronize()
    assert torch.equal(y, y0), "eqlinear_fwd_train changed y"
    assert torch.equal(dx, dx0), "eqlinear_bwd_x_train changed dx"
    if spectra and N > 0:
        dys, xs = spectrum_sections(N, Cp, Dp, T, xd.element_size())
        check_spectra(planes_of(ws_after, xs, N, T, dtype), planes_of(ws_ref, xs, N, T, dtype), x, T, dtype,
                      "x spectrum")
        if dys is not None:
            check_spectra(planes_of(ws_after, dys, N, T, dtype), planes_of(ws_ref, dys, N, T, dtype), dy, T,
                          dtype, "dy spectrum")
    return wl, x, dy, dw.cpu().numpy(), dw0.cpu().numpy()


CASES = [
    (4, "f16", 1000, 600, 600),    # separate path, 128-wide forward tiles
    (4, "f16", 777, 640, 1100),    # separate, ragged rows and tiles
    (4, "f16", 129, 1200, 520),    # separate, two row tiles, 256-wide weight-gradient tiles
    (4, "f16", 300, 96, 384),      # fused path (an MLP expansion's widths)
    (4, "f16", 4099, 64, 64),      # fused, narrow forward tiles, many row tiles
    (4, "f16", 3000, 40, 24),      # fused, one 32-channel block
    (4, "f16", 500, 601, 600),     # x rows not 16-byte aligned: separate transform for x
    (4, "f16", 1, 600, 600),       # one row
    (4, "f32", 300, 300, 520),     # fp32: separate transforms
    (8, "f16", 400, 300, 520),     # C8: separate transforms
    (3, "f32", 257, 33, 41),
    (2, "f16", 1000, 70, 132),     # fused path at T = 2
    (1, "f16", 333, 17, 40),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_%s_N%d_C%d_D%d" % c)
def test_train_trio_matches_plain_and_oracle(case):
    T, dtype, N, Cp, Dp = case
    wl, x, dy, dw, dw0 = run_case(T, dtype, N, Cp, Dp, seed=70 + T)
    ref = oracle.bwd_w(x, dy, T)
    assert rel_err(dw, ref) <= TOL[dtype]
    assert rel_err(dw0, ref) <= TOL[dtype]


def test_train_trio_no_rows():
    code = eql.EQL_F16
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    dw = torch.full((8, 6, 4), 7.0, dtype=torch.float16, device=DEV)
    eql.eqlinear_fwd_train(None, None, None, None, 0, 0, 6, 8, 4, code)
    eql.eqlinear_bwd_x_train(None, None, None, None, 0, 0, 6, 8, 4, code)
    eql.eqlinear_bwd_w_train(None, dw, ws, 0, 0, 6, 8, 4, code)
    torch.cuda.synchronize()
    assert not dw.any()


def test_train_rejects_short_workspace():
    code = eql.EQL_F16
    N, Cp, Dp, T = 64, 32, 32, 4
    nbytes = eql.eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    t = torch.empty((N, 128), dtype=torch.float16, device=DEV)
    w = torch.empty(eql.eqlinear_packed_weight_bytes(Dp, Cp, T, code), dtype=torch.uint8, device=DEV)
    dw = torch.empty((Dp, Cp, T), dtype=torch.float16, device=DEV)
    for call in (lambda: eql.eqlinear_fwd_train(t, w, t, ws, nbytes - 16, N, Cp, Dp, T, code),
                 lambda: eql.eqlinear_bwd_x_train(t, w, t, ws, nbytes - 16, N, Cp, Dp, T, code),
                 lambda: eql.eqlinear_bwd_w_train(t, dw, ws, nbytes - 16, N, Cp, Dp, T, code),
                 lambda: eql.eqlinear_fwd_train(t, w, t, None, nbytes, N, Cp, Dp, T, code)):
        with pytest.raises(eql.EqlError):
            call()


@pytest.mark.parametrize("key", ["c4", "c5"])
def test_train_full_size(key):
    """The two large workloads through the training entry points: y and dx bit-identical to
    the plain passes, every element of dw against the oracle (Frobenius and per-element
    bounds), and the spectra the forward kernel stored against the separate transform's."""
    from test_gpu_parity import Compare
    wl = W.WORKLOADS[key]
    print("case %s %s" % (key, wl.name), flush=True)
    wl, x, dy, dw, dw0 = run_case(wl.T, wl.dtype, wl.N, wl.Cp, wl.Dp, wl=wl)
    cmp = Compare(TOL[wl.dtype], "%s bwd_w_train" % key)
    cmp.add(dw.reshape(wl.Dp, -1), oracle.bwd_w(x, dy, wl.T).reshape(wl.Dp, -1))
    cmp.check()


@pytest.mark.parametrize("grads", ["both", "w_only", "x_only", "both_plain"])
def test_layer_autograd_through_training_entry_points(grads):
    """EQLinearFunction: with a weight gradient the forward keeps the workspace and the
    backward runs the training entry points (with only one gradient, or keep_spectra=False,
    the plain ones)."""
    from group_circulant_linear_p4_amd.layer import eqlinear
    T, N, Cp, Dp = 4, 333, 256, 520
    wl = W.Workload("t", "test", T, N, Cp, Dp, "f16", ("fwd", "bwd_x", "bwd_w"), seed=91)
    x_h, w_h, dy_h = W.make_x(wl), W.make_w(wl), W.make_dy(wl)
    x = torch.from_numpy(x_h).to(DEV).reshape(3, 111, Cp * T).requires_grad_(grads != "w_only")
    w = torch.from_numpy(w_h).to(DEV).requires_grad_(grads != "x_only")
    print("case layer %s" % grads, flush=True)
    y = eqlinear(x, w, keep_spectra=grads != "both_plain")
    y.backward(torch.from_numpy(dy_h).to(DEV).reshape(3, 111, Dp * T))
    torch.cuda.synchronize()
    assert rel_err(y.detach().cpu().numpy().reshape(N, -1), oracle.fwd(x_h, w_h)) <= TOL["f16"]
    if grads != "w_only":
        assert rel_err(x.grad.cpu().numpy().reshape(N, -1), oracle.bwd_x(dy_h, w_h)) <= TOL["f16"]
    else:
        assert x.grad is None
    if grads != "x_only":
        assert rel_err(w.grad.cpu().numpy(), oracle.bwd_w(x_h, dy_h, T)) <= TOL["f16"]
    else:
        assert w.grad is None


FUSED_TRAIN_CASES = [(4, "f16", 1000, 600, 600), (4, "f16", 300, 96, 384), (4, "f16", 500, 601, 600),
                     (3, "f32", 257, 33, 41), (8, "f16", 200, 130, 70)]


@pytest.mark.parametrize("case", FUSED_TRAIN_CASES, ids=lambda c: "T%d_%s_N%d_C%d_D%d" % c)
def test_fused_train_step(case):
    """eqlinear_fwd_fused_train (bias, GELU, residual, pre kept): y and pre bit-identical to
    eqlinear_fwd_fused, x's spectrum as the separate transform leaves it; then the epilogue
    backward and the training input and weight gradients on dpre against the oracle."""
    T, dtype, N, Cp, Dp = case
    code = DT[dtype]
    wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd", "bwd_x", "bwd_w"), seed=80 + T)
    x, w, dy, b, r = W.make_x(wl), W.make_w(wl), W.make_dy(wl), W.make_bias(wl), W.make_residual(wl)
    xd, wd, dyd, bd, rd = (torch.from_numpy(a).to(DEV) for a in (x, w, dy, b, r))
    wp = torch.empty(eql.eqlinear_packed_weight_bytes(Dp, Cp, T, code), dtype=torch.uint8, device=DEV)
    wpb = torch.empty(eql.eqlinear_packed_weight_bytes(Cp, Dp, T, code), dtype=torch.uint8, device=DEV)
    eql.eqlinear_pack_weight(wd, wp, Dp, Cp, T, code, eql.EQL_PACK_FWD)
    eql.eqlinear_pack_weight(wd, wpb, Dp, Cp, T, code, eql.EQL_PACK_BWDX)
    nbytes = eql.eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, code)
    ws = torch.full((max(nbytes, 16),), 0xFF, dtype=torch.uint8, device=DEV)
    ws_ref = torch.empty_like(ws)
    y, pre, y0, pre0, dpre = (torch.empty((N, Dp * T), dtype=xd.dtype, device=DEV) for _ in range(5))
    dx = torch.empty((N, Cp * T), dtype=xd.dtype, device=DEV)
    dw, dw0 = torch.empty((Dp, Cp, T), dtype=xd.dtype, device=DEV), torch.empty((Dp, Cp, T), dtype=xd.dtype,
                                                                                 device=DEV)
    db = torch.empty(Dp, dtype=xd.dtype, device=DEV)
    ebytes = eql.eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, code)
    ews = torch.empty(max(ebytes, 16), dtype=torch.uint8, device=DEV)
    print("case fused train T=%d %s N=%d C'=%d D'=%d" % case, flush=True)
    eql.eqlinear_fwd_fused_train(xd, wp, bd, rd, y, pre, ws, nbytes, N, Cp, Dp, T, code, eql.EQL_ACT_GELU)
    torch.cuda.synchronize()
    ws_after = ws.clone()
    eql.eqlinear_fused_epilogue_bwd(dyd, pre, dpre, db, ews, ebytes, N, Dp, T, code, eql.EQL_ACT_GELU)
    eql.eqlinear_bwd_x_train(dpre, wpb, dx, ws, nbytes, N, Cp, Dp, T, code)
    eql.eqlinear_bwd_w_train(dpre, dw, ws, nbytes, N, Cp, Dp, T, code)
    eql.eqlinear_fwd_fused(xd, wp, bd, rd, y0, pre0, N, Cp, Dp, T, code, eql.EQL_ACT_GELU)
    eql.eqlinear_bwd_w(xd, dpre, dw0, ws_ref, nbytes, N, Cp, Dp, T, code)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(pre, pre0), "eqlinear_fwd_fused_train changed y or pre"
    _, xs = spectrum_sections(N, Cp, Dp, T, xd.element_size())
    check_spectra(planes_of(ws_after, xs, N, T, dtype), planes_of(ws_ref, xs, N, T, dtype), x, T, dtype,
                  "x spectrum (fused forward)")
    dpre_h = dpre.cpu().numpy()
    assert rel_err(dx.cpu().numpy(), oracle.bwd_x(dpre_h, w)) <= TOL[dtype]
    assert rel_err(dw.cpu().numpy(), oracle.bwd_w(x, dpre_h, T)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [1, 3, 4, 8])
@pytest.mark.parametrize("shape", [(5, 3), (96, 384), (600, 520), (1024, 1024)], ids=lambda s: "D%d_C%d" % s)
def test_pack_weight_both_matches_two_packs(T, dtype, shape):
    """eqlinear_pack_weight_both: both packings bit-identical to two eqlinear_pack_weight calls."""
    Dp, Cp = shape
    code = DT[dtype]
    wl = W.Workload("t", "test", T, 1, Cp, Dp, dtype, ("fwd",), seed=5)
    wd = torch.from_numpy(W.make_w(wl)).to(DEV)
    nf = eql.eqlinear_packed_weight_bytes(Dp, Cp, T, code)
    nb = eql.eqlinear_packed_weight_bytes(Cp, Dp, T, code)
    a, b = torch.full((nf,), 0xAB, dtype=torch.uint8, device=DEV), torch.full((nb,), 0xAB, dtype=torch.uint8, device=DEV)
    a0, b0 = torch.empty_like(a), torch.empty_like(b)
    eql.eqlinear_pack_weight_both(wd, a, b, Dp, Cp, T, code)
    eql.eqlinear_pack_weight(wd, a0, Dp, Cp, T, code, eql.EQL_PACK_FWD)
    eql.eqlinear_pack_weight(wd, b0, Dp, Cp, T, code, eql.EQL_PACK_BWDX)
    torch.cuda.synchronize()
    assert torch.equal(a, a0) and torch.equal(b, b0)
