"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Error measure: relative Frobenius error ||got - ref|| / ||ref|| over the compared
elements, with the bounds fp32 <= 1e-5 and fp16 (fp32 accumulation) <= 3e-3.
Shapes span several tiles with ragged tails.  The five workloads run at their full
size in the launch configuration the benchmark uses and every output element is
compared with the oracle, under the Frobenius bound and a per-element bound
(Compare below).
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
NPDT = {"f32": np.float32, "f16": np.float16}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.cpu().numpy()


class Lib:
    """Runs each entry point on device copies of numpy inputs."""

    def __init__(self, T, dtype):
        self.T, self.dtype, self.code = T, dtype, DT[dtype]

    def pack(self, w_d, Dp, Cp, mode):
        out_ch, in_ch = (Dp, Cp) if mode == eql.EQL_PACK_FWD else (Cp, Dp)
        buf = torch.empty(eql.eqlinear_packed_weight_bytes(out_ch, in_ch, self.T, self.code),
                          dtype=torch.uint8, device=DEV)
        eql.eqlinear_pack_weight(w_d, buf, Dp, Cp, self.T, self.code, mode)
        return buf

    def fwd_d(self, x_d, wp, N, Cp, Dp):
        y = torch.empty((N, Dp * self.T), dtype=x_d.dtype, device=DEV)
        eql.eqlinear_fwd(x_d, wp, y, N, Cp, Dp, self.T, self.code)
        return y

    def bwd_x_d(self, dy_d, wpb, N, Cp, Dp):
        dx = torch.empty((N, Cp * self.T), dtype=dy_d.dtype, device=DEV)
        eql.eqlinear_bwd_x(dy_d, wpb, dx, N, Cp, Dp, self.T, self.code)
        return dx

    def bwd_w_d(self, x_d, dy_d, N, Cp, Dp):
        nbytes = eql.eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, self.T, self.code)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
        dw = torch.empty((Dp, Cp, self.T), dtype=x_d.dtype, device=DEV)
        eql.eqlinear_bwd_w(x_d, dy_d, dw, ws, nbytes, N, Cp, Dp, self.T, self.code)
        return dw

    def all_passes(self, x, w, dy):
        N, Dp, Cp = x.shape[0], w.shape[0], w.shape[1]
        x_d, w_d, dy_d = dev(x), dev(w), dev(dy)
        wp = self.pack(w_d, Dp, Cp, eql.EQL_PACK_FWD)
        wpb = self.pack(w_d, Dp, Cp, eql.EQL_PACK_BWDX)
        y = self.fwd_d(x_d, wp, N, Cp, Dp)
        dx = self.bwd_x_d(dy_d, wpb, N, Cp, Dp)
        dw = self.bwd_w_d(x_d, dy_d, N, Cp, Dp)
        torch.cuda.synchronize()
        return host(y), host(dx), host(dw)


def inputs(T, N, Cp, Dp, dtype, seed=0):
    wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd", "bwd_x", "bwd_w"), seed=seed)
    return W.make_x(wl), W.make_w(wl), W.make_dy(wl)


# ----------------------------------------------------------------- small shapes
SHAPES = [(197, 3, 5), (300, 33, 37), (1, 1, 1), (129, 2, 130), (257, 7, 9)]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "N%d_C%d_D%d" % s)
def test_all_passes_match_oracle(T, dtype, shape):
    N, Cp, Dp = shape
    print("case T=%d %s N=%d C'=%d D'=%d" % (T, dtype, N, Cp, Dp), flush=True)
    x, w, dy = inputs(T, N, Cp, Dp, dtype, seed=T)
    y, dx, dw = Lib(T, dtype).all_passes(x, w, dy)
    tol = TOL[dtype]
    assert rel_err(y, oracle.fwd(x, w)) <= tol
    assert rel_err(dx, oracle.bwd_x(dy, w)) <= tol
    assert rel_err(dw, oracle.bwd_w(x, dy, T)) <= tol


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("shape", [(1000, 96, 160), (640, 64, 64), (4096, 40, 24)],
                         ids=lambda s: "N%d_C%d_D%d" % s)
def test_p4_multi_tile(dtype, shape):
    N, Cp, Dp = shape
    print("case p4 %s N=%d C'=%d D'=%d" % (dtype, N, Cp, Dp), flush=True)
    x, w, dy = inputs(4, N, Cp, Dp, dtype, seed=7)
    y, dx, dw = Lib(4, dtype).all_passes(x, w, dy)
    assert rel_err(y, oracle.fwd(x, w)) <= TOL[dtype]
    assert rel_err(dx, oracle.bwd_x(dy, w)) <= TOL[dtype]
    assert rel_err(dw, oracle.bwd_w(x, dy, 4)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [3, 4, 8])
def test_multi_tile_ragged_channels(T, dtype):
    """Several 256-wide weight-gradient tiles in both channel axes, each with a
    ragged last tile, more rows than one k-step range, and for odd T a single real
    plane beside the complex pairs."""
    N, Cp, Dp = 700, 300, 520
    print("case T=%d %s N=%d C'=%d D'=%d" % (T, dtype, N, Cp, Dp), flush=True)
    x, w, dy = inputs(T, N, Cp, Dp, dtype, seed=11 + T)
    y, dx, dw = Lib(T, dtype).all_passes(x, w, dy)
    assert rel_err(y, oracle.fwd(x, w)) <= TOL[dtype]
    assert rel_err(dx, oracle.bwd_x(dy, w)) <= TOL[dtype]
    assert rel_err(dw, oracle.bwd_w(x, dy, T)) <= TOL[dtype]


# ------------------------------------------------------------ the five workloads
@pytest.mark.parametrize("key", ["c1", "c2", "c3"])
def test_workload_full_compare(key):
    wl = W.WORKLOADS[key]
    print("case %s %s" % (key, wl.name), flush=True)
    x, w, dy = W.make_x(wl), W.make_w(wl), W.make_dy(wl)
    y, dx, dw = Lib(wl.T, wl.dtype).all_passes(x, w, dy)
    tol = TOL[wl.dtype]
    for name, got, ref in (("fwd", y, oracle.fwd(x, w)), ("bwd_x", dx, oracle.bwd_x(dy, w)),
                           ("bwd_w", dw.reshape(wl.Dp, -1), oracle.bwd_w(x, dy, wl.T).reshape(wl.Dp, -1))):
        cmp = Compare(tol, "%s %s" % (key, name))
        cmp.add(got, ref)
        cmp.check()


# Per-element bound beside the Frobenius one: |got - ref| <= ELEM_K * tol * (|ref| + rms),
# rms the root mean square of the reference over the element's row (for dw, over the
# (c, t) entries of its output channel d).  One fp16 rounding of the output contributes
# at most 2^-11 |ref|; the rounded transforms contribute a random error of about
# 2^-11 * sqrt(2) * rms per element, whose largest value over 10^8 elements stays
# below 6 sigma.  ELEM_K = 4 puts the bound at 1.2e-2 (|ref| + rms) for fp16: a
# wrong element (off by a few percent of its row's scale or more) fails it even where
# a Frobenius norm over 10^8 elements would absorb it.
ELEM_K = 4.0


class Compare:
    """Accumulates the Frobenius error over chunks and checks every element."""

    def __init__(self, tol, what):
        self.tol, self.what = tol, what
        self.num = self.den = 0.0
        self.worst = 0.0
        self.count = 0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64).reshape(ref.shape[0], -1)
        ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
        d = got - ref
        self.num += float(np.sum(d * d))
        self.den += float(np.sum(ref * ref))
        rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
        ratio = np.abs(d) / (ELEM_K * self.tol * (np.abs(ref) + rms) + 1e-300)
        self.worst = max(self.worst, float(ratio.max()) if ratio.size else 0.0)
        self.count += ref.size
        assert np.isfinite(got).all(), "%s: non-finite output" % self.what

    def check(self):
        err = float(np.sqrt(self.num / self.den)) if self.den > 0 else float(np.sqrt(self.num))
        print("%s: %d elements, relative Frobenius error %.3g, worst element at %.3g of its bound"
              % (self.what, self.count, err, self.worst), flush=True)
        assert err <= self.tol, "%s: relative error %.3g > %.1g" % (self.what, err, self.tol)
        assert self.worst <= 1.0, "%s: an element exceeds %g * tol * (|ref| + row rms)" % (self.what, ELEM_K)


_FULL_CACHE = {}


def _full_outputs(key):
    """GPU outputs of every pass on the whole workload, in the benchmark's launch
    configuration (one run per workload, shared by the three pass tests)."""
    if key not in _FULL_CACHE:
        _FULL_CACHE.clear()
        wl = W.WORKLOADS[key]
        x, w, dy = W.make_x(wl), W.make_w(wl), W.make_dy(wl)
        y, dx, dw = Lib(wl.T, wl.dtype).all_passes(x, w, dy)
        _FULL_CACHE[key] = (wl, x, w, dy, y, dx, dw)
    return _FULL_CACHE[key]


@pytest.mark.parametrize("pass_", ["fwd", "bwd_x", "bwd_w"])
@pytest.mark.parametrize("key", ["c4", "c5"])
def test_workload_full_size(key, pass_):
    """Every output element of the two large workloads (all rows of y and dx, all of
    dw, so every row tile of every persistent round and, for c5, every x16 row)
    against the oracle, in 8192-row chunks."""
    print("case %s %s %s" % (key, pass_, W.WORKLOADS[key].name), flush=True)
    wl, x, w, dy, y, dx, dw = _full_outputs(key)
    tol = TOL[wl.dtype]
    cmp = Compare(tol, "%s %s" % (key, pass_))
    if pass_ == "bwd_w":
        cmp.add(dw.reshape(wl.Dp, -1), oracle.bwd_w(x, dy, wl.T).reshape(wl.Dp, -1))
    else:
        got, src = (y, x) if pass_ == "fwd" else (dx, dy)
        ref_fn = oracle.fwd if pass_ == "fwd" else oracle.bwd_x
        for r0 in range(0, wl.N, 8192):
            cmp.add(got[r0:r0 + 8192], ref_fn(src[r0:r0 + 8192], w))
    cmp.check()
    if key == "c5" and pass_ == "fwd":
        hot = W.hot_rows(wl)
        assert hot.size == 655
        hc = Compare(tol, "c5 fwd, the x16 rows")
        hc.add(y[hot], oracle.fwd(x[hot], w))
        hc.check()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_two_block_tile(T, dtype):
    """157 row tiles x 64 output channels: on a 256-CU device the tile-width model
    picks the 64-column tile for the forward (D' = 64) and the input gradient
    (C' = 40): one round of tiles where 32-column tiles would need two."""
    N, Cp, Dp = 20000, 40, 64
    print("case two-block tile T=%d %s" % (T, dtype), flush=True)
    x, w, dy = inputs(T, N, Cp, Dp, dtype, seed=40 + T)
    y, dx, dw = Lib(T, dtype).all_passes(x, w, dy)
    tol = TOL[dtype]
    assert rel_err(y, oracle.fwd(x, w)) <= tol
    assert rel_err(dx, oracle.bwd_x(dy, w)) <= tol
    assert rel_err(dw, oracle.bwd_w(x, dy, T)) <= tol


# -------------------------------------------------------------- fused epilogue
def fused_d(T, dtype, x_d, wp, b_d, r_d, y, N, Cp, Dp, act):
    eql.eqlinear_fwd_fused(x_d, wp, b_d, r_d, y, None, N, Cp, Dp, T, DT[dtype],
                           eql.EQL_ACT_GELU if act == "gelu" else eql.EQL_ACT_NONE)
    return y


FUSED_CASES = [(True, "gelu", False), (True, "none", True), (False, "gelu", True), (True, "gelu", True)]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [3, 4, 8, 16])
@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "b%d_%s_r%d" % (c[0], c[1], c[2]))
def test_fwd_fused_matches_oracle(T, dtype, case):
    use_b, act, use_r = case
    N, Cp, Dp = 300, 33, 70                      # three row tiles, ragged channel counts
    print("case fused T=%d %s %s" % (T, dtype, case), flush=True)
    wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd",), seed=21 + T)
    x, w = W.make_x(wl), W.make_w(wl)
    b = W.make_bias(wl) if use_b else None
    r = W.make_residual(wl) if use_r else None
    L = Lib(T, dtype)
    x_d, w_d = dev(x), dev(w)
    wp = L.pack(w_d, Dp, Cp, eql.EQL_PACK_FWD)
    y = torch.empty((N, Dp * T), dtype=x_d.dtype, device=DEV)
    fused_d(T, dtype, x_d, wp, dev(b) if use_b else None, dev(r) if use_r else None, y, N, Cp, Dp, act)
    ref = oracle.fwd_fused(x, w, bias=b, residual=r, act=act)
    assert rel_err(host(y), ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_fwd_fused_in_place_residual_and_plain_equivalence(dtype):
    T, N, Cp, Dp = 4, 261, 40, 96
    print("case fused in-place %s" % dtype, flush=True)
    wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd",), seed=5)
    x, w, b, r = W.make_x(wl), W.make_w(wl), W.make_bias(wl), W.make_residual(wl)
    L = Lib(T, dtype)
    x_d, w_d = dev(x), dev(w)
    wp = L.pack(w_d, Dp, Cp, eql.EQL_PACK_FWD)
    y = dev(r).clone()                                       # residual buffer doubles as the output
    fused_d(T, dtype, x_d, wp, dev(b), y, y, N, Cp, Dp, "gelu")
    assert rel_err(host(y), oracle.fwd_fused(x, w, bias=b, residual=r, act="gelu")) <= TOL[dtype]
    # Nothing fused: bitwise the plain forward.
    y0 = L.fwd_d(x_d, wp, N, Cp, Dp)
    y1 = torch.empty_like(y0)
    fused_d(T, dtype, x_d, wp, None, None, y1, N, Cp, Dp, "none")
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_fwd_fused_matches_torch_fp32_epilogue(dtype):
    """Against plain PyTorch fp32 ops applied to the unfused kernel's fp32-rounded
    output: F.gelu(y + b) + r."""
    T, N, Cp, Dp = 4, 520, 64, 160
    print("case fused vs torch %s" % dtype, flush=True)
    wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd",), seed=8)
    x, w, b, r = W.make_x(wl), W.make_w(wl), W.make_bias(wl), W.make_residual(wl)
    L = Lib(T, dtype)
    x_d, w_d, b_d, r_d = dev(x), dev(w), dev(b), dev(r)
    wp = L.pack(w_d, Dp, Cp, eql.EQL_PACK_FWD)
    y = torch.empty((N, Dp * T), dtype=x_d.dtype, device=DEV)
    fused_d(T, dtype, x_d, wp, b_d, r_d, y, N, Cp, Dp, "gelu")
    plain = L.fwd_d(x_d, wp, N, Cp, Dp).float()
    ref = torch.nn.functional.gelu(plain + b_d.float().repeat_interleave(T)) + r_d.float()
    torch.cuda.synchronize()
    assert rel_err(host(y.float()), host(ref)) <= TOL[dtype]


def test_fwd_fused_mlp_expansion_full_size():
    """The EQ-ViT-S MLP expansion (c2) at full size with bias and GELU; every row."""
    wl = W.WORKLOADS["c2"]
    T, N, Cp, Dp = wl.T, wl.N, wl.Cp, wl.Dp
    print("case fused %s" % wl.name, flush=True)
    x, w, b = W.make_x(wl), W.make_w(wl), W.make_bias(wl)
    L = Lib(T, wl.dtype)
    x_d, w_d = dev(x), dev(w)
    wp = L.pack(w_d, Dp, Cp, eql.EQL_PACK_FWD)
    y = torch.empty((N, Dp * T), dtype=x_d.dtype, device=DEV)
    fused_d(T, wl.dtype, x_d, wp, dev(b), None, y, N, Cp, Dp, "gelu")
    cmp = Compare(TOL[wl.dtype], "c2 fused bias + GELU")
    cmp.add(host(y), oracle.fwd_fused(x, w, bias=b, act="gelu"))
    cmp.check()


# ------------------------------------------------------------------ pack layout
def unpack(buf, out_ch, in_ch, T, dtype):
    """Planes of the packed weight in the documented layout: output channels in blocks
    of 32; per block and stage of two 16-byte input groups one chunk of T*64 units,
    ordered [plane][channel of the block][group of the stage XOR bit 3 of the channel]."""
    G = 16 // np.dtype(NPDT[dtype]).itemsize
    jin = -(-(-(-in_ch // G)) // 4) * 4          # ceil(in / G) rounded up to a multiple of 4
    opad = -(-out_ch // 32) * 32
    a = host(buf).view(NPDT[dtype]).astype(np.float64)
    assert a.size == opad * jin * T * G
    a = a.reshape(opad // 32, jin // 2, T, 32, 2, G)  # [block][stage][plane][channel][half'][element]
    ol = np.arange(32)
    swz = (ol >> 3) & 1
    halves = np.stack([a[:, :, :, ol, h ^ swz, :] for h in (0, 1)], axis=4)  # undo the XOR: [.., ol, half, G]
    planes = halves.transpose(0, 3, 1, 4, 5, 2).reshape(opad, jin * G, T)  # [o][input channel][plane]
    assert np.all(planes[out_ch:] == 0) and np.all(planes[:, in_ch:, :] == 0)
    planes = planes[:out_ch, :in_ch, :]
    nr = 2 if (T % 2 == 0 and T > 1) else 1
    planes[:, :, :nr] *= T                         # stored with the inverse's 1/T ...
    planes[:, :, nr:] *= T / 2.0                   # ... and 2/T on the complex planes
    spec = np.zeros((out_ch, in_ch, T // 2 + 1), dtype=np.complex128)
    spec[:, :, 0] = planes[:, :, 0]
    if nr == 2:
        spec[:, :, T // 2] = planes[:, :, 1]
    for q in range((T - nr) // 2):
        spec[:, :, q + 1] = planes[:, :, nr + 2 * q] + 1j * planes[:, :, nr + 2 * q + 1]
    return spec


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8, 16])
def test_pack_weight_is_half_spectrum(T, dtype):
    Dp, Cp = 5, 11
    _, w, _ = inputs(T, 1, Cp, Dp, dtype, seed=3)
    L = Lib(T, dtype)
    w_d = dev(w)
    ref = oracle.half_spectrum(w)                                   # [D', C', K]
    fwd = unpack(L.pack(w_d, Dp, Cp, eql.EQL_PACK_FWD), Dp, Cp, T, dtype)
    bwd = unpack(L.pack(w_d, Dp, Cp, eql.EQL_PACK_BWDX), Cp, Dp, T, dtype)
    # One rounding of an fp32 value to the element type (plus fp32 sums).
    tol = 1e-6 if dtype == "f32" else 2.0 ** -10
    scale = np.abs(w.astype(np.float64)).sum(axis=2, keepdims=True)
    assert np.all(np.abs(fwd - ref) <= tol * scale + 1e-12)
    assert np.all(np.abs(bwd - np.conj(ref).transpose(1, 0, 2)) <= tol * scale.transpose(1, 0, 2) + 1e-12)


# ---------------------------------------------------------- equivariance, misc
def roll_group(a, s, T):
    n = a.shape[0]
    return np.roll(a.reshape(n, -1, T), s, axis=2).reshape(n, -1)


@pytest.mark.parametrize("dtype,T", [("f16", 4), ("f32", 4), ("f32", 8), ("f16", 8), ("f32", 3)])
def test_equivariance_residual(dtype, T):
    N, Cp, Dp = 384, 40, 72
    x, w, dy = inputs(T, N, Cp, Dp, dtype, seed=9)
    L = Lib(T, dtype)
    w_d = dev(w)
    wp = L.pack(w_d, Dp, Cp, eql.EQL_PACK_FWD)
    y = host(L.fwd_d(dev(x), wp, N, Cp, Dp))
    dw = host(L.bwd_w_d(dev(x), dev(dy), N, Cp, Dp)).astype(np.float64)
    for s in sorted({1, T - 1}):
        ys = host(L.fwd_d(dev(roll_group(x, s, T)), wp, N, Cp, Dp))
        rho = rel_err(ys, roll_group(y, s, T).astype(np.float64))
        assert rho <= TOL[dtype]
        if T == 4:
            # p4: the butterflies map a shift to an exact permutation / negation of
            # the planes and the MFMA chains are ordered symmetrically, so the
            # residual only reflects the matrix cores' internal rounding of negated
            # operands (measured ~1e-7, orders below the tolerance).
            assert rho <= 1e-5, "p4 residual %g" % rho
        dws = host(L.bwd_w_d(dev(roll_group(x, s, T)), dev(roll_group(dy, s, T)), N, Cp, Dp))
        assert rel_err(dws, dw) <= TOL[dtype]


def test_deterministic_repeat():
    T, N, Cp, Dp = 4, 2048, 64, 96
    x, w, dy = inputs(T, N, Cp, Dp, "f16", seed=2)
    L = Lib(T, "f16")
    a = L.all_passes(x, w, dy)
    b = L.all_passes(x, w, dy)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_zero_rows():
    T, Cp, Dp = 4, 8, 8
    L = Lib(T, "f16")
    w_d = dev(inputs(T, 1, Cp, Dp, "f16")[1])
    wp = L.pack(w_d, Dp, Cp, eql.EQL_PACK_FWD)
    y = torch.full((1, Dp * T), 7.0, dtype=torch.float16, device=DEV)
    eql.eqlinear_fwd(y, wp, y[:0], 0, Cp, Dp, T, eql.EQL_F16)       # no-op
    x0 = torch.empty((0, Cp * T), dtype=torch.float16, device=DEV)
    dw = L.bwd_w_d(x0, torch.empty((0, Dp * T), dtype=torch.float16, device=DEV), 0, Cp, Dp)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    assert torch.all(dw == 0)


def test_misaligned_buffer_is_rejected():
    T, Cp, Dp, N = 4, 4, 4, 8
    L = Lib(T, "f32")
    w_d = dev(inputs(T, 1, Cp, Dp, "f32")[1])
    wp = L.pack(w_d, Dp, Cp, eql.EQL_PACK_FWD)
    big = torch.zeros(N * Cp * T + 2, dtype=torch.float32, device=DEV)
    y = torch.empty((N, Dp * T), dtype=torch.float32, device=DEV)
    with pytest.raises(eql.EqlError) as ei:
        eql.eqlinear_fwd(big[1:].data_ptr(), wp, y, N, Cp, Dp, T, eql.EQL_F32)
    assert ei.value.status == eql.EQL_EALIGN


def _sweep_cases(n=30, seed=2024):
    """Seeded shapes over every T and both dtypes (oracle work <= ~5e8 MACs each), plus
    large-N / few-channel shapes for which the tile-width model picks two-block tiles."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        T = int(rng.integers(1, 17))
        dtype = ["f32", "f16"][int(rng.integers(0, 2))]
        N = int(rng.integers(1, 1500))
        Cp = int(rng.integers(1, 90))
        Dp = int(rng.integers(1, 90))
        if N * Cp * Dp * T * T <= 5e8:
            cases.append((T, dtype, N, Cp, Dp))
    cases += [(4, "f16", 14000, 24, 80), (2, "f32", 20000, 16, 60), (1, "f16", 30000, 40, 48),
              (3, "f16", 17000, 20, 96), (4, "f32", 12800, 96, 40), (4, "f16", 16500, 70, 33)]
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "T%d_%s_N%d_C%d_D%d" % c)
def test_random_shape_sweep(case):
    T, dtype, N, Cp, Dp = case
    print("case sweep T=%d %s N=%d C'=%d D'=%d" % case, flush=True)
    x, w, dy = inputs(T, N, Cp, Dp, dtype, seed=N % 97 + T)
    y, dx, dw = Lib(T, dtype).all_passes(x, w, dy)
    tol = TOL[dtype]
    assert rel_err(y, oracle.fwd(x, w)) <= tol
    assert rel_err(dx, oracle.bwd_x(dy, w)) <= tol
    assert rel_err(dw, oracle.bwd_w(x, dy, T)) <= tol
    # The fused epilogue on the same shape (bias + GELU + residual).
    wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd",), seed=3)
    b, r = W.make_bias(wl), W.make_residual(wl)
    L = Lib(T, dtype)
    x_d = dev(x)
    wp = L.pack(dev(w), Dp, Cp, eql.EQL_PACK_FWD)
    yf = torch.empty((N, Dp * T), dtype=x_d.dtype, device=DEV)
    fused_d(T, dtype, x_d, wp, dev(b), dev(r), yf, N, Cp, Dp, "gelu")
    torch.cuda.synchronize()
    assert rel_err(host(yf), oracle.fwd_fused(x, w, bias=b, residual=r, act="gelu")) <= tol
    # The epilogue's backward on the same shape (GELU, bias gradient), r standing in for pre.
    dy_d, r_d = dev(dy), dev(r)
    dpre = torch.empty_like(dy_d)
    db = epi_bwd_d(T, dtype, dy_d, r_d, dpre, True, N, Dp, "gelu")
    torch.cuda.synchronize()
    ref_dpre, ref_db = oracle.fused_epilogue_bwd(dy, r, T, act="gelu")
    assert rel_err(host(dpre), ref_dpre) <= tol
    assert rel_err(host(db), ref_db) <= tol


def epi_bwd_d(T, dtype, dy_d, pre_d, dpre, with_bias, N, Dp, act):
    code = DT[dtype]
    nbytes = eql.eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, code)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    db = torch.empty(Dp, dtype=dy_d.dtype, device=DEV) if with_bias else None
    eql.eqlinear_fused_epilogue_bwd(dy_d, pre_d, dpre, db, ws, nbytes, N, Dp, T, code,
                                    eql.EQL_ACT_GELU if act == "gelu" else eql.EQL_ACT_NONE)
    return db


# Rows of (D'T) elements stream in chunks of 16, 8, 4 or 2 bytes (the widest power of
# two dividing the row); between them these shapes take every chunk width, and
# dozens of ragged row blocks.
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [3, 4, 8])
@pytest.mark.parametrize("act", ["gelu", "none"])
@pytest.mark.parametrize("shape", [(700, 70), (1301, 7)], ids=lambda s: "N%d_D%d" % s)
def test_fused_epilogue_bwd_matches_oracle(T, dtype, act, shape):
    N, Dp = shape
    print("case epilogue bwd T=%d %s %s N=%d D'=%d" % (T, dtype, act, N, Dp), flush=True)
    wl = W.Workload("t", "test", T, N, 8, Dp, dtype, ("fwd",), seed=31 + T)
    dy, pre = W.make_dy(wl), W.make_residual(wl)
    dy_d, pre_d = dev(dy), dev(pre)
    dpre = torch.empty_like(dy_d)
    db = epi_bwd_d(T, dtype, dy_d, pre_d if act == "gelu" else None, dpre, True, N, Dp, act)
    torch.cuda.synchronize()
    ref_dpre, ref_db = oracle.fused_epilogue_bwd(dy, pre, T, act=act)
    assert rel_err(host(dpre), ref_dpre) <= TOL[dtype]
    assert rel_err(host(db), ref_db) <= TOL[dtype]
    # In place (dpre = dy) gives the same result, bias gradient included (without an
    # activation the kernel then stores nothing and only sums).
    dyi = dy_d.clone()
    dbi = epi_bwd_d(T, dtype, dyi, pre_d if act == "gelu" else None, dyi, True, N, Dp, act)
    torch.cuda.synchronize()
    assert torch.equal(dyi, dpre)
    assert torch.equal(dbi, db)


def test_fused_epilogue_bwd_full_size():
    """The epilogue backward at the benchmark's size (p4 fp16, N=65536, D'T=4096: 8
    blocks of 64 16-byte chunks across, 256 row blocks of 256 rows): every row of dpre
    and the bias gradient against the oracle, and the bias gradient also against an
    fp64 sum of the kernel's own dpre over every row."""
    wl = W.WORKLOADS["c5"]
    T, N, Dp = wl.T, wl.N, wl.Dp
    print("case epilogue bwd full size %s" % wl.name, flush=True)
    dy, pre = W.make_dy(wl), W.make_residual(wl)
    dy_d, pre_d = dev(dy), dev(pre)
    dpre = torch.empty_like(dy_d)
    db = epi_bwd_d(T, wl.dtype, dy_d, pre_d, dpre, True, N, Dp, "gelu")
    torch.cuda.synchronize()
    got = host(dpre)
    cmp = Compare(TOL[wl.dtype], "c5 epilogue bwd dpre")
    ref_db = np.zeros(Dp)
    for r0 in range(0, N, 8192):
        ref_dpre, part = oracle.fused_epilogue_bwd(dy[r0:r0 + 8192], pre[r0:r0 + 8192], T, act="gelu")
        cmp.add(got[r0:r0 + 8192], ref_dpre)
        ref_db += part
    cmp.check()
    assert rel_err(host(db), ref_db) <= TOL[wl.dtype]
    total = torch.zeros(Dp, dtype=torch.float64, device=DEV)
    for r0 in range(0, N, 8192):
        total += dpre[r0:r0 + 8192].view(-1, Dp, T).double().sum(dim=(0, 2))
    torch.cuda.synchronize()
    assert rel_err(host(db), host(total)) <= TOL[wl.dtype]


def test_fused_epilogue_bwd_empty_and_pre_out():
    """N = 0 writes a zero bias gradient; pre_out of the fused forward is x W^T + b."""
    dy_d = torch.empty((0, 40), dtype=torch.float32, device=DEV)
    db = epi_bwd_d(4, "f32", dy_d, None, dy_d, True, 0, 10, "none")
    torch.cuda.synchronize()
    assert torch.equal(db, torch.zeros(10, device=DEV))
    T, N, Cp, Dp, dtype = 4, 333, 24, 50, "f16"
    wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd",), seed=12)
    x, w, b = W.make_x(wl), W.make_w(wl), W.make_bias(wl)
    L = Lib(T, dtype)
    x_d = dev(x)
    wp = L.pack(dev(w), Dp, Cp, eql.EQL_PACK_FWD)
    y = torch.empty((N, Dp * T), dtype=x_d.dtype, device=DEV)
    pre = torch.empty_like(y)
    eql.eqlinear_fwd_fused(x_d, wp, dev(b), None, y, pre, N, Cp, Dp, T, DT[dtype], eql.EQL_ACT_GELU)
    torch.cuda.synchronize()
    assert rel_err(host(pre), oracle.fwd_fused(x, w, bias=b)) <= TOL[dtype]
    assert rel_err(host(y), oracle.fwd_fused(x, w, bias=b, act="gelu")) <= TOL[dtype]


@pytest.mark.parametrize("mode", ["plain", "fused_bias_gelu", "train", "fused_train"])
def test_graph_replay_matches_eager(mode):
    """One training step captured in a HIP graph and replayed three times: pack, forward,
    input gradient and weight gradient; with `fused`, the forward with bias + GELU that
    keeps pre, the epilogue's backward (dpre, dbias), and both gradients on dpre; with
    `train`, the training entry points (spectra kept in the workspace between the passes,
    on a shape whose weight gradient takes the separate path).
    Between replays the inputs are rewritten in place and other eager work runs; every
    replay must equal the eager result for the same inputs bit for bit (the library
    allocates nothing and records no memset, so the captured step is the eager one)."""
    fused, train = mode.startswith("fused"), mode.endswith("train")
    T, N, Cp, Dp, dtype = (4, 700, 600, 520, "f16") if train else (4, 700, 72, 96, "f16")
    print("case graph replay %s" % mode, flush=True)
    code = DT[dtype]
    bufs = [inputs(T, N, Cp, Dp, dtype, seed=60 + i) for i in range(4)]
    biases = [W.make_bias(W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd",), seed=70 + i)) for i in range(4)]
    x_d, w_d, dy_d = (dev(a) for a in bufs[0])
    b_d = dev(biases[0])
    wp = torch.empty(eql.eqlinear_packed_weight_bytes(Dp, Cp, T, code), dtype=torch.uint8, device=DEV)
    wpb = torch.empty(eql.eqlinear_packed_weight_bytes(Cp, Dp, T, code), dtype=torch.uint8, device=DEV)
    y = torch.empty((N, Dp * T), dtype=x_d.dtype, device=DEV)
    pre, dpre = torch.empty_like(y), torch.empty_like(y)
    db = torch.empty_like(b_d)
    dx = torch.empty((N, Cp * T), dtype=x_d.dtype, device=DEV)
    dw = torch.empty_like(w_d)
    nbytes = eql.eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, code)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    ebytes = eql.eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, code)
    ews = torch.empty(max(ebytes, 16), dtype=torch.uint8, device=DEV)

    def step():
        eql.eqlinear_pack_weight(w_d, wp, Dp, Cp, T, code, eql.EQL_PACK_FWD)
        eql.eqlinear_pack_weight(w_d, wpb, Dp, Cp, T, code, eql.EQL_PACK_BWDX)
        if fused:
            if train:
                eql.eqlinear_fwd_fused_train(x_d, wp, b_d, None, y, pre, ws, nbytes, N, Cp, Dp, T, code,
                                             eql.EQL_ACT_GELU)
            else:
                eql.eqlinear_fwd_fused(x_d, wp, b_d, None, y, pre, N, Cp, Dp, T, code, eql.EQL_ACT_GELU)
            eql.eqlinear_fused_epilogue_bwd(dy_d, pre, dpre, db, ews, ebytes, N, Dp, T, code, eql.EQL_ACT_GELU)
            g_out = dpre
        else:
            if train:
                eql.eqlinear_fwd_train(x_d, wp, y, ws, nbytes, N, Cp, Dp, T, code)
            else:
                eql.eqlinear_fwd(x_d, wp, y, N, Cp, Dp, T, code)
            g_out = dy_d
        if train:
            eql.eqlinear_bwd_x_train(g_out, wpb, dx, ws, nbytes, N, Cp, Dp, T, code)
            eql.eqlinear_bwd_w_train(g_out, dw, ws, nbytes, N, Cp, Dp, T, code)
        else:
            eql.eqlinear_bwd_x(g_out, wpb, dx, N, Cp, Dp, T, code)
            eql.eqlinear_bwd_w(x_d, g_out, dw, ws, nbytes, N, Cp, Dp, T, code)

    outs = (y, dx, dw) + ((pre, dpre, db) if fused else ())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(1, 4):
        xh, wh, dyh = bufs[i]
        x_d.copy_(dev(xh)); w_d.copy_(dev(wh)); dy_d.copy_(dev(dyh)); b_d.copy_(dev(biases[i]))
        junk = torch.randn(1 << 20, device=DEV).sum()          # other eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = tuple(t.clone() for t in outs)
        step()                                                  # eager, same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert torch.equal(a, b)
        if fused:
            assert rel_err(host(got[0]), oracle.fwd_fused(xh, wh, bias=biases[i], act="gelu")) <= TOL[dtype]
        else:
            assert rel_err(host(got[0]), oracle.fwd(xh, wh)) <= TOL[dtype]
        assert bool(torch.isfinite(junk))


def test_layer_fused_forward_matches_oracle():
    from group_circulant_linear_p4_amd.layer import eqlinear_fused
    T, N, Cp, Dp = 4, 3 * 37, 24, 40
    print("case layer fused", flush=True)
    wl = W.Workload("t", "test", T, N, Cp, Dp, "f32", ("fwd",), seed=17)
    x, w, b, r = W.make_x(wl), W.make_w(wl), W.make_bias(wl), W.make_residual(wl)
    y = eqlinear_fused(dev(x).reshape(3, 37, Cp * T), dev(w), dev(b), dev(r), act="gelu")
    assert tuple(y.shape) == (3, 37, Dp * T)
    ref = oracle.fwd_fused(x, w, bias=b, residual=r, act="gelu")
    assert rel_err(host(y).reshape(N, Dp * T), ref) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("act", ["gelu", "none"])
def test_layer_fused_training_with_residual(act, dtype):
    """eqlinear_fused(x, w, b, r, act) trains: gradients of x, w, b and r against the
    oracle's chain rule (dr = dy; without an activation dpre is dy itself)."""
    from group_circulant_linear_p4_amd.layer import eqlinear_fused
    T, N, Cp, Dp = 4, 2 * 65, 20, 28
    print("case layer fused training act=%s %s" % (act, dtype), flush=True)
    wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("fwd",), seed=23)
    x, w, b, r, dy = W.make_x(wl), W.make_w(wl), W.make_bias(wl), W.make_residual(wl), W.make_dy(wl)
    xt, wt, bt, rt = (dev(a).requires_grad_() for a in (x, w, b, r))
    y = eqlinear_fused(xt.reshape(2, 65, Cp * T), wt, bt, rt, act=act)
    y.backward(dev(dy).reshape(2, 65, Dp * T))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert rel_err(host(y.detach()).reshape(N, Dp * T), oracle.fwd_fused(x, w, bias=b, residual=r, act=act)) <= tol
    dpre, db = oracle.fused_epilogue_bwd(dy, oracle.fwd_fused(x, w, bias=b), T, act=act)
    assert rel_err(host(bt.grad), db) <= tol
    assert rel_err(host(xt.grad), oracle.bwd_x(dpre, w)) <= tol
    assert rel_err(host(wt.grad), oracle.bwd_w(x, dpre, T)) <= tol
    assert np.array_equal(host(rt.grad), dy)


def test_layer_bias_gelu_training_matches_oracle():
    """EQLinear(bias=True, activation='gelu'): the fused forward and the epilogue
    backward + input and weight gradients against the oracle's chain rule."""
    from group_circulant_linear_p4_amd.layer import EQLinear
    T, N, Cp, Dp = 4, 260, 20, 36
    print("case layer bias+gelu training", flush=True)
    layer = EQLinear(Cp, Dp, T, bias=True, activation="gelu", device=DEV, dtype=torch.float32)
    wl = W.Workload("t", "test", T, N, Cp, Dp, "f32", ("fwd",), seed=44)
    with torch.no_grad():
        layer.bias.copy_(dev(W.make_bias(wl)))
    xn, dyn = W.make_x(wl), W.make_dy(wl)
    x = dev(xn).requires_grad_()
    y = layer(x)
    y.backward(dev(dyn))
    torch.cuda.synchronize()
    w, b = host(layer.weight.detach()), host(layer.bias.detach())
    assert rel_err(host(y.detach()), oracle.fwd_fused(xn, w, bias=b, act="gelu")) <= 1e-5
    pre = oracle.fwd_fused(xn, w, bias=b)
    dpre, db = oracle.fused_epilogue_bwd(dyn, pre, T, act="gelu")
    assert rel_err(host(layer.bias.grad), db) <= 1e-5
    assert rel_err(host(x.grad), oracle.bwd_x(dpre, w)) <= 1e-5
    assert rel_err(host(layer.weight.grad), oracle.bwd_w(xn, dpre, T)) <= 1e-5
    with torch.no_grad():                     # inference: no pre kept, same output
        y2 = layer(dev(xn))
    torch.cuda.synchronize()
    assert torch.equal(y2, y.detach())


def test_layer_autograd_matches_oracle():
    from group_circulant_linear_p4_amd.layer import EQLinear
    T, N, Cp, Dp = 4, 200, 6, 10
    torch.manual_seed(0)
    layer = EQLinear(Cp, Dp, T, device=DEV, dtype=torch.float32)
    x = torch.randn(2, N // 2, Cp * T, device=DEV, requires_grad=True)
    y = layer(x)
    dy = torch.randn_like(y)
    y.backward(dy)
    w = host(layer.weight.detach())
    xn, dyn = host(x.detach()).reshape(N, -1), host(dy).reshape(N, -1)
    assert rel_err(host(y.detach()).reshape(N, -1), oracle.fwd(xn, w)) <= 1e-5
    assert rel_err(host(x.grad).reshape(N, -1), oracle.bwd_x(dyn, w)) <= 1e-5
    assert rel_err(host(layer.weight.grad), oracle.bwd_w(xn, dyn, T)) <= 1e-5


# ------------------------------------------------- weight gradient: both paths
_PATH_CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import group_circulant_linear_p4_amd as eql
import oracle, workloads as W
out = {}
for (T, dtype, N, Cp, Dp) in json.loads(sys.argv[2]):
    wl = W.Workload("t", "test", T, N, Cp, Dp, dtype, ("bwd_w",), seed=50 + T)
    x, dy = W.make_x(wl), W.make_dy(wl)
    code = eql.EQL_F16 if dtype == "f16" else eql.EQL_F32
    xd, dyd = torch.from_numpy(x).cuda(), torch.from_numpy(dy).cuda()
    nbytes = eql.eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, code)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    dw = torch.empty((Dp, Cp, T), dtype=xd.dtype, device="cuda")
    print("case T=%d %s N=%d C'=%d D'=%d" % (T, dtype, N, Cp, Dp), flush=True)
    eql.eqlinear_bwd_w(xd, dyd, dw, ws, nbytes, N, Cp, Dp, T, code)
    torch.cuda.synchronize()
    ref = oracle.bwd_w(x, dy, T)
    got = dw.cpu().numpy().astype(np.float64)
    out["%d/%s/%d/%d/%d" % (T, dtype, N, Cp, Dp)] = [float(np.linalg.norm(got - ref) / np.linalg.norm(ref)), nbytes]
print("RESULT " + json.dumps(out), flush=True)
"""

# Shapes with 16-byte dy rows (the fused path's condition): ragged d and c tiles, partial
# last k-steps, and enough rows for several row ranges.
_PATH_CASES = [(4, "f16", 700, 300, 520), (4, "f16", 20000, 64, 64), (2, "f16", 1000, 70, 132),
               (1, "f16", 333, 17, 40), (4, "f32", 257, 33, 41), (2, "f32", 129, 5, 130), (1, "f32", 1100, 200, 132)]


@pytest.mark.parametrize("path", ["fused", "separate"])
def test_bwd_w_both_paths(path):
    """eqlinear_bwd_w through each of its two paths (the transform of dy inside the
    GEMM, or both spectra first), selected with EQL_BWDW_PATH in a child process (the
    library reads it once), against the oracle."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, EQL_BWDW_PATH=path)
    r = subprocess.run([sys.executable, "-c", _PATH_CHILD, root, json.dumps(_PATH_CASES)], env=env,
                       capture_output=True, text=True, timeout=170)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0
    res = json.loads([l for l in r.stdout.splitlines() if l.startswith("RESULT ")][-1][7:])
    assert len(res) == len(_PATH_CASES)
    for key, (err, nbytes) in res.items():
        assert err <= TOL[key.split("/")[1]], (key, err)


# Shapes whose channel axes take 256-wide GEMM tiles on the separate weight-gradient path
# (ragged tiles on both axes, T with and without complex pairs, both dtypes, one row, a
# partial k-step, several row ranges).
_WAVE_CASES = [(8, "f16", 600, 200, 500), (8, "f32", 300, 256, 256), (4, "f16", 1000, 256, 400),
               (6, "f32", 257, 230, 450), (2, "f16", 900, 300, 260), (4, "f16", 1, 256, 256),
               (8, "f32", 15, 300, 210), (3, "f16", 4000, 512, 256)]


@pytest.mark.parametrize("waves", ["4", "8"])
def test_bwd_w_gemm_wave_arrangements(waves):
    """The separate path's GEMMs on 256-wide tiles with 4 waves (one per SIMD) and with 8
    (two per SIMD, half the columns each), selected with EQL_BWDW_WAVES in a child process,
    against the oracle."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, EQL_BWDW_PATH="separate", EQL_BWDW_WAVES=waves)
    r = subprocess.run([sys.executable, "-c", _PATH_CHILD, root, json.dumps(_WAVE_CASES)], env=env,
                       capture_output=True, text=True, timeout=170)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0
    res = json.loads([l for l in r.stdout.splitlines() if l.startswith("RESULT ")][-1][7:])
    assert len(res) == len(_WAVE_CASES)
    for key, (err, nbytes) in res.items():
        assert err <= TOL[key.split("/")[1]], (key, err)
