"""Pins for the fp64 oracle (CPU only).

The oracle is the plain definition of the layer (dense unroll, fp64 matmul).  Each
test below checks it against something that is not the oracle itself: the
hand-worked fixtures, scipy's circulant matrix, torch's circular conv1d and its
autograd, numpy's FFT (convolution theorem), closed forms for special inputs, and
the adjoint / gradient identities.  The mutation tests at the end plant plausible
mistakes in a copy of the oracle and show that at least one pin catches each.
"""
import types

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from oracle import eqlinear_oracle as O
from tests._golden import load_cases

RNG = np.random.default_rng(1234)
TS = [1, 2, 3, 4, 5, 6, 8]


def rand(*shape):
    return RNG.standard_normal(shape)


def _ns(**over):
    base = dict(unroll=O.unroll, fwd=O.fwd, bwd_x=O.bwd_x, bwd_w=O.bwd_w, half_spectrum=O.half_spectrum,
                gelu=O.gelu, fwd_fused=O.fwd_fused, gelu_grad=O.gelu_grad,
                fused_epilogue_bwd=O.fused_epilogue_bwd)
    base.update(over)
    return types.SimpleNamespace(**base)


# --------------------------------------------------------------------------- pins
def pin_golden(o):
    for c in load_cases():
        if not np.allclose(o.fwd(c["x"], c["w"]), c["y"], atol=1e-12):
            return False
        if "dx" in c and not np.allclose(o.bwd_x(c["dy"], c["w"]), c["dx"], atol=1e-12):
            return False
        if "dw" in c and not np.allclose(o.bwd_w(c["x"], c["dy"], c["T"]), c["dw"], atol=1e-12):
            return False
    return True


def pin_circulant(o, T=5, Dp=3, Cp=2):
    """Each (d, c) block of the unrolled weight is scipy's circulant of w[d, c]."""
    w = rand(Dp, Cp, T)
    W = o.unroll(w)
    for d in range(Dp):
        for c in range(Cp):
            blk = W[d * T:(d + 1) * T, c * T:(c + 1) * T]
            if not np.array_equal(blk, scipy.linalg.circulant(w[d, c])):
                return False
    return True


def _torch_layer(x, w, T):
    """Circular convolution over the group axis via torch conv1d (cross-correlation
    with a flipped kernel and circular left padding of T-1)."""
    N = x.shape[0]
    Dp, Cp, _ = w.shape
    xin = x.reshape(N, Cp, T)
    xpad = torch.cat([xin[:, :, 1:], xin], dim=2) if T > 1 else xin   # left pad by T-1, circular
    y = torch.nn.functional.conv1d(xpad, torch.flip(w, dims=[2]))
    return y.reshape(N, Dp * T)


def pin_torch_autograd(o, T=4, N=6, Cp=3, Dp=2):
    x = torch.tensor(rand(N, Cp * T), requires_grad=True)
    w = torch.tensor(rand(Dp, Cp, T), requires_grad=True)
    dy = torch.tensor(rand(N, Dp * T))
    y = _torch_layer(x, w, T)
    y.backward(dy)
    ok = np.allclose(o.fwd(x.detach().numpy(), w.detach().numpy()), y.detach().numpy(), atol=1e-12)
    ok &= np.allclose(o.bwd_x(dy.numpy(), w.detach().numpy()), x.grad.numpy(), atol=1e-12)
    ok &= np.allclose(o.bwd_w(x.detach().numpy(), dy.numpy(), T), w.grad.numpy(), atol=1e-12)
    return bool(ok)


def pin_fft(o, T=6, N=5, Cp=3, Dp=4):
    """Convolution theorem with numpy's FFT: y = irfft(sum_c rfft(w) * rfft(x))."""
    x = rand(N, Cp * T)
    w = rand(Dp, Cp, T)
    X = np.fft.rfft(x.reshape(N, Cp, T), axis=-1)            # [N, C', K]
    Wf = np.fft.rfft(w, axis=-1)                              # [D', C', K]
    Y = np.einsum("dck,nck->ndk", Wf, X)
    y = np.fft.irfft(Y, n=T, axis=-1).reshape(N, Dp * T)
    return bool(np.allclose(o.fwd(x, w), y, atol=1e-12))


def pin_adjoint(o, T=4, N=7, Cp=3, Dp=3):
    x, w, dy = rand(N, Cp * T), rand(Dp, Cp, T), rand(N, Dp * T)
    lhs = np.sum(o.fwd(x, w) * dy)
    rhs = np.sum(x * o.bwd_x(dy, w))
    return bool(abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs)))


def pin_weight_gradient(o, T=4, N=9, Cp=2, Dp=3):
    """<y(x; w'), dy> = <dw(x, dy), w'> for any w': dw is the gradient of a linear form."""
    x, dy = rand(N, Cp * T), rand(N, Dp * T)
    dw = o.bwd_w(x, dy, T)
    for _ in range(3):
        wp = rand(Dp, Cp, T)
        if abs(np.sum(o.fwd(x, wp) * dy) - np.sum(dw * wp)) > 1e-10:
            return False
    return True


def pin_equivariance(o, T=4, N=5, Cp=3, Dp=2):
    x, w = rand(N, Cp * T), rand(Dp, Cp, T)
    y = o.fwd(x, w).reshape(N, Dp, T)
    for s in range(T):
        xs = np.roll(x.reshape(N, Cp, T), s, axis=2).reshape(N, Cp * T)
        if not np.allclose(o.fwd(xs, w).reshape(N, Dp, T), np.roll(y, s, axis=2), atol=1e-12):
            return False
    return True


def pin_spectrum(o, T=7):
    v = rand(3, 4, T)
    return bool(np.allclose(o.half_spectrum(v), np.fft.rfft(v, axis=-1), atol=1e-12))


# Fused epilogue (bias broadcast over g, GELU, residual).
def pin_gelu_table(o):
    """GELU(v) = v Phi(v) against the standard normal distribution table (5 digits):
    Phi(1) = 0.84134, Phi(2) = 0.97725, Phi(-0.5) = 0.30854, Phi(0) = 0.5."""
    table = {1.0: 0.84134, 2.0: 0.97725, -0.5: 0.30854, 0.0: 0.5}
    v = np.array(sorted(table))
    want = v * np.array([table[k] for k in sorted(table)])
    return bool(np.all(np.abs(o.gelu(v) - want) <= 1e-5 * np.maximum(1.0, np.abs(v))))


def pin_gelu_odd_part(o):
    """Phi(v) + Phi(-v) = 1, so GELU(v) - GELU(-v) = v for every v."""
    v = np.linspace(-6.0, 6.0, 97)
    return bool(np.allclose(o.gelu(v) - o.gelu(-v), v, atol=1e-12))


def pin_fused_brute_force(o, T=3, N=2, Cp=2, Dp=2):
    """Plain loops with math.erf: y[n, dT+g] = gelu(sum_{c,h} x[n, cT+h] w[d, c, (g-h) mod T]
    + b[d]) + r[n, dT+g]."""
    import math
    x, w, b, r = rand(N, Cp * T), rand(Dp, Cp, T), rand(Dp), rand(N, Dp * T)
    got = o.fwd_fused(x, w, bias=b, residual=r, act="gelu")
    for n in range(N):
        for d in range(Dp):
            for g in range(T):
                acc = sum(x[n, c * T + h] * w[d, c, (g - h) % T] for c in range(Cp) for h in range(T)) + b[d]
                want = 0.5 * acc * (1.0 + math.erf(acc / math.sqrt(2.0))) + r[n, d * T + g]
                if abs(got[n, d * T + g] - want) > 1e-12 * max(1.0, abs(want)):
                    return False
    return True


def pin_fused_equivariance(o, T=4, N=5, Cp=3, Dp=2):
    """A shared per-channel bias and a pointwise activation commute with the group
    action: shifting x and the residual along the group axis shifts y."""
    x, w, b, r = rand(N, Cp * T), rand(Dp, Cp, T), rand(Dp), rand(N, Dp * T)
    y = o.fwd_fused(x, w, bias=b, residual=r, act="gelu").reshape(N, Dp, T)
    for s in range(1, T):
        xs = np.roll(x.reshape(N, Cp, T), s, axis=2).reshape(N, Cp * T)
        rs = np.roll(r.reshape(N, Dp, T), s, axis=2).reshape(N, Dp * T)
        ys = o.fwd_fused(xs, w, bias=b, residual=rs, act="gelu").reshape(N, Dp, T)
        if not np.allclose(ys, np.roll(y, s, axis=2), atol=1e-12):
            return False
    return True


def pin_fused_reduces_to_fwd(o, T=4, N=4, Cp=3, Dp=2):
    x, w = rand(N, Cp * T), rand(Dp, Cp, T)
    return bool(np.array_equal(o.fwd_fused(x, w), o.fwd(x, w)))


def pin_gelu_grad_finite_difference(o):
    """GELU' against central differences of GELU itself (error O(h^2) ~ 1e-10)."""
    v = np.linspace(-5.0, 5.0, 81)
    h = 1e-5
    fd = (o.gelu(v + h) - o.gelu(v - h)) / (2 * h)
    return bool(np.allclose(o.gelu_grad(v), fd, atol=1e-8))


def pin_gelu_grad_identities(o):
    """GELU'(v) + GELU'(-v) = 1 (Phi(v) + Phi(-v) = 1, phi even) and GELU'(0) = 1/2."""
    v = np.linspace(-6.0, 6.0, 61)
    return bool(np.allclose(o.gelu_grad(v) + o.gelu_grad(-v), 1.0, atol=1e-12) and
                abs(o.gelu_grad(np.array([0.0]))[0] - 0.5) < 1e-15)


def pin_epilogue_bwd_loops(o, T=3, N=4, Dp=2):
    """dbias by plain loops, dpre elementwise."""
    dy, pre = rand(N, Dp * T), rand(N, Dp * T)
    dpre, db = o.fused_epilogue_bwd(dy, pre, T, act="gelu")
    g = o.gelu_grad(pre)
    for d in range(Dp):
        want = sum(dy[n, d * T + k] * g[n, d * T + k] for n in range(N) for k in range(T))
        if abs(db[d] - want) > 1e-12 * max(1.0, abs(want)):
            return False
    return bool(np.allclose(dpre, dy * g, atol=1e-14))


def pin_fused_layer_autograd(o, T=4, N=5, Cp=3, Dp=2):
    """The whole training step of y = gelu(x W^T + b) + r through torch autograd in
    fp64: conv1d layer, F.gelu (exact form), bias broadcast over g."""
    x = torch.tensor(rand(N, Cp * T), requires_grad=True)
    w = torch.tensor(rand(Dp, Cp, T), requires_grad=True)
    b = torch.tensor(rand(Dp), requires_grad=True)
    r = torch.tensor(rand(N, Dp * T), requires_grad=True)
    dy = torch.tensor(rand(N, Dp * T))
    pre_t = _torch_layer(x, w, T) + b.repeat_interleave(T)
    y = torch.nn.functional.gelu(pre_t) + r
    y.backward(dy)
    xn, wn, bn, rn = (t.detach().numpy() for t in (x, w, b, r))
    ok = np.allclose(o.fwd_fused(xn, wn, bias=bn, residual=rn, act="gelu"), y.detach().numpy(), atol=1e-12)
    pre = o.fwd_fused(xn, wn, bias=bn)
    dpre, db = o.fused_epilogue_bwd(dy.numpy(), pre, T, act="gelu")
    ok &= np.allclose(db, b.grad.numpy(), atol=1e-10)
    ok &= np.allclose(o.bwd_x(dpre, wn), x.grad.numpy(), atol=1e-10)
    ok &= np.allclose(o.bwd_w(xn, dpre, T), w.grad.numpy(), atol=1e-10)
    ok &= np.allclose(dy.numpy(), r.grad.numpy())
    return bool(ok)


ALL_PINS = [pin_golden, pin_circulant, pin_torch_autograd, pin_fft, pin_adjoint,
            pin_weight_gradient, pin_equivariance, pin_spectrum, pin_gelu_table, pin_gelu_odd_part,
            pin_fused_brute_force, pin_fused_equivariance, pin_fused_reduces_to_fwd,
            pin_gelu_grad_finite_difference, pin_gelu_grad_identities, pin_epilogue_bwd_loops,
            pin_fused_layer_autograd]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(_ns())


# ------------------------------------------------------------------ per-T sweeps
@pytest.mark.parametrize("T", TS)
def test_unroll_blocks_are_circulant(T):
    assert pin_circulant(_ns(), T=T)


@pytest.mark.parametrize("T", TS)
def test_fwd_matches_fft_convolution_theorem(T):
    assert pin_fft(_ns(), T=T)


@pytest.mark.parametrize("T", TS)
def test_fwd_and_grads_match_torch_conv1d_autograd(T):
    assert pin_torch_autograd(_ns(), T=T)


@pytest.mark.parametrize("T", TS)
def test_brute_force_loops(T):
    """Direct circular-convolution sums in pure Python on a tiny shape."""
    N, Cp, Dp = 2, 2, 3
    x, w, dy = rand(N, Cp * T), rand(Dp, Cp, T), rand(N, Dp * T)
    y = np.zeros((N, Dp * T))
    dx = np.zeros((N, Cp * T))
    dw = np.zeros((Dp, Cp, T))
    for n in range(N):
        for d in range(Dp):
            for g in range(T):
                for c in range(Cp):
                    for h in range(T):
                        t = (g - h) % T
                        y[n, d * T + g] += w[d, c, t] * x[n, c * T + h]
                        dx[n, c * T + h] += w[d, c, t] * dy[n, d * T + g]
                        dw[d, c, t] += dy[n, d * T + g] * x[n, c * T + h]
    assert np.allclose(O.fwd(x, w), y, atol=1e-12)
    assert np.allclose(O.bwd_x(dy, w), dx, atol=1e-12)
    assert np.allclose(O.bwd_w(x, dy, T), dw, atol=1e-12)


@pytest.mark.parametrize("T", TS)
def test_equivariance_every_shift(T):
    assert pin_equivariance(_ns(), T=T)


@pytest.mark.parametrize("T", TS)
def test_weight_gradient_shift_invariant(T):
    """dw(roll_s x, roll_s dy) = dw(x, dy): shifting both operands leaves the tied sums unchanged."""
    N, Cp, Dp = 5, 3, 2
    x, dy = rand(N, Cp * T), rand(N, Dp * T)
    dw = O.bwd_w(x, dy, T)
    for s in range(1, T):
        xs = np.roll(x.reshape(N, Cp, T), s, axis=2).reshape(N, -1)
        dys = np.roll(dy.reshape(N, Dp, T), s, axis=2).reshape(N, -1)
        assert np.allclose(O.bwd_w(xs, dys, T), dw, atol=1e-12)


# ------------------------------------------------------------ special cases
def test_T1_is_plain_linear():
    x, w = rand(6, 5), rand(4, 5, 1)
    assert np.allclose(O.fwd(x, w), x @ w[:, :, 0].T, atol=1e-12)


@pytest.mark.parametrize("T", TS)
def test_constant_over_group_uses_only_k0(T):
    """x[n,c,h] = u[n,c] for all h  =>  y[n,d,g] = sum_c u[n,c] * sum_t w[d,c,t]."""
    N, Cp, Dp = 3, 4, 2
    u, w = rand(N, Cp), rand(Dp, Cp, T)
    x = np.repeat(u[:, :, None], T, axis=2).reshape(N, Cp * T)
    expect = (u @ w.sum(axis=2).T)[:, :, None].repeat(T, axis=2).reshape(N, Dp * T)
    assert np.allclose(O.fwd(x, w), expect, atol=1e-12)


@pytest.mark.parametrize("T", [2, 4, 6, 8])
def test_alternating_input_uses_only_nyquist(T):
    """x[n,c,h] = (-1)^h u[n,c]  =>  y[n,d,g] = (-1)^g sum_c u[n,c] sum_t (-1)^t w[d,c,t]."""
    N, Cp, Dp = 3, 4, 2
    u, w = rand(N, Cp), rand(Dp, Cp, T)
    sgn = (-1.0) ** np.arange(T)
    x = (u[:, :, None] * sgn).reshape(N, Cp * T)
    core = u @ (w * sgn).sum(axis=2).T
    expect = (core[:, :, None] * sgn).reshape(N, Dp * T)
    assert np.allclose(O.fwd(x, w), expect, atol=1e-12)


@pytest.mark.parametrize("T", TS)
def test_delta_input_returns_weight_column(T):
    Cp, Dp = 3, 2
    w = rand(Dp, Cp, T)
    for c0 in range(Cp):
        for h0 in range(T):
            x = np.zeros((1, Cp * T))
            x[0, c0 * T + h0] = 1.0
            y = O.fwd(x, w).reshape(Dp, T)
            expect = np.stack([[w[d, c0, (g - h0) % T] for g in range(T)] for d in range(Dp)])
            assert np.array_equal(y, expect)


def test_fp16_inputs_upcast_exactly():
    x = rand(4, 8).astype(np.float16)
    w = rand(2, 2, 4).astype(np.float16)
    ref = O.fwd(x.astype(np.float64), w.astype(np.float64))
    assert np.array_equal(O.fwd(x, w), ref)


def test_chunked_rows_match_unchunked(monkeypatch):
    x, w, dy = rand(50, 12), rand(3, 3, 4), rand(50, 12)
    full = (O.fwd(x, w), O.bwd_x(dy, w), O.bwd_w(x, dy, 4))
    monkeypatch.setattr(O, "_CHUNK_ROWS", 7)
    part = (O.fwd(x, w), O.bwd_x(dy, w), O.bwd_w(x, dy, 4))
    for a, b in zip(full, part):
        assert np.allclose(a, b, atol=1e-12)


# ------------------------------------------------------------ operation counts
def test_p4_needs_six_real_gemms():
    # p4 section: six real products instead of sixteen, a 16/6 reduction.
    assert oracle.real_gemm_count(4) == 6
    assert O.dense_equivalent_flops(1, 1, 1, 4) / O.actual_flops(1, 1, 1, 4) == pytest.approx(16 / 6)


@pytest.mark.parametrize("T", TS)
def test_real_gemm_count_matches_real_multiplies_of_half_spectrum(T):
    """Count the real multiplies in the pointwise half-spectrum product directly:
    a real frequency (imaginary part identically zero for real input) costs one,
    a complex frequency four."""
    v = rand(T)
    spec = np.fft.rfft(v)
    mults = 0
    for k, z in enumerate(spec):
        is_real = (k == 0) or (2 * k == T)
        assert (abs(z.imag) < 1e-12) == is_real     # random v: complex bins have nonzero Im
        mults += 1 if is_real else 4
    assert oracle.real_gemm_count(T) == mults


def test_macs_approach_2NDC_over_T():
    # "Abordagem Algoritmica", step 3: MACs fall from NDC to about 2NDC/T.
    for T in (4, 8, 16, 32):
        ratio = O.actual_flops(1, 1, 1, T) / O.dense_equivalent_flops(1, 1, 1, T)
        assert ratio == pytest.approx(2.0 / T, rel=1.0 / T)


# ------------------------------------------------------------ mutation tests
def _mut_unroll_correlation(w):
    w = np.asarray(w, dtype=np.float64)
    Dp, Cp, T = w.shape
    idx = (np.arange(T).reshape(1, T) - np.arange(T).reshape(T, 1)) % T   # (h - g): wrong
    return w[:, :, idx].transpose(0, 2, 1, 3).reshape(Dp * T, Cp * T)


def _mut_fwd_from(unroll_fn):
    return lambda x, w: np.asarray(x, dtype=np.float64) @ unroll_fn(w).T


def _mut_bwd_x_transposed(dy, w):
    return np.asarray(dy, dtype=np.float64) @ O.unroll(w).T                 # should be W, not W^T


def _mut_bwd_w_plus(x, dy, T):
    G = (np.asarray(dy, np.float64).T @ np.asarray(x, np.float64))
    Dp, Cp = G.shape[0] // T, G.shape[1] // T
    G4 = G.reshape(Dp, T, Cp, T)
    dw = np.zeros((Dp, Cp, T))
    for g in range(T):
        for h in range(T):
            dw[:, :, (g + h) % T] += G4[:, g, :, h]                         # sign of h flipped
    return dw


def _mut_bwd_w_dropped_term(x, dy, T):
    G = (np.asarray(dy, np.float64).T @ np.asarray(x, np.float64))
    Dp, Cp = G.shape[0] // T, G.shape[1] // T
    G4 = G.reshape(Dp, T, Cp, T)
    dw = np.zeros((Dp, Cp, T))
    for g in range(T - 1):                                                  # last g dropped
        for h in range(T):
            dw[:, :, (g - h) % T] += G4[:, g, :, h]
    return dw


def _mut_spectrum_sign(v):
    v = np.asarray(v, dtype=np.float64)
    T = v.shape[-1]
    t, k = np.arange(T).reshape(T, 1), np.arange(T // 2 + 1).reshape(1, -1)
    return v @ np.exp(+2j * np.pi * t * k / T)                              # wrong sign


def _mut_fused_bias_tiled(x, w, bias=None, residual=None, act="none"):
    y = O.fwd(x, w)
    T = np.asarray(w).shape[2]
    if bias is not None:
        y = y + np.tile(np.asarray(bias, np.float64), T)[None, :]          # b[(dT+g) mod D'], not b[d]
    y = O.gelu(y) if act == "gelu" else y
    return y + (0.0 if residual is None else np.asarray(residual, np.float64))


def _mut_gelu_tanh(v):
    v = np.asarray(v, dtype=np.float64)                                     # the tanh approximation
    return 0.5 * v * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (v + 0.044715 * v ** 3)))


def _mut_fused_residual_first(x, w, bias=None, residual=None, act="none"):
    y = O.fwd(x, w)
    T = np.asarray(w).shape[2]
    if bias is not None:
        y = y + np.repeat(np.asarray(bias, np.float64), T)[None, :]
    if residual is not None:
        y = y + np.asarray(residual, np.float64)                            # before the activation
    return O.gelu(y) if act == "gelu" else y


def _mut_gelu_grad_no_density(v):
    from scipy.special import erf
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * (1.0 + erf(v / np.sqrt(2.0)))                             # Phi only, v*phi dropped


def _mut_epilogue_bwd_bias_over_channels(dy, pre, T, act="none"):
    dpre, _ = O.fused_epilogue_bwd(dy, pre, T, act)
    N, DT = dpre.shape
    return dpre, dpre.reshape(N, T, DT // T).sum(axis=(0, 1))              # wrong grouping of d, g


MUTANTS = {
    "gelu_grad_without_density_term": dict(gelu_grad=_mut_gelu_grad_no_density),
    "epilogue_bwd_bias_wrong_grouping": dict(fused_epilogue_bwd=_mut_epilogue_bwd_bias_over_channels),
    "fused_bias_tiled_over_channels": dict(fwd_fused=_mut_fused_bias_tiled),
    "gelu_tanh_approximation": dict(gelu=_mut_gelu_tanh),
    "fused_residual_before_activation": dict(fwd_fused=_mut_fused_residual_first),
    "correlation_instead_of_convolution": dict(unroll=_mut_unroll_correlation,
                                               fwd=_mut_fwd_from(_mut_unroll_correlation)),
    "bwd_x_transposed_operand": dict(bwd_x=_mut_bwd_x_transposed),
    "bwd_w_wrong_shift_sign": dict(bwd_w=_mut_bwd_w_plus),
    "bwd_w_dropped_term": dict(bwd_w=_mut_bwd_w_dropped_term),
    "spectrum_wrong_sign": dict(half_spectrum=_mut_spectrum_sign),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    o = _ns(**MUTANTS[name])

    def holds(pin):
        try:
            return pin(o)
        except ValueError:          # a shape error is a caught mistake too
            return False

    failed = [p.__name__ for p in ALL_PINS if not holds(p)]
    assert failed, "no pin caught mutant %s" % name
