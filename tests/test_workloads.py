"""The seeded input generator: determinism, row-subset regeneration, recipe."""
import numpy as np

import workloads as W


def small(**kw):
    base = W.WORKLOADS["c5"].with_shape(N=3000, Cp=4, Dp=3)
    return base.with_shape(**kw) if kw else base


def test_deterministic():
    wl = small()
    assert np.array_equal(W.make_x(wl), W.make_x(wl))
    assert np.array_equal(W.make_w(wl), W.make_w(wl))
    assert np.array_equal(W.make_dy(wl), W.make_dy(wl))


def test_row_subset_equals_full_rows():
    wl = small()
    full_x, full_dy = W.make_x(wl), W.make_dy(wl)
    rows = np.array([0, 1, 1023, 1024, 2047, 2999, 17])
    assert np.array_equal(W.make_x(wl, rows), full_x[rows])
    assert np.array_equal(W.make_dy(wl, rows), full_dy[rows])
    assert np.array_equal(W.make_x(wl, slice(100, 2100)), full_x[100:2100])


def test_shapes_dtypes_and_scales():
    for key, wl in W.WORKLOADS.items():
        wl = wl.with_shape(N=min(wl.N, 700))
        x, w = W.make_x(wl), W.make_w(wl)
        assert x.shape == (wl.N, wl.Cp * wl.T) and x.dtype == wl.np_dtype
        assert w.shape == (wl.Dp, wl.Cp, wl.T) and w.dtype == wl.np_dtype
        assert abs(np.std(w.astype(np.float64)) * np.sqrt(wl.C) - 1.0) < 0.2


def test_hot_rows():
    wl = small()
    hr = W.hot_rows(wl)
    assert hr.size == 30 and np.unique(hr).size == 30
    base = W.WORKLOADS["c4"].with_shape(N=3000, Cp=4, Dp=3)
    assert W.hot_rows(base).size == 0
    x = W.make_x(wl).astype(np.float32)
    cold = np.setdiff1d(np.arange(wl.N), hr)
    assert np.abs(x[hr]).max() > 16 * 2.0 and np.abs(x[cold]).max() < 8.0


def test_bias_and_residual_streams():
    """The fused epilogue's inputs: deterministic, own streams (independent of dy, whose
    shape the residual shares), row subsets regenerate exactly."""
    wl = small()
    b, r = W.make_bias(wl), W.make_residual(wl)
    assert b.shape == (wl.Dp,) and b.dtype == wl.np_dtype
    assert r.shape == (wl.N, wl.Dp * wl.T) and r.dtype == wl.np_dtype
    assert np.array_equal(b, W.make_bias(wl)) and np.array_equal(r, W.make_residual(wl))
    assert not np.array_equal(r, W.make_dy(wl))
    rows = np.array([5, 1024, 2999])
    assert np.array_equal(W.make_residual(wl, rows), r[rows])
