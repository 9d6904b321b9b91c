"""Seeded synthetic inputs for the EQ-Linear layer.

This module draws random numbers and casts them; it holds none of the layer's
arithmetic, so both the fp64 oracle's tests and the HIP path's tests and benchmark
can take their inputs from it.

Recipe (shared by every consumer):
  * x, dy: N(0, 1); w: N(0, 1/C) with C = C'*T, the full input width.
  * Each tensor has its own stream.  x and dy are drawn in blocks of ROW_BLOCK rows;
    block b of tensor s comes from numpy.random.default_rng([seed, s, b]), so any
    row subset can be regenerated without drawing the whole tensor.
  * Values are drawn as float32 and rounded once (round-to-nearest-even) to the
    workload's dtype.
  * For workloads with ``hot_rows_frac`` > 0, a set of rows chosen without
    replacement from default_rng([seed, 3]) is multiplied by ``hot_rows_scale``
    before the cast (exact: the scale is a power of two).

The five workloads mirror the layer shapes of the equivariant ViT-S / Swin models
the pages evaluate (a p4 MLP expansion, a Swin MLP, a large square layer) plus a
tiny p4 case and a C8 case.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROW_BLOCK = 1024
_X, _W, _DY, _ROWS, _BIAS, _RES = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    name: str
    T: int
    N: int
    Cp: int
    Dp: int
    dtype: str            # "f32" or "f16"
    passes: tuple
    hot_rows_frac: float = 0.0
    hot_rows_scale: float = 1.0
    seed: int = 0

    @property
    def C(self) -> int:
        return self.Cp * self.T

    @property
    def D(self) -> int:
        return self.Dp * self.T

    @property
    def np_dtype(self):
        return np.float16 if self.dtype == "f16" else np.float32

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "c1": Workload("c1", "p4 fp32 tiny: N=256, C=D=64 (C'=D'=16)", 4, 256, 16, 16, "f32", ("fwd",)),
    "c2": Workload("c2", "p4 fp16 EQ-ViT-S MLP expansion: N=12608, C=384, D=1536", 4, 12608, 96, 384,
                   "f16", ("fwd",)),
    "c3": Workload("c3", "C8 fp32: N=16384, C=D=512 (C'=D'=64)", 8, 16384, 64, 64, "f32", ("fwd",)),
    "c4": Workload("c4", "p4 fp16 EQ-Swin MLP: N=100352, C=768, D=3072", 4, 100352, 192, 768, "f16",
                   ("fwd", "bwd_x", "bwd_w")),
    "c5": Workload("c5", "p4 fp16 large square: N=65536, C=D=4096 (1% rows x16)", 4, 65536, 1024, 1024,
                   "f16", ("fwd", "bwd_x", "bwd_w"), hot_rows_frac=0.01, hot_rows_scale=16.0),
}


def _block(seed: int, stream: int, b: int, rows: int, cols: int) -> np.ndarray:
    rng = np.random.default_rng([seed, stream, b])
    return rng.standard_normal((rows, cols), dtype=np.float32)


def _rows_f32(wl: Workload, stream: int, cols: int, rows) -> np.ndarray:
    """float32 draws for the requested rows (an index array) of tensor `stream`."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, cols), dtype=np.float32)
    if rows.size == 0:
        return out
    blocks = np.unique(rows // ROW_BLOCK)

    def one(b):
        r0 = b * ROW_BLOCK
        nr = min(ROW_BLOCK, wl.N - r0)
        blk = _block(wl.seed, stream, int(b), nr, cols)
        sel = np.nonzero((rows >= r0) & (rows < r0 + nr))[0]
        out[sel] = blk[rows[sel] - r0]

    if blocks.size > 4:
        with ThreadPoolExecutor(max_workers=8) as ex:
            list(ex.map(one, blocks))
    else:
        for b in blocks:
            one(b)
    return out


def hot_rows(wl: Workload) -> np.ndarray:
    """Sorted indices of the rows scaled by hot_rows_scale (empty if none)."""
    if wl.hot_rows_frac <= 0.0:
        return np.zeros(0, dtype=np.int64)
    k = int(wl.N * wl.hot_rows_frac)
    rng = np.random.default_rng([wl.seed, _ROWS])
    return np.sort(rng.choice(wl.N, k, replace=False)).astype(np.int64)


def _select(wl: Workload, rows):
    if rows is None:
        return np.arange(wl.N, dtype=np.int64)
    if isinstance(rows, slice):
        return np.arange(wl.N, dtype=np.int64)[rows]
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= wl.N):
        raise IndexError("row index out of range")
    return rows


def make_x(wl: Workload, rows=None) -> np.ndarray:
    """x[rows, C'*T] in the workload dtype (all rows when rows is None)."""
    idx = _select(wl, rows)
    a = _rows_f32(wl, _X, wl.C, idx)
    hr = hot_rows(wl)
    if hr.size:
        a[np.isin(idx, hr)] *= np.float32(wl.hot_rows_scale)
    return a.astype(wl.np_dtype)


def make_dy(wl: Workload, rows=None) -> np.ndarray:
    """dy[rows, D'*T] in the workload dtype."""
    idx = _select(wl, rows)
    return _rows_f32(wl, _DY, wl.D, idx).astype(wl.np_dtype)


def make_w(wl: Workload) -> np.ndarray:
    """w[D', C', T] ~ N(0, 1/C) in the workload dtype."""
    rng = np.random.default_rng([wl.seed, _W])
    a = rng.standard_normal((wl.Dp, wl.Cp, wl.T), dtype=np.float32)
    a *= np.float32(1.0 / np.sqrt(wl.C))
    return a.astype(wl.np_dtype)


def make_bias(wl: Workload) -> np.ndarray:
    """bias[D'] ~ N(0, 1) in the workload dtype: one value per output channel, shared
    by its T group elements (the fused forward epilogue)."""
    rng = np.random.default_rng([wl.seed, _BIAS])
    return rng.standard_normal(wl.Dp, dtype=np.float32).astype(wl.np_dtype)


def make_residual(wl: Workload, rows=None) -> np.ndarray:
    """residual[rows, D'*T] ~ N(0, 1) in the workload dtype (the fused forward epilogue)."""
    idx = _select(wl, rows)
    return _rows_f32(wl, _RES, wl.D, idx).astype(wl.np_dtype)

