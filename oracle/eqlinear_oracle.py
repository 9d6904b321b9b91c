"""fp64 CPU oracle for the EQ-Linear layer over the cyclic group C_T.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module; only
tests, the smoke check and the benchmark's CPU-baseline leg do. It shares no code
with the HIP library.

Source: "Resumo Tecnico: Flash EQ-Linear" (gist.science, arXiv 2607.21271), sections
"Definicao do Problema" and "Insight Central", and the abstract page "Flash EQ-Linear:
Accelerating Equivariant Linear Layers via Group-wise Discrete Fourier Transform".
The pages state that the layer's weight is a group-circulant matrix built by
replicating one set of learnable parameters under cyclic shifts, that the layer is
a circular convolution along the group axis composed with a linear map along the
channels, and that naive implementations unroll it into a dense matrix and call a
dense kernel. The method ("Abordagem Algoritmica", "Garantias Teoricas") is exact,
so the oracle is that plain definition: unroll, then multiply in fp64.

Conventions (readings where the pages are silent):
  * x has shape [N, C'*T], flat column index c*T + h (channel c, group element h);
    y has shape [N, D'*T], flat index d*T + g.  w has shape [D', C', T].
  * Convolution, not correlation:  W[d*T+g, c*T+h] = w[d, c, (g - h) mod T].
  * All arithmetic in float64; inputs given as fp16/fp32 are upcast exactly.

Functions:
  unroll(w)            dense (D'T) x (C'T) matrix (the "replicate" step)
  fwd(x, w)            y  = x W^T
  bwd_x(dy, w)         dx = dy W
  bwd_w(x, dy)         dw[d,c,t] = sum over tied entries of (dy^T x)
  half_spectrum(v)     DFT along the last axis, k = 0..floor(T/2)
  gelu(v)              v * Phi(v), the exact (erf) form
  fwd_fused(x, w, bias, residual, act)
                       y = act(x W^T + bias broadcast over g) + residual
  gelu_grad(v)         Phi(v) + v phi(v)
  fused_epilogue_bwd(dy, pre, T, act)
                       dpre = dy * act'(pre), dbias = sum of dpre over rows and g
  real_gemm_count(T)   per-frequency real products after conjugate symmetry
"""
from __future__ import annotations

import numpy as np

_CHUNK_ROWS = 8192


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    return a.astype(np.float64, copy=False)


def unroll(w) -> np.ndarray:
    """Replicate-and-shift: the dense (D'T) x (C'T) weight of the layer.

    W[d*T+g, c*T+h] = w[d, c, (g-h) mod T]  -- "Insight Central": a group-circulant
    matrix made of cyclically shifted copies of the shared parameters.
    """
    w = _f64(w)
    Dp, Cp, T = w.shape
    g = np.arange(T).reshape(T, 1)
    h = np.arange(T).reshape(1, T)
    idx = (g - h) % T                                  # [T(g), T(h)]
    blocks = w[:, :, idx]                              # [D', C', T(g), T(h)]
    return blocks.transpose(0, 2, 1, 3).reshape(Dp * T, Cp * T)


def fwd(x, w) -> np.ndarray:
    """y = x W^T with W = unroll(w)  ("Definicao do Problema": the dense product)."""
    x = _f64(x)
    W = unroll(w)
    if x.shape[1] != W.shape[1]:
        raise ValueError("x has %d columns, weight expects %d" % (x.shape[1], W.shape[1]))
    y = np.empty((x.shape[0], W.shape[0]), dtype=np.float64)
    for r0 in range(0, x.shape[0], _CHUNK_ROWS):
        y[r0:r0 + _CHUNK_ROWS] = x[r0:r0 + _CHUNK_ROWS] @ W.T
    return y


def bwd_x(dy, w) -> np.ndarray:
    """Gradient with respect to the input: dx = dy W (chain rule of y = x W^T)."""
    dy = _f64(dy)
    W = unroll(w)
    if dy.shape[1] != W.shape[0]:
        raise ValueError("dy has %d columns, weight expects %d" % (dy.shape[1], W.shape[0]))
    dx = np.empty((dy.shape[0], W.shape[1]), dtype=np.float64)
    for r0 in range(0, dy.shape[0], _CHUNK_ROWS):
        dx[r0:r0 + _CHUNK_ROWS] = dy[r0:r0 + _CHUNK_ROWS] @ W
    return dx


def bwd_w(x, dy, T: int) -> np.ndarray:
    """Gradient with respect to the shared parameters w[D', C', T].

    The dense gradient is G = dy^T x; every entry W[d*T+g, c*T+h] is the shared
    parameter w[d, c, (g-h) mod T], so dw[d,c,t] sums G over the positions tied to t.
    """
    x = _f64(x)
    dy = _f64(dy)
    if x.shape[0] != dy.shape[0]:
        raise ValueError("x and dy disagree on N")
    if x.shape[1] % T or dy.shape[1] % T:
        raise ValueError("widths must be multiples of T")
    Cp, Dp = x.shape[1] // T, dy.shape[1] // T
    G = np.zeros((Dp * T, Cp * T), dtype=np.float64)
    for r0 in range(0, x.shape[0], _CHUNK_ROWS):
        G += dy[r0:r0 + _CHUNK_ROWS].T @ x[r0:r0 + _CHUNK_ROWS]
    G4 = G.reshape(Dp, T, Cp, T)                       # [d, g, c, h]
    dw = np.zeros((Dp, Cp, T), dtype=np.float64)
    for g in range(T):
        for h in range(T):
            dw[:, :, (g - h) % T] += G4[:, g, :, h]
    return dw


def gelu(v) -> np.ndarray:
    """GELU in its exact form: v * Phi(v) = v/2 * (1 + erf(v / sqrt 2)), with Phi the
    standard normal distribution function (erf is the library routine)."""
    from scipy.special import erf
    v = _f64(v)
    return 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))


def fwd_fused(x, w, bias=None, residual=None, act: str = "none") -> np.ndarray:
    """y = act(x W^T + b) + r: the layer inside the MLP blocks of the transformers
    the pages build it into ("Nivel de Rede": Flash EQ-ViT, Flash EQ-Swin).

    bias has one entry per output channel d and is shared by the channel's T group
    elements (b_dense[d*T+g] = bias[d]); a bias that varied with g would not commute
    with the group action.  act is "none" or "gelu" (pointwise).  residual has y's
    shape and is added after the activation.  Readings where the pages are silent:
    the order bias -> activation -> residual, and GELU in its exact form.
    """
    y = fwd(x, w)
    T = np.asarray(w).shape[2]
    if bias is not None:
        y = y + np.repeat(_f64(bias), T)[None, :]
    if act == "gelu":
        y = gelu(y)
    elif act != "none":
        raise ValueError("act must be 'none' or 'gelu'")
    if residual is not None:
        y = y + _f64(residual)
    return y


def gelu_grad(v) -> np.ndarray:
    """Derivative of v * Phi(v): Phi(v) + v * phi(v), phi the standard normal density."""
    from scipy.special import erf
    v = _f64(v)
    return 0.5 * (1.0 + erf(v / np.sqrt(2.0))) + v * np.exp(-0.5 * v * v) / np.sqrt(2.0 * np.pi)


def fused_epilogue_bwd(dy, pre, T: int, act: str = "none"):
    """Chain rule through y = act(pre) + r with pre = x W^T + b (b shared over g):
    dpre = dy * act'(pre) and dbias[d] = sum over rows n and group elements g of
    dpre[n, d*T+g].  The input and weight gradients are bwd_x / bwd_w applied to dpre;
    the residual's gradient is dy."""
    dy = _f64(dy)
    if act == "gelu":
        dpre = dy * gelu_grad(pre)
    elif act == "none":
        dpre = dy.copy()
    else:
        raise ValueError("act must be 'none' or 'gelu'")
    N, DT = dpre.shape
    dbias = dpre.reshape(N, DT // T, T).sum(axis=(0, 2))
    return dpre, dbias


def half_spectrum(v) -> np.ndarray:
    """DFT along the last (group) axis, keeping k = 0..floor(T/2).

    V[..., k] = sum_t v[..., t] * exp(-2*pi*i*t*k/T)  ("Abordagem Algoritmica" step 2:
    real inputs have conjugate-symmetric spectra, so only this half is kept).
    """
    v = _f64(v)
    T = v.shape[-1]
    t = np.arange(T).reshape(T, 1)
    k = np.arange(T // 2 + 1).reshape(1, -1)
    F = np.exp(-2j * np.pi * ((t * k) % T) / T)        # [T, K]
    return v @ F


def real_gemm_count(T: int) -> int:
    """Real channel GEMMs per row block after the half-spectrum reduction.

    k = 0 (and k = T/2 for even T) are real frequencies: one real product each.
    Every other kept frequency is complex: four real products.  T = 4 gives
    1 + 1 + 4 = 6 real products where the dense layer needs T*T = 16 (section
    "Especializacao para o Grupo de Rotacao p4").
    """
    if T < 1:
        raise ValueError("T must be >= 1")
    n_real = 2 if T % 2 == 0 and T > 1 else 1
    n_complex = T // 2 + 1 - n_real
    return n_real + 4 * n_complex


def actual_flops(N: int, Cp: int, Dp: int, T: int) -> int:
    """FLOPs of the per-frequency products: 2 * (real GEMMs) * N * D' * C'."""
    return 2 * real_gemm_count(T) * N * Dp * Cp


def dense_equivalent_flops(N: int, Cp: int, Dp: int, T: int) -> int:
    """FLOPs of the unrolled dense layer, 2 * N * D * C with C = C'T, D = D'T."""
    return 2 * N * (Dp * T) * (Cp * T)
