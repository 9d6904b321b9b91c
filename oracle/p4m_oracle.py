"""fp64 CPU oracle for the equivariant linear layer over p4m's point group (dihedral D4).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module; only tests,
the smoke check and the benchmark's CPU-baseline leg may. It shares no code with the HIP
library (and none with the C_T oracle beyond NumPy).

Source: "Resumo Tecnico: Flash EQ-Linear", section "Limitacoes e Trabalho Futuro": the
implementation is specialised to p4 (90-degree rotations), and generalising it to other
transformation groups, reflection groups among them, is named as future work. The
layer's construction in "Definicao do Problema" and "Insight Central" (one set of
shared parameters replicated under the group action into a dense weight) is taken here
for the group of p4m's point symmetries: four rotations and four reflections.
Reading (the pages define no p4m layer): the group-convolution form of the cyclic layer,
W[(d,g),(c,h)] = w[d, c, g h^-1], which for C_T is w[d, c, (g - h) mod T].

Group D4: elements r^a s^b (a in Z_4, b in {0, 1}); r is the 90-degree rotation, s a
reflection, with r^4 = s^2 = e and s r s = r^-1, so
    (r^a1 s^b1)(r^a2 s^b2) = r^(a1 + (-1)^b1 a2) s^(b1 + b2).
Flattened group axis (a reading, chosen so the reflection coset is listed in the order
in which it pairs with the rotations):
    index j = 0..3 : r^j
    index j = 4..7 : r^-(j-4) s     (s, r^3 s, r^2 s, r s)
x has shape [N, C'*8] (flat index c*8 + j), y [N, D'*8], w [D', C', 8] (w[d, c, j] is
the parameter for group element j).  All arithmetic in float64.

Functions:
  element(j), index(a, b)   flattened index <-> (a, b)
  mul(i, j), inv(i)         group law on indices
  unroll(w)                 dense (8D') x (8C') weight, W[(d,g),(c,h)] = w[d,c, g h^-1]
  fwd(x, w)                 y  = x W^T
  bwd_x(dy, w)              dx = dy W
  bwd_w(x, dy)              dw[d,c,k] = sum over (g,h) with g h^-1 = k of (dy^T x)[(d,g),(c,h)]
  right_translate(v, a)     (R_a v)(h) = v(h a) on the group axis of [.., 8 ch] arrays
"""
from __future__ import annotations

import numpy as np

ORDER = 8


def element(j: int):
    """(a, b) of flattened index j: r^a s^b."""
    if j < 4:
        return j % 4, 0
    return (-(j - 4)) % 4, 1


def index(a: int, b: int) -> int:
    """Flattened index of r^a s^b."""
    a %= 4
    return a if b == 0 else 4 + ((-a) % 4)


def mul(i: int, j: int) -> int:
    """Index of e_i e_j:  r^a1 s^b1 r^a2 s^b2 = r^(a1 + (-1)^b1 a2) s^(b1 + b2)."""
    a1, b1 = element(i)
    a2, b2 = element(j)
    return index(a1 + (a2 if b1 == 0 else -a2), (b1 + b2) % 2)


def inv(i: int) -> int:
    """Index of e_i^-1: rotations invert the angle, reflections are involutions."""
    a, b = element(i)
    return index(-a, 0) if b == 0 else i


def _f64(a) -> np.ndarray:
    return np.asarray(a).astype(np.float64, copy=False)


def _table() -> np.ndarray:
    """K[g, h] = index of g h^-1."""
    return np.array([[mul(g, inv(h)) for h in range(ORDER)] for g in range(ORDER)], dtype=np.int64)


def unroll(w) -> np.ndarray:
    """Dense weight of the layer: W[d*8+g, c*8+h] = w[d, c, g h^-1]."""
    w = _f64(w)
    Dp, Cp, G = w.shape
    assert G == ORDER
    blocks = w[:, :, _table()]                  # [D', C', 8(g), 8(h)]
    return blocks.transpose(0, 2, 1, 3).reshape(Dp * ORDER, Cp * ORDER)


def fwd(x, w) -> np.ndarray:
    """y = x W^T."""
    return _f64(x) @ unroll(w).T


def bwd_x(dy, w) -> np.ndarray:
    """dx = dy W (the adjoint of fwd in x)."""
    return _f64(dy) @ unroll(w)


def bwd_w(x, dy) -> np.ndarray:
    """Gradient of the shared parameters: the dense gradient dy^T x summed over the
    entries each parameter is replicated into (weight sharing's chain rule)."""
    x, dy = _f64(x), _f64(dy)
    Cp, Dp = x.shape[1] // ORDER, dy.shape[1] // ORDER
    dense = (dy.T @ x).reshape(Dp, ORDER, Cp, ORDER).transpose(0, 2, 1, 3)  # [D', C', g, h]
    K = _table()
    dw = np.zeros((Dp, Cp, ORDER))
    for g in range(ORDER):
        for h in range(ORDER):
            dw[:, :, K[g, h]] += dense[:, :, g, h]
    return dw


def right_translate(v, a: int) -> np.ndarray:
    """(R_a v)(h) = v(h e_a) along the group axis of an array [..., ch*8]."""
    v = _f64(v)
    lead = v.shape[:-1]
    ch = v.shape[-1] // ORDER
    u = v.reshape(*lead, ch, ORDER)
    src = np.array([mul(h, a) for h in range(ORDER)])
    return u[..., src].reshape(*lead, ch * ORDER)
