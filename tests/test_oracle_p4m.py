"""Pins of the p4m (dihedral D4) oracle against facts other than its own formulas.

- The group law satisfies the group axioms and is D4's: order 8, non-abelian, r^4 = s^2 = e,
  s r s = r^-1, and exactly five elements of order 2 (this rules out Z8, Z4 x Z2, Z2^3 and
  the quaternion group).
- The layer is equivariant under right translation of the group axis, for every element.
- Convolution theorem through D4's two-dimensional irreducible representation (rotation
  by 90 degrees and a mirror as 2 x 2 matrices, checked to be a homomorphism of the law):
  y^(rho) = w^(rho) x^(rho).
- Restricted to rotation-only or reflection-only parameters, the layer's four
  rotation/reflection blocks are circular convolutions along Z_4, computed here with the
  independently written C_T oracle.
- Constant input over the group: every output element equals sum_c u_c sum_k w[d,c,k].
- Adjoint and linearity identities for the two gradients; the weight gradient is
  invariant under translating x and dy together.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import p4m_oracle as P

G = P.ORDER
E = P.index(0, 0)
R = P.index(1, 0)
S = P.index(0, 1)


def rng(seed):
    return np.random.default_rng(seed)


def test_group_axioms_and_d4_signature():
    els = range(G)
    for i in els:
        assert P.index(*P.element(i)) == i
        assert P.mul(E, i) == i and P.mul(i, E) == i
        assert P.mul(i, P.inv(i)) == E and P.mul(P.inv(i), i) == E
    for i, j, k in itertools.product(els, els, els):
        assert P.mul(P.mul(i, j), k) == P.mul(i, P.mul(j, k))
    # Generators and relations.
    r2 = P.mul(R, R)
    assert P.mul(r2, r2) == E and r2 != E
    assert P.mul(S, S) == E and S != E
    assert P.mul(P.mul(S, R), S) == P.inv(R)
    assert P.mul(R, S) != P.mul(S, R)
    order2 = [i for i in els if i != E and P.mul(i, i) == E]
    assert len(order2) == 5
    # Index layout: rotations first, then the reflections r^-m s for m = 0..3.
    assert [P.element(j) for j in range(G)] == [(0, 0), (1, 0), (2, 0), (3, 0), (0, 1), (3, 1), (2, 1), (1, 1)]


def test_unroll_matches_the_defining_sum():
    g = rng(1)
    N, Cp, Dp = 3, 2, 3
    x, w = g.standard_normal((N, Cp * G)), g.standard_normal((Dp, Cp, G))
    y = P.fwd(x, w)
    for n, d, gg in itertools.product(range(N), range(Dp), range(G)):
        ref = sum(w[d, c, P.mul(gg, P.inv(h))] * x[n, c * G + h] for c in range(Cp) for h in range(G))
        assert abs(y[n, d * G + gg] - ref) < 1e-12


@pytest.mark.parametrize("a", range(G))
def test_equivariant_under_right_translation(a):
    g = rng(2 + a)
    x, w = g.standard_normal((5, 3 * G)), g.standard_normal((4, 3, G))
    np.testing.assert_allclose(P.fwd(P.right_translate(x, a), w), P.right_translate(P.fwd(x, w), a), atol=1e-12)


def test_not_equivariant_under_left_translation():
    # D4 is not abelian: the layer commutes with right, not left, translations.
    g = rng(11)
    x, w = g.standard_normal((2, 2 * G)), g.standard_normal((2, 2, G))
    left = lambda v, a: v.reshape(v.shape[0], -1, G)[..., [P.mul(P.inv(a), h) for h in range(G)]].reshape(v.shape)
    assert np.abs(P.fwd(left(x, R), w) - left(P.fwd(x, w), R)).max() > 1e-3


def _rho(j):
    """Two-dimensional irreducible representation: r -> rotation by 90 degrees, s -> mirror."""
    Rm = np.array([[0.0, -1.0], [1.0, 0.0]])
    Sm = np.array([[1.0, 0.0], [0.0, -1.0]])
    a, b = P.element(j)
    return np.linalg.matrix_power(Rm, a) @ np.linalg.matrix_power(Sm, b)


def test_convolution_theorem_through_the_two_dimensional_irrep():
    for i, j in itertools.product(range(G), range(G)):
        np.testing.assert_allclose(_rho(P.mul(i, j)), _rho(i) @ _rho(j), atol=1e-15)
    g = rng(3)
    N, Cp, Dp = 4, 3, 2
    x, w = g.standard_normal((N, Cp * G)), g.standard_normal((Dp, Cp, G))
    y = P.fwd(x, w).reshape(N, Dp, G)
    xs = x.reshape(N, Cp, G)
    hat = lambda v: np.einsum("...j,jab->...ab", v, np.stack([_rho(j) for j in range(G)]))
    yh, wh, xh = hat(y), hat(w), hat(xs)                      # [N,D',2,2], [D',C',2,2], [N,C',2,2]
    np.testing.assert_allclose(yh, np.einsum("dcab,ncbe->ndae", wh, xh), atol=1e-11)


def test_rotation_and_reflection_blocks_are_c4_convolutions():
    """Rotation half r^a (indices 0..3) and reflection half r^-a s (indices 4..7): with
    rotation-only parameters each half maps to itself by a circular convolution (kernel
    w(r^k) on rotations, w(r^-k) on reflections); with reflection-only parameters the
    halves swap, with kernels w(r^k s) (reflections -> rotations) and w(r^-k s)
    (rotations -> reflections)."""
    g = rng(4)
    N, Cp, Dp = 5, 3, 2
    x = g.standard_normal((N, Cp, G))
    x_rot, x_ref = x[:, :, :4].reshape(N, -1), x[:, :, 4:].reshape(N, -1)
    k = np.arange(4)
    at = lambda w, a, b: w[:, :, [P.index(int(ai), b) for ai in a]]   # kernel k -> w(r^{a_k} s^b)
    w = g.standard_normal((Dp, Cp, G))
    w_rot, w_ref = w.copy(), w.copy()
    w_rot[:, :, 4:] = 0.0
    w_ref[:, :, :4] = 0.0
    y = P.fwd(x.reshape(N, -1), w_rot).reshape(N, Dp, G)
    np.testing.assert_allclose(y[:, :, :4].reshape(N, -1), oracle.fwd(x_rot, at(w_rot, k, 0)), atol=1e-12)
    np.testing.assert_allclose(y[:, :, 4:].reshape(N, -1), oracle.fwd(x_ref, at(w_rot, -k, 0)), atol=1e-12)
    y = P.fwd(x.reshape(N, -1), w_ref).reshape(N, Dp, G)
    np.testing.assert_allclose(y[:, :, :4].reshape(N, -1), oracle.fwd(x_ref, at(w_ref, k, 1)), atol=1e-12)
    np.testing.assert_allclose(y[:, :, 4:].reshape(N, -1), oracle.fwd(x_rot, at(w_ref, -k, 1)), atol=1e-12)


def test_constant_input_sees_the_parameter_sum():
    g = rng(5)
    u, w = g.standard_normal((3, 4)), g.standard_normal((2, 4, G))
    x = np.repeat(u[:, :, None], G, axis=2).reshape(3, -1)
    y = P.fwd(x, w).reshape(3, 2, G)
    ref = u @ w.sum(axis=2).T
    for gg in range(G):
        np.testing.assert_allclose(y[:, :, gg], ref, atol=1e-12)


def test_gradient_identities():
    g = rng(6)
    N, Cp, Dp = 7, 3, 4
    x, dy = g.standard_normal((N, Cp * G)), g.standard_normal((N, Dp * G))
    w, w2 = g.standard_normal((Dp, Cp, G)), g.standard_normal((Dp, Cp, G))
    # Adjoint in x: <x W^T, dy> = <x, dy W>.
    assert np.isclose(np.sum(P.fwd(x, w) * dy), np.sum(x * P.bwd_x(dy, w)), rtol=1e-12)
    # Linearity in w: <y(x; w2), dy> = <dw(x, dy), w2>.
    assert np.isclose(np.sum(P.fwd(x, w2) * dy), np.sum(P.bwd_w(x, dy) * w2), rtol=1e-12)
    for a in range(G):
        np.testing.assert_allclose(P.bwd_w(P.right_translate(x, a), P.right_translate(dy, a)), P.bwd_w(x, dy),
                                   atol=1e-11)
