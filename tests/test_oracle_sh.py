"""Pins of the oracle's spherical-harmonics basis against a library routine and quadrature."""
import numpy as np
import pytest
import scipy.special as sp

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def real_sh_from_scipy(l, m, theta, phi):
    """Real orthonormal SH from scipy's complex Y_l^m (theta = polar, phi = azimuth).

    The real basis removes the Condon-Shortley phase: for m > 0 it is sqrt(2) (-1)^m Re Y_l^m,
    for m < 0 sqrt(2) (-1)^m Im Y_l^|m|, and Y_l^0 for m = 0."""
    Y = sp.sph_harm_y(l, abs(m), theta, phi)
    if m > 0:
        return np.sqrt(2.0) * (-1.0) ** m * Y.real
    if m < 0:
        return np.sqrt(2.0) * (-1.0) ** m * Y.imag
    return Y.real


def test_sh_basis_matches_scipy(oracle_mod):
    rng = np.random.default_rng(7)
    d = rng.standard_normal((200, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    theta = np.arccos(np.clip(d[:, 2], -1, 1))
    phi = np.arctan2(d[:, 1], d[:, 0])
    Y = oracle_mod.sh_basis(3, d)
    for l in range(4):
        for m in range(-l, l + 1):
            ref = real_sh_from_scipy(l, m, theta, phi)
            np.testing.assert_allclose(Y[:, l * l + l + m], ref, rtol=1e-12, atol=1e-12, err_msg=f"l={l} m={m}")


def test_sh_orthonormal_by_quadrature(oracle_mod):
    # Gauss-Legendre in cos(theta) x uniform azimuth integrates products of degree <= 6 exactly.
    xg, wg = np.polynomial.legendre.leggauss(12)
    nphi = 24
    phi = (np.arange(nphi) + 0.5) * 2 * np.pi / nphi
    ct, ph = np.meshgrid(xg, phi, indexing="ij")
    w = (wg[:, None] * np.full(nphi, 2 * np.pi / nphi)[None, :]).ravel()
    st = np.sqrt(1 - ct ** 2)
    d = np.stack([st * np.cos(ph), st * np.sin(ph), ct], -1).reshape(-1, 3)
    Y = oracle_mod.sh_basis(3, d)
    gram = (Y * w[:, None]).T @ Y
    np.testing.assert_allclose(gram, np.eye(16), atol=1e-12)


def test_sh_lower_degrees_are_prefixes(oracle_mod):
    d = np.array([[0.3, -0.4, np.sqrt(1 - 0.25)]])
    full = oracle_mod.sh_basis(3, d)
    for deg in range(3):
        np.testing.assert_array_equal(oracle_mod.sh_basis(deg, d), full[:, : (deg + 1) ** 2])
