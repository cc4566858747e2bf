"""Pins for the offline transform fit (bit_quantized_decode_dqk_amd.calibrate):
the pair keeps dot products, the query basis is uncorrelated and ordered by
energy, alpha = 1 whitens the keys, alpha = 0 is a rotation, and diagonal
covariances give the closed forms (permutations and diagonal scalings)."""
import numpy as np
import pytest

from bit_quantized_decode_dqk_amd import calibrate as CAL


def _spd(rng, d, spread):
    v, _ = np.linalg.qr(rng.standard_normal((d, d)))
    w = np.exp(rng.uniform(0.0, np.log(spread), d))
    return (v * w) @ v.T


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.5, 1.0])
def test_pair_identity_and_orders(alpha):
    rng = np.random.default_rng(70)
    d = 64
    sk, sq = _spd(rng, d, 400.0), _spd(rng, d, 1e3)
    a, b, lam = CAL.fit_transforms(sk, sq, alpha, dtype=np.float64)
    assert np.allclose(a @ b.T, np.eye(d), atol=1e-9)                     # A B^T = I
    cq = a.T @ sq @ a
    assert np.allclose(cq, np.diag(lam), atol=1e-8 * lam[0])             # uncorrelated, energies lam
    assert np.all(np.diff(lam) <= 1e-12 * lam[0]) and lam[-1] > 0        # descending
    ck = b.T @ sk @ b
    ref = np.linalg.eigvalsh(CAL.sym_power(sk, 1.0 - alpha))
    assert np.allclose(np.sort(np.linalg.eigvalsh(ck)), np.sort(ref), rtol=1e-7)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    assert abs((q @ a) @ (k @ b) - q @ k) <= 1e-9 * np.linalg.norm(q) * np.linalg.norm(k)


def test_full_whitening_and_rotation_limits():
    rng = np.random.default_rng(71)
    d = 32
    sk, sq = _spd(rng, d, 100.0), _spd(rng, d, 50.0)
    a, b, _ = CAL.fit_transforms(sk, sq, 1.0, dtype=np.float64)
    assert np.allclose(b.T @ sk @ b, np.eye(d), atol=1e-9)               # alpha = 1: flat keys
    a0, b0, _ = CAL.fit_transforms(sk, sq, 0.0, dtype=np.float64)
    assert np.allclose(a0, b0) and np.allclose(a0.T @ a0, np.eye(d), atol=1e-12)   # a rotation


def test_diagonal_closed_forms():
    """S_k = I, S_q = diag(e): A = B = the permutation ordering e descending (up
    to signs).  S_k = diag(s^2), S_q = I: M = diag(s^(2 alpha)), so R orders s
    descending and B = diag(s^-alpha) R, A = diag(s^alpha) R."""
    d = 16
    e = np.arange(1, d + 1, dtype=np.float64)[np.random.default_rng(72).permutation(d)]
    a, b, lam = CAL.fit_transforms(np.eye(d), np.diag(e), 0.7, dtype=np.float64)
    perm = np.zeros((d, d))
    perm[np.argsort(-e), np.arange(d)] = 1.0
    assert np.allclose(np.abs(a), perm) and np.allclose(np.abs(b), perm)
    assert np.allclose(lam, np.sort(e)[::-1])
    s = np.exp(np.random.default_rng(73).uniform(0, 3, d))
    al = 0.5
    a, b, lam = CAL.fit_transforms(np.diag(s ** 2), np.eye(d), al, dtype=np.float64)
    order = np.argsort(-s)
    r = np.zeros((d, d))
    r[order, np.arange(d)] = 1.0
    assert np.allclose(np.abs(b), np.diag(s ** -al) @ r)
    assert np.allclose(np.abs(a), np.diag(s ** al) @ r)
    assert np.allclose(lam, np.sort(s ** (2 * al))[::-1])


def test_rotation_is_orthogonal_and_fp32_pair():
    a, b = CAL.rotation_transforms(128, seed=3)
    assert a.dtype == np.float32 and np.array_equal(a, b)
    assert np.allclose(a.astype(np.float64).T @ a.astype(np.float64), np.eye(128), atol=1e-5)
    rng = np.random.default_rng(74)
    sk, sq = _spd(rng, 128, 1600.0), _spd(rng, 128, 1e4)
    a32, b32, _ = CAL.fit_transforms(sk, sq, 0.5)
    assert a32.dtype == np.float32 and b32.dtype == np.float32
    assert np.abs(a32.astype(np.float64) @ b32.astype(np.float64).T - np.eye(128)).max() < 1e-4


def test_alpha_out_of_range():
    with pytest.raises(ValueError):
        CAL.fit_transforms(np.eye(4), np.eye(4), 1.5)
