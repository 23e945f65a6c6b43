"""Pins for the oracle's Haar rotation (FibQuant summary §1 and §2.1: one shared
random orthogonal Haar rotation)."""
import numpy as np
from scipy import stats

from oracle.rotation import haar_rotation, shared_rotation


def test_orthogonal_fp64_and_fp32():
    pi = haar_rotation(64, 0)
    assert np.max(np.abs(pi.T @ pi - np.eye(64))) < 1e-12
    assert np.max(np.abs(pi @ pi.T - np.eye(64))) < 1e-12
    p32 = shared_rotation(64, 0).astype(np.float64)
    assert np.max(np.abs(p32.T @ p32 - np.eye(64))) < 1e-6


def test_seed_determinism_and_distinct_seeds():
    assert np.array_equal(haar_rotation(64, 0), haar_rotation(64, 0))
    assert not np.allclose(haar_rotation(64, 0), haar_rotation(64, 1))


def _diag_sign_fractions(make, d=8, draws=2000):
    pos = np.zeros(d)
    for s in range(draws):
        pos += np.diag(make(d, s)) > 0
    return pos / draws


def test_haar_sign_fix_diagonal_signs_balanced():
    # Haar measure is invariant under sign flips of columns, so every diagonal
    # entry is positive with probability exactly 1/2.
    frac = _diag_sign_fractions(haar_rotation)
    for f in frac:
        assert stats.binomtest(int(round(f * 2000)), 2000, 0.5).pvalue > 1e-4


def test_sign_fix_test_catches_plain_qr():
    # Planted mistake: the Householder Q without the sign fix is not Haar; the
    # balanced-sign check above must reject it.
    def plain(d, seed):
        g = np.random.default_rng(seed).standard_normal((d, d))
        return np.linalg.qr(g)[0]

    frac = _diag_sign_fractions(plain)
    pvals = [stats.binomtest(int(round(f * 2000)), 2000, 0.5).pvalue for f in frac]
    assert min(pvals) < 1e-10


def test_first_column_uniform_on_sphere():
    # For Haar Π, every column is uniform on S^{d-1}, so Π_00² ~ Beta(1/2, (d-1)/2).
    d = 16
    v = np.array([haar_rotation(d, 10_000 + s)[0, 0] ** 2 for s in range(3000)])
    assert stats.kstest(v, stats.beta(0.5, (d - 1) / 2).cdf).pvalue > 1e-3
