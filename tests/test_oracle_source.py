"""Pins for the canonical source and Theorem 1 (FibQuant summary §2.1, §3.1):
after normalisation and a Haar rotation every k-block follows f_{d,k} on B^k,
i.e. ‖y_b‖² ~ Beta(k/2, (d-k)/2) with a uniform direction, for any nonzero input."""
import numpy as np
import pytest
from scipy import integrate, stats

import workloads
from oracle.codec import rotate_unit
from oracle.rotation import haar_rotation
from oracle.source import block_radius_sq_law, log_density, sample_canonical

D = 64


def _chi2_equiprobable(values, law, bins=50):
    edges = law.ppf(np.linspace(0, 1, bins + 1))
    counts, _ = np.histogram(values, bins=edges)
    expected = len(values) / bins
    chi2 = np.sum((counts - expected) ** 2 / expected)
    return stats.chi2.sf(chi2, bins - 1)


def _adversarial_inputs():
    e1 = np.zeros(D)
    e1[0] = 1.0
    outlier = np.ones(D)
    outlier[3] = 20.0
    heavy = workloads.gpt2_small_kv()[12345].astype(np.float64)
    return {"e1": e1, "outlier": outlier, "student_t": heavy}


@pytest.fixture(scope="module")
def haar_draws():
    return [haar_rotation(D, 50_000 + s) for s in range(6000)]


@pytest.mark.parametrize("name", ["e1", "outlier", "student_t"])
@pytest.mark.parametrize("k", [2, 8])
def test_theorem1_block_radius_law_over_rotations(haar_draws, name, k):
    # Fixed (adversarial) input, random Haar rotations: block 0's squared radius
    # must follow Beta(k/2, (d-k)/2) (chi-square, 50 equiprobable bins).
    x = _adversarial_inputs()[name]
    vals = []
    for pi in haar_draws:
        y, _ = rotate_unit(x[None, :], pi.astype(np.float32))
        vals.append(np.sum(y[0, :k] ** 2))
    assert _chi2_equiprobable(np.array(vals), block_radius_sq_law(D, k)) > 1e-3


def test_theorem1_angle_uniform_k2(haar_draws):
    x = _adversarial_inputs()["outlier"]
    ang = []
    for pi in haar_draws:
        y, _ = rotate_unit(x[None, :], pi.astype(np.float32))
        ang.append(np.arctan2(y[0, 1], y[0, 0]))
    assert _chi2_equiprobable(np.array(ang), stats.uniform(-np.pi, 2 * np.pi), bins=36) > 1e-3


def test_theorem1_detects_missing_normalisation(haar_draws):
    # Planted mistake: without the division by ν the block radius law is wrong.
    x = _adversarial_inputs()["outlier"]
    vals = [np.sum((pi @ x)[:2] ** 2) for pi in haar_draws[:2000]]
    assert _chi2_equiprobable(np.array(vals), block_radius_sq_law(D, 2)) < 1e-6


@pytest.mark.parametrize("k", [2, 4, 8])
def test_sampler_matches_beta_law(k):
    y = sample_canonical(D, k, 40_000, np.random.default_rng(7))
    assert stats.kstest(np.sum(y * y, axis=1), block_radius_sq_law(D, k).cdf).pvalue > 1e-3


def test_fixed_rotation_iid_gaussian_inputs():
    # The shared fixed Π on i.i.d. Gaussian inputs (which are themselves
    # rotation invariant): every block follows the law.
    x = workloads.iid_gaussian(4096, 101).astype(np.float64)
    y, _ = rotate_unit(x, haar_rotation(D, 0).astype(np.float32))
    vals = np.sum(y.reshape(-1, 2) ** 2, axis=1)[::32]  # one block per vector: independent
    assert _chi2_equiprobable(vals, block_radius_sq_law(D, 2), bins=30) > 1e-3


@pytest.mark.parametrize("k", [2, 4])
def test_density_integrates_to_one(k):
    # ∫_{B^k} f = ∫_0^1 f(r) · |S^{k-1}| r^{k-1} dr with |S^1| = 2π, |S^3| = 2π².
    area = {2: 2 * np.pi, 4: 2 * np.pi ** 2}[k]

    def integrand(r):
        y = np.zeros((1, k))
        y[0, 0] = r
        return np.exp(log_density(y, D, k)[0]) * area * r ** (k - 1)

    val, _ = integrate.quad(integrand, 0, 1, limit=200)
    assert abs(val - 1.0) < 1e-9
