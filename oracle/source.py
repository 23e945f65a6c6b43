"""Canonical spherical-Beta block source — oracle (test infrastructure only).

FibQuant summary §2.1 and §3.1 (Theorem 1): after normalisation and a Haar
rotation the vector is uniform on the sphere S^{d-1}, and every block of k
consecutive coordinates follows one spherical-Beta density f_{d,k} on the unit
ball B^k, whatever the input law was.

The pages name the density without printing it.  It is the textbook marginal
of k coordinates of a uniform point on S^{d-1}:

    f_{d,k}(y) = Γ(d/2) / (π^{k/2} Γ((d-k)/2)) · (1 - ‖y‖²)^{(d-k)/2 - 1},  ‖y‖ < 1, k < d,

so ‖y‖² ~ Beta(k/2, (d-k)/2) with an independent uniform direction.  For k = d
the block is the whole vector and lies on the sphere itself.
"""
from __future__ import annotations

import numpy as np
from scipy import special, stats


def sample_canonical(d: int, k: int, m: int, rng: np.random.Generator) -> np.ndarray:
    """m draws of a k-block of a uniform point on S^{d-1}: the first k
    coordinates of a normalised standard Gaussian d-vector (fp64 [m, k])."""
    g = rng.standard_normal((m, d))
    g /= np.sqrt(np.sum(g * g, axis=1, keepdims=True))
    return g[:, :k].copy()


def block_radius_sq_law(d: int, k: int):
    """Frozen SciPy law of ‖y_b‖² under f_{d,k}: Beta(k/2, (d-k)/2), k < d."""
    if not 0 < k < d:
        raise ValueError("block law defined for 0 < k < d")
    return stats.beta(k / 2.0, (d - k) / 2.0)


def log_density(y: np.ndarray, d: int, k: int) -> np.ndarray:
    """log f_{d,k}(y) for points y [m, k] strictly inside the unit ball."""
    t = np.sum(y * y, axis=-1)
    logc = special.gammaln(d / 2.0) - (k / 2.0) * np.log(np.pi) - special.gammaln((d - k) / 2.0)
    return logc + ((d - k) / 2.0 - 1.0) * np.log1p(-t)
