"""Offline FibQuant codebook construction — oracle (test infrastructure only).

FibQuant summary §2.2: one shared codebook matched to the spherical-Beta source
combines (1) radii r_n from the Bennett-Gersho companding rule applied to the
source's radial density (a closed form with Beta-quantile radii for k = 2),
(2) quasi-uniform directions u_n (planar Fibonacci spiral for k = 2, Fibonacci
sphere for k = 3, Roberts-Kronecker low-discrepancy sequence for k >= 4), and
(3) multi-restart Lloyd-Max refinement of that deterministic start for the
finite size N.  The codewords are c_n = r_n u_n before refinement.

Readings (the pages give the ingredients, not the formulas):
  * Companding: the high-resolution MSE-optimal point density is proportional
    to f^{k/(k+2)} (Bennett's integral).  For f_{d,k} ∝ (1-‖y‖²)^α with
    α = (d-k)/2 - 1 that density is radial, and the squared radius of the points
    follows Beta(k/2, 1 + α·k/(k+2)).  Codeword n takes the quantile of that law
    at (n + 1/2)/N (each codeword owns mass 1/N).  For k = 2 the law is
    Beta(1, β) whose quantile 1 - (1-p)^{1/β} is closed-form.  ``law="source"``
    gives the uncompanded source law Beta(k/2, (d-k)/2) instead.
    For k = d the block lies on the sphere, so every radius is 1.
  * k = 2 directions: angle n·π(3-√5) (the golden angle), i.e. the sunflower
    spiral with radius index n.
  * k >= 4 directions: Roberts' R_k sequence t_n = frac(1/2 + n·α), n = 1..N,
    α_j = φ_k^{-j} (j = 1..k) with φ_k the positive root of x^{k+1} = x + 1;
    mapped to the sphere by z = Φ^{-1}(t) (inverse normal CDF), u = z/‖z‖.
    Radius index n is paired with direction n.
  * k = 3 directions: Fibonacci sphere point n (height 1-(2n+1)/N, azimuth
    n × golden angle); its radius index is the rank of frac(n/φ) so that radius
    and height are not correlated.  (No workload uses k = 3.)
  * k = 1 (the scalar comparator of Theorem 2): signed quantiles of the
    companded law.
  * Lloyd: generalised Lloyd on M samples of f_{d,k} (M = max(256·N, 10^5)
    unless given), nearest-codeword assignment then cell means; an empty cell
    is re-seeded at the training sample with the largest current error.
    Restart r starts from init·H_rᵀ with H_r a seeded k×k Haar rotation (H_0 = I),
    valid because f_{d,k} is rotation invariant.  The restart with the lowest
    MSE on an independent validation set of the same size is kept.
  * The finished codebook is rounded to the nearest fp16-representable values
    (round-to-nearest-even), with values below the smallest normal fp16 (2^-14)
    flushed to zero, so that both the CPU oracle and fp16 matrix units see the
    exact same codewords.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
from scipy import special

from .rotation import haar_rotation
from .source import sample_canonical

GOLDEN_ANGLE = np.pi * (3.0 - np.sqrt(5.0))  # radians, ≈ 137.5077640500378°
GOLDEN_RATIO = (1.0 + np.sqrt(5.0)) / 2.0


# ---------------------------------------------------------------- radii
def radial_beta_params(d: int, k: int, law: str = "companded") -> tuple[float, float]:
    """Parameters (a, b) of the Beta law of r² for the codeword radii (k < d)."""
    if not 0 < k < d:
        raise ValueError("radial law defined for 0 < k < d")
    alpha = (d - k) / 2.0 - 1.0
    if law == "source":
        return k / 2.0, (d - k) / 2.0
    if law == "companded":
        return k / 2.0, 1.0 + (k / (k + 2.0)) * alpha
    raise ValueError(law)


def radii(d: int, k: int, N: int, law: str = "companded") -> np.ndarray:
    """r_n = sqrt(Q_{Beta(a,b)}((n + 1/2)/N)), n = 0..N-1; all ones when k = d."""
    if k == d:
        return np.ones(N)
    a, b = radial_beta_params(d, k, law)
    p = (np.arange(N) + 0.5) / N
    return np.sqrt(special.betaincinv(a, b, p))


# ---------------------------------------------------------------- directions
def spiral_directions(N: int) -> np.ndarray:
    """Planar Fibonacci spiral: unit vectors at angles n × golden angle."""
    th = np.arange(N) * GOLDEN_ANGLE
    return np.stack([np.cos(th), np.sin(th)], axis=1)


def fibonacci_sphere_directions(N: int) -> np.ndarray:
    """Fibonacci sphere on S²: height 1-(2n+1)/N, azimuth n × golden angle."""
    n = np.arange(N)
    z = 1.0 - (2.0 * n + 1.0) / N
    rho = np.sqrt(np.maximum(0.0, 1.0 - z * z))
    ph = n * GOLDEN_ANGLE
    return np.stack([rho * np.cos(ph), rho * np.sin(ph), z], axis=1)


def kronecker_phi(k: int) -> float:
    """Positive root of x^{k+1} = x + 1 (the generalised golden ratio), by bisection."""
    lo, hi = 1.0, 2.0  # g(x) = x^{k+1} - x - 1: g(1) = -1 < 0, g(2) > 0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid ** (k + 1) - mid - 1.0 < 0.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def roberts_points(k: int, N: int) -> np.ndarray:
    """Roberts' R_k low-discrepancy points in [0,1)^k: frac(1/2 + n α), n = 1..N."""
    phi = kronecker_phi(k)
    alpha = phi ** -np.arange(1, k + 1, dtype=np.float64)
    n = np.arange(1, N + 1, dtype=np.float64)[:, None]
    return np.mod(0.5 + n * alpha[None, :], 1.0)


def roberts_directions(k: int, N: int) -> np.ndarray:
    """Roberts-Kronecker points pushed to S^{k-1} through the inverse normal CDF."""
    z = special.ndtri(roberts_points(k, N))
    if not np.all(np.isfinite(z)):
        raise FloatingPointError("Roberts point on the cube boundary")
    return z / np.sqrt(np.sum(z * z, axis=1, keepdims=True))


def initial_codebook(d: int, k: int, N: int, law: str = "companded") -> np.ndarray:
    """Deterministic start c_n = r_n u_n (fp64 [N, k])."""
    if k == 1:
        a, b = radial_beta_params(d, 1, law)
        p = (np.arange(N) + 0.5) / N
        q = np.abs(2.0 * p - 1.0)
        return (np.sign(p - 0.5) * np.sqrt(special.betaincinv(a, b, q)))[:, None]
    r = radii(d, k, N, law)
    if k == 2:
        u = spiral_directions(N)
    elif k == 3:
        u = fibonacci_sphere_directions(N)
        rank = np.argsort(np.argsort(np.mod(np.arange(N) / GOLDEN_RATIO, 1.0), kind="stable"), kind="stable")
        r = r[rank]
    else:
        u = roberts_directions(k, N)
    return r[:, None] * u


# ---------------------------------------------------------------- Lloyd-Max
def assign(samples: np.ndarray, c: np.ndarray, chunk: int = 16384) -> tuple[np.ndarray, np.ndarray]:
    """Nearest codeword of every training sample (lowest index on ties) and the
    squared error to it.  Training-only helper: it ranks codewords by
    ‖c‖² - 2 y·c (a matrix product), then measures the error directly."""
    cn2 = np.sum(c * c, axis=1)
    idx = np.empty(len(samples), dtype=np.int64)
    for s in range(0, len(samples), chunk):
        y = samples[s:s + chunk]
        idx[s:s + chunk] = np.argmin(cn2[None, :] - 2.0 * (y @ c.T), axis=1)
    err = np.sum((samples - c[idx]) ** 2, axis=1)
    return idx, err


def lloyd(init: np.ndarray, train: np.ndarray, max_iter: int = 100, rel_tol: float = 1e-6):
    """Generalised Lloyd iteration.  Returns (codebook, mse history, assignment).

    history[i] is the training MSE of the assignment made after update i
    (history[0]: the initial codebook).  Stops when no assignment changes (the
    codewords are then exactly the cell means), when the relative decrease falls
    below ``rel_tol``, or after ``max_iter`` updates."""
    c = np.array(init, dtype=np.float64, copy=True)
    N, k = c.shape
    idx, err = assign(train, c)
    hist = [float(err.mean())]
    for _ in range(max_iter):
        counts = np.bincount(idx, minlength=N)
        new = c.copy()
        nz = counts > 0
        for j in range(k):
            s = np.bincount(idx, weights=train[:, j], minlength=N)
            new[nz, j] = s[nz] / counts[nz]
        empty = np.flatnonzero(~nz)
        if len(empty):
            worst = np.argsort(-err, kind="stable")[: len(empty)]
            new[empty] = train[worst]
        c = new
        new_idx, err = assign(train, c)
        hist.append(float(err.mean()))
        changed = bool(np.any(new_idx != idx))
        idx = new_idx
        if not changed:
            break
        if hist[-2] - hist[-1] <= rel_tol * hist[-1]:
            break
    return c, hist, idx


def to_fp16_grid(c: np.ndarray) -> np.ndarray:
    """Round to fp16-representable values (RNE), flush |v| < 2^-14 to 0; fp32 container."""
    h = np.asarray(c, dtype=np.float64).astype(np.float16)
    h[np.abs(h.astype(np.float64)) < 2.0 ** -14] = 0.0
    return h.astype(np.float32)


@dataclass
class Codebook:
    d: int
    k: int
    N: int
    codewords: np.ndarray          # fp32 [N, k], fp16-representable
    seed: int
    law: str
    restarts: int
    samples: int
    valid_mse: float               # per-block MSE of the rounded codebook on the validation set
    restart_valid_mse: list = field(default_factory=list)
    history: list = field(default_factory=list)  # training MSE history of the kept restart

    @property
    def normalised_mse(self) -> float:
        """Validation MSE divided by the block's mean energy k/d."""
        return self.valid_mse / (self.k / self.d)


def build_codebook(d: int, k: int, N: int, seed: int, restarts: int = 3, samples: int | None = None,
                   max_iter: int = 100, rel_tol: float = 1e-6, law: str = "companded",
                   init: np.ndarray | None = None) -> Codebook:
    """Full offline construction: deterministic start, multi-restart Lloyd, fp16 grid."""
    rng = np.random.default_rng(seed)
    m = samples if samples is not None else max(256 * N, 100_000)
    train = sample_canonical(d, k, m, rng)
    valid = sample_canonical(d, k, m, rng)
    c_init = initial_codebook(d, k, N, law) if init is None else np.asarray(init, dtype=np.float64)
    best = None
    vm = []
    for r in range(restarts):
        h = np.eye(k) if r == 0 else haar_rotation(k, seed * 1000 + r)
        c, hist, _ = lloyd(c_init @ h.T, train, max_iter=max_iter, rel_tol=rel_tol)
        v = float(assign(valid, c)[1].mean())
        vm.append(v)
        if best is None or v < best[0]:
            best = (v, c, hist)
    cw = to_fp16_grid(best[1])
    if len(np.unique(cw, axis=0)) != N:
        raise ValueError("fp16 rounding merged codewords")
    v_rounded = float(assign(valid, cw.astype(np.float64))[1].mean())
    return Codebook(d, k, N, cw, seed, law, restarts, m, v_rounded, vm, best[2])
