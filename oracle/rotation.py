"""Shared Haar rotation Π — oracle (test infrastructure only).

FibQuant summary §1 and §2.1: the codec applies one shared random orthogonal
(Haar) rotation to every normalised vector.

Reading: the rotation is drawn from a fixed seed as the orthogonal factor of the
QR decomposition of a d×d standard Gaussian matrix, with the sign fix
Π = Q · diag(sign(diag R)) that makes the factor exactly Haar-distributed (the
plain Householder Q is not).  Convention: y = Π x (Π acts on column vectors),
so rows of a batch rotate as X Πᵀ and the inverse rotation of a row is ŷ Π.
The artifact shared with the GPU is Π rounded to fp32; every oracle computation
uses those fp32 values exactly (as fp64).
"""
from __future__ import annotations

import numpy as np


def haar_rotation(d: int, seed: int) -> np.ndarray:
    """fp64 d×d Haar-distributed orthogonal matrix from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))  # diag(R) is nonzero with probability 1 for Gaussian G
    return q * s[None, :]


def shared_rotation(d: int = 64, seed: int = 0) -> np.ndarray:
    """The shared rotation artifact: :func:`haar_rotation` rounded to fp32."""
    return haar_rotation(d, seed).astype(np.float32)
