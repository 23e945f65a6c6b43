"""Dense decode attention over a decoded FibQuant cache — oracle (test infrastructure only).

FibQuant summary §5: because every key and value sits at a fixed address, the
decompression can be fused into the attention kernel.  The oracle does not
fuse anything: it decodes the whole cache in fp64 (no output rounding) and runs
plain softmax attention, which is what the fused kernel must reproduce.

Readings: one decode query per (batch, query head); query head h reads KV head
floor(h / (Hq/Hkv)) (contiguous grouped-query groups); no mask (the query sees
all T keys); logits are scale · q·k̂_j; softmax subtracts the row maximum.
"""
from __future__ import annotations

import numpy as np

from .codec import decode


def attention(q: np.ndarray, k_codes: np.ndarray, k_norms: np.ndarray, v_codes: np.ndarray,
              v_norms: np.ndarray, rotation: np.ndarray, codebook: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K̂ᵀ · scale) V̂ per (batch, query head), fp64.

    q [B, Hq, d]; k_codes / v_codes int [B, Hkv, T, d/k]; k_norms / v_norms
    stored norms [B, Hkv, T].  Returns fp64 [B, Hq, d]."""
    q64 = np.asarray(q, dtype=np.float64)
    B, Hq, d = q64.shape
    Hkv, T = k_codes.shape[1], k_codes.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for g in range(Hkv):
            kh = decode(k_codes[b, g], k_norms[b, g], rotation, codebook)
            vh = decode(v_codes[b, g], v_norms[b, g], rotation, codebook)
            for h in range(g * G, (g + 1) * G):
                s = (kh @ q64[b, h]) * scale
                s = s - np.max(s)
                p = np.exp(s)
                p = p / np.sum(p)
                out[b, h] = p @ vh
    return out
