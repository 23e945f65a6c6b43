"""Dense decode attention over a decoded FibQuant cache — oracle (test infrastructure only).

FibQuant summary §5: because every key and value sits at a fixed address, the
decompression can be fused into the attention kernel.  The oracle does not
fuse anything: it decodes the whole cache in fp64 (no output rounding) and runs
plain softmax attention, which is what the fused kernel must reproduce.

Readings: one decode query per (batch, query head); query head h reads KV head
floor(h / (Hq/Hkv)) (contiguous grouped-query groups); no mask (the query sees
all T keys); logits are scale · q·k̂_j; softmax subtracts the row maximum.
Growing cache (the append path of §5's decode loop): when per-batch lengths are
given, batch b sees only its first L_b keys (the ones written so far; the slab
has room for T), and with no key at all the output is 0 (a softmax over an empty
set has no value; zero is the reading taken).
Prefill (several queries per head): every query is scored like a decode query;
with the causal reading the Sq queries are the last Sq positions of the T keys,
so query i sees keys 0 .. T - Sq + i.
"""
from __future__ import annotations

import numpy as np

from .codec import decode


def attention(q: np.ndarray, k_codes: np.ndarray, k_norms: np.ndarray, v_codes: np.ndarray,
              v_norms: np.ndarray, rotation: np.ndarray, codebook: np.ndarray, scale: float,
              lengths=None) -> np.ndarray:
    """softmax(q K̂ᵀ · scale) V̂ per (batch, query head), fp64.

    q [B, Hq, d]; k_codes / v_codes int [B, Hkv, T, d/k]; k_norms / v_norms
    stored norms [B, Hkv, T]; lengths: None (every key) or int [B], batch b then
    using keys 0 .. min(max(lengths[b], 0), T) - 1.  Returns fp64 [B, Hq, d]."""
    q64 = np.asarray(q, dtype=np.float64)
    B, Hq, d = q64.shape
    Hkv, T = k_codes.shape[1], k_codes.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = T if lengths is None else min(max(int(lengths[b]), 0), T)
        if L == 0:
            continue  # no keys: the output stays 0
        for g in range(Hkv):
            kh = decode(k_codes[b, g, :L], k_norms[b, g, :L], rotation, codebook)
            vh = decode(v_codes[b, g, :L], v_norms[b, g, :L], rotation, codebook)
            for h in range(g * G, (g + 1) * G):
                s = (kh @ q64[b, h]) * scale
                s = s - np.max(s)
                p = np.exp(s)
                p = p / np.sum(p)
                out[b, h] = p @ vh
    return out


def prefill_attention(q: np.ndarray, k_codes: np.ndarray, k_norms: np.ndarray, v_codes: np.ndarray,
                      v_norms: np.ndarray, rotation: np.ndarray, codebook: np.ndarray, scale: float,
                      causal: bool) -> np.ndarray:
    """Sq queries per (batch, query head) over the decoded cache, fp64.

    q [B, Hq, Sq, d]; codes / norms as for :func:`attention`.  causal: query i sees
    keys 0 .. T - Sq + i (none when that is negative: output 0).  Returns fp64
    [B, Hq, Sq, d]."""
    q64 = np.asarray(q, dtype=np.float64)
    B, Hq, Sq, d = q64.shape
    Hkv, T = k_codes.shape[1], k_codes.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.zeros((B, Hq, Sq, d))
    for b in range(B):
        for g in range(Hkv):
            kh = decode(k_codes[b, g], k_norms[b, g], rotation, codebook)
            vh = decode(v_codes[b, g], v_norms[b, g], rotation, codebook)
            for h in range(g * G, (g + 1) * G):
                for i in range(Sq):
                    L = min(T, T - Sq + i + 1) if causal else T
                    if L <= 0:
                        continue
                    s = (kh[:L] @ q64[b, h, i]) * scale
                    s = s - np.max(s)
                    p = np.exp(s)
                    p = p / np.sum(p)
                    out[b, h, i] = p @ vh[:L]
    return out
