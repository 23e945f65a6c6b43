"""Seeded synthetic inputs for the FibQuant KV-cache codec.

This module only draws random tensors (NumPy ``default_rng``, i.e. PCG64) with
the shapes and value distributions of the workloads.  It holds none of the
codec's arithmetic (no norm, rotation, search, packing or attention), so the
CPU oracle, the tests and the benchmark can all take their inputs from here
without sharing any of the method's code.

Every generator draws in fp64 and casts round-to-nearest-even to the stored
dtype.  Draw order inside one generator is: per-slab scales (or outlier masks)
first, then the values, each in C order.

The pages (the FibQuant summary, section 4.2 and 4.3) measure on GPT-2 small and
TinyLlama-1.1B key/value caches.  Neither model nor any dataset is used here:
the generators below stand in for them with the model shapes and heavy-tailed /
outlier-channel value laws.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

D = 64  # head dimension of every workload


@dataclass(frozen=True)
class Workload:
    """Static description of one workload: sizes, dtypes and the code parameters."""

    name: str
    n: int            # number of d-dimensional vectors encoded
    in_dtype: str     # "f32" | "f16"
    norm_dtype: str   # "f32" | "f16"
    k: int            # block size
    N: int            # codebook size
    seed: int         # data seed
    codebook_seed: int


# Sizes are those of the five workloads; ``n`` counts d=64 vectors.
WORKLOADS = {
    "iid4096": Workload("iid4096", 4096, "f32", "f32", 2, 16, 101, 201),
    "gpt2s_kv": Workload("gpt2s_kv", 12 * 12 * 1024 * 2, "f16", "f16", 4, 256, 102, 202),
    "tinyllama_kv": Workload("tinyllama_kv", 22 * 4 * 2 * 8 * 4096, "f16", "f16", 8, 4096, 103, 203),
    "fullvec_kv": Workload("fullvec_kv", 1024 * 1024, "f16", "f16", 64, 4096, 104, 204),
    "attn_b16_t32k": Workload("attn_b16_t32k", 2 * 16 * 4 * 32768, "f16", "f16", 4, 256, 105, 202),
}

# Attention workload shape: batch, query heads, KV heads, context.
ATTN_B, ATTN_HQ, ATTN_HKV, ATTN_T = 16, 32, 4, 32768
# The GPT-2-small-shaped cache viewed as attention inputs: layers act as the
# batch dimension, 12 heads, multi-head (no grouping), 1024 tokens.
GPT2_L, GPT2_H, GPT2_T = 12, 12, 1024


def iid_gaussian(n: int = 4096, seed: int = 101, dtype=np.float32) -> np.ndarray:
    """[n, 64] i.i.d. N(0, 1), cast to ``dtype``."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, D)).astype(dtype)


def _student_t_slabs(rng, slab_shape, tokens, df=4.0, scale_sigma=0.5) -> np.ndarray:
    """Student-t(df) values times one lognormal(0, scale_sigma) scale per channel
    and per slab.  Returns fp64 array of shape slab_shape + (tokens, 64)."""
    z = rng.standard_normal(tuple(slab_shape) + (D,))
    sigma = np.exp(scale_sigma * z)
    t = rng.standard_t(df, size=tuple(slab_shape) + (tokens, D))
    t *= sigma[..., None, :]
    return t


def gpt2_small_kv(seed: int = 102) -> np.ndarray:
    """GPT-2-small-shaped KV vectors, fp16 [294912, 64].

    Layout [2 KV][12 layers][12 heads][1024 tokens][64]: the first half is the
    key cache and the second half the value cache, each [layer][head][token].
    Values: Student-t (4 degrees of freedom) times a per-channel lognormal(0, 0.5)
    scale, one scale vector per (KV, layer, head) slab.
    """
    rng = np.random.default_rng(seed)
    x = _student_t_slabs(rng, (2, GPT2_L, GPT2_H), GPT2_T)
    return x.reshape(-1, D).astype(np.float16)


def gpt2_small_queries(seed: int = 112) -> np.ndarray:
    """One decode query per (layer, head) of the GPT-2-small-shaped cache: fp16 [12, 12, 64] ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((GPT2_L, GPT2_H, D)).astype(np.float16)


def tinyllama_kv(seed: int = 103, outlier_p: float = 0.01, outlier_scale: float = 20.0) -> np.ndarray:
    """TinyLlama-1.1B-shaped KV vectors, fp16 [5767168, 64].

    Layout [22 layers][4 KV heads][2 KV][8 batch][4096 tokens][64], N(0,1) values.
    Each channel of each (layer, head, KV) slab is an outlier channel with
    probability ``outlier_p``; outlier channels are multiplied by ``outlier_scale``.
    """
    rng = np.random.default_rng(seed)
    mask = rng.random((22, 4, 2, D)) < outlier_p
    x = rng.standard_normal((22, 4, 2, 8 * 4096, D))
    mult = np.where(mask, outlier_scale, 1.0)
    x *= mult[:, :, :, None, :]
    return x.reshape(-1, D).astype(np.float16)


def fullvec_kv(seed: int = 104) -> np.ndarray:
    """Sub-one-bit workload, fp16 [1048576, 64]: 1024 slabs of 1024 tokens,
    Student-t(4) values times one lognormal(0, 0.5) channel-scale vector per slab."""
    rng = np.random.default_rng(seed)
    x = _student_t_slabs(rng, (1024,), 1024)
    return x.reshape(-1, D).astype(np.float16)


def attention_inputs(seed: int = 105, B: int = ATTN_B, Hq: int = ATTN_HQ, Hkv: int = ATTN_HKV, T: int = ATTN_T):
    """Decode-attention workload.

    Returns (q, kv): q fp16 [B, Hq, 64] ~ N(0,1); kv fp16 [2, B, Hkv, T, 64] with
    kv[0] the keys and kv[1] the values, drawn like :func:`gpt2_small_kv` with one
    channel-scale vector per (KV, batch, KV head) slab.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    kv = _student_t_slabs(rng, (2, B, Hkv), T).astype(np.float16)
    return q, kv


def random_code_store(nbytes: int, seed: int) -> np.ndarray:
    """Uniform random bytes.  Any bit pattern is a valid fixed-rate code store
    (every code value in [0, N) is a valid index), so this is a uniform random
    choice of codes for every block."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=nbytes, dtype=np.uint8)


def random_norms(n: int, seed: int, dtype=np.float16) -> np.ndarray:
    """Positive norms with the spread of the Student-t workloads: 8 * exp(0.5 z)."""
    rng = np.random.default_rng(seed)
    return (8.0 * np.exp(0.5 * rng.standard_normal(n))).astype(dtype)


def canonical_blocks(d: int, k: int, m: int, seed: int) -> np.ndarray:
    """Training blocks for the codebook construction: the first k coordinates of m
    points uniform on the unit sphere S^{d-1}, drawn as normalised standard
    Gaussian d-vectors (fp64 [m, k]).  A draw of the source, not a step of the
    codec."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((m, d))
    g /= np.sqrt(np.sum(g * g, axis=1, keepdims=True))
    return g[:, :k].copy()
