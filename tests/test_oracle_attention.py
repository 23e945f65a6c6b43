"""Pins for the oracle's dense decode attention over a decoded cache
(FibQuant summary §5: fixed addresses let decompression fuse into attention)."""
import math

import numpy as np

from oracle.attention import attention
from oracle.codec import decode
from oracle.codebook import initial_codebook, to_fp16_grid
from oracle.rotation import shared_rotation

D = 64
PI = shared_rotation(64, 0)
CB = to_fp16_grid(initial_codebook(D, 4, 16))


def _rand_cache(rng, B, Hkv, T, N=16, m=16):
    kc = rng.integers(0, N, size=(B, Hkv, T, m))
    vc = rng.integers(0, N, size=(B, Hkv, T, m))
    kn = (rng.uniform(0.5, 10, size=(B, Hkv, T))).astype(np.float16)
    vn = (rng.uniform(0.5, 10, size=(B, Hkv, T))).astype(np.float16)
    return kc, kn, vc, vn


def test_score_identity_rotated_query():
    # q·k̂_j = ν_j (Π q)·ĉ_j: scoring straight from the codes.
    rng = np.random.default_rng(1)
    q = rng.standard_normal(D)
    codes = rng.integers(0, 16, size=(20, 16))
    nus = rng.uniform(0.5, 5, size=20)
    khat = decode(codes, nus, PI, CB)
    qt = PI.astype(np.float64) @ q
    chat = CB.astype(np.float64)[codes].reshape(20, D)
    assert np.max(np.abs(khat @ q - nus * (chat @ qt))) < 1e-12


def test_single_token_returns_its_value():
    rng = np.random.default_rng(2)
    kc, kn, vc, vn = _rand_cache(rng, 1, 1, 1)
    q = rng.standard_normal((1, 2, D)).astype(np.float16)
    out = attention(q, kc, kn, vc, vn, PI, CB, 0.125)
    v0 = decode(vc[0, 0], vn[0, 0], PI, CB)[0]
    assert np.array_equal(out[0, 0], v0) and np.array_equal(out[0, 1], v0)


def test_equal_keys_give_mean_value():
    rng = np.random.default_rng(3)
    kc, kn, vc, vn = _rand_cache(rng, 1, 1, 9)
    kc[:] = kc[:, :, :1]
    kn[:] = kn[:, :, :1]
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    out = attention(q, kc, kn, vc, vn, PI, CB, 0.125)
    assert np.allclose(out[0, 0], decode(vc[0, 0], vn[0, 0], PI, CB).mean(axis=0), atol=1e-13)


def test_zero_query_uniform_average():
    rng = np.random.default_rng(4)
    kc, kn, vc, vn = _rand_cache(rng, 1, 1, 7)
    q = np.zeros((1, 1, D), dtype=np.float16)
    out = attention(q, kc, kn, vc, vn, PI, CB, 0.125)
    assert np.allclose(out[0, 0], decode(vc[0, 0], vn[0, 0], PI, CB).mean(axis=0), atol=1e-13)


def test_against_pure_python_loops_with_grouping():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, T = 2, 4, 2, 5
    kc, kn, vc, vn = _rand_cache(rng, B, Hkv, T)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    out = attention(q, kc, kn, vc, vn, PI, CB, 0.125)
    pi = PI.astype(np.float64)
    cb = CB.astype(np.float64)

    def dec(codes, nu):
        yh = [float(cb[codes[j // 4], j % 4]) for j in range(D)]
        return [float(nu) * math.fsum(pi[r, i] * yh[r] for r in range(D)) for i in range(D)]

    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            ks = [dec(kc[b, g, t], kn[b, g, t]) for t in range(T)]
            vs = [dec(vc[b, g, t], vn[b, g, t]) for t in range(T)]
            s = [0.125 * math.fsum(float(q[b, h, i]) * ks[t][i] for i in range(D)) for t in range(T)]
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            z = math.fsum(e)
            ref = [math.fsum(e[t] / z * vs[t][i] for t in range(T)) for i in range(D)]
            assert np.max(np.abs(out[b, h] - np.array(ref))) < 1e-11


# ------------------------------------------------------------------ growing cache (per-batch lengths)
def _python_attention_row(q, kc, kn, vc, vn, L, scale=0.125):
    """Pure-Python loops over the first L keys of one (batch, KV head) slab; 0 when L = 0."""
    if L == 0:
        return [0.0] * D
    pi = PI.astype(np.float64)
    cb = CB.astype(np.float64)

    def dec(codes, nu):
        yh = [float(cb[codes[j // 4], j % 4]) for j in range(D)]
        return [float(nu) * math.fsum(pi[r, i] * yh[r] for r in range(D)) for i in range(D)]

    ks = [dec(kc[t], kn[t]) for t in range(L)]
    vs = [dec(vc[t], vn[t]) for t in range(L)]
    s = [scale * math.fsum(float(q[i]) * ks[t][i] for i in range(D)) for t in range(L)]
    mx = max(s)
    e = [math.exp(v - mx) for v in s]
    z = math.fsum(e)
    return [math.fsum(e[t] / z * vs[t][i] for t in range(L)) for i in range(D)]


def test_lengths_against_pure_python_loops():
    # Each batch sees only its first L_b keys; keys past L_b carry values that would
    # change the result if they were read (huge norms).
    rng = np.random.default_rng(6)
    B, Hq, Hkv, T = 4, 4, 2, 6
    kc, kn, vc, vn = _rand_cache(rng, B, Hkv, T)
    lengths = np.array([0, 1, 4, 6])
    for b in range(B):
        kn[b, :, lengths[b]:] = 60000.0
        vn[b, :, lengths[b]:] = 60000.0
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    out = attention(q, kc, kn, vc, vn, PI, CB, 0.125, lengths=lengths)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            ref = _python_attention_row(q[b, h], kc[b, g], kn[b, g], vc[b, g], vn[b, g], int(lengths[b]))
            assert np.max(np.abs(out[b, h] - np.array(ref))) < 1e-11
    assert np.all(out[0] == 0.0)


def test_lengths_clamp_and_full_length_is_the_plain_call():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, T = 3, 2, 1, 5
    kc, kn, vc, vn = _rand_cache(rng, B, Hkv, T)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    full = attention(q, kc, kn, vc, vn, PI, CB, 0.125)
    assert np.array_equal(attention(q, kc, kn, vc, vn, PI, CB, 0.125, lengths=[T, T + 9, 10 ** 6]), full)
    neg = attention(q, kc, kn, vc, vn, PI, CB, 0.125, lengths=[-4, 0, T])
    assert np.all(neg[:2] == 0.0) and np.array_equal(neg[2], full[2])
    one = attention(q, kc, kn, vc, vn, PI, CB, 0.125, lengths=[1, 1, 1])
    for b in range(B):  # one key: the output is exactly that key's value
        v0 = decode(vc[b, 0, :1], vn[b, 0, :1], PI, CB)[0]
        assert np.array_equal(one[b, 0], v0) and np.array_equal(one[b, 1], v0)


# ------------------------------------------------------------------ prefill (several queries per head)
def test_prefill_noncausal_is_decode_per_query():
    from oracle.attention import prefill_attention

    rng = np.random.default_rng(8)
    B, Hq, Hkv, T, Sq = 2, 4, 2, 7, 3
    kc, kn, vc, vn = _rand_cache(rng, B, Hkv, T)
    q = rng.standard_normal((B, Hq, Sq, D)).astype(np.float16)
    out = prefill_attention(q, kc, kn, vc, vn, PI, CB, 0.125, causal=False)
    for i in range(Sq):
        assert np.array_equal(out[:, :, i], attention(q[:, :, i], kc, kn, vc, vn, PI, CB, 0.125))


def test_prefill_causal_against_pure_python_loops():
    # query i sees keys 0 .. T - Sq + i; the last query sees every key, Sq = T makes
    # query 0 see only key 0 (its output is exactly that value)
    from oracle.attention import prefill_attention

    rng = np.random.default_rng(9)
    B, Hq, Hkv, T, Sq = 1, 2, 1, 5, 5
    kc, kn, vc, vn = _rand_cache(rng, B, Hkv, T)
    q = rng.standard_normal((B, Hq, Sq, D)).astype(np.float16)
    out = prefill_attention(q, kc, kn, vc, vn, PI, CB, 0.125, causal=True)
    for h in range(Hq):
        for i in range(Sq):
            ref = _python_attention_row(q[0, h, i], kc[0, 0], kn[0, 0], vc[0, 0], vn[0, 0], i + 1)
            assert np.max(np.abs(out[0, h, i] - np.array(ref))) < 1e-11
    v0 = decode(vc[0, 0, :1], vn[0, 0, :1], PI, CB)[0]
    assert np.array_equal(out[0, 0, 0], v0)
    # more queries than keys: the first Sq - T queries see nothing
    out2 = prefill_attention(np.concatenate([q, q], axis=2), kc, kn, vc, vn, PI, CB, 0.125, causal=True)
    assert np.all(out2[:, :, :5] == 0.0) and np.array_equal(out2[:, :, 5:], out)
