"""GPU parity of fq_attn_prefill (several queries per head over the compressed
cache, FibQuant summary §5) against the oracle's prefill attention.

Bar: per (batch, query head, query) row ||o_gpu - o_ref||_inf <= 1e-3
||o_ref||_inf; rows with no visible key are exactly 0."""
import numpy as np
import pytest

import universal_vector_quantization_amd as fq
import workloads
from oracle import attention as oatt
from oracle import codec as oc

from gpu_util import D, artifact_or_skip, device, max_rel_rows, to_dev, unpack_sampled

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def cb4():
    cw, rot = artifact_or_skip(4, 256)
    return fq.Codebook(cw, rot), cw, rot


def _gpu_prefill(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, Sq, T, causal, scale=0.125):
    import torch

    out = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.float32, device=dev)
    wsb = fq.fq_attn_prefill_workspace_bytes(cb.handle, B, Hq, Hkv, Sq, T)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    fq.fq_attn_prefill(cb.handle, to_dev(q, dev), to_dev(kc, dev), to_dev(kn, dev), to_dev(vc, dev),
                       to_dev(vn, dev), B, Hq, Hkv, Sq, T, causal, scale, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _cache(B, Hkv, T, seed):
    n = B * Hkv * T
    return (workloads.random_code_store(n * 16, seed), workloads.random_norms(n, seed + 1),
            workloads.random_code_store(n * 16, seed + 2), workloads.random_norms(n, seed + 3))


@pytest.mark.parametrize("B,Hq,Hkv,Sq,T,causal", [
    (2, 8, 2, 5, 300, False),
    (2, 8, 2, 5, 300, True),
    (1, 4, 1, 37, 37, True),      # Sq = T: query 0 sees only key 0
    (2, 16, 2, 20, 1000, True),   # 160 rows per slab: workgroups of 64, 64 and 32 rows
    (1, 32, 2, 3, 777, False),    # 16 heads per KV head, 48 rows (one partial workgroup)
    (1, 8, 1, 70, 50, True),      # more queries than keys: the first 20 see nothing
    (3, 12, 12, 1, 129, True),    # one query per head (the decode step as a prefill)
])
def test_prefill_random_cache(dev, cb4, B, Hq, Hkv, Sq, T, causal):
    cb, cw, rot = cb4
    kc, kn, vc, vn = _cache(B, Hkv, T, 600 + T + Sq)
    q = np.random.default_rng(T * 7 + Sq).standard_normal((B, Hq, Sq, D)).astype(np.float16)
    print(f"[prefill parity] B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} T={T} causal={causal}", flush=True)
    got = _gpu_prefill(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, Sq, T, causal)
    n = B * Hkv * T
    unp = lambda s: oc.unpack_codes(s, n, 16, 8).reshape(B, Hkv, T, 16)
    ref = oatt.prefill_attention(q, unp(kc), kn.reshape(B, Hkv, T), unp(vc), vn.reshape(B, Hkv, T), rot, cw, 0.125,
                                 causal)
    assert max_rel_rows(got.reshape(-1, D), ref.reshape(-1, D)) <= TOL


def test_prefill_peaked_scores(dev, cb4):
    # large logits: nearly one-hot rows stress the running max across units and ranges
    cb, cw, rot = cb4
    B, Hq, Hkv, Sq, T = 1, 8, 1, 16, 3000
    kc, kn, vc, vn = _cache(B, Hkv, T, 700)
    kn = (kn.astype(np.float32) * 4).astype(np.float16)
    q = (np.random.default_rng(5).standard_normal((B, Hq, Sq, D)) * 3).astype(np.float16)
    got = _gpu_prefill(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, Sq, T, True, scale=1.0)
    n = B * Hkv * T
    unp = lambda s: oc.unpack_codes(s, n, 16, 8).reshape(B, Hkv, T, 16)
    ref = oatt.prefill_attention(q, unp(kc), kn.reshape(B, Hkv, T), unp(vc), vn.reshape(B, Hkv, T), rot, cw, 1.0,
                                 True)
    assert max_rel_rows(got.reshape(-1, D), ref.reshape(-1, D)) <= TOL


def test_prefill_full_size_sampled(dev, cb4):
    # The benchmark's launch: B=16, Hq=32, Hkv=4, T=32768, 64 causal queries per head
    # (a 64-token chunk appended to a 32k cache); sampled (batch, KV head) groups.
    cb, cw, rot = cb4
    B, Hq, Hkv, T, Sq = 16, 32, 4, 32768, 64
    kc, kn, vc, vn = _cache(B, Hkv, T, 800)
    q = np.random.default_rng(81).standard_normal((B, Hq, Sq, D)).astype(np.float16)
    print("[prefill full size] B=16 Hq=32 Hkv=4 Sq=64 T=32768 causal", flush=True)
    got = _gpu_prefill(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, Sq, T, True)
    G = Hq // Hkv
    for b, g in [(0, 0), (11, 3)]:
        idx = np.arange(T) + (b * Hkv + g) * T
        ref = oatt.prefill_attention(q[b:b + 1, g * G:(g + 1) * G], unpack_sampled(kc, idx, 16, 8).reshape(1, 1, T, 16),
                                     kn[idx].reshape(1, 1, T), unpack_sampled(vc, idx, 16, 8).reshape(1, 1, T, 16),
                                     vn[idx].reshape(1, 1, T), rot, cw, 0.125, True)
        assert max_rel_rows(got[b:b + 1, g * G:(g + 1) * G].reshape(-1, D), ref.reshape(-1, D)) <= TOL


def test_prefill_rejects_other_codebooks(dev):
    import torch

    cw, rot = artifact_or_skip(2, 16)
    cb = fq.Codebook(cw, rot)
    q = torch.zeros((1, 8, 4, D), dtype=torch.float16, device=dev)
    z = torch.zeros(16, dtype=torch.uint8, device=dev)
    out = torch.zeros((1, 8, 4, D), dtype=torch.float32, device=dev)
    with pytest.raises(fq.FQError) as e:
        fq.fq_attn_prefill(cb.handle, q, z, z, z, z, 1, 8, 1, 4, 10, True, 0.125, out, z)
    assert e.value.status == fq.FQ_ERR_UNSUPPORTED
