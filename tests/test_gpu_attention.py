"""GPU parity of fq_attn_decode (decode attention fused with decompression)
against the CPU oracle's dense attention over the fp64-decoded cache.

Bar: per (batch, query head) ||o_gpu - o_ref||_inf <= 1e-3 ||o_ref||_inf."""
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


def _gpu_attn(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale=0.125):
    import torch

    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    wsb = fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    fq.fq_attn_decode(cb.handle, to_dev(q, dev), to_dev(kc, dev), to_dev(kn, dev), to_dev(vc, dev), to_dev(vn, dev),
                      B, Hq, Hkv, T, scale, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _random_cache(B, Hkv, T, seed, m=16, bits=8):
    n = B * Hkv * T
    nbytes = (n * m * bits + 7) // 8
    return (workloads.random_code_store(nbytes, seed), workloads.random_norms(n, seed + 1),
            workloads.random_code_store(nbytes, seed + 2), workloads.random_norms(n, seed + 3))


def _oracle(q, kc, kn, vc, vn, B, Hkv, T, rot, cw, scale=0.125, m=16, bits=8):
    n = B * Hkv * T
    unp = lambda s: oc.unpack_codes(s, n, m, bits).reshape(B, Hkv, T, m)
    return oatt.attention(q, unp(kc), kn.reshape(B, Hkv, T), unp(vc), vn.reshape(B, Hkv, T), rot, cw, scale)


@pytest.mark.parametrize("B,Hq,Hkv,T", [
    (2, 16, 2, 1000),   # GQA 8:1, ragged against the 32-token tiles and the chunks
    (1, 8, 1, 1),       # a single key: the output is that key's value
    (1, 8, 1, 33),
    (3, 12, 12, 257),   # multi-head (group of 1), GPT-2-small-like
    (1, 32, 2, 4096),   # group of 16 (the most the MFMA columns hold)
    (2, 4, 1, 5000),
])
def test_attention_random_cache(dev, cb4, B, Hq, Hkv, T):
    cb, cw, rot = cb4
    kc, kn, vc, vn = _random_cache(B, Hkv, T, 1000 + T)
    q = np.random.default_rng(T).standard_normal((B, Hq, D)).astype(np.float16)
    print(f"[attention parity] B={B} Hq={Hq} Hkv={Hkv} T={T}", flush=True)
    got = _gpu_attn(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T)
    ref = _oracle(q, kc, kn, vc, vn, B, Hkv, T, rot, cw)
    assert max_rel_rows(got, ref) <= TOL


def test_attention_peaked_scores(dev, cb4):
    # Large logits (scale 1.0, big norms): the softmax is nearly one-hot, which
    # stresses the running-max rescaling across tiles and chunks.
    cb, cw, rot = cb4
    B, Hq, Hkv, T = 1, 8, 1, 3000
    kc, kn, vc, vn = _random_cache(B, Hkv, T, 77)
    kn = (kn.astype(np.float32) * 4).astype(np.float16)
    q = (np.random.default_rng(3).standard_normal((B, Hq, D)) * 3).astype(np.float16)
    got = _gpu_attn(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale=1.0)
    ref = _oracle(q, kc, kn, vc, vn, B, Hkv, T, rot, cw, scale=1.0)
    assert max_rel_rows(got, ref) <= TOL


def test_attention_full_size_sampled_heads(dev, cb4):
    # The benchmark's launch: B=16, Hq=32, Hkv=4, T=32768, on a random code store;
    # sampled (batch, KV head) groups checked against the oracle.
    cb, cw, rot = cb4
    B, Hq, Hkv, T = workloads.ATTN_B, workloads.ATTN_HQ, workloads.ATTN_HKV, workloads.ATTN_T
    kc, kn, vc, vn = _random_cache(B, Hkv, T, 4242)
    q = np.random.default_rng(9).standard_normal((B, Hq, D)).astype(np.float16)
    print("[attention full size] B=16 Hq=32 Hkv=4 T=32768", flush=True)
    got = _gpu_attn(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T)
    G = Hq // Hkv
    for b, g in [(0, 0), (7, 3), (15, 1)]:
        idx = np.arange(T) + (b * Hkv + g) * T
        sub = lambda s: oc.pack_codes(unpack_sampled(s, idx, 16, 8), 8)
        ref = oatt.attention(q[b:b + 1, g * G:(g + 1) * G], unpack_sampled(kc, idx, 16, 8).reshape(1, 1, T, 16),
                             kn[idx].reshape(1, 1, T), unpack_sampled(vc, idx, 16, 8).reshape(1, 1, T, 16),
                             vn[idx].reshape(1, 1, T), rot, cw, 0.125)
        assert max_rel_rows(got[b:b + 1, g * G:(g + 1) * G], ref) <= TOL


def test_attention_multi_chunk_workgroups(dev, cb4):
    # B=16, Hkv=4, T=16392: each workgroup of the fast path owns two 512-token
    # chunks and the last chunk holds 8 tokens (three of its four waves see none);
    # sampled (batch, KV head) groups checked against the oracle.
    cb, cw, rot = cb4
    B, Hq, Hkv, T = 16, 32, 4, 16392
    kc, kn, vc, vn = _random_cache(B, Hkv, T, 5151)
    q = np.random.default_rng(12).standard_normal((B, Hq, D)).astype(np.float16)
    print("[attention multi-chunk] B=16 Hq=32 Hkv=4 T=16392", flush=True)
    got = _gpu_attn(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T)
    G = Hq // Hkv
    for b, g in [(0, 0), (9, 2), (15, 3)]:
        idx = np.arange(T) + (b * Hkv + g) * T
        ref = oatt.attention(q[b:b + 1, g * G:(g + 1) * G], unpack_sampled(kc, idx, 16, 8).reshape(1, 1, T, 16),
                             kn[idx].reshape(1, 1, T), unpack_sampled(vc, idx, 16, 8).reshape(1, 1, T, 16),
                             vn[idx].reshape(1, 1, T), rot, cw, 0.125)
        assert max_rel_rows(got[b:b + 1, g * G:(g + 1) * G], ref) <= TOL


def test_attention_on_oracle_encoded_cache(dev, cb4):
    # Keys and values are real encodes (by the oracle) of the attention workload's
    # first (batch, KV head) slab, truncated to 4096 tokens.
    cb, cw, rot = cb4
    q, kv = workloads.attention_inputs(T=4096, B=1, Hkv=1, Hq=8)
    ke = oc.encode(kv[0, 0, 0], rot, cw, np.float16)
    ve = oc.encode(kv[1, 0, 0], rot, cw, np.float16)
    kc, vc = oc.pack_codes(ke.codes, 8), oc.pack_codes(ve.codes, 8)
    got = _gpu_attn(cb, dev, q, kc, ke.norms, vc, ve.norms, 1, 8, 1, 4096)
    ref = oatt.attention(q, ke.codes.reshape(1, 1, 4096, 16), ke.norms.reshape(1, 1, 4096),
                         ve.codes.reshape(1, 1, 4096, 16), ve.norms.reshape(1, 1, 4096), rot, cw, 0.125)
    assert max_rel_rows(got, ref) <= TOL


def test_attention_full_size_oracle_encoded_slabs(dev, cb4):
    # The benchmark's launch (B=16, Hq=32, Hkv=4, T=32768) on the GPU encode of the
    # attention workload's whole K and V draw.  For three (batch, KV head) slabs the
    # oracle encodes all 32,768 keys and values: the GPU's codes must meet the codec
    # bar there, and the attention rows of the slab's 8 query heads must match the
    # oracle's attention over those (accepted) codes.
    import torch

    cb, cw, rot = cb4
    B, Hq, Hkv, T = workloads.ATTN_B, workloads.ATTN_HQ, workloads.ATTN_HKV, workloads.ATTN_T
    G = Hq // Hkv
    q, kv = workloads.attention_inputs()
    n = B * Hkv * T
    print("[attention full size, oracle-encoded slabs] encode K and V on the GPU", flush=True)
    x = torch.from_numpy(kv.reshape(2 * n, D)).to(dev)
    codes = torch.empty(cb.code_bytes(2 * n), dtype=torch.uint8, device=dev)
    norms = torch.empty(2 * n, dtype=torch.float16, device=dev)
    fq.fq_encode(cb.handle, x, codes, norms)
    del x
    half = cb.code_bytes(n)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T), dtype=torch.uint8, device=dev)
    fq.fq_attn_decode(cb.handle, to_dev(q, dev), codes[:half], norms[:n], codes[half:], norms[n:], B, Hq, Hkv, T,
                      0.125, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    del codes, norms, ws
    for b, g in [(0, 0), (6, 2), (15, 3)]:
        idx = np.arange(T) + (b * Hkv + g) * T
        kx, vx = kv[0, b, g], kv[1, b, g]
        kcodes = unpack_sampled(gc[:half], idx, 16, 8)
        vcodes = unpack_sampled(gc[half:], idx, 16, 8)
        print(f"[attention full size, oracle-encoded slabs] oracle encode of slab b={b} g={g}", flush=True)
        for xx, cc, nn in ((kx, kcodes, gn[:n][idx]), (vx, vcodes, gn[n:][idx])):
            enc = oc.encode(xx, rot, cw, np.float16)
            mism = cc != enc.codes
            assert not (mism & ~enc.near_tie).any()
            assert oc.accepted(enc.y, cw, enc, cc).all()
            assert np.array_equal(nn.view(np.uint16), enc.norms.view(np.uint16))
        ref = oatt.attention(q[b:b + 1, g * G:(g + 1) * G], kcodes.reshape(1, 1, T, 16),
                             gn[:n][idx].reshape(1, 1, T), vcodes.reshape(1, 1, T, 16),
                             gn[n:][idx].reshape(1, 1, T), rot, cw, 0.125)
        assert max_rel_rows(got[b:b + 1, g * G:(g + 1) * G], ref) <= TOL


def test_attention_deterministic_and_workspace_errors(dev, cb4):
    import torch

    cb, cw, rot = cb4
    B, Hq, Hkv, T = 2, 16, 2, 2000
    kc, kn, vc, vn = _random_cache(B, Hkv, T, 31)
    q = np.random.default_rng(4).standard_normal((B, Hq, D)).astype(np.float16)
    a = _gpu_attn(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T)
    b = _gpu_attn(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    need = fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T)
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device=dev)
    small = torch.empty(need - 4, dtype=torch.uint8, device=dev)
    with pytest.raises(fq.FQError) as e:
        fq.fq_attn_decode(cb.handle, to_dev(q, dev), to_dev(kc, dev), to_dev(kn, dev), to_dev(vc, dev),
                          to_dev(vn, dev), B, Hq, Hkv, T, 0.125, out, small)
    assert e.value.status == fq.FQ_ERR_WORKSPACE
    with pytest.raises(fq.FQError) as e:  # group of 32 query heads per KV head is beyond the kernel
        fq.fq_attn_decode(cb.handle, to_dev(np.zeros((1, 32, D), np.float16), dev), to_dev(kc, dev),
                          to_dev(kn, dev), to_dev(vc, dev), to_dev(vn, dev), 1, 32, 1, 10, 0.125,
                          torch.zeros((1, 32, D), dtype=torch.float32, device=dev), small)
    assert e.value.status == fq.FQ_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert float(out.abs().sum()) == 0.0  # nothing was launched


def test_attention_T0_is_noop(dev, cb4):
    import torch

    cb, _, _ = cb4
    out = torch.full((1, 8, D), 7.0, dtype=torch.float32, device=dev)
    q = torch.zeros((1, 8, D), dtype=torch.float16, device=dev)
    L = fq.lib()
    assert L.fq_attn_decode(cb.handle, q.data_ptr(), None, None, None, None, 1, 8, 1, 0, 0.125, out.data_ptr(),
                            None, 0, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert float(out.min()) == 7.0
