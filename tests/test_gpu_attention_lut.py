"""GPU parity of decode attention for the full-vector code (FibQuant summary §5:
decompression fused into attention; for k = d a key's score is nu_j times one
entry (Pi q) . c_n) against the CPU oracle's dense attention over the
fp64-decoded cache.

Two kernels serve k = d: per-head lookup tables with LDS histograms of the value
weights, and the general kernel gathering codewords from the codebook in global
memory; the library picks one by shape, and FQ_ATTN_KERNEL=lut / gather at load
time forces it, so every case here runs through both.  FQ_ATTN_KERNEL=lut also
takes the k = 4, N = 256 code through the tables (the head-to-head comparison
with the gather kernel).
Bar: per (batch, query head) ||o_gpu - o_ref||_inf <= 1e-3 ||o_ref||_inf."""
import os

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


_cbs = {}


def codebook(k, N, initial=False, kernel=None):
    """kernel: None (the library's choice), "lut" or "gather" (forced at load time)."""
    key = (k, N, initial, kernel)
    if key not in _cbs:
        if initial:
            try:
                cw, rot = fq.load_artifact(k, N, initial=True)
            except FileNotFoundError:
                pytest.skip(f"artifact k={k} N={N} missing")
        else:
            cw, rot = artifact_or_skip(k, N)
        if kernel:
            os.environ["FQ_ATTN_KERNEL"] = kernel
        try:
            _cbs[key] = (fq.Codebook(cw, rot), cw, rot)
        finally:
            os.environ.pop("FQ_ATTN_KERNEL", None)
    return _cbs[key]


KERNELS = ["lut", "gather"]


def _cache(cb, B, Hkv, T, seed):
    n = B * Hkv * T
    nb = cb.code_bytes(n)
    B_bits = (D // cb.k) * cb.bits
    kc, vc = workloads.random_code_store(nb, seed), workloads.random_code_store(nb, seed + 2)
    if (n * B_bits) % 8:  # pad bits of the store are zero
        for s in (kc, vc):
            s[-1] &= (1 << ((n * B_bits) % 8)) - 1
    return kc, workloads.random_norms(n, seed + 1), vc, workloads.random_norms(n, seed + 3)


def _run(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale=0.125, lens=None):
    import torch

    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T), 16), dtype=torch.uint8, device=dev)
    args = (cb.handle, to_dev(q, dev), to_dev(kc, dev), to_dev(kn, dev), to_dev(vc, dev), to_dev(vn, dev))
    if lens is None:
        fq.fq_attn_decode(*args, B, Hq, Hkv, T, scale, out, ws)
    else:
        fq.fq_attn_decode_varlen(*args, to_dev(np.asarray(lens, np.int32), dev), B, Hq, Hkv, T, scale, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(cb, rot, cw, q, kc, kn, vc, vn, B, Hkv, T, scale=0.125, lens=None):
    n = B * Hkv * T
    m, bits = D // cb.k, cb.bits
    unp = lambda s: oc.unpack_codes(s, n, m, bits).reshape(B, Hkv, T, m)
    return oatt.attention(q, unp(kc), kn.reshape(B, Hkv, T), unp(vc), vn.reshape(B, Hkv, T), rot, cw, scale,
                          lengths=lens)


@pytest.mark.parametrize("B,Hq,Hkv,T", [
    (2, 16, 2, 1000),   # GQA 8:1 (two sets of 4 heads per KV head), ragged
    (1, 8, 1, 1),       # one key: the output is that key's value
    (1, 8, 1, 65),
    (3, 12, 12, 257),   # multi-head (group of 1)
    (1, 32, 2, 3000),   # group of 16
    (2, 6, 2, 700),     # group of 3: sets of one head
])
@pytest.mark.parametrize("kernel", KERNELS)
def test_full_vector_attention(dev, B, Hq, Hkv, T, kernel):
    cb, cw, rot = codebook(64, 4096, kernel=kernel)
    kc, kn, vc, vn = _cache(cb, B, Hkv, T, 3000 + T)
    q = np.random.default_rng(T + 1).standard_normal((B, Hq, D)).astype(np.float16)
    print(f"[full-vector attention, {kernel}] k=64 N=4096 B={B} Hq={Hq} Hkv={Hkv} T={T}", flush=True)
    got = _run(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T)
    ref = _oracle(cb, rot, cw, q, kc, kn, vc, vn, B, Hkv, T)
    assert max_rel_rows(got, ref) <= TOL


@pytest.mark.parametrize("kernel", KERNELS)
def test_full_vector_attention_34x_point(dev, kernel):
    # k = d, N = 16384: 14-bit records; the tables take one head per workgroup (64 KiB)
    cb, cw, rot = codebook(64, 16384, initial=True, kernel=kernel)
    B, Hq, Hkv, T = 2, 8, 2, 1500
    kc, kn, vc, vn = _cache(cb, B, Hkv, T, 41)
    q = np.random.default_rng(5).standard_normal((B, Hq, D)).astype(np.float16)
    got = _run(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T)
    ref = _oracle(cb, rot, cw, q, kc, kn, vc, vn, B, Hkv, T)
    assert max_rel_rows(got, ref) <= TOL


@pytest.mark.parametrize("kernel", KERNELS)
def test_full_vector_attention_peaked_scores_and_lengths(dev, kernel):
    # large logits (scale 1, norms x4): a nearly one-hot softmax; per-batch lengths
    # including an empty batch and one key
    cb, cw, rot = codebook(64, 4096, kernel=kernel)
    B, Hq, Hkv, T = 4, 16, 2, 2000
    kc, kn, vc, vn = _cache(cb, B, Hkv, T, 51)
    kn = (kn.astype(np.float32) * 4).astype(np.float16)
    q = (np.random.default_rng(6).standard_normal((B, Hq, D)) * 3).astype(np.float16)
    lens = [2000, 0, 1, 1234]
    got = _run(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T, scale=1.0, lens=lens)
    ref = _oracle(cb, rot, cw, q, kc, kn, vc, vn, B, Hkv, T, scale=1.0, lens=lens)
    assert np.all(got[1] == 0)
    assert max_rel_rows(got, ref) <= TOL


@pytest.mark.parametrize("kernel", [None, "gather"])
def test_full_vector_attention_full_size_sampled(dev, kernel):
    # the attention workload's shape (B=16, Hq=32, Hkv=4, T=32768) on the full-vector
    # code (the library's choice there: the tables): GPU encode of the workload's K
    # and V draws, three slabs checked
    import torch

    cb, cw, rot = codebook(64, 4096, kernel=kernel)
    B, Hq, Hkv, T = workloads.ATTN_B, workloads.ATTN_HQ, workloads.ATTN_HKV, workloads.ATTN_T
    G = Hq // Hkv
    q, kv = workloads.attention_inputs()
    n = B * Hkv * T
    x = torch.from_numpy(kv.reshape(2 * n, D)).to(dev)
    codes = torch.zeros(cb.code_bytes(2 * n), dtype=torch.uint8, device=dev)
    norms = torch.empty(2 * n, dtype=torch.float16, device=dev)
    fq.fq_encode(cb.handle, x, codes, norms)
    del x
    half = cb.code_bytes(n)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T), dtype=torch.uint8, device=dev)
    print(f"[full-vector attention full size, {kernel or 'auto'}] B=16 Hq=32 Hkv=4 T=32768 k=64 N=4096", flush=True)
    fq.fq_attn_decode(cb.handle, to_dev(q, dev), codes[:half], norms[:n], codes[half:], norms[n:], B, Hq, Hkv, T,
                      0.125, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    for b, g in [(0, 0), (9, 1), (15, 3)]:
        idx = np.arange(T) + (b * Hkv + g) * T
        kcod = unpack_sampled(gc[:half], idx, 1, 12)
        vcod = unpack_sampled(gc[half:], idx, 1, 12)
        ref = oatt.attention(q[b:b + 1, g * G:(g + 1) * G], kcod.reshape(1, 1, T, 1), gn[:n][idx].reshape(1, 1, T),
                             vcod.reshape(1, 1, T, 1), gn[n:][idx].reshape(1, 1, T), rot, cw, 0.125)
        assert max_rel_rows(got[b:b + 1, g * G:(g + 1) * G], ref) <= TOL


@pytest.mark.parametrize("B,Hq,Hkv,T", [(2, 16, 2, 1000), (1, 4, 1, 33)])
def test_lut_attention_forced_for_k4(dev, B, Hq, Hkv, T):
    cb, cw, rot = codebook(4, 256, kernel="lut")
    kc, kn, vc, vn = _cache(cb, B, Hkv, T, 61 + T)
    q = np.random.default_rng(7).standard_normal((B, Hq, D)).astype(np.float16)
    got = _run(cb, dev, q, kc, kn, vc, vn, B, Hq, Hkv, T)
    ref = _oracle(cb, rot, cw, q, kc, kn, vc, vn, B, Hkv, T)
    assert max_rel_rows(got, ref) <= TOL
