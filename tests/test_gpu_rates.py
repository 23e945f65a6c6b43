"""GPU parity along the rate axis (FibQuant summary §2.3: b = log2(N)/k; §3.3 and
§4.1: a dense rate axis, fractional and sub-one-bit rates included): encode,
decode, scattered encode and decode attention at (k, N) points away from the
four workload codebooks, against the CPU oracle.

The codec is exact for any fp16-exact codebook, so these tests use the frozen
rate-axis artifacts: the construction's initial codebooks (companded radii and
spiral / Roberts directions, rounded to the fp16 grid) without the Lloyd
refinement, which changes codeword values, not what the kernels compute.

Bars as for the workload codebooks: codes equal the oracle's outside its
near-ties (accepted codes inside), norms bit-exact, decoded vectors and
attention rows within 1e-3 relative in the max norm."""
import numpy as np
import pytest

import universal_vector_quantization_amd as fq
import workloads
from oracle import attention as oatt
from oracle import codec as oc

from gpu_util import D, check_encode, device, gpu_decode, gpu_encode, max_rel_rows, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-3

# (k, N): rate b = log2(N) / k bits per coordinate
RATES = [
    (1, 16),      # b = 4: the scalar (k = 1) specialisation
    (2, 32),      # b = 2.5
    (2, 128),     # b = 3.5
    (4, 1024),    # b = 2.5
    (4, 16384),   # b = 3.5
    (16, 1024),   # b = 0.625
    (32, 512),    # b = 0.28125
    (64, 16384),  # b = 0.21875: 64 coordinates in 14 bits (+ a 16-bit norm: 34.1x)
]
# every rate-axis point has an attention kernel: the general one holds the fp16 codebook
# in LDS (N k <= 65536 on gfx950) or gathers from global memory, the full-vector code
# goes through lookup tables or the global gathers
ATTN_RATES = RATES


@pytest.fixture(scope="module")
def dev():
    return device()


_cbs = {}


def codebook(k, N):
    if (k, N) not in _cbs:
        try:
            cw, rot = fq.load_artifact(k, N, initial=True)
        except FileNotFoundError:
            pytest.skip(f"rate-axis artifact k={k} N={N} not built")
        _cbs[(k, N)] = (fq.Codebook(cw, rot), cw, rot)
    return _cbs[(k, N)]


def _x(n, dtype, off=3000):
    return workloads.gpt2_small_kv()[off:off + n].astype(dtype)


@pytest.mark.parametrize("k,N", RATES)
@pytest.mark.parametrize("n,dtype", [(131, np.float16), (3001, np.float16), (2085, np.float32)])
def test_encode_rate_axis(dev, k, N, n, dtype):
    # 131 vectors: the small-batch encoder where the shape allows it; 2085 / 3001:
    # the throughput encoders (fp32 / fp16 input)
    if N >= 16384 and n > 1000:
        n = 1007  # the oracle's brute force at N = 16384 dominates the test time
    cb, cw, rot = codebook(k, N)
    x = _x(n, dtype)
    print(f"[rate encode] k={k} N={N} b={np.log2(N) / k:.4g} n={n} x={np.dtype(dtype).name}", flush=True)
    gc, gn = gpu_encode(cb, x, dev, dtype)
    check_encode(x, rot, cw, gc, gn, dtype, k, N)


@pytest.mark.parametrize("k,N", RATES)
def test_decode_rate_axis(dev, k, N):
    # decode of the oracle's codes and norms (ragged: 32 k + 19 vectors)
    cb, cw, rot = codebook(k, N)
    x = _x(1043, np.float16)
    enc = oc.encode(x, rot, cw, np.float16)
    packed = oc.pack_codes(enc.codes, oc.code_bits(N))
    print(f"[rate decode] k={k} N={N}", flush=True)
    got = gpu_decode(cb, packed, enc.norms, dev, np.float16)
    ref = oc.decode(enc.codes, enc.norms, rot, cw)
    assert max_rel_rows(got, ref) <= TOL


@pytest.mark.parametrize("k,N", [(k, N) for k, N in RATES if (D // k) * oc.code_bits(N) % 8 == 0])
def test_scatter_rate_axis(dev, k, N):
    import torch

    cb, cw, rot = codebook(k, N)
    bits, m = oc.code_bits(N), D // k
    cap, n = 997, 200
    x = _x(n, np.float16, off=9000)
    slots = np.random.default_rng(k + N).choice(cap, n, replace=False).astype(np.int64)
    store0 = workloads.random_code_store(cb.code_bytes(cap), 5)
    norms0 = workloads.random_norms(cap, 6)
    codes, norms = to_dev(store0, dev), to_dev(norms0, dev)
    fq.fq_encode_scatter(cb.handle, to_dev(x, dev), to_dev(slots, dev), cap, codes, norms)
    torch.cuda.synchronize()
    got_c = oc.unpack_codes(codes.cpu().numpy(), cap, m, bits)
    enc = oc.encode(x, rot, cw, np.float16)
    exp_c, exp_n = oc.write_records(oc.unpack_codes(store0, cap, m, bits), norms0, enc.codes, enc.norms, slots)
    assert np.array_equal(norms.cpu().numpy().view(np.uint16), exp_n.view(np.uint16))
    assert not ((got_c != exp_c) & ~oc.write_records(np.zeros_like(exp_c, dtype=bool), norms0, enc.near_tie,
                                                       enc.norms, slots)[0]).any()


@pytest.mark.parametrize("k,N", ATTN_RATES)
def test_attention_rate_axis(dev, k, N):
    import torch

    cb, cw, rot = codebook(k, N)
    bits, m = oc.code_bits(N), D // k
    B, Hq, Hkv, T = 2, 8, 2, 333
    n = B * Hkv * T
    nbytes = (n * m * bits + 7) // 8
    kc, vc = workloads.random_code_store(nbytes, 40 + k), workloads.random_code_store(nbytes, 41 + k)
    kn, vn = workloads.random_norms(n, 42), workloads.random_norms(n, 43)
    q = np.random.default_rng(N).standard_normal((B, Hq, D)).astype(np.float16)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T), 16), dtype=torch.uint8, device=dev)
    print(f"[rate attention] k={k} N={N} B={B} Hq={Hq} Hkv={Hkv} T={T}", flush=True)
    fq.fq_attn_decode(cb.handle, to_dev(q, dev), to_dev(kc, dev), to_dev(kn, dev), to_dev(vc, dev), to_dev(vn, dev),
                      B, Hq, Hkv, T, 0.125, out, ws)
    torch.cuda.synchronize()
    unp = lambda s: oc.unpack_codes(s, n, m, bits).reshape(B, Hkv, T, m)
    ref = oatt.attention(q, unp(kc), kn.reshape(B, Hkv, T), unp(vc), vn.reshape(B, Hkv, T), rot, cw, 0.125)
    assert max_rel_rows(out.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("k,N", [(2, 65536), (4, 32768), (8, 16384), (16, 8192), (32, 4096)])
def test_attention_beyond_lds(dev, k, N):
    # Codebooks whose fp16 copy does not fit one workgroup's LDS beside the general
    # kernel's buffers (N k > 65536 on gfx950; k = 4, N = 16384 is the last that does)
    # are gathered from global memory: k = 2 and 4 several codes per 8 dimensions,
    # k = 8, 16 and 32 through the prefetching loop.  Random fp16-exact codebooks;
    # parity against the oracle.
    import torch

    at, _, _ = codebook(4, 16384)
    assert fq.fq_attn_workspace_bytes(at.handle, 1, 8, 1, 4) > 0
    rng = np.random.default_rng(17 + k)
    cw = (rng.standard_normal((N, k)) * 0.15).astype(np.float16).astype(np.float32)
    cw[np.abs(cw) < 2.0 ** -14] = 0.0
    _, rot = fq.load_artifact(4, 256)
    cb = fq.Codebook(cw, rot)
    try:
        bits, m = oc.code_bits(N), D // k
        B, Hq, Hkv, T = 2, 8, 2, 333
        n = B * Hkv * T
        nbytes = (n * m * bits + 7) // 8
        kc, vc = workloads.random_code_store(nbytes, 60 + k), workloads.random_code_store(nbytes, 61 + k)
        kn, vn = workloads.random_norms(n, 62), workloads.random_norms(n, 63)
        q = np.random.default_rng(N + k).standard_normal((B, Hq, D)).astype(np.float16)
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
        ws = torch.empty(fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T), dtype=torch.uint8, device=dev)
        print(f"[attention beyond LDS] k={k} N={N} B={B} Hq={Hq} Hkv={Hkv} T={T}", flush=True)
        fq.fq_attn_decode(cb.handle, to_dev(q, dev), to_dev(kc, dev), to_dev(kn, dev), to_dev(vc, dev),
                          to_dev(vn, dev), B, Hq, Hkv, T, 0.125, out, ws)
        torch.cuda.synchronize()
        unp = lambda s: oc.unpack_codes(s, n, m, bits).reshape(B, Hkv, T, m)
        ref = oatt.attention(q, unp(kc), kn.reshape(B, Hkv, T), unp(vc), vn.reshape(B, Hkv, T), rot, cw, 0.125)
        assert max_rel_rows(out.cpu().numpy(), ref) <= TOL
    finally:
        cb.close()
