"""Shared helpers for the GPU parity tests (device plumbing and comparisons only)."""
import os

import numpy as np
import pytest

import universal_vector_quantization_amd as fq
from oracle import codec as oc

D = 64


def device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(fq.library_path):
        raise RuntimeError("libfq.so missing on a GPU machine: build before testing")
    return torch.device("cuda:0")


def artifact_or_skip(k, N):
    try:
        return fq.load_artifact(k, N)
    except FileNotFoundError:
        pytest.skip(f"codebook artifact k={k} N={N} not built")


def to_dev(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_encode(cb, x_np, dev, norm_dtype):
    import torch

    x = to_dev(x_np, dev)
    n = x_np.shape[0]
    codes = torch.empty(max(cb.code_bytes(n), 1), dtype=torch.uint8, device=dev)
    norms = torch.empty(max(n, 1), dtype=torch.float16 if norm_dtype == np.float16 else torch.float32, device=dev)
    fq.fq_encode(cb.handle, x, codes, norms[:n] if n else norms[:0])
    torch.cuda.synchronize()
    return codes.cpu().numpy()[: cb.code_bytes(n)], norms.cpu().numpy()[:n]


def gpu_decode(cb, codes_np, norms_np, dev, out_dtype):
    import torch

    n = len(norms_np)
    out = torch.empty((n, D), dtype=torch.float16 if out_dtype == np.float16 else torch.float32, device=dev)
    fq.fq_decode(cb.handle, to_dev(codes_np, dev), to_dev(norms_np, dev), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_encode(x_np, rot, cw, gcodes_bytes, gnorms, norm_dtype, k, N):
    """Codes equal the oracle outside near-ties and accepted inside; norms bit-exact.
    Returns (number of near-tie blocks, number of those that differ)."""
    n = x_np.shape[0]
    enc = oc.encode(x_np, rot, cw, norm_dtype)
    g = oc.unpack_codes(gcodes_bytes, n, D // k, oc.code_bits(N))
    mism = g != enc.codes
    assert not (mism & ~enc.near_tie).any(), (
        f"{int((mism & ~enc.near_tie).sum())} non-near-tie blocks differ, first at "
        f"{np.argwhere(mism & ~enc.near_tie)[:5].tolist()}")
    assert oc.accepted(enc.y, cw, enc, g).all()
    assert np.array_equal(gnorms.view(np.uint16 if norm_dtype == np.float16 else np.uint32),
                          enc.norms.view(np.uint16 if norm_dtype == np.float16 else np.uint32)), "norms differ"
    # pad bits of the store are zero
    B = (D // k) * oc.code_bits(N)
    if (n * B) % 8:
        assert gcodes_bytes[-1] >> ((n * B) % 8) == 0
    return int(enc.near_tie.sum()), int(mism.sum())


def max_rel_rows(got, ref):
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows with ref = 0 must match exactly)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    axis = tuple(range(1, ref.ndim))
    den = np.abs(ref).max(axis=axis)
    num = np.abs(got - ref).max(axis=axis)
    zero = den == 0
    assert np.all(num[zero] == 0)
    return float((num[~zero] / den[~zero]).max()) if (~zero).any() else 0.0


def unpack_sampled(store, idx, m, bits):
    """Codes [len(idx), m] of the vectors ``idx`` read from a fixed-address store
    (each vector at bit i*B, LSB-first), touching only their own bytes."""
    B = m * bits
    out = np.empty((len(idx), m), dtype=np.int64)
    w = np.int64(1) << np.arange(bits, dtype=np.int64)
    for r, i in enumerate(idx):
        b0 = (int(i) * B) // 8
        b1 = ((int(i) + 1) * B + 7) // 8
        bitarr = np.unpackbits(store[b0:b1], bitorder="little")
        off = int(i) * B - 8 * b0
        out[r] = (bitarr[off:off + B].reshape(m, bits).astype(np.int64) * w).sum(axis=1)
    return out
