"""Every matrix-core encoder, forced at load time (FQ_ENCODE_KERNEL), on the edge
cases of the nearest-codeword search (FibQuant summary §2.3 encoder; readings: the
lowest index on exact ties, ν = 0 gives the smallest-norm codes, fp16 overflow of
the norm stores +inf).  Each case asserts which kernel ran (fq_encode_kernel) and
meets the codec bar: codes equal the oracle's outside its near-ties and are
accepted inside them, norms bit-exact."""
import os

import numpy as np
import pytest

import universal_vector_quantization_amd as fq
import workloads
from oracle import codec as oc

from gpu_util import D, artifact_or_skip, check_encode, device, gpu_encode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _forced(cw, rot, kernel):
    os.environ["FQ_ENCODE_KERNEL"] = kernel
    try:
        return fq.Codebook(cw, rot)
    finally:
        del os.environ["FQ_ENCODE_KERNEL"]


def _tie_codebook(k, N, seed):
    # fp16-exact normal-or-zero codewords at the scale of a unit vector's k-block; codewords
    # 3 and 5 are negatives of each other and the two shortest, so a zero vector (every
    # block at distance ||c_3||^2 from both) is an exact tie the search must settle as 3
    rng = np.random.default_rng(seed)
    c = (rng.standard_normal((N, k)) * np.sqrt(1.0 / D) * 1.2).astype(np.float16).astype(np.float32)
    c[np.abs(c) < 2.0 ** -14] = 0.0
    c[3] = (c[3] * np.float32(2.0 ** -6)).astype(np.float16).astype(np.float32)
    c[3][np.abs(c[3]) < 2.0 ** -14] = 0.0
    if np.abs(c[3]).max() == 0:
        c[3, 0] = 2.0 ** -10
    c[5] = -c[3]
    assert len(np.unique(c, axis=0)) == N
    return c


def _edge_inputs(n_plain, seed):
    """Workload vectors with, interleaved: zero vectors, vectors whose norm overflows
    fp16 (stored +inf), vectors of fp16 subnormals only, and vectors mixing subnormal
    and normal coordinates."""
    x = workloads.gpt2_small_kv()[seed * 1000: seed * 1000 + n_plain].copy()
    rng = np.random.default_rng(seed)
    x[3::11] = np.float16(10000.0) * np.sign(rng.standard_normal((len(x[3::11]), D))).astype(np.float16)
    sub = (rng.integers(1, 1024, size=(len(x[5::13]), D)) * rng.choice([-1, 1], size=(len(x[5::13]), D)))
    x[5::13] = (sub * 2.0 ** -24).astype(np.float16)  # every coordinate an fp16 subnormal
    mix = x[9::17].astype(np.float32)
    mix[:, ::3] = (rng.integers(1, 1024, size=mix[:, ::3].shape) * 2.0 ** -24)
    x[9::17] = mix.astype(np.float16)
    x[::7] = 0  # last, so that every 7th vector is zero
    return x


CASES = [("h16", 4, 32), ("h16", 4, 256), ("h16", 4, 2048), ("h16", 4, 4096),  # 4096: codebook streamed
         ("h16", 8, 32), ("h16", 8, 64), ("h16", 8, 512), ("h16", 8, 2048), ("h16", 8, 4096),
         ("mfma", 4, 32), ("mfma", 4, 1024), ("mfma", 8, 32), ("mfma", 8, 4096),
         ("full", 64, 32), ("full", 64, 4096),
         ("full", 32, 32), ("full", 32, 512), ("full", 32, 2048),    # two blocks per vector
         ("full", 16, 32), ("full", 16, 1024), ("full", 16, 4096),   # four blocks, two codebook passes
         ("valu", 4, 256), ("small", 8, 512)]
NAMES = {"h16": "encode_h16", "mfma": "encode_mfma", "full": "encode_full", "valu": "encode_valu",
         "small": "encode_wave"}


@pytest.mark.parametrize("kernel,k,N", CASES)
def test_forced_encoder_ties_zeros_overflow_subnormals(dev, kernel, k, N):
    _, rot = artifact_or_skip(4, 256)
    cw = _tie_codebook(k, N, 7000 + 10 * k + N)
    cb = _forced(cw, rot, kernel)
    for n in (1, 37, 700 + 9):
        x = _edge_inputs(n, 3)
        for dt in ((np.float16, np.float32) if kernel in ("mfma", "valu") else (np.float16,)):
            xs = x.astype(dt)
            xd = fq.FQ_F16 if dt == np.float16 else fq.FQ_F32
            assert fq.fq_encode_kernel(cb.handle, xd, n) == NAMES[kernel]
            print(f"[{NAMES[kernel]}] k={k} N={N} n={n} x={np.dtype(dt).name}", flush=True)
            with np.errstate(over="ignore"):
                gc, gn = gpu_encode(cb, xs, dev, np.float16)
                check_encode(xs, rot, cw, gc, gn, np.float16, k, N)
            g = oc.unpack_codes(gc, n, D // k, oc.code_bits(N))
            assert (g[::7] == 3).all(), "zero vectors must take the lower of the two tied codewords"
            if n > 3:
                assert np.isinf(gn[3]) and gn[3] > 0
    cb.close()


@pytest.mark.parametrize("kernel,k,N", [("h16", 4, 256), ("h16", 8, 4096), ("mfma", 8, 4096), ("full", 64, 4096)])
def test_forced_encoder_workload_codebook_many_groups(dev, kernel, k, N):
    # the frozen workload codebooks over enough vectors that every wave of the persistent
    # grid sees several groups, with a ragged tail
    cw, rot = artifact_or_skip(k, N)
    cb = _forced(cw, rot, kernel)
    x = {4: workloads.gpt2_small_kv, 8: workloads.tinyllama_kv, 64: workloads.fullvec_kv}[k]()
    m = 40000 + 13 if k == 4 else 3000 + 13  # the oracle's search at N = 4096 takes about 2 ms per vector
    x = x[::max(1, len(x) // m)][:m]
    assert fq.fq_encode_kernel(cb.handle, fq.FQ_F16, len(x)) == NAMES[kernel]
    print(f"[{NAMES[kernel]}] workload codebook k={k} N={N} n={len(x)}", flush=True)
    gc, gn = gpu_encode(cb, x, dev, np.float16)
    check_encode(x, rot, cw, gc, gn, np.float16, k, N)
    cb.close()


def test_automatic_encoder_choice(dev):
    cw, rot = artifact_or_skip(4, 256)
    cb = fq.Codebook(cw, rot)
    assert fq.fq_encode_kernel(cb.handle, fq.FQ_F16, 2048) == "encode_wave"
    assert fq.fq_encode_kernel(cb.handle, fq.FQ_F16, 2049) == "encode_h16"
    assert fq.fq_encode_kernel(cb.handle, fq.FQ_F32, 2049) == "encode_mfma"
    cb.close()
    cw, rot = artifact_or_skip(64, 4096)
    cb = fq.Codebook(cw, rot)
    assert fq.fq_encode_kernel(cb.handle, fq.FQ_F16, 100000) == "encode_full"
    assert fq.fq_encode_kernel(cb.handle, fq.FQ_F32, 100000) == "encode_valu"
    cb.close()
    for k, N in [(16, 1024), (32, 512)]:
        cw, rot = fq.load_artifact(k, N, initial=True)
        cb = fq.Codebook(cw, rot)
        assert fq.fq_encode_kernel(cb.handle, fq.FQ_F16, 100000) == "encode_full"
        assert fq.fq_encode_kernel(cb.handle, fq.FQ_F32, 100000) == "encode_valu"
        cb.close()
    # a forced kernel that does not cover the call leaves the automatic choice
    cw, rot = artifact_or_skip(4, 256)
    cb = _forced(cw, rot, "full")
    assert fq.fq_encode_kernel(cb.handle, fq.FQ_F16, 100000) == "encode_h16"
    cb.close()


def test_streamed_codebook_many_rounds_sampled(dev):
    # k = 4, N = 16384 (the b = 3.5 rate-axis codebook, 256 KiB of records): the fp16
    # encoder streams it through LDS; 100,013 vectors give every workgroup several
    # rounds; sampled vectors (both ends and random ones) against the oracle
    from gpu_util import unpack_sampled

    try:
        cw, rot = fq.load_artifact(4, 16384, initial=True)
    except FileNotFoundError:
        pytest.skip("rate-axis artifact k=4 N=16384 missing")
    cb = fq.Codebook(cw, rot)
    x = workloads.tinyllama_kv()[: 100_000 + 13]
    n = len(x)
    assert fq.fq_encode_kernel(cb.handle, fq.FQ_F16, n) == "encode_h16"
    print(f"[streamed codebook] k=4 N=16384 n={n}", flush=True)
    gc, gn = gpu_encode(cb, x, dev, np.float16)
    rng = np.random.default_rng(8)
    idx = np.unique(np.concatenate([rng.choice(n, 600, replace=False), np.arange(16), np.arange(n - 16, n)]))
    g = unpack_sampled(gc, idx, 16, 14)
    enc = oc.encode(x[idx], rot, cw, np.float16)
    assert not ((g != enc.codes) & ~enc.near_tie).any()
    assert oc.accepted(enc.y, cw, enc, g).all()
    assert np.array_equal(gn[idx].view(np.uint16), enc.norms.view(np.uint16))
    cb.close()


@pytest.mark.parametrize("k,N", [(16, 1024), (32, 512)])
def test_block_encoder_many_rounds_sampled(dev, k, N):
    # the rate-axis codebooks of k = 16 and 32 on the matrix core: 100,013 vectors give
    # every workgroup several rounds; sampled vectors (both ends and random ones) against
    # the oracle
    from gpu_util import unpack_sampled

    cw, rot = fq.load_artifact(k, N, initial=True)
    cb = fq.Codebook(cw, rot)
    x = workloads.gpt2_small_kv()[: 100_000 + 13]
    n = len(x)
    assert fq.fq_encode_kernel(cb.handle, fq.FQ_F16, n) == "encode_full"
    print(f"[block encoder] k={k} N={N} n={n}", flush=True)
    gc, gn = gpu_encode(cb, x, dev, np.float16)
    rng = np.random.default_rng(9 + k)
    idx = np.unique(np.concatenate([rng.choice(n, 1500, replace=False), np.arange(40), np.arange(n - 40, n)]))
    g = unpack_sampled(gc, idx, D // k, oc.code_bits(N))
    enc = oc.encode(x[idx], rot, cw, np.float16)
    assert not ((g != enc.codes) & ~enc.near_tie).any()
    assert oc.accepted(enc.y, cw, enc, g).all()
    assert np.array_equal(gn[idx].view(np.uint16), enc.norms.view(np.uint16))
    cb.close()
