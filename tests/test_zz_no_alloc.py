"""fq_attn_decode_noalloc (the decode-attention entry point that allocates nothing:
its workspace is the library's fixed per-device buffer) through the C ABI, against
the entry points that take a caller's workspace: the same results on calls in a
row, each smaller than the one before, on the buffer the previous call left
behind; sizes past the buffer are refused before any launch."""
import numpy as np
import pytest

import universal_vector_quantization_amd as fq
import workloads

from gpu_util import D, artifact_or_skip, device, max_rel_rows, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def dev():
    return device()


def _cache(cb, B, Hkv, T, seed):
    n = B * Hkv * T
    nb = cb.code_bytes(n)
    return (workloads.random_code_store(nb, seed), workloads.random_norms(n, seed + 1),
            workloads.random_code_store(nb, seed + 2), workloads.random_norms(n, seed + 3))


def _pair(cb, dev, B, Hq, Hkv, T, seed, lens=None):
    """(no-allocation output, caller-workspace output) for one random cache."""
    import torch

    kc, kn, vc, vn = (to_dev(a, dev) for a in _cache(cb, B, Hkv, T, seed))
    q = to_dev(np.random.default_rng(seed).standard_normal((B, Hq, D)).astype(np.float16), dev)
    ln = None if lens is None else to_dev(np.asarray(lens, dtype=np.int32), dev)
    a = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    b = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    print(f"[no-alloc attention] k={cb.k} N={cb.N} B={B} Hq={Hq} Hkv={Hkv} T={T} lens={lens is not None}",
          flush=True)
    fq.fq_attn_decode_noalloc(cb.handle, q, kc, kn, vc, vn, B, Hq, Hkv, T, 0.125, a, lens=ln)
    ws = torch.empty(max(fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T), 16), dtype=torch.uint8, device=dev)
    if lens is None:
        fq.fq_attn_decode(cb.handle, q, kc, kn, vc, vn, B, Hq, Hkv, T, 0.125, b, ws)
    else:
        fq.fq_attn_decode_varlen(cb.handle, q, kc, kn, vc, vn, ln, B, Hq, Hkv, T, 0.125, b, ws)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_matches_workspace_entry_points_on_successive_calls(dev):
    assert fq.fq_attn_noalloc_max_workspace_bytes() == 16 << 20
    cw, rot = artifact_or_skip(4, 256)
    cb = fq.Codebook(cw, rot)
    # 1: the k = 4, 8-bit fast kernel, all keys
    a, b = _pair(cb, dev, 4, 32, 4, 8192, 11)
    assert np.isfinite(a).all() and max_rel_rows(a, b) <= TOL and np.array_equal(a, b)
    # 2: smaller, per-batch lengths (one batch empty), on the buffer call 1 left behind
    a, b = _pair(cb, dev, 3, 16, 2, 1000, 12, lens=[1000, 0, 517])
    assert max_rel_rows(a, b) <= TOL and np.array_equal(a, b)
    assert np.all(a[1] == 0)
    cb.close()
    # 3: smaller again, the general kernel (k = 2, N = 16)
    cw2, rot2 = artifact_or_skip(2, 16)
    cb2 = fq.Codebook(cw2, rot2)
    a, b = _pair(cb2, dev, 2, 8, 2, 700, 13)
    assert np.isfinite(a).all() and max_rel_rows(a, b) <= TOL and np.array_equal(a, b)
    cb2.close()


def test_noalloc_refuses_sizes_past_its_buffer(dev):
    import torch

    cw, rot = artifact_or_skip(4, 256)
    cb = fq.Codebook(cw, rot)
    B, Hq, Hkv, T = 16, 32, 4, 262144  # 69 MB of partial records
    assert fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T) > fq.fq_attn_noalloc_max_workspace_bytes()
    z = torch.zeros(64, dtype=torch.uint8, device=dev)
    q = torch.zeros((B, Hq, D), dtype=torch.float16, device=dev)
    out = torch.full((B, Hq, D), 3.0, dtype=torch.float32, device=dev)
    with pytest.raises(fq.FQError) as e:
        fq.fq_attn_decode_noalloc(cb.handle, q, z, z, z, z, B, Hq, Hkv, T, 0.125, out)
    assert e.value.status == fq.FQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(out.min()) == 3.0  # nothing was launched
    cb.close()
