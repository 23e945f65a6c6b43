"""Seeded synthetic inputs: shapes, dtypes, determinism and the stated laws."""
import numpy as np
from scipy import stats

import workloads as w


def test_iid_gaussian():
    x = w.iid_gaussian(4096, 101)
    assert x.shape == (4096, 64) and x.dtype == np.float32
    assert np.array_equal(x, w.iid_gaussian(4096, 101))
    assert stats.kstest(x[:, 0], "norm").pvalue > 1e-3


def test_gpt2_small_kv_shape_and_slab_scales():
    x = w.gpt2_small_kv()
    assert x.shape == (294912, 64) and x.dtype == np.float16
    assert np.array_equal(x[:1000], w.gpt2_small_kv()[:1000])
    slabs = x.astype(np.float64).reshape(2, 12, 12, 1024, 64)
    # one channel-scale vector per slab: channel spreads differ across channels
    # within a slab but are shared by the slab's tokens
    iqr = stats.iqr(slabs[0, 0, 0], axis=0)
    assert iqr.max() / iqr.min() > 2
    assert np.isfinite(x.astype(np.float32)).all()


def test_queries_and_random_stores():
    q = w.gpt2_small_queries()
    assert q.shape == (12, 12, 64) and q.dtype == np.float16
    s = w.random_code_store(1000, 1)
    assert s.dtype == np.uint8 and len(s) == 1000
    nrm = w.random_norms(100, 2)
    assert nrm.dtype == np.float16 and (nrm > 0).all()


def test_workload_table():
    assert w.WORKLOADS["gpt2s_kv"].n == 294912
    assert w.WORKLOADS["tinyllama_kv"].n == 5767168
    assert w.WORKLOADS["fullvec_kv"].n == 1048576
    assert w.WORKLOADS["attn_b16_t32k"].n == 2 * w.ATTN_B * w.ATTN_HKV * w.ATTN_T


def test_canonical_blocks_agree_with_the_oracle_source():
    # two implementations of the same draw (uniform points on the sphere, first k
    # coordinates): the generator here and the oracle's own
    from oracle.source import sample_canonical

    for k in (1, 4, 64):
        a = w.canonical_blocks(64, k, 1000, 7)
        b = sample_canonical(64, k, 1000, np.random.default_rng(7))
        assert a.shape == (1000, k) and np.array_equal(a, b)
    assert np.allclose(np.sum(w.canonical_blocks(64, 64, 10, 1) ** 2, axis=1), 1.0)
