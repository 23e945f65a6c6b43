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
