"""The C-ABI library loads and exports every entry point include/fq.h declares;
host-side argument checks answer without a GPU (no compute call is made)."""
import ctypes
import os
import re

import numpy as np
import pytest

import universal_vector_quantization_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fq.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fq_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fq.library_path):
        pytest.skip("libfq.so not built")
    return fq.lib()


def test_header_declares_the_boundary():
    assert _declared() == sorted(["fq_attn_decode", "fq_attn_decode_noalloc", "fq_attn_decode_varlen",
                                  "fq_attn_noalloc_max_workspace_bytes", "fq_attn_prefill",
                                  "fq_attn_prefill_workspace_bytes", "fq_attn_workspace_bytes",
                                  "fq_code_bytes", "fq_codebook_free", "fq_codebook_load", "fq_decode",
                                  "fq_codebook_train", "fq_codebook_train_workspace_bytes",
                                  "fq_encode", "fq_encode_kernel", "fq_encode_scatter", "fq_status_string"])


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {fq.library_path}").read()
    exported = set(re.findall(r" T (fq_\w+)", out))
    assert set(_declared()) <= exported
    # nothing else leaks from the library's own namespace
    assert exported == set(_declared())


def test_status_strings(L):
    assert fq.fq_status_string(fq.FQ_OK) == "ok"
    for st in range(1, 5):
        assert fq.fq_status_string(st) != "ok"
    assert fq.fq_status_string(99) == "unknown status"


def test_null_handle_paths_without_gpu(L):
    vp = ctypes.c_void_p
    assert L.fq_code_bytes(None, 10) == -1
    L.fq_encode_kernel.restype = ctypes.c_char_p
    assert L.fq_encode_kernel(None, fq.FQ_F16, 10) is None
    assert L.fq_encode(None, vp(16), fq.FQ_F16, 1, vp(16), vp(16), fq.FQ_F16, None) == fq.FQ_ERR_ARG
    assert L.fq_decode(None, vp(16), vp(16), fq.FQ_F16, 1, vp(16), fq.FQ_F16, None) == fq.FQ_ERR_ARG
    assert L.fq_attn_workspace_bytes(None, 1, 8, 1, 10) == 0
    assert L.fq_attn_decode(None, vp(16), vp(16), vp(16), vp(16), vp(16), 1, 8, 1, 10, 0.125, vp(16), vp(16),
                            1 << 20, None) == fq.FQ_ERR_ARG
    assert L.fq_encode_scatter(None, vp(16), fq.FQ_F16, 1, vp(16), 10, vp(16), vp(16), fq.FQ_F16,
                               None) == fq.FQ_ERR_ARG
    assert L.fq_attn_decode_varlen(None, vp(16), vp(16), vp(16), vp(16), vp(16), vp(16), 1, 8, 1, 10, 0.125,
                                   vp(16), vp(16), 1 << 20, None) == fq.FQ_ERR_ARG
    assert L.fq_attn_prefill_workspace_bytes(None, 1, 8, 1, 4, 10) == 0
    assert L.fq_attn_prefill(None, vp(16), vp(16), vp(16), vp(16), vp(16), 1, 8, 1, 4, 10, 1, 0.125, vp(16),
                             vp(16), 1 << 20, None) == fq.FQ_ERR_ARG
    assert L.fq_codebook_train_workspace_bytes(3, 16, 100, 100) == 0  # k not a power of two
    assert L.fq_codebook_train_workspace_bytes(4, 16, 100, 100) > 0
    dbl = ctypes.c_double
    L.fq_codebook_train.argtypes = [ctypes.c_int, ctypes.c_int, vp, ctypes.c_int64, vp, ctypes.c_int64, vp,
                                    ctypes.c_int, ctypes.c_int, dbl, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    assert L.fq_codebook_train(4, 16, None, 100, vp(16), 100, vp(16), 1, 10, 1e-6, vp(16), None, None, None, None,
                               None, vp(16), 1 << 20, None) == fq.FQ_ERR_ARG
    assert L.fq_codebook_train(4, 16, vp(16), 100, vp(16), 100, vp(16), 1, 10, -1.0, vp(16), None, None, None,
                               None, None, vp(16), 1 << 20, None) == fq.FQ_ERR_ARG
    assert L.fq_codebook_train(4, 16, vp(16), 100, vp(16), 100, vp(16), 1, 10, 1e-6, vp(16), None, None, None,
                               None, None, vp(16), 16, None) == fq.FQ_ERR_WORKSPACE
    L.fq_codebook_free(None)  # ignored


def test_codebook_load_rejects_bad_arguments_before_any_hip_call(L):
    h = ctypes.c_void_p()
    cw = np.full((16, 2), 0.25, dtype=np.float32)
    rot = np.eye(64, dtype=np.float32)
    load = lambda d, k, N, c, r: L.fq_codebook_load(d, k, N, c.ctypes.data, r.ctypes.data, ctypes.byref(h))
    assert load(63, 2, 16, cw, rot) == fq.FQ_ERR_UNSUPPORTED      # d != 64
    assert load(64, 3, 16, cw, rot) == fq.FQ_ERR_ARG              # k does not divide d
    assert load(64, 2, 12, cw, rot) == fq.FQ_ERR_ARG              # N not a power of two
    assert load(64, 2, 1, cw, rot) == fq.FQ_ERR_ARG               # N < 2
    bad = cw.copy()
    bad[3, 1] = 0.1                                               # not fp16-representable
    assert load(64, 2, 16, bad, rot) == fq.FQ_ERR_ARG
    sub = cw.copy()
    sub[0, 0] = 2.0 ** -20                                        # fp16 subnormal
    assert load(64, 2, 16, sub, rot) == fq.FQ_ERR_ARG
    nanrot = rot.copy()
    nanrot[1, 2] = np.nan
    assert load(64, 2, 16, cw, nanrot) == fq.FQ_ERR_ARG
    assert L.fq_codebook_load(64, 2, 16, None, rot.ctypes.data, ctypes.byref(h)) == fq.FQ_ERR_ARG
    assert h.value is None
