"""Python binding of libfq, the FibQuant KV-cache codec for AMD MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/fq.h``: every function has
the C name and forwards device pointers (``torch.Tensor.data_ptr()``), sizes
and the current HIP stream.  All arithmetic runs in the HIP kernels of the
library; nothing here computes a result, and there is no CPU fallback — if the
library is missing the import of any entry point raises.

PyTorch serves only as the owner of device memory and streams.
"""
from __future__ import annotations

import ctypes
import json
import os

import numpy as np

__all__ = [
    "FQ_OK", "FQ_ERR_ARG", "FQ_ERR_UNSUPPORTED", "FQ_ERR_WORKSPACE", "FQ_ERR_HIP", "FQ_F32", "FQ_F16",
    "FQError", "lib", "library_path", "fq_status_string", "fq_codebook_load", "fq_codebook_free", "fq_code_bytes",
    "fq_encode", "fq_encode_kernel", "fq_encode_scatter", "fq_decode", "fq_attn_workspace_bytes", "fq_attn_decode",
    "fq_attn_decode_varlen", "fq_attn_noalloc_max_workspace_bytes", "fq_attn_decode_noalloc",
    "fq_attn_prefill_workspace_bytes", "fq_attn_prefill",
    "fq_codebook_train_workspace_bytes", "fq_codebook_train", "Codebook",
    "load_artifact",
    "artifact_dir",
]

FQ_OK, FQ_ERR_ARG, FQ_ERR_UNSUPPORTED, FQ_ERR_WORKSPACE, FQ_ERR_HIP = 0, 1, 2, 3, 4
FQ_F32, FQ_F16 = 0, 1

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libfq.so")
_lib = None


class FQError(RuntimeError):
    """A libfq call returned a status other than FQ_OK."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {fq_status_string(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libfq (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"libfq.so not built at {library_path}; run __graft_entry__.build() "
                              "or python -m universal_vector_quantization_amd.build_lib")
        L = ctypes.CDLL(library_path)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.fq_status_string.argtypes, L.fq_status_string.restype = [i32], ctypes.c_char_p
        L.fq_codebook_load.argtypes = [i32, i32, i32, vp, vp, ctypes.POINTER(vp)]
        L.fq_codebook_load.restype = i32
        L.fq_codebook_free.argtypes, L.fq_codebook_free.restype = [vp], None
        L.fq_code_bytes.argtypes, L.fq_code_bytes.restype = [vp, i64], i64
        L.fq_encode.argtypes = [vp, vp, i32, i64, vp, vp, i32, vp]
        L.fq_encode.restype = i32
        L.fq_encode_kernel.argtypes, L.fq_encode_kernel.restype = [vp, i32, i64], ctypes.c_char_p
        L.fq_encode_scatter.argtypes = [vp, vp, i32, i64, vp, i64, vp, vp, i32, vp]
        L.fq_encode_scatter.restype = i32
        L.fq_decode.argtypes = [vp, vp, vp, i32, i64, vp, i32, vp]
        L.fq_decode.restype = i32
        L.fq_attn_workspace_bytes.argtypes, L.fq_attn_workspace_bytes.restype = [vp, i32, i32, i32, i64], sz
        L.fq_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, ctypes.c_float, vp, vp, sz, vp]
        L.fq_attn_decode.restype = i32
        L.fq_attn_decode_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, ctypes.c_float, vp, vp,
                                            sz, vp]
        L.fq_attn_decode_varlen.restype = i32
        L.fq_attn_noalloc_max_workspace_bytes.argtypes, L.fq_attn_noalloc_max_workspace_bytes.restype = [], sz
        L.fq_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, ctypes.c_float, vp, vp]
        L.fq_attn_decode_noalloc.restype = i32
        L.fq_attn_prefill_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, i64]
        L.fq_attn_prefill_workspace_bytes.restype = sz
        L.fq_attn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, ctypes.c_float, vp, vp,
                                      sz, vp]
        L.fq_attn_prefill.restype = i32
        L.fq_codebook_train_workspace_bytes.argtypes = [i32, i32, i64, i64]
        L.fq_codebook_train_workspace_bytes.restype = sz
        dbl = ctypes.c_double
        L.fq_codebook_train.argtypes = [i32, i32, vp, i64, vp, i64, vp, i32, i32, dbl, vp, vp, vp, vp, vp, vp, vp,
                                        sz, vp]
        L.fq_codebook_train.restype = i32
        _lib = L
    return _lib


def fq_status_string(status: int) -> str:
    return lib().fq_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != FQ_OK:
        raise FQError(fn, status)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return FQ_F16
    if t.dtype == torch.float32:
        return FQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors must be contiguous device tensors")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def fq_codebook_load(d: int, k: int, N: int, codewords: np.ndarray, rotation: np.ndarray) -> int:
    """Upload a codebook [N, k] and rotation [d, d] (host fp32); returns the handle."""
    cw = np.ascontiguousarray(codewords, dtype=np.float32)
    rot = np.ascontiguousarray(rotation, dtype=np.float32)
    if cw.shape != (N, k) or rot.shape != (d, d):
        raise ValueError("codewords must be [N, k] and rotation [d, d]")
    h = ctypes.c_void_p()
    _check("fq_codebook_load", lib().fq_codebook_load(d, k, N, cw.ctypes.data, rot.ctypes.data, ctypes.byref(h)))
    return h.value


def fq_codebook_free(cb: int) -> None:
    lib().fq_codebook_free(cb)


def fq_code_bytes(cb: int, n: int) -> int:
    return int(lib().fq_code_bytes(cb, n))


def fq_encode(cb: int, x, codes, norms, stream=None) -> None:
    """x: [n, 64] fp16/fp32; codes: uint8 [fq_code_bytes(n)]; norms: [n] fp16/fp32."""
    n = x.shape[0] if x.dim() else 0
    _check("fq_encode", lib().fq_encode(cb, _ptr(x), _dtype_code(x), n, _ptr(codes), _ptr(norms),
                                        _dtype_code(norms), _stream(stream)))


def fq_encode_kernel(cb: int, x_dtype: int, n: int) -> str:
    """Name of the encoder kernel fq_encode launches for n vectors of x_dtype (FQ_F16 / FQ_F32)."""
    r = lib().fq_encode_kernel(cb, int(x_dtype), int(n))
    if r is None:
        raise ValueError("invalid arguments")
    return r.decode()


def fq_encode_scatter(cb: int, x, slots, capacity: int, codes, norms, stream=None) -> None:
    """x: [n, 64] fp16/fp32; slots: int64 [n] record slots (outside [0, capacity) = skip);
    codes: uint8 store of `capacity` records; norms: [capacity] fp16/fp32."""
    import torch

    n = x.shape[0] if x.dim() else 0
    if slots.dtype != torch.int64 or slots.numel() != n:
        raise ValueError("slots must be int64 [n]")
    _check("fq_encode_scatter", lib().fq_encode_scatter(cb, _ptr(x), _dtype_code(x), n, _ptr(slots), int(capacity),
                                                        _ptr(codes), _ptr(norms), _dtype_code(norms),
                                                        _stream(stream)))


def fq_decode(cb: int, codes, norms, x_out, stream=None) -> None:
    """codes: uint8 store; norms: [n]; x_out: [n, 64] fp16/fp32 (written)."""
    n = x_out.shape[0]
    _check("fq_decode", lib().fq_decode(cb, _ptr(codes), _ptr(norms), _dtype_code(norms), n, _ptr(x_out),
                                        _dtype_code(x_out), _stream(stream)))


def fq_attn_workspace_bytes(cb: int, B: int, Hq: int, Hkv: int, T: int) -> int:
    return int(lib().fq_attn_workspace_bytes(cb, B, Hq, Hkv, T))


def fq_attn_decode(cb: int, q, k_codes, k_norms, v_codes, v_norms, B: int, Hq: int, Hkv: int, T: int,
                   scale: float, out, workspace, stream=None) -> None:
    """q fp16 [B, Hq, 64]; codes/norms of a [B, Hkv, T] cache; out fp32 [B, Hq, 64]."""
    ws_ptr = None if workspace is None else _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("fq_attn_decode", lib().fq_attn_decode(cb, _ptr(q), _ptr(k_codes), _ptr(k_norms), _ptr(v_codes),
                                                  _ptr(v_norms), B, Hq, Hkv, T, float(scale), _ptr(out), ws_ptr,
                                                  ws_bytes, _stream(stream)))


def fq_attn_decode_varlen(cb: int, q, k_codes, k_norms, v_codes, v_norms, lens, B: int, Hq: int, Hkv: int, T: int,
                          scale: float, out, workspace, stream=None) -> None:
    """As fq_attn_decode over a cache of capacity T; batch b attends to its first lens[b] keys
    (lens: int32 [B] device tensor)."""
    import torch

    if lens.dtype != torch.int32 or lens.numel() != B:
        raise ValueError("lens must be int32 [B]")
    ws_ptr = None if workspace is None else _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("fq_attn_decode_varlen",
           lib().fq_attn_decode_varlen(cb, _ptr(q), _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms),
                                       _ptr(lens), B, Hq, Hkv, T, float(scale), _ptr(out), ws_ptr, ws_bytes,
                                       _stream(stream)))


def fq_attn_noalloc_max_workspace_bytes() -> int:
    return int(lib().fq_attn_noalloc_max_workspace_bytes())


def fq_attn_decode_noalloc(cb: int, q, k_codes, k_norms, v_codes, v_norms, B: int, Hq: int, Hkv: int, T: int,
                           scale: float, out, lens=None, stream=None) -> None:
    """As fq_attn_decode (lens None) or fq_attn_decode_varlen (lens int32 [B]) with the
    workspace in the library's fixed device buffer: no allocation."""
    import torch

    if lens is not None and (lens.dtype != torch.int32 or lens.numel() != B):
        raise ValueError("lens must be int32 [B]")
    _check("fq_attn_decode_noalloc",
           lib().fq_attn_decode_noalloc(cb, _ptr(q), _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms),
                                        _ptr(lens), B, Hq, Hkv, T, float(scale), _ptr(out), _stream(stream)))


def fq_attn_prefill_workspace_bytes(cb: int, B: int, Hq: int, Hkv: int, Sq: int, T: int) -> int:
    return int(lib().fq_attn_prefill_workspace_bytes(cb, B, Hq, Hkv, Sq, T))


def fq_attn_prefill(cb: int, q, k_codes, k_norms, v_codes, v_norms, B: int, Hq: int, Hkv: int, Sq: int, T: int,
                    causal: bool, scale: float, out, workspace, stream=None) -> None:
    """q fp16 [B, Hq, Sq, 64]; codes/norms of a [B, Hkv, T] cache; out fp32 [B, Hq, Sq, 64]."""
    ws_ptr = None if workspace is None else _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("fq_attn_prefill", lib().fq_attn_prefill(cb, _ptr(q), _ptr(k_codes), _ptr(k_norms), _ptr(v_codes),
                                                    _ptr(v_norms), B, Hq, Hkv, Sq, T, 1 if causal else 0,
                                                    float(scale), _ptr(out), ws_ptr, ws_bytes, _stream(stream)))


def fq_codebook_train_workspace_bytes(k: int, N: int, m_train: int, m_valid: int) -> int:
    return int(lib().fq_codebook_train_workspace_bytes(k, N, m_train, m_valid))


def fq_codebook_train(train, valid, starts, max_iter: int, rel_tol: float, codewords, codewords64=None,
                      workspace=None, stream=None) -> dict:
    """Generalised Lloyd on the GPU.  train [m_train, k] / valid [m_valid, k] fp64, starts
    [restarts, N, k] fp64 device tensors; codewords fp32 [N, k] (written).  Returns the
    per-restart validation MSE, the rounded codebook's validation MSE and the kept run's
    training-MSE history (host values the call produced)."""
    import torch

    R, N, k = starts.shape
    mt, mv = train.shape[0], valid.shape[0]
    if train.shape[1] != k or valid.shape[1] != k or codewords.shape != (N, k):
        raise ValueError("shape mismatch")
    if workspace is None:
        workspace = torch.empty(max(fq_codebook_train_workspace_bytes(k, N, mt, mv), 16), dtype=torch.uint8,
                                device=train.device)
    rmse = (ctypes.c_double * R)()
    vmse = ctypes.c_double()
    hist = (ctypes.c_double * (max_iter + 1))()
    hlen = ctypes.c_int()
    _check("fq_codebook_train", lib().fq_codebook_train(
        k, N, _ptr(train), mt, _ptr(valid), mv, _ptr(starts), R, max_iter, float(rel_tol), _ptr(codewords),
        _ptr(codewords64), rmse, ctypes.byref(vmse), hist, ctypes.byref(hlen), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return {"restart_valid_mse": list(rmse), "valid_mse": vmse.value, "history": list(hist)[: hlen.value]}


# --------------------------------------------------------------- artifacts
artifact_dir = os.path.join(_PKG, "codebooks")


def load_artifact(k: int, N: int, d: int = 64, initial: bool = False):
    """(codewords fp32 [N, k], rotation fp32 [d, d]) from the frozen artifact files;
    initial=True: the rate-axis codebooks frozen before any Lloyd refinement."""
    man = json.load(open(os.path.join(artifact_dir, "MANIFEST.json")))
    name = f"fq_d{d}_k{k}_n{N}{'_init' if initial else ''}.npz"
    if name not in man:
        raise FileNotFoundError(f"no codebook artifact {name}")
    cw = np.load(os.path.join(artifact_dir, name), allow_pickle=False)["codewords"]
    rot = np.load(os.path.join(artifact_dir, f"rotation_d{d}_seed0.npz"), allow_pickle=False)["rotation"]
    return cw, rot


class Codebook:
    """Owner of one device codebook handle (freed on close / garbage collection)."""

    def __init__(self, codewords: np.ndarray, rotation: np.ndarray):
        self.N, self.k = codewords.shape
        self.d = rotation.shape[0]
        self.bits = int(self.N).bit_length() - 1
        self.handle = fq_codebook_load(self.d, self.k, self.N, codewords, rotation)

    @classmethod
    def from_artifact(cls, k: int, N: int, d: int = 64, initial: bool = False) -> "Codebook":
        return cls(*load_artifact(k, N, d, initial))

    def code_bytes(self, n: int) -> int:
        return fq_code_bytes(self.handle, n)

    def close(self) -> None:
        if getattr(self, "handle", None):
            fq_codebook_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
