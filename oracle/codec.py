"""FibQuant encode / decode, brute force in fp64 — oracle (test infrastructure only).

FibQuant summary §2.3: the encoder computes the norm ν = ‖x‖₂, rotates the unit
vector Πx/ν, splits it into d/k blocks of k coordinates and looks up the nearest
codeword of each block in the shared codebook; the decoder gathers the
codewords, concatenates the blocks, applies the inverse rotation and scales by
the norm.  The rate is b = log2(N)/k bits per coordinate.  §1: codes are stored
at fixed addresses so every token decodes alone by address arithmetic.

Readings:
  * ν is accumulated in fp64 on the exact input values and stored
    round-to-nearest-even in the norm dtype, converted straight from fp64.
    The unit vector uses the unrounded fp64 ν.  ν = 0 gives the zero unit vector
    (every block then takes the smallest-norm codeword) and decodes to exactly 0.
  * Blocks are k consecutive coordinates of the rotated vector.
  * The nearest codeword is the definition itself: squared distance
    Σ_i (y_i - c_{n,i})² in fp64 for every codeword, lowest index on exact ties.
    Several codes are correct at a near-tie: when the two smallest distances
    d1 <= d2 satisfy d2 - d1 < 1e-6·d2 the block is flagged, and any code n with
    d_n - d1 <= 1e-6·d_n is accepted.
  * Fixed-address store: B = (d/k)·log2 N bits per vector; vector i starts at
    bit i·B, its block j at bit i·B + j·log2 N; bits are LSB-first inside
    little-endian bytes; the store has ceil(n·B/8) bytes, pad bits are 0.
  * Decode works in fp64 from the stored norm and rounds once (RNE) to the
    output dtype.
"""
from __future__ import annotations

import math

import numpy as np

NEAR_TIE_REL = 1e-6


# ---------------------------------------------------------------- rate
def code_bits(N: int) -> int:
    """log2 N for a power-of-two codebook size (fixed-rate codes need it integral)."""
    b = int(N).bit_length() - 1
    if N < 2 or (1 << b) != N:
        raise ValueError("N must be a power of two >= 2")
    return b


def rate_bits_per_coordinate(k: int, N: int) -> float:
    """b = log2(N) / k."""
    return math.log2(N) / k


def bits_per_vector(d: int, k: int, N: int) -> int:
    """B = (d/k) · log2 N."""
    if d % k:
        raise ValueError("k must divide d")
    return (d // k) * code_bits(N)


def code_bytes(n: int, d: int, k: int, N: int) -> int:
    """Size of the fixed-address store for n vectors: ceil(n·B/8)."""
    return (n * bits_per_vector(d, k, N) + 7) // 8


# ---------------------------------------------------------------- encode
def vector_norms(x: np.ndarray) -> np.ndarray:
    """ν = sqrt(Σ x_i²) in fp64 (inputs are exact in fp64)."""
    x64 = np.asarray(x, dtype=np.float64)
    return np.sqrt(np.sum(x64 * x64, axis=1))


def store_norms(nu: np.ndarray, dtype) -> np.ndarray:
    """Round fp64 norms to the storage dtype (NumPy casts fp64 -> fp16/fp32 directly, RNE)."""
    return np.asarray(nu, dtype=np.float64).astype(dtype)


def rotate_unit(x: np.ndarray, rotation: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """y = Π (x/ν) for every row (fp64), and ν.  Rows with ν = 0 give y = 0."""
    x64 = np.asarray(x, dtype=np.float64)
    nu = vector_norms(x64)
    u = np.zeros_like(x64)
    nz = nu > 0
    u[nz] = x64[nz] / nu[nz, None]
    pi = np.asarray(rotation, dtype=np.float64)
    return u @ pi.T, nu


def nearest_codewords(blocks: np.ndarray, codebook: np.ndarray, chunk: int = 4096):
    """Brute-force nearest codeword for every block (fp64 direct form).

    blocks [m, k], codebook [N, k].  Returns (code, d1, d2, near_tie) where d1 <= d2
    are the two smallest squared distances."""
    y = np.asarray(blocks, dtype=np.float64)
    c = np.asarray(codebook, dtype=np.float64)
    m, k = y.shape
    N = c.shape[0]
    code = np.empty(m, dtype=np.int64)
    d1 = np.empty(m)
    d2 = np.empty(m)
    for s in range(0, m, chunk):
        yc = y[s:s + chunk]
        dist = np.zeros((len(yc), N))
        for i in range(k):
            dist += (yc[:, i, None] - c[None, :, i]) ** 2
        code[s:s + chunk] = np.argmin(dist, axis=1)
        two = np.sort(np.partition(dist, 1, axis=1)[:, :2], axis=1)
        d1[s:s + chunk] = two[:, 0]
        d2[s:s + chunk] = two[:, 1]
    near_tie = ((d2 - d1) < NEAR_TIE_REL * d2) | (d2 == 0.0)
    return code, d1, d2, near_tie


def block_distances(blocks: np.ndarray, codebook: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Squared distance of each block to the codeword ``codes`` names (fp64 direct form)."""
    y = np.asarray(blocks, dtype=np.float64)
    c = np.asarray(codebook, dtype=np.float64)[np.asarray(codes)]
    return np.sum((y - c) ** 2, axis=1)


class Encoded:
    """Result of :func:`encode` (all arrays indexed by vector, then block)."""

    def __init__(self, codes, norms, nu, d1, d2, near_tie, y):
        self.codes = codes          # int64 [n, d/k]
        self.norms = norms          # stored norms, norm dtype [n]
        self.nu = nu                # fp64 norms [n]
        self.d1 = d1                # fp64 [n, d/k]
        self.d2 = d2
        self.near_tie = near_tie    # bool [n, d/k]
        self.y = y                  # rotated unit vectors, fp64 [n, d]


def encode(x: np.ndarray, rotation: np.ndarray, codebook: np.ndarray, norm_dtype) -> Encoded:
    """Encode rows of x: stored norms and one code per block (FibQuant summary §2.3)."""
    n, d = x.shape
    N, k = codebook.shape
    if d % k:
        raise ValueError("k must divide d")
    y, nu = rotate_unit(x, rotation)
    code, d1, d2, nt = nearest_codewords(y.reshape(n * (d // k), k), codebook)
    shp = (n, d // k)
    return Encoded(code.reshape(shp), store_norms(nu, norm_dtype), nu, d1.reshape(shp), d2.reshape(shp),
                   nt.reshape(shp), y)


def accepted(y: np.ndarray, codebook: np.ndarray, enc: Encoded, other_codes: np.ndarray) -> np.ndarray:
    """Whether each code in ``other_codes`` [n, d/k] is a correct answer: equal to the
    oracle code, or (at a near-tie only) within 1e-6 relative of the best distance."""
    n, m = other_codes.shape
    k = codebook.shape[1]
    dn = block_distances(y.reshape(n * m, k), codebook, other_codes.reshape(-1)).reshape(n, m)
    ok_tie = enc.near_tie & ((dn - enc.d1) <= NEAR_TIE_REL * dn)
    return (other_codes == enc.codes) | ok_tie


# ---------------------------------------------------------------- fixed-address store
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes [n, m] into the LSB-first little-endian bitstream."""
    c = np.asarray(codes, dtype=np.int64).reshape(-1)
    if np.any(c < 0) or np.any(c >= (1 << bits)):
        raise ValueError("code out of range")
    bitarr = ((c[:, None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(bitarr, bitorder="little")


def unpack_codes(buf: np.ndarray, n: int, m: int, bits: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`: [n, m] int64 codes from the bitstream."""
    total = n * m * bits
    bitarr = np.unpackbits(np.asarray(buf, dtype=np.uint8), bitorder="little")[:total]
    b = bitarr.reshape(n * m, bits).astype(np.int64)
    return (b << np.arange(bits)).sum(axis=1).reshape(n, m)


def write_records(codes: np.ndarray, norms: np.ndarray, new_codes: np.ndarray, new_norms: np.ndarray,
                  slots) -> tuple[np.ndarray, np.ndarray]:
    """The append step on a fixed-address store (FibQuant summary §1: each record has a
    fixed size and place, so one record changes without touching the others; §5: the
    decode loop adds one token per step).  codes [capacity, m] and norms [capacity] are
    the store; new vector i (codes new_codes[i], norm new_norms[i]) replaces record
    slots[i]; a slot outside [0, capacity) writes nothing.  Slots must be distinct.
    Returns new arrays; the inputs are not modified."""
    out_c = np.array(codes, copy=True)
    out_n = np.array(norms, copy=True)
    cap = out_c.shape[0]
    used = set()
    for i, s in enumerate(np.asarray(slots, dtype=np.int64).tolist()):
        if not 0 <= s < cap:
            continue
        if s in used:
            raise ValueError(f"slot {s} given twice")
        used.add(s)
        out_c[s] = new_codes[i]
        out_n[s] = new_norms[i]
    return out_c, out_n


# ---------------------------------------------------------------- decode
def decode(codes: np.ndarray, norms: np.ndarray, rotation: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """x̂ = ν · Πᵀ concat(c_code) in fp64 from stored norms (FibQuant summary §2.3)."""
    codes = np.asarray(codes)
    n, m = codes.shape
    c = np.asarray(codebook, dtype=np.float64)
    yhat = c[codes].reshape(n, m * c.shape[1])
    pi = np.asarray(rotation, dtype=np.float64)
    nu = np.asarray(norms).astype(np.float64)
    return nu[:, None] * (yhat @ pi)


def round_output(x64: np.ndarray, dtype) -> np.ndarray:
    """Round an fp64 reconstruction once (RNE) to the output dtype."""
    return np.asarray(x64, dtype=np.float64).astype(dtype)
