"""Plain CPU oracle of the FP8 index-vector producer: Hadamard rotation, then
per-row ue8m0-scaled E4M3 quantisation.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the bench's cpu_baseline leg may import or run this module; the library's
product path never calls it and shares no code with it.

What it computes and where it comes from:

  1. Rotation.  The HF model doc "DeepSeek-V3.2", section "DeepSeek Sparse
     Attention (DSA)", item 1: the indexer runs in FP8 after a Hadamard
     transform ("rotate_activation") of its query and key vectors, and the
     transform is orthogonal, so rotated dot products equal the plain ones.
     Reading used here: the Sylvester-ordered Hadamard matrix of order
     D = 128 scaled by 1/sqrt(D) (the orthonormal Walsh-Hadamard transform),
     applied to every D-element index vector (each head of q, each key).
  2. Quantisation.  The released configuration excerpt on the atlas
     "DeepSeek-V3.2-Exp" token-ids page gives "scale_fmt: ue8m0"; the drose
     page names F8_E4M3 as the FP8 format.  Reading: one power-of-two scale
     per row, the smallest 2^e with max|y| / 2^e <= 448 (the largest E4M3
     value), stored as the byte e + 127 (an all-zero row uses e = 0; e is
     clamped at -127, the byte's range, for rows below about 2^-118); codes
     are E4M3 ("fn": bias 7, no infinities) of y / 2^e, rounded to nearest
     with ties to even.

Two forms of the rotation are given: `rotate_exact` (fp64 matrix product, the
definition) and `rotate_fwht_f32` (the butterfly network in fp32 in a fixed
order).  Codes are decided by rounding, so the comparison with a kernel uses
the fp32 form, which takes the same decisions in the same precision; the
pins tie the fp32 form to the exact one.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two): H_1 = [1],
    H_2m = [[H_m, H_m], [H_m, -H_m]].  Entries are +-1."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_exact(x: np.ndarray) -> np.ndarray:
    """y = H x / sqrt(D) for every row x (last axis of length D), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    return x @ hadamard(d).T / math.sqrt(d)


def rotate_fwht_f32(x: np.ndarray) -> np.ndarray:
    """The same rotation as a butterfly network in fp32: for h = 1, 2, 4, ...,
    D/2, every pair (j, j + h) inside each block of 2h becomes
    (x_j + x_{j+h}, x_j - x_{j+h}); then every element is multiplied by the
    fp32 value of 1/sqrt(D).  The result is H x / sqrt(D) up to fp32
    rounding (the Sylvester matrix factors into these stages)."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return y * np.float32(1.0 / math.sqrt(d))


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax / 2^e <= 448 (e = 0 where amax == 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    e[nz] = np.ceil(np.log2(amax[nz] / E4M3_MAX)).astype(np.int64)
    # guard the floating-point log: step to the smallest exponent that fits
    fix_up = nz & (amax / np.exp2(e.astype(np.float64)) > E4M3_MAX)
    e[fix_up] += 1
    fix_dn = nz & (amax / np.exp2((e - 1).astype(np.float64)) <= E4M3_MAX)
    e[fix_dn] -= 1
    return e


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """E4M3 ("fn") code of each value: round to nearest, ties to even,
    magnitudes above 448 saturate to 448.  -0.0 keeps its sign bit.
    Written from the format: normal values 2^(E-7) * (1 + m/8) for exponent
    field E = 1..15 (except E = 15, m = 7, which is NaN), subnormal values
    m/8 * 2^-6."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.uint8)
    # subnormal range: multiples of 2^-9 below 2^-6
    sub = a < 2.0 ** -6
    n = np.rint(a[sub] * 512.0)                 # numpy rint: ties to even
    out[sub] = n.astype(np.uint8)               # n = 8 is the code of 2^-6 (E = 1, m = 0)
    nor = ~sub
    an = np.minimum(a[nor], E4M3_MAX)
    ex = np.floor(np.log2(an)).astype(np.int64)
    # guard the floating-point log at exact powers of two
    ex = np.where(np.exp2(ex.astype(np.float64)) > an, ex - 1, ex)
    ex = np.where(np.exp2((ex + 1).astype(np.float64)) <= an, ex + 1, ex)
    m = np.rint(an / np.exp2(ex.astype(np.float64)) * 8.0) - 8.0   # 0..8, ties to even
    carry = m >= 8
    ex = np.where(carry, ex + 1, ex)
    m = np.where(carry, 0, m)
    code = ((ex + 7) << 3) + m.astype(np.int64)
    code = np.minimum(code, 0x7E)               # 448 is the largest finite value
    out[nor] = code.astype(np.uint8)
    return out | sign


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code (NaN for the two NaN codes)."""
    c = np.asarray(c, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def quantize_rows(y: np.ndarray):
    """Per-row ue8m0 scale byte and E4M3 codes of rows y (last axis).  The
    exponent is clamped to the byte's range (e >= -127), which only matters
    for rows whose maximum is below about 2^-118."""
    y = np.asarray(y, dtype=np.float64)
    amax = np.abs(y).max(axis=-1)
    e = np.clip(scale_exponent(amax), -127, 127)
    codes = e4m3_encode(y / np.exp2(e.astype(np.float64))[..., None])
    return codes, (e + 127).astype(np.uint8)


def rotate_quantize(x: np.ndarray):
    """Codes and scale bytes of the rotated rows, rotation in fp32 (the
    precision in which the codes are decided)."""
    return quantize_rows(rotate_fwht_f32(x).astype(np.float64))
