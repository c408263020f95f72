"""Pins of the FP8 producer oracle (Hadamard rotation + ue8m0/E4M3
quantisation) against the mathematics and independent library routines."""
import math

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from oracle import fp8_producer as P


def test_hadamard_small_orders_by_hand():
    assert np.array_equal(P.hadamard(1), [[1.0]])
    assert np.array_equal(P.hadamard(2), [[1, 1], [1, -1]])
    assert np.array_equal(P.hadamard(4), [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])


def test_hadamard_128_is_orthogonal_symmetric_pm1():
    h = P.hadamard(128)
    assert set(np.unique(h)) == {-1.0, 1.0}
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h.T, 128 * np.eye(128))
    assert np.all(h[0] == 1) and np.all(h[:, 0] == 1)


def test_rotation_preserves_dot_products():
    # HF doc, DSA item 1: the transform is orthogonal, so Hq . Hk = q . k
    rng = np.random.default_rng(11)
    q, k = rng.standard_normal((64, 128)), rng.standard_normal((300, 128))
    assert np.allclose(P.rotate_exact(q) @ P.rotate_exact(k).T, q @ k.T, atol=1e-10)
    assert np.allclose(np.linalg.norm(P.rotate_exact(q), axis=1), np.linalg.norm(q, axis=1))


def test_rotated_index_scores_equal_plain_scores():
    rng = np.random.default_rng(12)
    H, D, L = 4, 128, 40
    q = rng.standard_normal((1, L, H, D))
    k = rng.standard_normal((1, L, D))
    w = rng.standard_normal((1, L, H)) / H
    plain = O.index_scores(q, k, w, L, L)
    rot = O.index_scores(P.rotate_exact(q), P.rotate_exact(k), w, L, L)
    fin = np.isfinite(plain)
    assert np.array_equal(fin, np.isfinite(rot))
    assert np.allclose(rot[fin], plain[fin], atol=1e-10)


def test_fwht_f32_matches_exact_rotation_and_basis_vectors():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    ref = P.rotate_exact(x)
    got = P.rotate_fwht_f32(x).astype(np.float64)
    assert np.max(np.abs(got - ref)) < 2e-5 * max(1.0, np.max(np.abs(ref)))
    # e_j maps to column j of H / sqrt(D), exactly (one nonzero input)
    eye = np.eye(128, dtype=np.float32)
    cols = P.rotate_fwht_f32(eye).astype(np.float64)
    assert np.array_equal(cols, (P.hadamard(128).T / math.sqrt(128)).astype(np.float32).astype(np.float64))


def test_e4m3_codes_round_trip_and_grid():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = P.e4m3_decode(codes)
    assert np.array_equal(P.e4m3_encode(vals), codes)
    # the decoder agrees with the dsa oracle's independent E4M3 decoder
    assert np.array_equal(vals, O.e4m3_decode(codes))
    assert P.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert P.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert P.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6


def test_e4m3_ties_go_to_even_and_large_values_saturate():
    pos = np.array([c for c in range(0x7E)], dtype=np.uint8)
    lo, hi = P.e4m3_decode(pos), P.e4m3_decode(pos + 1)
    mid = (lo + hi) / 2
    got = P.e4m3_encode(mid)
    want = np.where((pos & 1) == 0, pos, pos + 1)          # the neighbour with an even mantissa
    assert np.array_equal(got, want)
    assert np.array_equal(P.e4m3_encode(np.array([448.0, 460.0, 1e6, -1e6, -0.0])),
                          np.array([0x7E, 0x7E, 0x7E, 0xFE, 0x80], dtype=np.uint8))


def test_e4m3_encode_matches_torch_float8_cast():
    rng = np.random.default_rng(14)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 1e-2,
                        rng.standard_normal(20000) * 1e-4]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(P.e4m3_encode(v.astype(np.float64)), ref)


def test_scale_rule():
    rng = np.random.default_rng(15)
    amax = np.exp(rng.uniform(-30, 30, 5000))
    e = P.scale_exponent(amax)
    r = amax / np.exp2(e.astype(np.float64))
    assert np.all(r <= 448.0) and np.all(r > 224.0)
    k = np.arange(-20, 21)
    assert np.array_equal(P.scale_exponent(448.0 * np.exp2(k.astype(np.float64))), k)
    assert P.scale_exponent(np.array([0.0]))[0] == 0


def test_quantize_rows_dequantise_within_half_step():
    rng = np.random.default_rng(16)
    y = rng.standard_normal((500, 128)) * np.exp(rng.uniform(-5, 5, (500, 1)))
    codes, sb = P.quantize_rows(y)
    scale = np.exp2(sb.astype(np.float64) - 127)[:, None]
    deq = P.e4m3_decode(codes) * scale
    # E4M3 has 3 mantissa bits: relative error <= 2^-4 for normals; absolute
    # error <= 2^-10 * scale in the subnormal range
    err = np.abs(deq - y)
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, scale * 2.0 ** -10) + 1e-300)
    assert np.all(np.abs(P.e4m3_decode(codes)).max(axis=1) >= 224.0)  # the scale uses the range


def test_all_zero_row_and_single_spike():
    codes, sb = P.quantize_rows(np.zeros((1, 128)))
    assert sb[0] == 127 and np.all(codes == 0)
    # worked by hand: amax 3e5 -> 3e5 / 448 = 669.6 -> e = ceil(log2 669.6) = 10,
    # byte 137; -3e5 / 1024 = -292.97 = -256 * 1.1444 -> mantissa 1.1444 * 8 - 8
    # = 1.155 -> 1, exponent field 8 + 7 = 15: code 0x80 | 15 << 3 | 1 = 0xF9
    # (-288 * 1024 = -294912 after dequantisation)
    y = np.zeros((1, 128))
    y[0, 5] = -3.0e5
    codes, sb = P.quantize_rows(y)
    assert sb[0] == 137 and codes[0, 5] == 0xF9
    assert P.e4m3_decode(codes[0, 5:6])[0] * 2.0 ** (int(sb[0]) - 127) == -294912.0
    assert np.all(codes[0, np.arange(128) != 5] == 0)


@pytest.mark.parametrize("seed", [0, 1])
def test_rotate_quantize_keeps_scores_within_fp8_error(seed):
    rng = np.random.default_rng(20 + seed)
    H, D, L = 8, 128, 64
    q = rng.standard_normal((1, L, H, D)).astype(np.float32)
    k = rng.standard_normal((1, L, D)).astype(np.float32)
    w = (rng.standard_normal((1, L, H)) / H).astype(np.float32)
    qc, qs = P.rotate_quantize(q.reshape(-1, D))
    kc, ks = P.rotate_quantize(k.reshape(-1, D))
    qf, kf = O.as_f64_index_inputs(qc.reshape(1, L, H, D), qs.reshape(1, L, H), kc.reshape(1, L, D), ks.reshape(1, L))
    got = O.index_scores(qf, kf, w.astype(np.float64), L, L)
    ref = O.index_scores(q.astype(np.float64), k.astype(np.float64), w.astype(np.float64), L, L)
    fin = np.isfinite(ref)
    # E4M3 relative step 2^-3 per element: the score error stays a small
    # fraction of the score scale
    assert np.max(np.abs(got[fin] - ref[fin])) < 0.15 * np.max(np.abs(ref[fin]))
