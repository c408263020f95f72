"""Pins of the projections oracle (index query from the query latent, head
weights from the hidden state, per-head un-absorption of the attention
output) against hand-worked values and identities of the method."""
import json
import math
import os

import numpy as np

from oracle import dsa_oracle as O
from oracle import projections as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "projections_small.json")


def test_hand_worked_fixture():
    g = json.load(open(GOLDEN))
    iq = g["index_q"]
    assert np.array_equal(P.index_q_from_latent(iq["cq"], iq["wq_b"], iq["heads"], iq["dim"]), iq["q"])
    hw = g["head_weights"]
    assert np.array_equal(P.head_weights_from_hidden(hw["x"], hw["w_proj"]), hw["w"])
    ua = g["unabsorb"]
    assert np.array_equal(P.unabsorb_output(ua["o_lat"], ua["w_uv"]), ua["out"])


def test_index_q_is_head_major_over_the_weight_rows():
    # a selection matrix: output row h*D + d copies latent entry (7h + 3d) % R,
    # so a swapped head/dim order or a transposed weight picks other entries
    H, D, R = 4, 8, 37
    w = np.zeros((H * D, R))
    for h in range(H):
        for d in range(D):
            w[h * D + d, (7 * h + 3 * d) % R] = 1.0
    cq = np.random.default_rng(1).standard_normal((5, R))
    q = P.index_q_from_latent(cq, w, H, D)
    for t in range(5):
        for h in range(H):
            for d in range(D):
                assert q[t, h, d] == cq[t, (7 * h + 3 * d) % R]


def test_index_q_feeds_scores_linearly():
    # scaling the latent scales every head dot product; ReLU is positively
    # homogeneous, so index scores scale by the same factor and the top-k set
    # is unchanged
    rng = np.random.default_rng(2)
    H, D, R, L = 4, 16, 24, 30
    cq = rng.standard_normal((1, L, R))
    w = rng.standard_normal((H * D, R)) / math.sqrt(R)
    k = rng.standard_normal((1, L, D))
    hw = rng.standard_normal((1, L, H)) / H
    s1 = O.index_scores(P.index_q_from_latent(cq, w, H, D), k, hw, L, L)
    s2 = O.index_scores(P.index_q_from_latent(2.5 * cq, w, H, D), k, hw, L, L)
    fin = np.isfinite(s1)
    assert np.allclose(s2[fin], 2.5 * s1[fin], rtol=1e-12, atol=1e-12)
    assert np.array_equal(O.topk(s1, L, L, 5), O.topk(s2, L, L, 5))


def test_head_weights_single_feature():
    # x = e_i picks column i of the projection for every head
    Hd, dim = 6, 50
    wp = np.random.default_rng(3).standard_normal((Hd, dim))
    for i in (0, 17, 49):
        x = np.zeros((1, dim))
        x[0, i] = 1.0
        assert np.array_equal(P.head_weights_from_hidden(x, wp)[0], wp[:, i])


def test_unabsorb_with_leading_identity_returns_leading_dims():
    # W_UV[a] = c_a [I_V | 0]: head a returns c_a times its first V latent dims,
    # so a mixed-up head index or contraction axis fails
    NH, V, C = 5, 4, 12
    w = np.zeros((NH, V, C))
    for a in range(NH):
        w[a, :, :V] = (a + 1) * np.eye(V)
    o = np.random.default_rng(4).standard_normal((3, NH, C))
    out = P.unabsorb_output(o, w)
    for a in range(NH):
        assert np.array_equal(out[:, a], (a + 1) * o[:, a, :V])


def test_unabsorbed_absorbed_attention_equals_attention_with_per_head_values():
    # absorbed attention followed by W_UV equals attention whose values are
    # W_UV[a] kv_j[0:C], written here as an explicit per-head softmax loop
    rng = np.random.default_rng(5)
    NH, Dqk, C, V, Lk = 3, 10, 8, 4, 20
    qa = rng.standard_normal((NH, Dqk))
    kv = rng.standard_normal((Lk, Dqk))
    w_uv = rng.standard_normal((NH, V, C)) / math.sqrt(C)
    sel = np.array([1, 4, 5, 11, 19, -1])
    scale = 1 / math.sqrt(Dqk)
    o_lat, _ = O.sparse_attention_row(qa, kv, sel, scale, C)
    got = P.unabsorb_output(o_lat[None], w_uv)[0]
    chosen = [j for j in sel if j >= 0]
    for a in range(NH):
        z = [scale * sum(qa[a, d] * kv[j, d] for d in range(Dqk)) for j in chosen]
        m = max(z)
        e = [math.exp(x - m) for x in z]
        tot = sum(e)
        for v in range(V):
            want = sum(e[t] / tot * sum(w_uv[a, v, c] * kv[j, c] for c in range(C)) for t, j in enumerate(chosen))
            assert abs(got[a, v] - want) < 1e-12


def test_shape_checks():
    import pytest
    with pytest.raises(ValueError):
        P.index_q_from_latent(np.zeros((2, 5)), np.zeros((8, 4)), 2, 4)
    with pytest.raises(ValueError):
        P.unabsorb_output(np.zeros((1, 2, 3)), np.zeros((2, 4, 5)))
