"""Pins for the oracle's rotary embedding by branch depth.

Checked against: rotation matrices written out for 2 and 4 channels, the complex
form of the rotary embedding (pair j as the complex number x_j + i x_{j+rot/2}
times e^{i pos theta_j}), the transformers library's rotate-half application,
and the properties that make RoPE a position code (scores depend only on the
distance of positions; rotations compose; position 0 is the identity).
"""

import numpy as np
import pytest

from oracle import attention as oattn
from oracle import rope as orope


def test_two_channels_is_a_plane_rotation():
    x = np.array([0.3, -1.7])
    for p in (0, 1, 5, 1000):
        c, s = np.cos(p), np.sin(p)
        want = np.array([[c, -s], [s, c]]) @ x
        np.testing.assert_allclose(orope.rope(x[None], np.array([p]), 2, 10000.0)[0], want, rtol=0, atol=1e-12)


def test_four_channels_pair_layout_and_frequencies():
    # theta = 100, rot = 4: pair (0, 2) turns by p, pair (1, 3) by p / 10
    p = 3
    e = np.eye(4)
    got = orope.rope(e, np.full(4, p), 4, 100.0)
    a0, a1 = p * 1.0, p * 0.1
    want = np.array([[np.cos(a0), 0, np.sin(a0), 0],
                     [0, np.cos(a1), 0, np.sin(a1)],
                     [-np.sin(a0), 0, np.cos(a0), 0],
                     [0, -np.sin(a1), 0, np.cos(a1)]])
    np.testing.assert_allclose(got, want, atol=1e-12)


@pytest.mark.parametrize("D,rot", [(8, 8), (64, 16), (256, 64), (128, 128)])
def test_complex_form(D, rot):
    rng = np.random.default_rng(D + rot)
    x = rng.standard_normal((5, 3, D))
    pos = rng.integers(0, 140000, 5)
    got = orope.rope(x, pos, rot, 1e6)
    h = rot // 2
    z = x[..., :h] + 1j * x[..., h:rot]
    freq = 1e6 ** (-np.arange(h) / h)
    zr = z * np.exp(1j * pos[:, None, None] * freq)
    np.testing.assert_allclose(got[..., :h], zr.real, atol=1e-9)
    np.testing.assert_allclose(got[..., h:rot], zr.imag, atol=1e-9)
    np.testing.assert_array_equal(got[..., rot:], x[..., rot:])


def test_matches_transformers_rotate_half():
    import torch
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb

    rng = np.random.default_rng(0)
    T, H, D = 7, 2, 16
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((T, H, D))
    pos = np.array([40, 41, 41, 42, 43, 42, 44])
    freq = np.outer(pos, 500.0 ** (-np.arange(0, D, 2) / D))
    emb = np.concatenate([freq, freq], axis=-1)                      # the library's cos/sin layout
    cos, sin = torch.from_numpy(np.cos(emb)), torch.from_numpy(np.sin(emb))
    qt, kt = (torch.from_numpy(a).transpose(0, 1)[None] for a in (q, k))  # [1][H][T][D]
    qr, kr = apply_rotary_pos_emb(qt, kt, cos[None], sin[None])
    np.testing.assert_allclose(orope.rope(q, pos, D, 500.0), qr[0].transpose(0, 1).numpy(), atol=1e-12)
    np.testing.assert_allclose(orope.rope(k, pos, D, 500.0), kr[0].transpose(0, 1).numpy(), atol=1e-12)


def test_scores_depend_only_on_distance_and_rotations_compose():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((2, 64))
    ref = orope.rope(q[None], [100], 64, 1e4)[0] @ orope.rope(k[None], [93], 64, 1e4)[0]
    for shift in (1, 17, 12345):
        got = orope.rope(q[None], [100 + shift], 64, 1e4)[0] @ orope.rope(k[None], [93 + shift], 64, 1e4)[0]
        assert abs(got - ref) < 1e-9
    a = orope.rope(orope.rope(q[None], [7], 64, 1e4), [30], 64, 1e4)
    np.testing.assert_allclose(a, orope.rope(q[None], [37], 64, 1e4), atol=1e-12)
    np.testing.assert_array_equal(orope.rope(q[None], [0], 64, 1e4), q[None])
    assert abs(np.linalg.norm(orope.rope(q[None], [999], 64, 1e4)) - np.linalg.norm(q)) < 1e-12


def test_positions_follow_branch_depth():
    # a chain tree sits at consecutive positions; siblings share one
    np.testing.assert_array_equal(orope.tree_positions(50, np.arange(5)), 50 + np.arange(5))
    depth = np.array([[0, 1, 1, 2, 1], [0, 1, 2, 3, 4]])
    np.testing.assert_array_equal(orope.tree_positions(np.array([10, 3]), depth),
                                  [[10, 11, 11, 12, 11], [3, 4, 5, 6, 7]])


def test_chain_tree_equals_sequential_decoding():
    # a chain tree verified in one pass equals attention of a plain sequence whose
    # keys were rotated one token at a time at positions P, P+1, ...
    rng = np.random.default_rng(5)
    P, T, Hq, Hkv, D, rot = 6, 4, 2, 1, 16, 8
    pos_all = np.arange(P + T)
    k_all = rng.standard_normal((P + T, Hkv, D))
    v_all = rng.standard_normal((P + T, Hkv, D))
    q = rng.standard_normal((T, Hq, D))
    k_rot = np.stack([orope.rope(k_all[t], np.full(Hkv, t), rot, 1e4) for t in range(P + T)])
    anc = np.array([0] + [(1 << i) - 1 for i in range(1, T)], dtype=np.uint64)  # row i: rows 1..i
    depth = np.arange(T)
    qr, kt, vt = orope.rope_tree_inputs(q, k_all[P:], v_all[P:], P, depth, rot, 1e4)
    o = oattn.tree_attention(qr, k_rot[:P].transpose(1, 0, 2), v_all[:P].transpose(1, 0, 2), P, kt, vt, anc)
    for i in range(T):
        qi = orope.rope(q[i], np.full(Hq, P + i), rot, 1e4)
        keys, vals = k_rot[:P + i + 1, 0], v_all[:P + i + 1, 0]
        for h in range(Hq):
            s = keys @ qi[h] / np.sqrt(D)
            w = np.exp(s - s.max())
            np.testing.assert_allclose(o[i, h], (w / w.sum()) @ vals, atol=1e-12)
