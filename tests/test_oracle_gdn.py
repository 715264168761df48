"""Pins for the oracle's short conv + Gated DeltaNet tree step.

Checked against: a separately written sequential chain replay of every
root-to-leaf path (conv through np.convolve, state update in the matrix form
S_t = g S_{t-1} (I - beta k k^T) + beta v k^T), closed forms (beta=0 & g=1
keeps the state; beta=1 with unit k stores v exactly; a hand-computed 2x2
update; an identity tap turns the conv into SiLU), exact copies in the conv
scratch, and branch locality (a sibling's inputs never reach a node).
"""

import numpy as np
import pytest
from scipy.special import expit

from oracle import gdn as ogdn
from tree_speculative_decoding_ddt_amd import synth


def paths_to_leaves(parent):
    T = len(parent)
    kids = {i: [] for i in range(T)}
    for i in range(1, T):
        kids[int(parent[i])].append(i)
    out = []
    for leaf in (i for i in range(T) if not kids[i]):
        p = [leaf]
        while p[-1] != 0:
            p.append(int(parent[p[-1]]))
        out.append(p[::-1])
    return out


def chain_replay(path, x, conv_w, conv_state, v, beta, g, S0, H, dk):
    """Sequential replay of one root path; returns per-position (o, S, conv window)."""
    W = conv_w.shape[1]
    C = x.shape[1]
    xs = np.asarray(x[path], np.float64)  # [m][C]
    hist = np.concatenate([np.asarray(conv_state, np.float64), xs])  # [W-1+m][C]
    y = np.stack([np.convolve(hist[:, c], np.asarray(conv_w[c], np.float64)[::-1], mode="valid")
                  for c in range(C)], axis=1)
    y = y * expit(y)
    S = np.asarray(S0, np.float64).copy()
    res = []
    for t, r in enumerate(path):
        o = np.empty((H, v.shape[2]))
        for h in range(H):
            q = y[t, h * dk:(h + 1) * dk] / np.sqrt(dk)
            k = y[t, H * dk + h * dk: H * dk + (h + 1) * dk]
            k = k / np.sqrt(k @ k + 1e-6)
            I = np.eye(dk)
            S[h] = g[r, h] * S[h] @ (I - beta[r, h] * np.outer(k, k)) + beta[r, h] * np.outer(v[r, h], k)
            o[h] = S[h] @ q
        res.append((o, S.copy(), hist[t + 1: t + W]))
    return res


@pytest.mark.parametrize("seed", range(3))
def test_tree_matches_chain_replay(seed):
    rng = np.random.default_rng(seed)
    B, L, H, dk, W = 10, 4, 2, 8, 4
    parent, _ = synth.random_parents(rng, B, L)
    x = {k: v[0] if k != "conv_w" else v for k, v in synth.gdn_inputs(rng, 1, B + 1, H, dk, dk, W).items()}
    o, S, cs = ogdn.gdn_tree_step(x["x"], x["conv_w"], x["conv_state"], x["v"], x["beta"], x["g"],
                                  x["S"], parent, H, dk)
    for path in paths_to_leaves(parent):
        rep = chain_replay(path, x["x"], x["conv_w"], x["conv_state"], x["v"], x["beta"], x["g"],
                           x["S"], H, dk)
        for r, (o_r, S_r, win) in zip(path, rep):
            np.testing.assert_allclose(o[r], o_r, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(S[r], S_r, rtol=1e-10, atol=1e-12)
            np.testing.assert_array_equal(cs[r], win)  # the conv scratch is an exact copy


def test_conv_scratch_exact_copies_short_path():
    # a depth-1 node's conv scratch holds the last two committed rows then its own input
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 6))
    st = rng.standard_normal((3, 6))
    w = rng.standard_normal((6, 4))
    _, cs = ogdn.short_conv_tree(x, w, st, np.array([-1, 0, 1]))
    np.testing.assert_array_equal(cs[0], np.stack([st[1], st[2], x[0]]))
    np.testing.assert_array_equal(cs[1], np.stack([st[2], x[0], x[1]]))
    np.testing.assert_array_equal(cs[2], np.stack([x[0], x[1], x[2]]))


def test_identity_tap_is_silu():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 8)) * 3
    w = np.zeros((8, 4))
    w[:, 3] = 1.0
    y, _ = ogdn.short_conv_tree(x, w, rng.standard_normal((3, 8)), np.array([-1, 0, 0, 1, 2]))
    np.testing.assert_allclose(y, x * expit(x), rtol=1e-14, atol=0)


def test_zero_beta_unit_gate_keeps_state():
    rng = np.random.default_rng(7)
    T, H, dk = 6, 2, 4
    parent = np.array([-1, 0, 1, 0, 3, 2])
    q, k, v = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk))
    S0 = rng.standard_normal((H, dk, dk))
    o, S = ogdn.gated_delta_tree(q, k, v, np.zeros((T, H)), np.ones((T, H)), S0, parent)
    for i in range(T):
        np.testing.assert_array_equal(S[i], S0)
        np.testing.assert_allclose(o[i], np.einsum("hvk,hk->hv", S0, q[i]), rtol=1e-14)


def test_unit_beta_stores_value():
    rng = np.random.default_rng(8)
    T, H, dk = 5, 3, 6
    parent = np.array([-1, 0, 1, 1, 3])
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dk))
    _, S = ogdn.gated_delta_tree(rng.standard_normal((T, H, dk)), k, v, np.ones((T, H)),
                                 rng.uniform(0.9, 1, (T, H)), rng.standard_normal((H, dk, dk)), parent)
    for i in range(T):
        np.testing.assert_allclose(np.einsum("hvk,hk->hv", S[i], k[i]), v[i], rtol=1e-12, atol=1e-12)


def test_hand_computed_update():
    # S0 = [[1,2],[3,4]], k = e1, v = [5,6], beta = g = 1/2, q = [1,1]:
    # S' = [[.5,1],[1.5,2]], u = [.5,1.5], S = S' + .5*[4.5,4.5] e1^T = [[2.75,1],[3.75,2]], o = [3.75,5.75]
    o, S = ogdn.gated_delta_tree(np.array([[[1.0, 1.0]]]), np.array([[[1.0, 0.0]]]),
                                 np.array([[[5.0, 6.0]]]), np.array([[0.5]]), np.array([[0.5]]),
                                 np.array([[[1.0, 2.0], [3.0, 4.0]]]), np.array([-1]))
    np.testing.assert_allclose(S[0, 0], [[2.75, 1.0], [3.75, 2.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], [3.75, 5.75], rtol=0, atol=1e-15)


def test_branch_locality():
    rng = np.random.default_rng(9)
    B, H, dk, W = 9, 1, 8, 4
    parent = np.array([-1, 0, 0, 1, 2, 3, 4, 1, 2, 7])
    x = {k: v[0] if k != "conv_w" else v for k, v in synth.gdn_inputs(rng, 1, B + 1, H, dk, dk, W).items()}
    o, S, cs = ogdn.gdn_tree_step(x["x"], x["conv_w"], x["conv_state"], x["v"], x["beta"], x["g"],
                                  x["S"], parent, H, dk)
    # change every input of row 2's subtree; rows on the other branch must not move
    sub = [2, 4, 6, 8]
    x2 = dict(x)
    x2["x"] = x["x"].copy(); x2["x"][sub] += 1.0
    x2["v"] = x["v"].copy(); x2["v"][sub] -= 2.0
    o2, S2, cs2 = ogdn.gdn_tree_step(x2["x"], x["conv_w"], x["conv_state"], x2["v"], x["beta"], x["g"],
                                     x["S"], parent, H, dk)
    for r in (0, 1, 3, 5, 7, 9):
        np.testing.assert_array_equal(o2[r], o[r])
        np.testing.assert_array_equal(S2[r], S[r])
        np.testing.assert_array_equal(cs2[r], cs[r])
