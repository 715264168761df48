"""Branch-local short conv + Gated DeltaNet over the draft tree (oracle).

Sources: "DDTree on vLLM: candid research notes", section "Why hybrid
attention makes it hard": Gated DeltaNet layers carry a fixed-size recurrent
state plus a short convolution state, and for a tree every node reads both
from its parent and writes its own to scratch, never to the committed state.
"The architecture of speculation", section "The DDTree Integration
Challenge": the recurrent state cannot be shared across branches.

The pages never write the recurrence down.  Readings:
  * conv: depthwise causal, width W, no bias, SiLU after.  Tap W-1 multiplies
    the current input; the state is the last W-1 inputs, oldest first.
    Channels C = 2*H*dk hold [q | k]; v, beta and g bypass the conv.
  * delta rule, per head, state S [dv][dk]:
        S' = g * S_parent;  u = S' k;  S = S' + beta (v - u) k^T;  o = S q
    with k L2-normalised as k / sqrt(sum k^2 + 1e-6) and q scaled by dk**-0.5.
  * the root (parent -1) reads the committed conv state and S.
Rows are processed in increasing order; a parent row always precedes its
children (the tree build numbers rows in pop order).
"""

import numpy as np

K_NORM_EPS = 1e-6


def silu(x):
    return x / (1.0 + np.exp(-x))


def short_conv_tree(x, conv_w, conv_state, parent):
    """x [T][C], conv_w [C][W], conv_state [W-1][C] -> y [T][C], conv_scratch [T][W-1][C]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(conv_w, dtype=np.float64)
    state0 = np.asarray(conv_state, dtype=np.float64)
    T, C = x.shape
    W = w.shape[1]
    scratch = np.empty((T, W - 1, C), dtype=np.float64)
    y = np.empty((T, C), dtype=np.float64)
    for i in range(T):
        assert parent[i] < i, "a parent row must precede its child"
        prev = state0 if parent[i] < 0 else scratch[parent[i]]
        window = np.concatenate([prev, x[i][None, :]], axis=0)  # [W][C], last = current
        y[i] = silu(np.einsum("jc,cj->c", window, w))
        scratch[i] = window[1:]
    return y, scratch


def gated_delta_tree(q, k, v, beta, g, S0, parent):
    """q, k [T][H][dk] (already scaled / normalised), v [T][H][dv], beta, g [T][H],
    S0 [H][dv][dk] -> o [T][H][dv], S_scratch [T][H][dv][dk]."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    beta, g = np.asarray(beta, np.float64), np.asarray(g, np.float64)
    S0 = np.asarray(S0, dtype=np.float64)
    T, H, dk = k.shape
    dv = v.shape[2]
    S = np.empty((T, H, dv, dk), dtype=np.float64)
    o = np.empty((T, H, dv), dtype=np.float64)
    for i in range(T):
        assert parent[i] < i, "a parent row must precede its child"
        Sp = S0 if parent[i] < 0 else S[parent[i]]
        for h in range(H):
            Sd = g[i, h] * Sp[h]
            u = Sd @ k[i, h]
            S[i, h] = Sd + beta[i, h] * np.outer(v[i, h] - u, k[i, h])
            o[i, h] = S[i, h] @ q[i, h]
    return o, S


def split_qk(y, H, dk):
    """Split conv output [T][2*H*dk] into per-head q (scaled) and k (L2-normalised)."""
    T = y.shape[0]
    q = y[:, : H * dk].reshape(T, H, dk) * dk ** -0.5
    k = y[:, H * dk: 2 * H * dk].reshape(T, H, dk)
    k = k / np.sqrt((k * k).sum(axis=-1, keepdims=True) + K_NORM_EPS)
    return q, k


def gdn_tree_step(x, conv_w, conv_state, v, beta, g, S0, parent, H, dk):
    """One GDN layer over the tree for one sequence.

    Returns (o [T][H][dv], S_scratch [T][H][dv][dk], conv_scratch [T][W-1][C]).
    """
    y, conv_scratch = short_conv_tree(x, conv_w, conv_state, parent)
    q, k = split_qk(y, H, dk)
    o, S_scratch = gated_delta_tree(q, k, v, beta, g, S0, parent)
    return o, S_scratch, conv_scratch


def gdn_tree_step_batch(x, conv_w, conv_state, v, beta, g, S0, parent, H, dk):
    outs = [gdn_tree_step(x[s], conv_w, conv_state[s], v[s], beta[s], g[s], S0[s],
                          parent[s], H, dk) for s in range(len(x))]
    return tuple(np.stack([o[j] for o in outs]) for j in range(3))
