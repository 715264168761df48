"""Rotary position embedding by branch depth, for the tree rows (oracle).

Sources: "DDTree on vLLM: candid research notes", section "What broke along the
way" and "Where the next step is": the positions of tree nodes, and RoPE applied
at those positions, must follow the branch depth, not the row order of the
flattened tree.  "From DDTree to drafter training", section "The Architecture of
DDTree": the whole tree is verified in one pass over the committed prefix.

Readings: a tree row at depth d of a sequence with committed prefix
length P sits at position P + d (nodes at one depth share a position; the root,
depth 0, is the token right after the prefix).  RoPE is the rotary embedding of
Su et al. (RoFormer) in the rotate-half layout: the first rot_dim channels of a
head form the rot_dim/2 pairs (j, j + rot_dim/2); pair j turns by the angle
pos * theta**(-2j/rot_dim); channels from rot_dim on pass unchanged.  Queries
and the tree rows' own keys are rotated; values are not.
"""

import numpy as np


def tree_positions(prefix_len, depth):
    """Position of every tree row: prefix_len + depth (depth [T] or [n][T])."""
    depth = np.asarray(depth, dtype=np.int64)
    prefix_len = np.asarray(prefix_len, dtype=np.int64)
    if depth.ndim == 2:
        return prefix_len[:, None] + depth
    return prefix_len + depth


def angles(pos, rot_dim, theta):
    """[..., rot_dim/2] rotation angles pos * theta^(-2j/rot_dim), in float64."""
    j = np.arange(rot_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * j / rot_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x, pos, rot_dim, theta):
    """Rotate x [..., D] at positions pos (shape x.shape[:-2] -- one position per
    token, shared by the heads of axis -2 -- or x.shape[:-1])."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert rot_dim % 2 == 0 and 0 < rot_dim <= D
    half = rot_dim // 2
    pos = np.asarray(pos, dtype=np.float64)
    if pos.ndim == x.ndim - 2:
        pos = pos[..., None]                  # one position for every head of a token
    a = angles(pos, rot_dim, theta)           # broadcasts against x[..., :half]
    c, s = np.cos(a), np.sin(a)
    lo, hi = x[..., :half], x[..., half:rot_dim]
    out = x.copy()
    out[..., :half] = lo * c - hi * s
    out[..., half:rot_dim] = hi * c + lo * s
    return out


def rope_tree_inputs(q, k_new, v_new, prefix_len, depth, rot_dim, theta):
    """One sequence: pre-rotation q [T][Hq][D], k_new, v_new [T][Hkv][D] (token-major,
    as a projection writes them) -> (q rotated [T][Hq][D], k_tree [Hkv][T][D] rotated,
    v_tree [Hkv][T][D]), the tree attention's inputs and the scratch the commit copies."""
    pos = tree_positions(prefix_len, depth)
    qr = rope(q, pos, rot_dim, theta)
    kr = rope(k_new, pos, rot_dim, theta)
    return qr, np.ascontiguousarray(kr.transpose(1, 0, 2)), \
        np.ascontiguousarray(np.asarray(v_new, np.float64).transpose(1, 0, 2))
