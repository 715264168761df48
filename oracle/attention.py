"""Tree-masked attention as a dense masked softmax (oracle).

Sources: "DDTree on vLLM: candid research notes", section "Why hybrid
attention makes it hard": every candidate row attends to the committed prefix
plus its own ancestors and never to its siblings.  "From DDTree to drafter
training", section "The Architecture of DDTree": the whole tree is verified in
one target pass with an ancestor-only attention mask.

Readings: query head h reads kv head h // (Hq/Hkv); scale defaults
to D**-0.5; row i sees prefix keys [0, P), tree row 0 (the root), and tree row
j+1 for every set bit j of anc[i] (which includes row i itself).  Tree keys and
values sit in their own buffers, separate from the committed cache.
"""

import numpy as np


def visible_tree_rows(anc_i):
    """Tree rows visible to a row whose ancestor-or-self mask is anc_i."""
    anc_i = int(anc_i)
    return [0] + [j + 1 for j in range(64) if (anc_i >> j) & 1]


def tree_attention(q, k_cache, v_cache, prefix_len, k_tree, v_tree, anc, scale=None):
    """One sequence, one layer.

    q       [T][Hq][D]     queries of the tree rows
    k_cache [Hkv][>=P][D]  committed keys (rows >= prefix_len are ignored)
    v_cache [Hkv][>=P][D]
    k_tree  [Hkv][T][D]    keys/values of the tree rows themselves
    v_tree  [Hkv][T][D]
    anc     [T] uint64     ancestor-or-self masks
    Returns o [T][Hq][D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = k_cache.shape[0]
    G = Hq // Hkv
    P = int(prefix_len)
    scale = D ** -0.5 if scale is None else scale

    mask = np.zeros((T, P + T), dtype=bool)
    mask[:, :P] = True
    for i in range(T):
        for j in visible_tree_rows(anc[i]):
            mask[i, P + j] = True

    o = np.empty((T, Hq, D), dtype=np.float64)
    for h in range(Hq):
        kvh = h // G
        keys = np.concatenate([np.asarray(k_cache[kvh, :P], np.float64),
                               np.asarray(k_tree[kvh], np.float64)], axis=0)
        vals = np.concatenate([np.asarray(v_cache[kvh, :P], np.float64),
                               np.asarray(v_tree[kvh], np.float64)], axis=0)
        s = scale * (q[:, h, :] @ keys.T)
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ vals
    return o


def tree_attention_batch(q, k_cache, v_cache, prefix_len, k_tree, v_tree, anc, scale=None):
    """Batch form: leading dimension n on every array argument."""
    return np.stack([tree_attention(q[s], k_cache[s], v_cache[s], prefix_len[s],
                                    k_tree[s], v_tree[s], anc[s], scale)
                     for s in range(len(q))])


def tree_attention_row(q_row, k_cache, v_cache, prefix_len, k_tree, v_tree, anc_i, scale=None):
    """A single tree row (q_row [Hq][D]); used to sample large parity cases."""
    q_row = np.asarray(q_row, dtype=np.float64)
    Hq, D = q_row.shape
    Hkv = k_cache.shape[0]
    G = Hq // Hkv
    P = int(prefix_len)
    scale = D ** -0.5 if scale is None else scale
    rows = visible_tree_rows(anc_i)
    o = np.empty((Hq, D), dtype=np.float64)
    for h in range(Hq):
        kvh = h // G
        keys = np.concatenate([np.asarray(k_cache[kvh, :P], np.float64),
                               np.asarray(k_tree[kvh, rows], np.float64)], axis=0)
        vals = np.concatenate([np.asarray(v_cache[kvh, :P], np.float64),
                               np.asarray(v_tree[kvh, rows], np.float64)], axis=0)
        s = scale * (keys @ q_row[h])
        s = s - s.max()
        p = np.exp(s)
        o[h] = (p / p.sum()) @ vals
    return o
