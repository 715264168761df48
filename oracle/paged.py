"""Paged KV cache: the committed prefix held in fixed-size pages named by a block
table, read through a page gather (oracle).

Sources: "DDTree on vLLM: candid research notes", sections "Why hybrid attention
makes it hard" and "Where the next step is": the tree's ancestor-mask attention is
to run over the serving engine's paged KV blocks, and the accepted path is then
written into the committed KV.  "From DDTree to drafter training", section "The
Architecture of DDTree": the cache keeps only the accepted path's entries.

Readings: a page holds page_size consecutive positions of every kv
head, pool layout [num_pages][Hkv][page_size][D]; position p of sequence s lives in
page block_table[s][p // page_size] at slot p % page_size.  Attention and commit
are exactly those of the contiguous cache after this gather (and its inverse
scatter for the commit).
"""

import numpy as np

from . import attention as _attention
from . import commit as _commit


def gather(pages, block_table, length):
    """Pool [num_pages][Hkv][ps][D] + one sequence's block table -> [Hkv][length][D]."""
    pages = np.asarray(pages)
    ps = pages.shape[2]
    pos = np.arange(length)
    return np.ascontiguousarray(pages[np.asarray(block_table)[pos // ps], :, pos % ps, :].transpose(1, 0, 2))


def scatter(pages, block_table, start, rows):
    """Write rows [Hkv][m][D] at positions start.. of one sequence into a copy of the pool."""
    out = np.array(pages, copy=True)
    ps = out.shape[2]
    for j in range(rows.shape[1]):
        p = start + j
        out[block_table[p // ps], :, p % ps, :] = rows[:, j, :]
    return out


def tree_attention_paged(q, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree, anc, scale=None):
    """One sequence: the tree attention of the contiguous cache read through the pages."""
    P = int(prefix_len)
    return _attention.tree_attention(q, gather(k_pages, block_table, P), gather(v_pages, block_table, P), P,
                                     k_tree, v_tree, anc, scale)


def commit_paged(acc_rows, acc_len, prefix_len, k_tree, v_tree, k_pages, v_pages, block_table):
    """One sequence, one layer: the contiguous commit of the accepted rows, with the
    capacity len(block_table) * page_size, scattered into the pages.
    Returns (new_prefix_len, new_acc_len, k_pages, v_pages) (copies)."""
    ps = np.shape(k_pages)[2]
    cap = len(block_table) * ps
    a, P = int(acc_len), int(prefix_len)
    if a < 0 or P + a + 1 > cap:
        return P, -1, np.array(k_pages, copy=True), np.array(v_pages, copy=True)
    rows = [int(r) for r in acc_rows[: a + 1]]
    Hkv, _, D = np.shape(k_tree)
    # the contiguous commit into an empty cache of the capacity, then its new rows moved to the pages
    empty = np.zeros((Hkv, cap, D))
    p1, a1, kv_new, _ = _commit.commit(acc_rows, acc_len, P,
                                       [dict(k_tree=k_tree, v_tree=v_tree, k_cache=empty, v_cache=empty)], [], cap)
    assert (p1, a1) == (P + a + 1, a)
    kn, vn = kv_new[0]["k_cache"][:, P:P + a + 1], kv_new[0]["v_cache"][:, P:P + a + 1]
    assert len(rows) == kn.shape[1]
    return p1, a1, scatter(k_pages, block_table, P, kn), scatter(v_pages, block_table, P, vn)
