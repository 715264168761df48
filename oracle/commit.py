"""Accepted-path commit into the contiguous committed buffers (oracle).

Sources: "DDTree on vLLM: candid research notes", section "Why hybrid
attention makes it hard": once a path is accepted, only that path is copied
into the contiguous KV and recurrent buffers; section "Where the next step is":
an explicit accepted-branch commit keyed by node and parent ids.  "From DDTree
to drafter training", section "The Architecture of DDTree": the KV cache keeps
only the accepted path's entries.

Readings: the root plus the a accepted rows land at cache
positions P..P+a; the recurrent and conv state of the deepest accepted row
(the root when a = 0) replace the committed state; prefix_len grows by a+1.
A sequence whose prefix would exceed the cache capacity Pmax is left
untouched and reported with acc_len = -1, as is a sequence whose acc_len is
already negative or one of whose accepted rows is not a tree row (malformed
input, reading R23: nothing is written for it).
"""

import numpy as np


def _copy64(a):
    """Copy promoted to float64, so that copying float64 scratch is exact."""
    return np.array(a, dtype=np.float64, copy=True)


def commit(acc_rows, acc_len, prefix_len, kv_layers, gdn_layers, Pmax, T=None):
    """One sequence.  T (tree rows) defaults to the rows of the layers' scratch.

    kv_layers:  list of dicts with k_tree, v_tree [Hkv][T][D], k_cache, v_cache [Hkv][Pmax][D]
    gdn_layers: list of dicts with S_scratch [T][H][dv][dk], S [H][dv][dk],
                conv_scratch [T][W-1][C], conv_state [W-1][C]
    Returns (new_prefix_len, new_acc_len, new_kv_layers, new_gdn_layers); the
    inputs are not modified.
    """
    a = int(acc_len)
    P = int(prefix_len)
    kv_out = [{k: _copy64(v) for k, v in lay.items()} for lay in kv_layers]
    gdn_out = [{k: _copy64(v) for k, v in lay.items()} for lay in gdn_layers]
    if T is None:
        T = (kv_layers[0]["k_tree"].shape[1] if kv_layers else
             gdn_layers[0]["S_scratch"].shape[0] if gdn_layers else None)
    if a < 0 or P + a + 1 > Pmax:
        return P, -1, kv_out, gdn_out
    rows = [int(r) for r in acc_rows[: a + 1]]
    if len(rows) < a + 1 or (T is not None and any(r < 0 or r >= T for r in rows)):
        return P, -1, kv_out, gdn_out
    for lay in kv_out:
        for j, r in enumerate(rows):
            lay["k_cache"][:, P + j, :] = lay["k_tree"][:, r, :]
            lay["v_cache"][:, P + j, :] = lay["v_tree"][:, r, :]
    last = rows[-1]
    for lay in gdn_out:
        lay["S"][...] = lay["S_scratch"][last]
        lay["conv_state"][...] = lay["conv_scratch"][last]
    return P + a + 1, a, kv_out, gdn_out
