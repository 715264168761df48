"""Target argmax and greedy tree walk (oracle).

Sources: "From DDTree to drafter training", section "The Architecture of
DDTree": after the verify pass, walk down the tree from the root while the
target's token at the current node matches one of its children.  "DDTree on
vLLM: candid research notes", section "What broke along the way": accepted and
emitted tokens are kept apart -- the bonus token is emitted but is not an
accepted draft node.

Readings: greedy acceptance; argmax ties go to the lowest token
id; a = number of accepted non-root nodes; acc_rows lists the root then the
accepted rows, padded with -1 to L+1 entries; bonus = target argmax at the last
accepted row.  Sibling tokens are distinct, so at most one child can match.
"""

import numpy as np


def argmax_lowest(row):
    row = np.asarray(row)
    return int(np.flatnonzero(row == row.max())[0])


def tree_accept(target_logits, tok, parent, L):
    """target_logits [T][V], tok/parent [T] -> (acc_rows [L+1], a, bonus)."""
    return walk([argmax_lowest(target_logits[i]) for i in range(len(tok))], tok, parent, L)


def walk(t, tok, parent, L):
    """The walk given the target's token t[i] of every row -> (acc_rows [L+1], a, bonus)."""
    T = len(tok)
    path = [0]
    cur = 0
    while True:
        match = [c for c in range(1, T) if parent[c] == cur and tok[c] == t[cur]]
        assert len(match) <= 1, "sibling tokens must be distinct"
        if not match:
            break
        cur = match[0]
        path.append(cur)
    a = len(path) - 1
    acc_rows = np.full(L + 1, -1, dtype=np.int64)
    acc_rows[: len(path)] = path
    return acc_rows, a, t[cur]


def tree_accept_batch(target_logits, tok, parent, L):
    outs = [tree_accept(target_logits[s], tok[s], parent[s], L) for s in range(len(tok))]
    return (np.stack([o[0] for o in outs]), np.array([o[1] for o in outs]),
            np.array([o[2] for o in outs]))
