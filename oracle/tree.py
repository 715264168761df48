"""Draft-tree construction: per-depth top-K and best-first expansion (oracle).

Source: "From DDTree to drafter training" (magik.net), section "The
Architecture of DDTree": a block drafter emits one distribution per future
position in a single pass; the tree takes the top-K tokens and their
log-probabilities at every depth, seeds a max-heap with the best depth-1 token,
repeatedly pops the globally best node, pushes that node's next-ranked sibling
and its best child, and stops once the node budget is spent.  The same section
flattens the tree into ids, per-depth positions and an ancestor-only mask.

"DDTree on vLLM: candid research notes" (lotusmake.com), section "What broke
along the way": the drafter's per-depth logits are not conditioned on the
branch, so a node's score is the sum of its path's per-depth log-probs.

Readings where the pages are silent:
  * score(node) = sum over its path of full-vocabulary log-softmax values.
  * K defaults to B, which makes the result exactly the B best prefixes.
  * Heap order: score descending, then token id ascending (the configured tie
    rule), then parent row ascending.  (parent row, token) is unique among
    frontier entries, so this order is total.
  * Row 0 is the root (the caller's token, depth 0, score 0, empty mask);
    popped nodes take rows 1..B in pop order.
  * anc[i] is a 64-bit mask with bit j set when row j+1 is an ancestor of row
    i or row i itself; the root is implicit in every row's mask.
  * If fewer than B prefixes exist, unused rows hold token -1, parent -1,
    depth -1, score -inf and mask 0.
"""

import heapq

import numpy as np


def log_softmax(z):
    """Full-vocabulary log-softmax of each row of ``z`` (float64)."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=-1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True))
    return z - lse


def topk_per_depth(lp, K):
    """Top-K token ids and log-probs per depth, ordered by (lp desc, id asc)."""
    lp = np.asarray(lp, dtype=np.float64)
    L, V = lp.shape
    K = min(K, V)
    ids = np.empty((L, K), dtype=np.int64)
    vals = np.empty((L, K), dtype=np.float64)
    tok = np.arange(V)
    for d in range(L):
        order = np.lexsort((tok, -lp[d]))  # primary -lp, secondary id
        ids[d] = order[:K]
        vals[d] = lp[d, order[:K]]
    return ids, vals


def build_tree(draft_logits, B, root_token, K=None):
    """Best-first draft tree for one sequence.

    draft_logits: [L][V] drafter logits (row d is the distribution of depth d+1).
    Returns a dict of arrays with T = B+1 rows: tok, parent, depth (int64),
    score (float64), anc (uint64).
    """
    z = np.asarray(draft_logits, dtype=np.float64)
    L, V = z.shape
    K = B if K is None else K
    lp = log_softmax(z)
    ids, vals = topk_per_depth(lp, K)
    K = ids.shape[1]
    T = B + 1
    tok = np.full(T, -1, dtype=np.int64)
    parent = np.full(T, -1, dtype=np.int64)
    depth = np.full(T, -1, dtype=np.int64)
    score = np.full(T, -np.inf, dtype=np.float64)
    anc = [0] * T
    tok[0], depth[0], score[0] = int(root_token), 0, 0.0

    # entry: (-score, token, parent row, depth, rank); heapq pops the smallest,
    # i.e. the highest score, then the lowest token, then the lowest parent row.
    frontier = []
    if B > 0 and L > 0:
        heapq.heappush(frontier, (-(0.0 + vals[0, 0]), int(ids[0, 0]), 0, 1, 0))
    rows = 1
    while rows < T and frontier:
        neg, t, p, d, r = heapq.heappop(frontier)
        i = rows
        rows += 1
        tok[i], parent[i], depth[i], score[i] = t, p, d, -neg
        anc[i] = anc[p] | (1 << (i - 1))
        if r + 1 < K:  # next-ranked sibling under the same parent
            heapq.heappush(frontier, (-(score[p] + vals[d - 1, r + 1]),
                                      int(ids[d - 1, r + 1]), p, d, r + 1))
        if d < L:  # best child one depth further down
            heapq.heappush(frontier, (-(score[i] + vals[d, 0]), int(ids[d, 0]), i, d + 1, 0))
    # masks of trees wider than 64 nodes (used only by the gap guard) stay Python ints
    anc = np.array(anc, dtype=np.uint64 if B <= 64 else object)
    return {"tok": tok, "parent": parent, "depth": depth, "score": score, "anc": anc}


def build_tree_batch(draft_logits, B, root_token, K=None):
    """build_tree over a batch: draft_logits [n][L][V], root_token [n]."""
    outs = [build_tree(draft_logits[s], B, root_token[s], K) for s in range(len(draft_logits))]
    return {k: np.stack([o[k] for o in outs]) for k in outs[0]}


def ancestor_masks(parent):
    """Ancestor-or-self bitmask per row from a parent array (root = row 0)."""
    parent = np.asarray(parent)
    anc = [0] * len(parent)
    for i in range(1, len(parent)):
        if parent[i] >= 0:
            anc[i] = anc[parent[i]] | (1 << (i - 1))
    return np.array(anc, dtype=np.uint64)

