"""Score-gap guard for seeded draft logits (test infrastructure).

The tree topology must come out bit-identical from the fp32 GPU build and the
fp64 oracle.  Scores are sums of log-probs, so two prefixes whose scores lie
within rounding of each other could be ordered differently by the two sides.
The workloads therefore only use drafter logits whose best B+1 prefixes, in
heap order, are separated by more than ``eps`` -- except pairs whose per-depth
logit values are identical, which both sides tie exactly and break by token id
and parent row.  ``first_gapped_seed`` redraws with seed+1, seed+2, ... until
that holds.
"""

import numpy as np

from . import tree as _tree


def path_values(z, tree, i):
    """Drafter logit values along row i's root path, root excluded."""
    vals = []
    while i > 0:
        vals.append(float(z[tree["depth"][i] - 1, tree["tok"][i]]))
        i = int(tree["parent"][i])
    return tuple(reversed(vals))


def gaps_ok(draft_logits, B, eps=1e-4):
    """True when every adjacent pair among the best B+1 prefixes is separated by
    more than eps or is an exact tie of identical per-depth values."""
    z = np.asarray(draft_logits, dtype=np.float64)
    t = _tree.build_tree(z, B + 1, root_token=0)
    for i in range(1, B + 1):
        if t["tok"][i + 1] < 0:
            break
        if t["score"][i] - t["score"][i + 1] > eps:
            continue
        if path_values(z, t, i) != path_values(z, t, i + 1):
            return False
    return True


def batch_gaps_ok(draft_logits, B, eps=1e-4):
    return all(gaps_ok(draft_logits[s], B, eps) for s in range(len(draft_logits)))


def first_gapped_seed(make, B, seed, eps=1e-4, max_tries=200):
    """Call make(seed) -> (draft logits as seen by the kernels [n][L][V], extra)
    for seed, seed+1, ... and return (seed, logits, extra) of the first draw
    whose every sequence passes gaps_ok."""
    for s in range(seed, seed + max_tries):
        z, extra = make(s)
        if batch_gaps_ok(z, B, eps):
            return s, z, extra
    raise RuntimeError("no gapped draw within %d seeds from %d" % (max_tries, seed))
