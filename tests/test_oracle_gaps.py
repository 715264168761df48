"""Pins for the oracle's score-gap guard (oracle/gaps.py) and its ancestor masks.

The guard decides which drafter draws the bit-exact topology claim covers: the
best B+1 prefixes must be pairwise more than 1e-4 apart in heap order, unless two
of them carry identical per-depth logit values (an exact tie that both sides break
by token id).  It is pinned here against hand-built draws whose gaps are known by
construction, and against an independent brute-force enumeration of every prefix
of a tiny vocabulary.

Source: "From DDTree to drafter training", section "The Architecture of DDTree"
(best-first tree of the B best prefixes, ties to the lower token id).
"""

import itertools

import numpy as np
import pytest
from scipy.special import log_softmax as sp_log_softmax

from oracle import gaps, tree as otree


def one_depth(values, V=12, low=-30.0):
    """A single-depth draw whose best logits are `values` (token ids 0, 1, ...), the
    rest far below: score differences equal logit differences exactly."""
    z = np.full((1, V), low)
    z[0, : len(values)] = values
    return z


def test_gap_below_eps_fails():
    assert not gaps.gaps_ok(one_depth([0.0, -5e-5]), B=1)


def test_gap_above_eps_passes():
    assert gaps.gaps_ok(one_depth([0.0, -2e-4]), B=1)


def test_exact_tie_of_identical_values_passes():
    # tokens 0 and 1 carry the same logit: scores tie exactly, values identical
    assert gaps.gaps_ok(one_depth([0.0, 0.0, -1.0]), B=2)


def test_exact_tie_of_different_values_fails():
    # two depths: (a, b) and (b, a) sum to the same score with different per-depth values
    z = np.full((2, 8), -30.0)
    z[0, 0], z[0, 1] = 0.0, -0.5
    z[1, 0], z[1, 1] = 0.0, -0.5
    # prefixes by score: (0) , (0,0), (1), (0,1), (1,0) ... ; (0,1) and (1,0) tie
    t = otree.build_tree(z, 6, root_token=0)
    assert gaps.path_values(z, t, 4) != gaps.path_values(z, t, 5)
    assert t["score"][4] == t["score"][5]
    assert not gaps.gaps_ok(z, B=4)   # the tied pair is rows 4, 5: inside the best B+1 = 5
    assert gaps.gaps_ok(z, B=3)       # only rows 1..4 matter: the tie sits past them


def test_near_tie_only_matters_up_to_b_plus_one():
    # four well separated prefixes, then a near tie between the 4th and 5th best
    vals = [0.0, -1.0, -2.0, -3.0, -3.00005, -9.0]
    z = one_depth(vals)
    assert not gaps.gaps_ok(z, B=5)   # rows 4 and 5 both inside the tree
    assert not gaps.gaps_ok(z, B=4)   # the B-th and (B+1)-th best: the boundary pair
    assert gaps.gaps_ok(z, B=3)       # the near tie lies past the best B+1 = 4


def test_gap_measured_on_summed_scores():
    # depth-1 values well apart; at depth 2 the child of token 0 lands 5e-5 from token 1
    z = np.full((2, 8), -30.0)
    z[0, 0], z[0, 1] = 0.0, -0.7
    z[1, 0] = 0.0
    lp = sp_log_softmax(z, axis=-1)
    # choose depth-2 token 1 so that lp(0) + lp2(1) = lp(1) - 5e-5
    want = lp[0, 1] - 5e-5 - lp[0, 0]
    # solve log_softmax(z1)[1] = want with the other entries fixed: z1[1] = want + lse
    z1 = z[1].copy()
    for _ in range(60):  # fixed point: lse depends weakly on z1[1]
        lse = np.log(np.exp(z1 - z1.max()).sum()) + z1.max()
        z1[1] = want + lse
    z[1] = z1
    lp = sp_log_softmax(z, axis=-1)
    assert abs((lp[0, 0] + lp[1, 1]) - (lp[0, 1] - 5e-5)) < 1e-12
    assert not gaps.gaps_ok(z, B=3)


def brute_force_gaps_ok(z, B, eps=1e-4):
    """Independent check: every prefix of the whole vocabulary, scored with scipy,
    sorted by score; the best B+1 must be pairwise > eps apart when adjacent unless
    their per-depth values are identical."""
    lp = sp_log_softmax(np.asarray(z, np.float64), axis=-1)
    L, V = lp.shape
    pref = []
    for d in range(1, L + 1):
        for toks in itertools.product(range(V), repeat=d):
            pref.append((sum(lp[e, toks[e]] for e in range(d)), toks))
    pref.sort(key=lambda s: -s[0])
    top = pref[: B + 1]
    for (s0, t0), (s1, t1) in zip(top, top[1:]):
        if s0 - s1 > eps:
            continue
        if tuple(z[e, t0[e]] for e in range(len(t0))) != tuple(z[e, t1[e]] for e in range(len(t1))):
            return False
    return True


@pytest.mark.parametrize("seed", range(8))
def test_guard_equals_brute_force(seed):
    # V 8, L 4 (4680 prefixes); some draws carry planted near ties and exact ties
    rng = np.random.default_rng(500 + seed)
    z = rng.standard_normal((4, 8)) * 1.5
    o0, o2 = np.argsort(-z[0]), np.argsort(-z[2])
    if seed % 4 == 1:
        z[0, o0[1]] = z[0, o0[0]] - 3e-5         # near tie of the two best at depth 1
    if seed % 4 == 2:
        z[1, 5] = z[1, 6]                        # exact tie of values at depth 2
        z[2, o2[2]] = z[2, o2[1]] - 2e-5         # near tie of ranks 1 and 2 at depth 3
    if seed % 4 == 3:
        z[0, :] = np.round(z[0, :], 0)           # many exact ties
    for B in (3, 6, 12, 25):
        assert gaps.gaps_ok(z, B) == brute_force_gaps_ok(z, B), (seed, B)


def test_first_gapped_seed_skips_ungapped_draws():
    # seeds 0 and 1 draw a near tie; seed 2 is the first clean draw
    def make(s):
        vals = [0.0, -5e-5] if s < 2 else [0.0, -1.0]
        return one_depth(vals)[None], s
    s, z, extra = gaps.first_gapped_seed(make, 1, 0)
    assert s == 2 and extra == 2 and gaps.gaps_ok(z[0], 1)


def test_ancestor_masks_match_the_parent_chain():
    # hand-made parents; bit j <-> row j+1; root implicit
    parent = np.array([-1, 0, 0, 1, 3, 2, 1])
    want = [0, 0b1, 0b10, 0b101, 0b1101, 0b10010, 0b100001]
    assert [int(a) for a in otree.ancestor_masks(parent)] == want
    # and equal to the masks the tree build writes
    rng = np.random.default_rng(9)
    t = otree.build_tree(rng.standard_normal((5, 40)), 30, root_token=0)
    assert [int(a) for a in otree.ancestor_masks(t["parent"])] == [int(a) for a in t["anc"]]
