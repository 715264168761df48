"""Pins for the oracle's tree build (per-depth top-K + best-first expansion).

The oracle's heap is checked against things other than itself: brute-force
enumeration of prefixes (scored with scipy's log_softmax), full enumeration of
the whole vocabulary on a tiny case, a hand-worked example with exact ties,
special cases with a known answer, and structural invariants.
"""

import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import log_softmax as sp_log_softmax

from oracle import tree as otree
from tree_speculative_decoding_ddt_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def row_paths(t):
    """Token path (root excluded) of every used row."""
    paths = []
    for i in range(len(t["tok"])):
        if t["tok"][i] < 0:
            break
        p, j = [], i
        while j > 0:
            p.append(int(t["tok"][j]))
            j = int(t["parent"][j])
        paths.append(tuple(reversed(p)))
    return paths


def brute_force_top(z, B, max_rank=None):
    """Enumerate every prefix (tokens restricted to the max_rank best per depth
    when given), score it by summed log-softmax, return the B best token paths."""
    lp = sp_log_softmax(np.asarray(z, np.float64), axis=-1)
    L, V = lp.shape
    cands = [np.argsort(-lp[d], kind="stable")[: (max_rank or V)] for d in range(L)]
    scored = []
    for d in range(1, L + 1):
        for toks in itertools.product(*cands[:d]):
            scored.append((sum(lp[e, toks[e]] for e in range(d)), toks))
    scored.sort(key=lambda s: -s[0])
    return [s[1] for s in scored[:B]], [s[0] for s in scored[:B]]


@pytest.mark.parametrize("seed", range(4))
def test_heap_equals_brute_force_rank_limited(seed):
    # config[0] drafter shape: V=512, L=4, B=8 -> 4680 candidate prefixes
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((4, 512)) * 2.0
    t = otree.build_tree(z, 8, root_token=7)
    paths, scores = brute_force_top(z, 8, max_rank=8)
    assert row_paths(t)[1:] == paths
    np.testing.assert_allclose(t["score"][1:], scores, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed,B", [(0, 8), (1, 20), (2, 5)])
def test_heap_equals_full_enumeration(seed, B):
    # whole vocabulary, no rank limit: also pins that K = B candidates suffice
    rng = np.random.default_rng(100 + seed)
    z = rng.standard_normal((4, 16)) * 1.5
    t = otree.build_tree(z, B, root_token=0)
    paths, scores = brute_force_top(z, B)
    assert row_paths(t)[1:] == paths
    np.testing.assert_allclose(t["score"][1:], scores, rtol=0, atol=1e-12)


def test_hand_worked_example_with_ties():
    g = json.load(open(os.path.join(GOLDEN, "tree_hand_example.json")))
    z = np.log(np.array(g["logits_ln"], dtype=np.float64))
    t = otree.build_tree(z, g["B"], root_token=g["root_token"])
    assert t["tok"].tolist() == g["tok"]
    assert t["parent"].tolist() == g["parent"]
    assert t["depth"].tolist() == g["depth"]
    np.testing.assert_allclose(np.exp(t["score"]), g["prob"], rtol=1e-12)
    want = [sum(1 << b for b in bits) for bits in g["anc_bits"]]
    assert [int(a) for a in t["anc"]] == want


def check_invariants(z, t, B):
    lp = sp_log_softmax(np.asarray(z, np.float64), axis=-1)
    T = B + 1
    assert len(t["tok"]) == T
    used = int((t["tok"] >= 0).sum())
    assert t["parent"][0] == -1 and t["depth"][0] == 0 and t["score"][0] == 0 and t["anc"][0] == 0
    for i in range(1, used):
        p = int(t["parent"][i])
        assert 0 <= p < i, "parents precede children"
        assert t["depth"][i] == t["depth"][p] + 1
        np.testing.assert_allclose(t["score"][i], t["score"][p] + lp[t["depth"][i] - 1, t["tok"][i]],
                                   rtol=0, atol=1e-12)
        assert t["score"][i] <= t["score"][i - 1] + 1e-12, "pop order is best-first"
        # ancestor closure recomputed by walking the parent chain
        want, j = 0, i
        while j > 0:
            want |= 1 << (j - 1)
            j = int(t["parent"][j])
        assert int(t["anc"][i]) == want
    # siblings carry distinct tokens; the tree is prefix-closed by construction of parents
    sib = {}
    for i in range(1, used):
        key = (int(t["parent"][i]), int(t["tok"][i]))
        assert key not in sib
        sib[key] = i
    paths = row_paths(t)
    assert len(set(paths)) == len(paths)
    for pth in paths[1:]:
        assert pth[:-1] in set(paths)


@pytest.mark.parametrize("seed", range(3))
def test_invariants_config1_shape(seed):
    # config[1]-like drafter logits (bf16-rounded, planted peaks) at a reduced vocab
    rng = np.random.default_rng(seed)
    z = synth.draft_logits(rng, 1, 15, 4096, 3.0, plant_p=0.6)
    _, zf = synth.quantize(z, "bf16")
    for B in (32, 64):
        t = otree.build_tree(zf[0], B, root_token=1)
        assert (t["tok"] >= 0).all()
        check_invariants(zf[0], t, B)


def test_single_depth_is_top_b_of_one_row():
    rng = np.random.default_rng(3)
    z = rng.integers(-3, 4, size=(1, 50)).astype(np.float64)  # many exact ties
    t = otree.build_tree(z, 12, root_token=0)
    want = np.argsort(-z[0], kind="stable")[:12]  # stable: equal values keep id order
    assert t["tok"][1:].tolist() == want.tolist()
    assert (t["parent"][1:] == 0).all()


def test_dominant_peaks_give_top1_chain():
    rng = np.random.default_rng(4)
    L, V = 6, 300
    z = rng.standard_normal((L, V))
    peaks = rng.integers(0, V, size=L)
    z[np.arange(L), peaks] = 30.0
    t = otree.build_tree(z, L, root_token=0)
    assert t["tok"][1:].tolist() == peaks.tolist()
    assert t["parent"].tolist() == [-1] + list(range(L))


def test_small_tree_leaves_unused_rows():
    # V=2, L=2 has only 6 prefixes: a budget of 10 leaves 4 rows unused
    z = np.array([[0.0, 1.0], [2.0, 0.0]])
    t = otree.build_tree(z, 10, root_token=0)
    assert (t["tok"][7:] == -1).all() and (t["parent"][7:] == -1).all()
    assert np.isneginf(t["score"][7:]).all() and (t["anc"][7:] == 0).all()
    assert sorted(row_paths(t)[1:]) == sorted([(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)])

