"""The oracle's whole verify step on the tiny CPU-checkable workload.

Drafter fp32 N(0,2) vocab 512 depth 4, budget 8; target N(0,2) with the
drafter top-1 planted at p=0.7; one full-attention layer (2 q heads, 1 kv head,
head_dim 64, prefix 128) and one GDN layer (1 head, dk=dv=32, conv width 4 over
64 channels).  Checks the wiring of the composed step against its parts'
contracts: the committed rows are the accepted tree rows, the committed state
is the deepest accepted row's scratch, and a decode over the committed cache
reproduces the accepted rows' attention.
"""

import numpy as np
import pytest

from oracle import gaps
from oracle import step as ostep
from tree_speculative_decoding_ddt_amd import synth


def tiny_inputs(seed, n=2):
    L, V, B, P, Pmax = 4, 512, 8, 128, 160

    def make(s):
        rng = np.random.default_rng(s)
        return synth.draft_logits(rng, n, L, V, 2.0), rng

    s, z, rng = gaps.first_gapped_seed(make, B, seed)
    from oracle import tree as otree
    t = otree.build_tree_batch(z, B, np.zeros(n, np.int64))
    y = synth.target_logits(rng, n, B + 1, V, 2.0, t["depth"], synth.draft_top1(z), 0.7)
    at = synth.attention_inputs(rng, n, B + 1, 2, 1, 64, Pmax)
    gi = synth.gdn_inputs(rng, n, B + 1, 1, 32, 32, 4)
    return dict(z=z, y=y, at=at, gi=gi, L=L, B=B, P=np.full(n, P), Pmax=Pmax)


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_step_wiring(seed):
    d = tiny_inputs(seed)
    gl = {k: v for k, v in d["gi"].items()}
    r = ostep.verify_step(d["z"], np.zeros(2, np.int64), d["B"], [d["at"]], [gl], d["y"],
                          d["P"], d["Pmax"], H=1, dk=32)
    for s in range(2):
        a = r["acc_len"][s]
        assert 0 <= a <= d["L"] and r["prefix_len"][s] == d["P"][s] + a + 1
        rows = r["acc_rows"][s, : a + 1]
        P = d["P"][s]
        np.testing.assert_array_equal(r["kv_after"][0]["k_cache"][s][:, P:P + a + 1],
                                      d["at"]["k_tree"][s][:, rows])
        np.testing.assert_array_equal(r["gdn_after"][0]["S"][s], r["S_scratch"][0][s][rows[-1]])
        np.testing.assert_array_equal(r["gdn_after"][0]["conv_state"][s], r["conv_scratch"][0][s][rows[-1]])
        for j, row in enumerate(rows):
            # a decode of the accepted row over the first P+j+1 committed rows
            kk = r["kv_after"][0]["k_cache"][s][0, : P + j + 1].astype(np.float64)
            vv = r["kv_after"][0]["v_cache"][s][0, : P + j + 1].astype(np.float64)
            for h in range(2):
                sc = kk @ d["at"]["q"][s][row, h].astype(np.float64) / 8.0
                p = np.exp(sc - sc.max())
                np.testing.assert_allclose((p / p.sum()) @ vv, r["attn_out"][0][s][row, h],
                                           rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_step_with_rope_commits_keys_rotated_at_their_cache_position(seed):
    # pre-rotation tree inputs: after the commit, the key at cache position P + j is the
    # accepted row's key rotated at P + j, and a decode of the accepted row at position
    # P + j over the committed cache reproduces its tree attention
    from oracle import rope as orope
    d = tiny_inputs(seed)
    rng = np.random.default_rng(100 + seed)
    n, T, D = 2, d["B"] + 1, 64
    lay = dict(d["at"])
    lay["k_new"] = rng.standard_normal((n, T, 1, D))
    lay["v_new"] = rng.standard_normal((n, T, 1, D))
    rot, theta = 32, 1e4
    r = ostep.verify_step(d["z"], np.zeros(n, np.int64), d["B"], [lay], [dict(d["gi"])], d["y"],
                          d["P"], d["Pmax"], H=1, dk=32, rope=(rot, theta))
    for s in range(n):
        a = r["acc_len"][s]
        rows = r["acc_rows"][s, : a + 1]
        P = d["P"][s]
        kc = r["kv_after"][0]["k_cache"][s]
        vc = r["kv_after"][0]["v_cache"][s]
        for j, row in enumerate(rows):
            np.testing.assert_allclose(kc[0, P + j], orope.rope(lay["k_new"][s][row], [P + j], rot, theta)[0],
                                       atol=1e-12)
            np.testing.assert_array_equal(vc[0, P + j], lay["v_new"][s][row, 0])
            qr = orope.rope(lay["q"][s][row], np.full(2, P + j), rot, theta)
            kk, vv = kc[0, : P + j + 1], vc[0, : P + j + 1]
            for h in range(2):
                sc = kk @ qr[h] / 8.0
                p = np.exp(sc - sc.max())
                np.testing.assert_allclose((p / p.sum()) @ vv, r["attn_out"][0][s][row, h], rtol=1e-10, atol=1e-12)


def test_uncommitted_sequence_keeps_its_root():
    # sequence 1's cache is full: its round is not committed, so it keeps root 5 for the
    # next round; sequence 0 commits and continues from its bonus token
    d = tiny_inputs(0)
    P = np.array([d["P"][0], d["Pmax"] - 1])
    r = ostep.verify_step(d["z"], np.array([3, 5]), d["B"], [d["at"]], [dict(d["gi"])], d["y"],
                          P, d["Pmax"], H=1, dk=32)
    assert r["acc_len"][0] >= 0 and r["acc_len"][1] == -1
    assert r["next_root"].tolist() == [r["bonus"][0], 5]
    assert r["prefix_len"].tolist() == [P[0] + r["acc_len"][0] + 1, P[1]]
