"""GPU parity of ddt_gdn_replay (the committed GDN / conv state advanced along the
accepted path) against the oracle's stored node state of the path's deepest row.

A tree step run without node-state storage must give the same o; replaying the
path r_0..r_a on the committed state must give the oracle's S of row r_a within
the fp32 tolerance (1e-5) and its conv rows bit-exact (copies of stored values).
"""

import numpy as np
import pytest
import torch

from oracle import gdn as ogdn
from tests.gpu_util import assert_close, down, say, up, up_int
from tree_speculative_decoding_ddt_amd import ddt, synth

pytestmark = pytest.mark.gpu


def path_to(parents, r):
    out = [r]
    while parents[out[-1]] >= 0:
        out.append(int(parents[out[-1]]))
    return out[::-1]


def make_layer(rng, n, B, H, dk, W, dtype):
    x = synth.gdn_inputs(rng, n, B + 1, H, dk, dk, W)
    xt, xe = up(x["x"], dtype)
    vt, ve = up(x["v"], dtype)
    cst, cse = up(x["conv_state"], dtype)
    f32 = lambda a: up(a, "f32")
    (bt, be), (gt, ge), (St, Se), (wt, we) = f32(x["beta"]), f32(x["g"]), f32(x["S"]), f32(x["conv_w"])
    dev_ = dict(x=xt, v=vt, conv_state=cst, beta=bt, g=gt, S=St, conv_w=wt)
    ref = dict(x=xe, v=ve, conv_state=cse, beta=be, g=ge, S=Se, conv_w=we)
    return dev_, ref


def run_case(seed, n, B, L, H, dk, W, dtype, kind="random", n_layers=1, targets=None, skip=()):
    """targets[s]: the row whose root path is accepted for sequence s (default: a random row);
    sequences in `skip` get acc_len = -1 and must be left untouched."""
    rng = np.random.default_rng(seed)
    if kind == "chain":
        parents = np.stack([np.arange(-1, B)] * n)
    else:
        parents = np.stack([synth.random_parents(rng, B, L)[0] for _ in range(n)])
    layers = [make_layer(rng, n, B, H, dk, W, dtype) for _ in range(n_layers)]
    if targets is None:
        targets = [int(rng.integers(0, B + 1)) for _ in range(n)]
    acc_rows = np.full((n, L + 1), 1 << 20, dtype=np.int64)  # unread past acc_len: out of range on purpose
    acc_len = np.zeros(n, dtype=np.int64)
    for s in range(n):
        p = path_to(parents[s], targets[s])
        assert len(p) <= L + 1
        acc_rows[s, :len(p)] = p
        acc_len[s] = -1 if s in skip else len(p) - 1
    pt = up_int(parents)
    before = [(down(d["S"]), down(d["conv_state"])) for d, _ in layers]
    for d, _ in layers:
        out = ddt.gdn_tree_step(d["x"], d["conv_w"], d["conv_state"], d["v"], d["beta"], d["g"], d["S"], pt, L,
                                store_states=False)
        d["o"] = out["o"]
    ddt.gdn_replay(up_int(acc_rows), up_int(acc_len),
                   [(d["x"], d["conv_w"], d["v"], d["beta"], d["g"], d["S"], d["conv_state"]) for d, _ in layers], B)
    torch.cuda.synchronize()
    for li, (d, e) in enumerate(layers):
        o, S, cs = down(d["o"]), down(d["S"]), down(d["conv_state"])
        for s in range(n):
            ro, rS, rc = ogdn.gdn_tree_step(e["x"][s], e["conv_w"], e["conv_state"][s], e["v"][s], e["beta"][s],
                                            e["g"][s], e["S"][s], parents[s], H, dk)
            assert_close(o[s], ro, dtype, "o layer %d seq %d (no node-state storage)" % (li, s))
            if s in skip:
                np.testing.assert_array_equal(S[s], before[li][0][s], err_msg="skipped seq %d: S touched" % s)
                np.testing.assert_array_equal(cs[s], before[li][1][s], err_msg="skipped seq %d: conv touched" % s)
                continue
            last = targets[s]
            assert_close(S[s], rS[last], "f32", "replayed S layer %d seq %d (row %d)" % (li, s, last))
            np.testing.assert_array_equal(cs[s], rc[last], err_msg="replayed conv layer %d seq %d" % (li, s))


@pytest.mark.parametrize("seed", range(3))
def test_tiny_fp32(seed):
    say("replay tiny fp32 seed", seed)
    run_case(seed, 3, 8, 4, 1, 32, 4, "f32")


@pytest.mark.parametrize("dk", [32, 64, 128])
def test_head_sizes_fp32(dk):
    say("replay fp32 dk", dk)
    run_case(20 + dk, 2, 24, 6, 3, dk, 4, "f32")


@pytest.mark.parametrize("W", [2, 3, 8])
def test_conv_widths(W):
    # paths both shorter and longer than the conv window: root only, depth 1, deep rows
    say("replay conv width", W)
    run_case(40 + W, 4, 12, 12, 2, 64, W, "f32", kind="chain", targets=[0, 1, W - 1, 12])


def test_bf16_workload_heads():
    # the workload's layer shape at a small batch: 32 heads of 128, conv width 4, budget 64, depth 15
    say("replay bf16 32x128")
    run_case(7, 2, 64, 15, 32, 128, 4, "bf16")


def test_skipped_sequences_untouched():
    say("replay skip")
    run_case(8, 4, 16, 6, 2, 64, 4, "bf16", skip=(1, 3))


def test_more_layers_than_one_launch_holds():
    # 18 layers: two launches of the per-launch layer table
    say("replay 18 layers")
    run_case(9, 2, 12, 5, 1, 32, 4, "f32", n_layers=18)


def test_deep_chain_full_depth():
    # a depth-31 path, the deepest tree the tree step walks
    say("replay depth 31")
    run_case(10, 1, 31, 31, 2, 64, 4, "f32", kind="chain", targets=[31])
