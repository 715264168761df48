"""GPU parity of ddt_gdn_tree_step against the oracle's tree recurrence.

o within the activation dtype's tolerance (fp32 1e-5; bf16 2e-2 / 1e-2); the fp32
state scratch within 1e-5 (its inputs are exact in both dtypes, so only fp32
rounding separates it from the fp64 oracle); the conv scratch bit-exact (copies).
"""

import numpy as np
import pytest
import torch

from oracle import gdn as ogdn
from tests.gpu_util import assert_close, down, say, up, up_int
from tree_speculative_decoding_ddt_amd import ddt, synth

pytestmark = pytest.mark.gpu


def run_case(seed, n, B, L, H, dk, W, dtype, kind="random", check_heads=None):
    rng = np.random.default_rng(seed)
    if kind == "lopsided":
        parents = np.stack([synth.lopsided_parents()[0]] * n)
    elif kind == "chain":
        parents = np.stack([np.arange(-1, B)] * n)  # row i's parent is row i-1: depth i
    elif kind == "star":
        parents = np.stack([np.r_[-1, np.zeros(B, dtype=np.int64)]] * n)  # every node a child of the root
    elif kind == "deep":
        # each row hangs off one of the 2 rows before it: depths around 40 at B 64, with
        # branch points all the way down
        parents = np.full((n, B + 1), -1, dtype=np.int64)
        for s in range(n):
            dep = [0]
            for i in range(1, B + 1):
                cands = [j for j in range(max(0, i - 2), i) if dep[j] < L] or \
                    [j for j in range(i) if dep[j] < L]
                p = int(cands[rng.integers(0, len(cands))])
                parents[s, i] = p
                dep.append(dep[p] + 1)
    elif kind == "unused":
        parents = np.stack([synth.random_parents(rng, B, L)[0] for _ in range(n)])
        parents[:, B - 3:] = -1  # rows left unused by the build read the committed state
    else:
        parents = np.stack([synth.random_parents(rng, B, L)[0] for _ in range(n)])
    x = synth.gdn_inputs(rng, n, B + 1, H, dk, dk, W)
    xt, xe = up(x["x"], dtype)
    vt, ve = up(x["v"], dtype)
    cst, cse = up(x["conv_state"], dtype)
    f32 = lambda a: up(a, "f32")
    (bt, be), (gt, ge), (St, Se), (wt, we) = f32(x["beta"]), f32(x["g"]), f32(x["S"]), f32(x["conv_w"])
    out = ddt.gdn_tree_step(xt, wt, cst, vt, bt, gt, St, up_int(parents), L)
    torch.cuda.synchronize()
    o, Ssc, csc = down(out["o"]), down(out["S_scratch"]), down(out["conv_scratch"])
    for s in range(n):
        ro, rS, rc = ogdn.gdn_tree_step(xe[s], we, cse[s], ve[s], be[s], ge[s], Se[s], parents[s], H, dk)
        hs = slice(None) if check_heads is None else check_heads
        assert_close(o[s][:, hs], ro[:, hs], dtype, "o seq %d" % s)
        assert_close(Ssc[s][:, hs], rS[:, hs], "f32", "S_scratch seq %d" % s)
        np.testing.assert_array_equal(csc[s], rc, err_msg="conv_scratch seq %d" % s)
    return out


@pytest.mark.parametrize("seed", range(3))
def test_tiny_fp32(seed):
    # 1 head, dk = dv = 32, conv width 4 over 64 channels, budget 8
    say("gdn tiny fp32 seed", seed)
    run_case(seed, 2, 8, 4, 1, 32, 4, "f32")


@pytest.mark.parametrize("dk", [32, 64, 128])
def test_head_sizes_fp32(dk):
    run_case(10 + dk, 2, 20, 6, 2, dk, 4, "f32")


@pytest.mark.parametrize("W", [2, 3, 8])
def test_conv_widths(W):
    run_case(20 + W, 2, 16, 10, 2, 32, W, "bf16")


def test_bf16_config_shape():
    # 32 heads, dk = dv = 128, conv width 4 over 8192 channels, 65 rows, depth <= 15
    say("gdn bf16 H=32 dk=128 C=8192 B=64 n=2")
    run_case(30, 2, 64, 15, 32, 128, 4, "bf16")


def test_lopsided_and_unused_rows():
    run_case(31, 1, 64, 15, 4, 128, 4, "bf16", kind="lopsided")
    run_case(32, 2, 24, 8, 2, 64, 4, "f32", kind="unused")


def test_full_batch_sampled_heads():
    say("gdn bf16 n=8 H=32 dk=128 (heads 0, 17, 31 checked)")
    run_case(33, 8, 64, 15, 32, 128, 4, "bf16", check_heads=[0, 17, 31])


def test_full_batch_all_heads_reduced_budget():
    # the workload's batch and heads (8 sequences, 32 heads of 128) at budget 24: every
    # head's o and state scratch compared
    say("gdn bf16 n=8 H=32 dk=128 B=24, all heads")
    run_case(34, 8, 24, 10, 32, 128, 4, "bf16")


def test_deep_chain_and_deep_trees():
    # every row is processed whatever its depth: a 64-deep chain (all 65 rows, depth bound
    # 63), 63-deep chains, and random trees about 40 deep with many branch points
    say("gdn chain depth 64 / 63, deep random trees")
    run_case(40, 2, 64, 63, 2, 128, 4, "bf16", kind="chain")
    run_case(44, 1, 63, 63, 1, 64, 3, "f32", kind="chain")
    out = run_case(45, 3, 64, 63, 2, 128, 4, "bf16", kind="deep")
    run_case(46, 2, 64, 40, 1, 32, 4, "f32", kind="deep")
    run_case(41, 1, 40, 31, 1, 64, 3, "f32")  # random tree


def test_star_and_root_only():
    run_case(42, 2, 64, 1, 2, 128, 4, "bf16", kind="star")
    run_case(43, 2, 0, 1, 2, 64, 4, "f32")    # B = 0: the root alone


def test_chunk_form_states():
    # bf16 activations with the depth bound at most 16 form the node states from the chunk
    # form (w and k of each path node); a tree deeper than the bound given still comes out
    # right (the bound only picks the path).  The deep trees at bound 16 have paths of up
    # to 17 rows (three batches of the states kernel), the chain 65 (nine).
    say("gdn stored states, chunk form: chain 64 deep at bound 15, deep trees dk 64 at bound 16, root alone, W 5")
    run_case(50, 2, 64, 15, 2, 128, 4, "bf16", kind="chain")
    run_case(51, 3, 64, 16, 2, 64, 4, "bf16", kind="deep")
    run_case(52, 2, 0, 1, 2, 128, 4, "bf16")
    run_case(53, 2, 40, 12, 3, 64, 5, "bf16")


def test_chunk_form_matches_walk_states():
    # the same inputs through both ways of storing states (bound 15: chunk form; bound 63:
    # the walk): states within fp32 rounding of each other, conv scratch identical
    say("gdn stored states: chunk form vs walk")
    rng = np.random.default_rng(54)
    n, B, L, H, dk = 3, 64, 15, 4, 128
    parents = np.stack([synth.random_parents(rng, B, L)[0] for _ in range(n)])
    x = synth.gdn_inputs(rng, n, B + 1, H, dk, dk, 4)
    dev = {k: up(x[k], "bf16" if k in ("x", "v", "conv_state") else "f32")[0] for k in x}
    pt = up_int(parents)
    args = (dev["x"], dev["conv_w"], dev["conv_state"], dev["v"], dev["beta"], dev["g"], dev["S"], pt)
    a = ddt.gdn_tree_step(*args, 15)
    b = ddt.gdn_tree_step(*args, 63)
    torch.cuda.synchronize()
    assert_close(down(a["S_scratch"]), down(b["S_scratch"]), "f32", "states chunk form vs walk")
    assert_close(down(a["o"]), down(b["o"]), "bf16", "o chunk form vs walk")
    np.testing.assert_array_equal(down(a["conv_scratch"]), down(b["conv_scratch"]))


@pytest.mark.parametrize("kind", ["random", "chain"])
def test_deferred_state_write_matches_the_call(kind):
    # ddt_gdn_tree_step_deferred + ddt_gdn_tree_states (the latter on a second stream after
    # an event) leave exactly what one ddt_gdn_tree_step call (chunk form) leaves, also for
    # a 64-deep chain (paths of up to 65 rows; the chunk form itself is checked against the
    # oracle on that chain in test_chunk_form_states)
    say("gdn deferred state write on a second stream vs the single call, %s tree" % kind)
    rng = np.random.default_rng(55)
    n, B, L, H, dk = 2, 64, 15, 4, 128
    if kind == "chain":
        parents = np.stack([np.arange(-1, B)] * n)
    else:
        parents = np.stack([synth.random_parents(rng, B, L)[0] for _ in range(n)])
    x = synth.gdn_inputs(rng, n, B + 1, H, dk, dk, 4)
    dev = {k: up(x[k], "bf16" if k in ("x", "v", "conv_state") else "f32")[0] for k in x}
    pt = up_int(parents)
    args = (dev["x"], dev["conv_w"], dev["conv_state"], dev["v"], dev["beta"], dev["g"], dev["S"], pt)
    ref = ddt.gdn_tree_step(*args, L)
    ws = torch.empty(ddt.gdn_tree_step_workspace(n, B, H, dk), dtype=torch.uint8, device="cuda")
    out = ddt.gdn_tree_step_deferred(*args, L, ws)
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record()
    side.wait_event(ev)
    ddt.gdn_tree_states(dev["S"], out["S_scratch"], ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for key in ("o", "conv_scratch", "S_scratch"):
        assert torch.equal(out[key], ref[key]), key
