"""A whole verify round captured once in a HIP graph and replayed: every replay must
leave exactly the state an identical step object reaches by running the same rounds
eagerly (the library allocates nothing, synchronises nothing and issues no memset, so
its calls are capturable).  Eager work runs between the replays."""

import pytest
import torch

from tests.gpu_util import say
from tree_speculative_decoding_ddt_amd.step import HybridConfig, HybridVerifyStep

pytestmark = pytest.mark.gpu


def state(step):
    out = {"tok": step.tree["tok"], "parent": step.tree["parent"], "anc": step.tree["anc"],
           "acc_rows": step.acc["acc_rows"], "acc_len": step.acc["acc_len"], "bonus": step.acc["bonus"],
           "prefix_len": step.prefix_len, "root": step.root_token}
    for j, a in enumerate(step.attn):
        out["attn%d" % j] = a["out"]
        out["k_cache%d" % j] = a["k_cache"]
        out["v_cache%d" % j] = a["v_cache"]
    for j, g in enumerate(step.gdn):
        out["gdn_o%d" % j] = g["out"]["o"]
        out["S%d" % j] = g["S"]
        out["conv%d" % j] = g["conv_state"]
    return {k: v.clone() for k, v in out.items()}


def run(cfg, seed, replays=3):
    a, b = HybridVerifyStep(cfg), HybridVerifyStep(cfg)
    a.fill_random(seed=seed)
    b.fill_random(seed=seed)
    a()          # one eager round each: every kernel and attribute initialised before capture
    b()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        a()
    for k in range(replays):
        graph.replay()
        b()
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        sa, sb = state(a), state(b)
        for key in sa:
            assert torch.equal(sa[key], sb[key]), "replay %d: %s differs from the eager round" % (k, key)
        del junk


def test_graph_replay_stored_states():
    say("graph replay: stored node states, bf16")
    run(HybridConfig(n=2, V=4096, L=6, B=16, prefix=256, extra_cap=64, n_attn=1, n_gdn=2, Hq=8, Hkv=2, D=128,
                     H=4, dk=64, W=4), seed=1)


def test_graph_replay_next_paths():
    say("graph replay: replay + RoPE + sampled walk, then paged + replay")
    run(HybridConfig(n=2, V=4096, L=6, B=16, prefix=256, extra_cap=64, n_attn=1, n_gdn=2, Hq=8, Hkv=2, D=128,
                     H=4, dk=64, W=4, replay=True, rope=(64, 10000.0), sampled=True), seed=2)
    run(HybridConfig(n=2, V=4096, L=6, B=16, prefix=256, extra_cap=64, n_attn=1, n_gdn=2, Hq=8, Hkv=2, D=128,
                     H=4, dk=64, W=4, replay=True, page_size=16), seed=3)


def test_graph_replay_overlapped_state_writes():
    # the node-state writes on a second stream (joined before the attention layer and the
    # commit) captured with the round: the committed state the commit copies from them
    # must match the eager rounds after every replay
    say("graph replay: node states written on a second stream")
    run(HybridConfig(n=2, V=4096, L=6, B=16, prefix=256, extra_cap=64, n_attn=1, n_gdn=2, Hq=8, Hkv=2, D=128,
                     H=4, dk=64, W=4, overlap_states=True), seed=4)
