"""GPU parity of whole verify rounds (tree build -> hybrid layers -> walk -> commit)
against the oracle's composed step, over two consecutive rounds (the first round's
bonus token is the second round's root; its commit grows the prefix)."""

import numpy as np
import pytest
import torch

from oracle import gaps
from oracle import step as ostep
from oracle import tree as otree
from tests.gpu_util import anc_numpy, assert_close, down, say, up
from tree_speculative_decoding_ddt_amd import synth
from tree_speculative_decoding_ddt_amd.step import HybridConfig, HybridVerifyStep

pytestmark = pytest.mark.gpu


def load_inputs(step, seed, dtype):
    """Fill the step's buffers from numpy draws; return the exact float64 views."""
    c = step.cfg

    def make(t):
        r = np.random.default_rng(t)
        z = synth.draft_logits(r, c.n, c.L, c.V, 2.0 if c.V <= 4096 else 3.0,
                               plant_p=None if c.V <= 4096 else 0.6)
        return synth.quantize(z, dtype)[1], (z, r)

    _, zq, (z, rng) = gaps.first_gapped_seed(make, c.B, seed)
    zt, ze = up(z, dtype)
    step.draft_logits.copy_(zt)
    t = otree.build_tree_batch(ze, c.B, np.zeros(c.n, np.int64))
    y = synth.target_logits(rng, c.n, c.T, c.V, 2.0, t["depth"], synth.draft_top1(ze), 0.7)
    yt, ye = up(y, dtype)
    step.target_logits.copy_(yt)
    ex = {"z": ze, "y": ye, "attn": [], "gdn": []}
    if c.sampled:
        g = rng.gumbel(size=(c.n, c.T, c.V)).astype(np.float32)
        temps = np.array([0.8, 0.0, 1.3, 2.0][: c.n] + [1.0] * max(0, c.n - 4), np.float32)
        step.gumbel.copy_(torch.from_numpy(g))
        step.temperature.copy_(torch.from_numpy(temps))
        ex["sample"] = (g, temps)
    for a in step.attn:
        x = synth.attention_inputs(rng, c.n, c.T, c.Hq, c.Hkv, c.D, c.Pmax)
        if c.rope:  # the tree rows' own keys/values come token-major, before rotation
            x["k_new"] = np.ascontiguousarray(x.pop("k_tree").transpose(0, 2, 1, 3))
            x["v_new"] = np.ascontiguousarray(x.pop("v_tree").transpose(0, 2, 1, 3))
        lay = {}
        for k, v in x.items():
            tt, ee = up(v, dtype)
            if step.block_table is not None and k in ("k_cache", "v_cache"):
                tt = to_pages(tt, step)  # the same cache, held in the step's pages
            a[k].copy_(tt)
            lay[k] = ee
        ex["attn"].append(lay)
    for g in step.gdn:
        x = synth.gdn_inputs(rng, c.n, c.T, c.H, c.dk, c.dk, c.W)
        lay = {}
        for k, v in x.items():
            dtk = dtype if k in ("x", "v", "conv_state") else "f32"
            tt, ee = up(v, dtk)
            g[k].copy_(tt)
            lay[k] = ee
        ex["gdn"].append(lay)
    return ex


def to_pages(cache, step):
    """Contiguous [n][Hkv][Pmax][D] device tensor -> the step's page pool layout."""
    ps = step.cfg.page_size
    bt = step.block_table.cpu().numpy()
    pool = torch.zeros(step.num_pages, cache.shape[1], ps, cache.shape[3], dtype=cache.dtype, device=cache.device)
    for s in range(cache.shape[0]):
        for b in range(bt.shape[1]):
            pool[int(bt[s, b])] = cache[s, :, b * ps:(b + 1) * ps]
    return pool


def committed(step, t):
    """A committed cache as contiguous [n][Hkv][Pmax][D] float64 (read through the pages if paged)."""
    if step.block_table is None:
        return down(t)
    from oracle import paged as opaged
    pool, bt = down(t), step.block_table.cpu().numpy()
    return np.stack([opaged.gather(pool, bt[s], step.cfg.Pmax) for s in range(bt.shape[0])])


def check_round(step, ex, ref, dtype, rows_only=None):
    for key in ("tok", "parent", "depth"):
        np.testing.assert_array_equal(down(step.tree[key]), ref["tree"][key], err_msg=key)
    np.testing.assert_array_equal(anc_numpy(step.tree["anc"]), ref["tree"]["anc"])
    for j, a in enumerate(step.attn):
        got = down(a["out"])
        want = ref["attn_out"][j]
        if rows_only is not None:
            got, want = got[:, rows_only], want[:, rows_only]
        assert_close(got, want, dtype, "attn layer %d" % j)
    for j, g in enumerate(step.gdn):
        assert_close(down(g["out"]["o"]), ref["gdn_o"][j], dtype, "gdn o layer %d" % j)
        if g["out"]["S_scratch"] is None:  # replay mode stores no node state
            continue
        assert_close(down(g["out"]["S_scratch"]), ref["S_scratch"][j], "f32", "S_scratch layer %d" % j)
        np.testing.assert_array_equal(down(g["out"]["conv_scratch"]), ref["conv_scratch"][j])
    np.testing.assert_array_equal(down(step.acc["acc_rows"]), ref["acc_rows"])
    np.testing.assert_array_equal(down(step.acc["acc_len"]), ref["acc_len"])
    np.testing.assert_array_equal(down(step.prefix_len), ref["prefix_len"])
    for j, a in enumerate(step.attn):
        if ref["attn_tree"] is not None:
            # rotated on the GPU in fp32 and rounded to the storage dtype; values are copies
            assert_close(down(a["k_tree"]), ref["attn_tree"][j]["k_tree"], dtype, "rotated k_tree layer %d" % j)
            np.testing.assert_array_equal(down(a["v_tree"]), ref["attn_tree"][j]["v_tree"])
            assert_close(committed(step, a["k_cache"]), ref["kv_after"][j]["k_cache"], dtype, "k_cache layer %d" % j)
        else:
            np.testing.assert_array_equal(committed(step, a["k_cache"]), ref["kv_after"][j]["k_cache"])
        np.testing.assert_array_equal(committed(step, a["v_cache"]), ref["kv_after"][j]["v_cache"])
    for j, g in enumerate(step.gdn):
        assert_close(down(g["S"]), ref["gdn_after"][j]["S"], "f32", "committed S layer %d" % j)
        np.testing.assert_array_equal(down(g["conv_state"]), ref["gdn_after"][j]["conv_state"])


def run_rounds(cfg, dtype, seed, rounds=2, rows_only=None):
    step = HybridVerifyStep(cfg)
    ex = load_inputs(step, seed, dtype)
    root = np.zeros(cfg.n, np.int64)
    prefix = np.full(cfg.n, cfg.prefix, np.int64)
    attn_in = [dict(lay) for lay in ex["attn"]]
    gdn_in = [dict(lay) for lay in ex["gdn"]]
    for r in range(rounds):
        say("round", r)
        step()
        torch.cuda.synchronize()
        ref = ostep.verify_step(ex["z"], root, cfg.B, attn_in, gdn_in,
                                ex["y"], prefix, cfg.Pmax, cfg.H, cfg.dk, rope=cfg.rope,
                                sample=ex.get("sample"))
        check_round(step, ex, ref, dtype, rows_only)
        # next round: committed buffers, grown prefix, bonus as root where committed
        np.testing.assert_array_equal(down(step.root_token), ref["next_root"])
        root = ref["next_root"]
        prefix = ref["prefix_len"]
        for j, lay in enumerate(attn_in):
            lay["k_cache"] = ref["kv_after"][j]["k_cache"]
            lay["v_cache"] = ref["kv_after"][j]["v_cache"]
        for j, lay in enumerate(gdn_in):
            lay["S"] = ref["gdn_after"][j]["S"]
            lay["conv_state"] = ref["gdn_after"][j]["conv_state"]
    return step


def test_tiny_step_two_rounds():
    # drafter fp32 vocab 512 depth 4, budget 8; 1 attention layer (2/1 heads, D 64, prefix 128);
    # 1 GDN layer (1 head, dk = dv = 32, conv width 4 over 64 channels)
    say("step tiny fp32")
    cfg = HybridConfig(n=2, V=512, L=4, B=8, prefix=128, extra_cap=16, n_attn=1, n_gdn=1, Hq=2, Hkv=1, D=64,
                       H=1, dk=32, W=4, dtype=torch.float32)
    run_rounds(cfg, "f32", seed=3)


def test_bf16_hybrid_step_reduced():
    # config-4 layer shapes, fewer layers and a shorter prefix so that the oracle stays quick
    say("step bf16 hybrid reduced: n=2 V=151936 L=15 B=64 prefix 640, 1 attn + 3 gdn")
    cfg = HybridConfig(n=2, V=151936, L=15, B=64, prefix=640, extra_cap=32, n_attn=1, n_gdn=3)
    run_rounds(cfg, "bf16", seed=5, rounds=2)


def test_tiny_step_replay_two_rounds():
    # as the tiny step, with no node-state storage: the commit replays the accepted path
    say("step tiny fp32 replay")
    cfg = HybridConfig(n=2, V=512, L=4, B=8, prefix=128, extra_cap=16, n_attn=1, n_gdn=1, Hq=2, Hkv=1, D=64,
                       H=1, dk=32, W=4, dtype=torch.float32, replay=True)
    run_rounds(cfg, "f32", seed=3)


def test_bf16_hybrid_step_reduced_replay():
    say("step bf16 hybrid reduced replay: n=2 V=151936 L=15 B=64 prefix 640, 1 attn + 3 gdn")
    cfg = HybridConfig(n=2, V=151936, L=15, B=64, prefix=640, extra_cap=32, n_attn=1, n_gdn=3, replay=True)
    run_rounds(cfg, "bf16", seed=5, rounds=3)


def test_tiny_step_rope_two_rounds():
    # pre-rotation attention inputs: RoPE at prefix + depth inside the attention call,
    # the rotated tree keys committed at their positions, then a second round over them
    say("step tiny fp32 rope")
    cfg = HybridConfig(n=2, V=512, L=4, B=8, prefix=128, extra_cap=16, n_attn=2, n_gdn=1, Hq=2, Hkv=1, D=64,
                       H=1, dk=32, W=4, dtype=torch.float32, rope=(32, 10000.0))
    run_rounds(cfg, "f32", seed=6)


def test_bf16_hybrid_step_reduced_rope_replay():
    # the workload's layer shapes with RoPE on a quarter of the channels and GDN replay on commit
    say("step bf16 hybrid reduced rope + replay")
    cfg = HybridConfig(n=2, V=151936, L=15, B=64, prefix=640, extra_cap=32, n_attn=1, n_gdn=3, replay=True,
                       rope=(64, 1e7))
    run_rounds(cfg, "bf16", seed=7, rounds=2)


def test_tiny_step_paged_two_rounds():
    # the committed KV in pages of 16 scattered over a pool; the commit writes through the table
    say("step tiny fp32 paged")
    cfg = HybridConfig(n=2, V=512, L=4, B=8, prefix=128, extra_cap=32, n_attn=2, n_gdn=1, Hq=2, Hkv=1, D=64,
                       H=1, dk=32, W=4, dtype=torch.float32, page_size=16)
    run_rounds(cfg, "f32", seed=8)


def test_bf16_hybrid_step_reduced_paged_replay():
    say("step bf16 hybrid reduced paged + replay")
    cfg = HybridConfig(n=2, V=151936, L=15, B=64, prefix=640, extra_cap=64, n_attn=1, n_gdn=3, replay=True,
                       page_size=32)
    run_rounds(cfg, "bf16", seed=9, rounds=2)


def test_tiny_step_sampled_two_rounds():
    # the walk over sampled target tokens (temperatures 0.8 and greedy), fp32
    say("step tiny fp32 sampled")
    cfg = HybridConfig(n=2, V=512, L=4, B=8, prefix=128, extra_cap=16, n_attn=1, n_gdn=1, Hq=2, Hkv=1, D=64,
                       H=1, dk=32, W=4, dtype=torch.float32, sampled=True)
    run_rounds(cfg, "f32", seed=10)


def test_bf16_hybrid_step_reduced_all_next_paths():
    # sampled walk + RoPE inside attention + GDN replay, at the workload's layer shapes
    say("step bf16 hybrid reduced: sampled + rope + replay")
    cfg = HybridConfig(n=4, V=151936, L=15, B=64, prefix=640, extra_cap=64, n_attn=1, n_gdn=2, replay=True,
                       rope=(256, 10000.0), sampled=True)
    run_rounds(cfg, "bf16", seed=12, rounds=2)


def test_replay_matches_stored_commit_on_overflow():
    # a cache with room for a single commit: the second round's sequences overflow and
    # are left untouched (acc_len -1) in both commit modes
    say("step replay overflow")
    cfg = HybridConfig(n=2, V=512, L=4, B=8, prefix=128, extra_cap=5, n_attn=1, n_gdn=2, Hq=2, Hkv=1, D=64,
                       H=1, dk=32, W=4, dtype=torch.float32, replay=True)
    run_rounds(cfg, "f32", seed=4, rounds=3)


def test_full_size_hybrid_round_sampled():
    """One round at the full hybrid shapes (8 sequences, vocab 151936, depth 15, B 64,
    prefix 16384, 16 attention + 48 GDN layers), inputs drawn on the device as the
    benchmark draws them; the oracle checks sampled outputs one by one."""
    from oracle import accept as oacc
    from oracle import attention as oattn
    from oracle import gdn as ogdn

    say("step full size: n=8 prefix 16384, 16 attn + 48 gdn (sampled oracle checks)")
    cfg = HybridConfig(n=8, prefix=16384, extra_cap=64)
    step = HybridVerifyStep(cfg)
    step.fill_random(seed=11)
    P0 = cfg.prefix
    g0 = step.gdn[0]
    S_before = down(g0["S"][0])
    cs_before = down(g0["conv_state"][0])
    tail_before = down(step.attn[3]["k_cache"][:, :, P0 + cfg.L + 1:P0 + cfg.L + 5])
    step()
    torch.cuda.synchronize()

    z = down(step.draft_logits)
    tree = {k: down(step.tree[k]) for k in ("tok", "parent", "depth")}
    anc = anc_numpy(step.tree["anc"])
    acc_rows, acc_len = down(step.acc["acc_rows"]), down(step.acc["acc_len"])
    bonus, prefix = down(step.acc["bonus"]), down(step.prefix_len)

    # tree topology, bit-exact, on the sequences whose draws keep the stated score gaps
    checked = 0
    for s in range(cfg.n):
        if not gaps.gaps_ok(z[s], cfg.B):
            continue
        ref = otree.build_tree(z[s], cfg.B, 0)
        for key in ("tok", "parent", "depth"):
            np.testing.assert_array_equal(tree[key][s], ref[key], err_msg="%s seq %d" % (key, s))
        np.testing.assert_array_equal(anc[s], ref["anc"], err_msg="anc seq %d" % s)
        checked += 1
    say("tree checked on", checked, "of", cfg.n, "sequences")
    assert checked == cfg.n, "draws of seed 11 should keep the score gaps on every sequence"

    # walk against the target argmaxes, bit-exact (the bonus is the next root)
    for s in (0, 3, 7):
        y = down(step.target_logits[s])
        rows, a, b = oacc.tree_accept(y, tree["tok"][s], tree["parent"][s], cfg.L)
        np.testing.assert_array_equal(acc_rows[s], rows)
        assert acc_len[s] == a and bonus[s] == b
    np.testing.assert_array_equal(down(step.root_token), bonus)

    # attention: sampled rows of the first and last layer (the commit only wrote rows >= P0)
    for j in (0, cfg.n_attn - 1):
        lay = step.attn[j]
        for s in (0, 5):
            kc, vc = down(lay["k_cache"][s]), down(lay["v_cache"][s])
            kt, vt = down(lay["k_tree"][s]), down(lay["v_tree"][s])
            q, out = down(lay["q"][s]), down(lay["out"][s])
            for i in (0, 17, cfg.B):
                ref = oattn.tree_attention_row(q[i], kc, vc, P0, kt, vt, anc[s][i])
                assert_close(out[i], ref, "bf16", "attn layer %d seq %d row %d" % (j, s, i))

    # GDN layer 0, sequence 0, every head, from the state before the commit
    ro, rS, rc = ogdn.gdn_tree_step(down(g0["x"][0]), down(g0["conv_w"]), cs_before, down(g0["v"][0]),
                                    down(g0["beta"][0]), down(g0["g"][0]), S_before, tree["parent"][0],
                                    cfg.H, cfg.dk)
    assert_close(down(g0["out"]["o"][0]), ro, "bf16", "gdn o")
    assert_close(down(g0["out"]["S_scratch"][0]), rS, "f32", "gdn S_scratch")
    np.testing.assert_array_equal(down(g0["out"]["conv_scratch"][0]), rc)

    # commit: prefix growth, exact KV rows of the accepted path, deepest row's states
    np.testing.assert_array_equal(prefix, P0 + acc_len + 1)
    for j in (0, 3, cfg.n_attn - 1):
        lay = step.attn[j]
        for s in range(cfg.n):
            a = int(acc_len[s])
            rows = acc_rows[s][:a + 1].astype(np.int64)
            for name, tree_name in (("k_cache", "k_tree"), ("v_cache", "v_tree")):
                got = lay[name][s][:, P0:P0 + a + 1]
                want = lay[tree_name][s][:, torch.as_tensor(rows, device=got.device)]
                assert torch.equal(got, want), (name, j, s)
    np.testing.assert_array_equal(down(step.attn[3]["k_cache"][:, :, P0 + cfg.L + 1:P0 + cfg.L + 5]), tail_before)
    for j in (0, 24, cfg.n_gdn - 1):
        g = step.gdn[j]
        for s in range(cfg.n):
            r = int(acc_rows[s][int(acc_len[s])])
            assert torch.equal(g["S"][s], g["out"]["S_scratch"][s, r]), ("S", j, s)
            assert torch.equal(g["conv_state"][s], g["out"]["conv_scratch"][s, r]), ("conv", j, s)


def test_overlapped_state_writes_match():
    # the round with each layer's node-state write on a second stream (the default) leaves
    # exactly what the round with every call on one stream leaves, over two rounds
    say("step bf16: state writes overlapped on a second stream vs one stream")
    kw = dict(n=2, V=151936, L=15, B=64, prefix=640, extra_cap=32, n_attn=1, n_gdn=3)
    a = HybridVerifyStep(HybridConfig(overlap_states=True, **kw))
    b = HybridVerifyStep(HybridConfig(overlap_states=False, **kw))
    a.fill_random(seed=6)
    b.fill_random(seed=6)
    for r in range(2):
        a()
        b()
        torch.cuda.synchronize()
        for j, (ga, gb) in enumerate(zip(a.gdn, b.gdn)):
            for key in ("o", "S_scratch", "conv_scratch"):
                assert torch.equal(ga["out"][key], gb["out"][key]), "round %d layer %d %s" % (r, j, key)
            assert torch.equal(ga["S"], gb["S"]), "round %d committed S layer %d" % (r, j)
            assert torch.equal(ga["conv_state"], gb["conv_state"]), "round %d conv state layer %d" % (r, j)
        assert torch.equal(a.prefix_len, b.prefix_len) and torch.equal(a.root_token, b.root_token)
        for la, lb in zip(a.attn, b.attn):
            assert torch.equal(la["k_cache"], lb["k_cache"]) and torch.equal(la["v_cache"], lb["v_cache"])
