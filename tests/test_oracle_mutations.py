"""The pins must catch plausible mistakes in the oracle.

Each case rewrites one line of an oracle function on the CPU (a dropped term,
a wrong sign, a wrong index, a flipped tie rule ...) and checks that at least
one pin test then fails.  Nothing here touches a GPU.
"""

import inspect
import textwrap

import pytest

import oracle.accept
import oracle.attention
import oracle.commit
import oracle.gaps
import oracle.gdn
import oracle.paged
import oracle.rope
import oracle.sampled
import oracle.tree
from tests import test_oracle_accept_commit as t_ac
from tests import test_oracle_attention as t_attn
from tests import test_oracle_gaps as t_gaps
from tests import test_oracle_gdn as t_gdn
from tests import test_oracle_paged as t_paged
from tests import test_oracle_rope as t_rope
from tests import test_oracle_sampled as t_smp
from tests import test_oracle_tree as t_tree


def mutated(module, name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, name)))
    assert old in src, (name, old)
    ns = dict(vars(module))
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), ns)
    return ns[name]


def run_pins(pins):
    """True if at least one pin fails (a wrong answer, or an error the mistake causes;
    every pin passes on the unmodified oracle)."""
    for pin in pins:
        try:
            pin()
        except Exception:
            return True
    return False


TREE_PINS = [lambda: t_tree.test_heap_equals_brute_force_rank_limited(0),
             lambda: t_tree.test_heap_equals_full_enumeration(1, 20),
             t_tree.test_hand_worked_example_with_ties,
             t_tree.test_single_depth_is_top_b_of_one_row]
ATTN_PINS = [lambda: t_attn.test_matches_per_path_replay(0), t_attn.test_chain_tree_equals_causal_attention,
             t_attn.test_closed_forms]
GDN_PINS = [lambda: t_gdn.test_tree_matches_chain_replay(0), t_gdn.test_hand_computed_update,
            t_gdn.test_identity_tap_is_silu, t_gdn.test_conv_scratch_exact_copies_short_path,
            t_gdn.test_unit_beta_stores_value]
ACC_PINS = [lambda: t_ac.test_walk_matches_brute_force(0), t_ac.test_argmax_ties_take_lowest_id,
            lambda: t_ac.test_commit_copies_replay_and_decode(0)]

ROPE_PINS = [t_rope.test_two_channels_is_a_plane_rotation, t_rope.test_four_channels_pair_layout_and_frequencies,
             lambda: t_rope.test_complex_form(64, 16), t_rope.test_positions_follow_branch_depth,
             t_rope.test_chain_tree_equals_sequential_decoding]

PAGED_PINS = [t_paged.test_hand_example_two_pages, lambda: t_paged.test_identity_and_permuted_tables_equal_contiguous_attention(16),
              lambda: t_paged.test_paged_commit_equals_contiguous_commit(14, 5),
              lambda: t_paged.test_paged_commit_equals_contiguous_commit(58, 5), t_paged.test_paged_commit_overflow_leaves_pages]

SMP_PINS = [lambda: t_smp.test_draws_follow_the_tempered_softmax(0.5), t_smp.test_zero_temperature_and_zero_noise_are_greedy,
            t_smp.test_power_of_two_rescaling_is_exact, t_smp.test_sampled_tokens_decide_the_path,
            t_smp.test_walk_emits_target_samples_along_a_chain]

GAPS_PINS = [t_gaps.test_gap_below_eps_fails, t_gaps.test_gap_above_eps_passes,
             t_gaps.test_exact_tie_of_identical_values_passes, t_gaps.test_exact_tie_of_different_values_fails,
             t_gaps.test_near_tie_only_matters_up_to_b_plus_one, lambda: t_gaps.test_guard_equals_brute_force(1),
             lambda: t_gaps.test_guard_equals_brute_force(2), t_gaps.test_ancestor_masks_match_the_parent_chain]

CASES = [
    (oracle.tree, "build_tree", "int(ids[0, 0]), 0, 1, 0", "int(ids[0, 0]), 0, 1, 1", TREE_PINS),
    (oracle.tree, "build_tree", "score[p] + vals[d - 1, r + 1]", "score[p] + vals[d - 1, r]", TREE_PINS),
    (oracle.tree, "build_tree", "score[i] + vals[d, 0]", "score[p] + vals[d, 0]", TREE_PINS),
    (oracle.tree, "build_tree", "-(score[i] + vals[d, 0]), int(ids[d, 0])", "-(score[i] + vals[d, 0]), -int(ids[d, 0])", TREE_PINS),
    (oracle.tree, "build_tree", "anc[p] | (1 << (i - 1))", "anc[p] | (1 << i)", TREE_PINS),
    (oracle.tree, "topk_per_depth", "np.lexsort((tok, -lp[d]))", "np.lexsort((-tok, -lp[d]))", TREE_PINS),
    (oracle.tree, "log_softmax", "z - lse", "z - m", TREE_PINS),
    (oracle.attention, "tree_attention", "mask[:, :P] = True", "mask[:, :P - 1] = True", ATTN_PINS),
    (oracle.attention, "tree_attention", "kvh = h // G", "kvh = h % Hkv", ATTN_PINS),
    (oracle.attention, "tree_attention", "scale = D ** -0.5 if", "scale = D ** -1.0 if", ATTN_PINS),
    (oracle.attention, "visible_tree_rows", "[0] + [j + 1", "[j + 1", ATTN_PINS),
    (oracle.attention, "visible_tree_rows", "[j + 1 for", "[j for", ATTN_PINS),
    (oracle.gdn, "gated_delta_tree", "np.outer(v[i, h] - u, k[i, h])", "np.outer(v[i, h] + u, k[i, h])", GDN_PINS),
    (oracle.gdn, "gated_delta_tree", "Sd = g[i, h] * Sp[h]", "Sd = Sp[h]", GDN_PINS),
    (oracle.gdn, "gated_delta_tree", "o[i, h] = S[i, h] @ q[i, h]", "o[i, h] = S[i, h].T @ q[i, h]", GDN_PINS),
    (oracle.gdn, "short_conv_tree", 'np.einsum("jc,cj->c", window, w)', 'np.einsum("jc,cj->c", window[::-1], w)', GDN_PINS),
    (oracle.gdn, "short_conv_tree", "scratch[i] = window[1:]", "scratch[i] = window[:-1]", GDN_PINS),
    (oracle.gdn, "split_qk", "+ K_NORM_EPS)", "+ 1.0)", GDN_PINS),
    (oracle.gdn, "split_qk", "* dk ** -0.5", "* 1.0", GDN_PINS),
    (oracle.accept, "argmax_lowest", "[0])", "[-1])", ACC_PINS),
    (oracle.accept, "walk", "tok[c] == t[cur]", "tok[c] == t[c]", ACC_PINS),
    (oracle.commit, "commit", 'lay["k_cache"][:, P + j, :] = lay["k_tree"][:, r, :]',
     'lay["k_cache"][:, P + j + 1, :] = lay["k_tree"][:, r, :]', ACC_PINS),
    (oracle.commit, "commit", "last = rows[-1]", "last = rows[0]", ACC_PINS),
    (oracle.commit, "commit", "any(r < 0 or r >= T for r in rows)", "any(r < 0 for r in rows)",
     ACC_PINS + [t_ac.test_commit_capacity_guard]),
    (oracle.commit, "commit", "P + a + 1 > Pmax", "P + a > Pmax", ACC_PINS + [t_ac.test_commit_capacity_guard]),
    (oracle.rope, "rope", "hi * c + lo * s", "hi * c - lo * s", ROPE_PINS),
    (oracle.rope, "rope", "lo * c - hi * s", "lo * c + hi * s", ROPE_PINS),
    (oracle.rope, "rope", "lo, hi = x[..., :half], x[..., half:rot_dim]",
     "lo, hi = x[..., 0:rot_dim:2], x[..., 1:rot_dim:2]", ROPE_PINS),
    (oracle.rope, "angles", "-2.0 * j / rot_dim", "-1.0 * j / rot_dim", ROPE_PINS),
    (oracle.rope, "tree_positions", "return prefix_len + depth", "return prefix_len + depth + 1", ROPE_PINS),
    (oracle.paged, "gather", "[pos // ps], :, pos % ps", "[pos // ps - 1], :, pos % ps", PAGED_PINS),
    (oracle.paged, "gather", "[pos // ps], :, pos % ps", "[pos // ps], :, (pos + 1) % ps", PAGED_PINS),
    (oracle.paged, "scatter", "p = start + j", "p = start + j + 1", PAGED_PINS),
    (oracle.paged, "commit_paged", "P + a + 1 > cap", "P + a > cap", PAGED_PINS),
    (oracle.sampled, "sample_token", "* inv", "* np.float32(temperature)", SMP_PINS),
    (oracle.sampled, "sample_token", "key + np.asarray(g_row", "key - np.asarray(g_row", SMP_PINS),
    (oracle.sampled, "sample_token", "if temperature <= 0:", "if temperature < 0:", SMP_PINS),
    (oracle.sampled, "tree_accept_sampled", "gumbel[i], temperature)", "gumbel[0], temperature)", SMP_PINS),
    (oracle.gaps, "gaps_ok", "for i in range(1, B + 1):", "for i in range(1, B):", GAPS_PINS),
    (oracle.gaps, "gaps_ok", "if path_values(z, t, i) != path_values(z, t, i + 1):", "if True:", GAPS_PINS),
    (oracle.gaps, "gaps_ok", "if path_values(z, t, i) != path_values(z, t, i + 1):", "if False:", GAPS_PINS),
    (oracle.gaps, "gaps_ok", '"score"][i + 1] > eps', '"score"][i + 1] > 0', GAPS_PINS),
    (oracle.gaps, "gaps_ok", '"score"][i + 1] > eps', '"score"][i + 1] > 10 * eps', GAPS_PINS),
    (oracle.gaps, "path_values", "z[tree[\"depth\"][i] - 1, tree[\"tok\"][i]]", "z[tree[\"depth\"][i], tree[\"tok\"][i]]", GAPS_PINS),
    (oracle.tree, "ancestor_masks", "anc[parent[i]] | (1 << (i - 1))", "anc[parent[i]] | (1 << i)", GAPS_PINS),
    (oracle.tree, "ancestor_masks", "anc[parent[i]] | (1 << (i - 1))", "(1 << (i - 1))", GAPS_PINS),
    # the mistake the pages warn of: positions by flattened row order instead of depth
    (oracle.rope, "tree_positions", "prefix_len[:, None] + depth", "prefix_len[:, None] + np.arange(depth.shape[1])",
     ROPE_PINS),
]


@pytest.mark.parametrize("case", range(len(CASES)), ids=lambda i: "%s.%s#%d" % (CASES[i][0].__name__.split(".")[-1], CASES[i][1], i))
def test_pins_catch_planted_mistake(case, monkeypatch):
    module, name, old, new, pins = CASES[case]
    monkeypatch.setattr(module, name, mutated(module, name, old, new))
    assert run_pins(pins), "no pin caught: %s.%s %r -> %r" % (module.__name__, name, old, new)
