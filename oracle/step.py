"""The whole DDTree verification step composed from the oracle parts.

Sources: "DDTree on vLLM: candid research notes", section "Why hybrid
attention makes it hard" (the three surfaces: tree attention, branch-local
recurrent state, accepted-path commit); "The architecture of speculation",
section "The DDTree Integration Challenge" (drafting, tree construction, tree
attention, compaction); "From DDTree to drafter training", section "The
Architecture of DDTree" (heap build, flatten, verify, walk, compaction).

Order: build the tree -> every layer in the given pattern ("attn" or "gdn") ->
walk against the target argmaxes -> commit the accepted path.  The layers' own
inputs are given (the pages name no hidden size, so there are no projections
between layers).
"""

import numpy as np

from . import accept as _accept
from . import attention as _attention
from . import commit as _commit
from . import gdn as _gdn
from . import rope as _rope
from . import sampled as _sampled
from . import tree as _tree


def verify_step(draft_logits, root_token, B, attn_layers, gdn_layers, target_logits,
                prefix_len, Pmax, H, dk, scale=None, rope=None, sample=None):
    """Batch of n sequences.

    attn_layers: list of dicts q [n][T][Hq][D], k_tree, v_tree [n][Hkv][T][D],
                 k_cache, v_cache [n][Hkv][Pmax][D]
                 With rope = (rot_dim, theta): q is before rotation and the tree rows'
                 keys and values come as k_new, v_new [n][T][Hkv][D]; they are rotated
                 at positions prefix_len + depth (the tree just built) and the
                 rotated k_tree / v_tree are what the attention reads and the commit
                 copies (returned as "attn_tree").
    sample:      None for the greedy walk, or (gumbel [n][T][V], temperature [n]) for
                 the walk over sampled target tokens.
    gdn_layers:  list of dicts x [n][T][C], v [n][T][H][dv], beta, g [n][T][H],
                 S [n][H][dv][dk], conv_state [n][W-1][C], conv_w [C][W]
    Returns a dict with the tree, per-layer outputs, the walk and the
    committed buffers.
    """
    n, L, _ = np.shape(draft_logits)
    tree = _tree.build_tree_batch(draft_logits, B, root_token)
    attn_tree = None
    if rope is not None:
        rot_dim, theta = rope
        attn_tree, rotated = [], []
        for lay in attn_layers:
            parts = [_rope.rope_tree_inputs(lay["q"][s], lay["k_new"][s], lay["v_new"][s], prefix_len[s],
                                            tree["depth"][s], rot_dim, theta) for s in range(n)]
            q, kt, vt = (np.stack([p[i] for p in parts]) for i in range(3))
            attn_tree.append({"q": q, "k_tree": kt, "v_tree": vt})
            rotated.append(dict(lay, q=q, k_tree=kt, v_tree=vt))
        attn_layers = rotated
    attn_out = [_attention.tree_attention_batch(lay["q"], lay["k_cache"], lay["v_cache"],
                                                prefix_len, lay["k_tree"], lay["v_tree"],
                                                tree["anc"], scale)
                for lay in attn_layers]
    gdn_out = [_gdn.gdn_tree_step_batch(lay["x"], lay["conv_w"], lay["conv_state"], lay["v"],
                                        lay["beta"], lay["g"], lay["S"], tree["parent"], H, dk)
               for lay in gdn_layers]
    if sample is None:
        acc_rows, acc_len, bonus = _accept.tree_accept_batch(target_logits, tree["tok"], tree["parent"], L)
    else:
        acc_rows, acc_len, bonus = _sampled.tree_accept_sampled_batch(target_logits, sample[0], sample[1],
                                                                      tree["tok"], tree["parent"], L)
    new_prefix, new_acc = np.empty(n, np.int64), np.empty(n, np.int64)
    kv_after = [dict(k_cache=[], v_cache=[]) for _ in attn_layers]
    gdn_after = [dict(S=[], conv_state=[]) for _ in gdn_layers]
    for s in range(n):
        kv = [dict(k_tree=lay["k_tree"][s], v_tree=lay["v_tree"][s],
                   k_cache=lay["k_cache"][s], v_cache=lay["v_cache"][s]) for lay in attn_layers]
        gd = [dict(S_scratch=gdn_out[j][1][s], S=gdn_layers[j]["S"][s],
                   conv_scratch=gdn_out[j][2][s], conv_state=gdn_layers[j]["conv_state"][s])
              for j in range(len(gdn_layers))]
        p, a, kv_new, gd_new = _commit.commit(acc_rows[s], acc_len[s], prefix_len[s], kv, gd, Pmax)
        new_prefix[s], new_acc[s] = p, a
        for j, lay in enumerate(kv_new):
            kv_after[j]["k_cache"].append(lay["k_cache"])
            kv_after[j]["v_cache"].append(lay["v_cache"])
        for j, lay in enumerate(gd_new):
            gdn_after[j]["S"].append(lay["S"])
            gdn_after[j]["conv_state"].append(lay["conv_state"])
    kv_after = [{k: np.stack(v) for k, v in d.items()} for d in kv_after]
    gdn_after = [{k: np.stack(v) for k, v in d.items()} for d in gdn_after]
    return {"tree": tree, "attn_out": attn_out, "attn_tree": attn_tree,
            "gdn_o": [g[0] for g in gdn_out], "S_scratch": [g[1] for g in gdn_out],
            "conv_scratch": [g[2] for g in gdn_out],
            "acc_rows": acc_rows, "acc_len_walk": acc_len, "bonus": bonus,
            # the next round's root: the bonus token where the round was committed; a
            # sequence that was not (acc_len -1) keeps its root and repeats the round
            "next_root": np.where(new_acc >= 0, bonus, np.asarray(root_token)),
            "acc_len": new_acc, "prefix_len": new_prefix,
            "kv_after": kv_after, "gdn_after": gdn_after}
