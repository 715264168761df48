"""Sampled (stochastic) tree acceptance (oracle).

Sources: "DDTree on vLLM: candid research notes", section "What broke along the
way": the tree walk compares sampled tokens, and testing with greedy decoding only
hid anomalies.  "From DDTree to drafter training", section "The Architecture of
DDTree": walk down from the root while the target's token at the current node
matches a child; the last target token is the bonus.

Readings: the pages give no acceptance rule beyond comparing sampled
tokens, so the walk is the greedy walk with each row's argmax replaced by a draw
from the target's distribution at that row, softmax(z / temperature).  Every
emitted token is then a plain sample of the target at its own context, so the
output distribution is the target's whatever the drafter proposed.  The draw is
Gumbel-max: t = argmax_v (z_v * (1/temperature) + G_v), with the Gumbel noise G
an input (the random numbers the method draws), ties to the lowest token id.  The
key is formed in float32 exactly as written -- 1/temperature rounded once, the
product rounded, the sum rounded -- so that a device doing the same IEEE float32
operations takes the same decision.  temperature <= 0 is greedy (argmax of z).
"""

import numpy as np

from . import accept as _accept


def sample_token(z_row, g_row, temperature):
    """One row's target token: a Gumbel-max draw from softmax(z / temperature)."""
    if temperature <= 0:
        return _accept.argmax_lowest(z_row)
    inv = np.float32(1.0) / np.float32(temperature)
    key = np.asarray(z_row, dtype=np.float32) * inv      # float32 product, rounded
    key = key + np.asarray(g_row, dtype=np.float32)      # float32 sum, rounded
    return _accept.argmax_lowest(key)


def tree_accept_sampled(target_logits, gumbel, temperature, tok, parent, L):
    """One sequence: target_logits, gumbel [T][V], temperature (scalar) -> (acc_rows, a, bonus)."""
    t = [sample_token(target_logits[i], gumbel[i], temperature) for i in range(len(tok))]
    return _accept.walk(t, tok, parent, L)


def tree_accept_sampled_batch(target_logits, gumbel, temperature, tok, parent, L):
    outs = [tree_accept_sampled(target_logits[s], gumbel[s], temperature[s], tok[s], parent[s], L)
            for s in range(len(tok))]
    return (np.stack([o[0] for o in outs]), np.array([o[1] for o in outs]),
            np.array([o[2] for o in outs]))
