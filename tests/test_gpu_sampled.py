"""GPU parity of ddt_tree_accept_sampled against the oracle's sampled walk.

Both sides form every Gumbel-max key with the same float32 operations (1/t, the
product, the sum, each rounded once), so the draws, the path, acc_len and the bonus
must agree exactly.  Targets are planted so that a row's draw often lands on one of
its children (deep paths), with per-sequence temperatures including 0 (greedy).
"""

import numpy as np
import pytest
import torch

from oracle import sampled as osmp
from oracle import tree as otree
from tests.gpu_util import dev, down, say, up, up_int
from tree_speculative_decoding_ddt_amd import ddt, synth

pytestmark = pytest.mark.gpu


def make_case(seed, n, L, V, B, boost):
    rng = np.random.default_rng(seed)
    # the workload's drafter plant at full vocab (else the best-first tree is a star)
    z = synth.draft_logits(rng, n, L, V, 3.0, plant_p=0.6) if V > 4096 else synth.draft_logits(rng, n, L, V, 2.0)
    t = otree.build_tree_batch(z, B, np.zeros(n, np.int64))
    y = rng.standard_normal((n, B + 1, V)).astype(np.float32)
    for s in range(n):
        for c in range(1, B + 1):           # a child's token gets a boost at its parent row
            if rng.random() < 0.5:
                y[s, t["parent"][s][c], t["tok"][s][c]] += boost
    g = rng.gumbel(size=(n, B + 1, V)).astype(np.float32)
    return t, y, g


def run(t, y, g, temps, L, dtype):
    yt, ye = up(y, dtype)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())
    out = ddt.tree_accept_sampled(yt, f32(g), f32(temps), up_int(t["tok"]), up_int(t["parent"]), L)
    torch.cuda.synchronize()
    rows, alen, bonus = down(out["acc_rows"]), down(out["acc_len"]), down(out["bonus"])
    ref = osmp.tree_accept_sampled_batch(ye.astype(np.float32), g, temps, t["tok"], t["parent"], L)
    np.testing.assert_array_equal(rows, ref[0])
    np.testing.assert_array_equal(alen, ref[1])
    np.testing.assert_array_equal(bonus, ref[2])
    return alen


@pytest.mark.parametrize("seed", range(4))
def test_tiny_fp32(seed):
    say("sampled walk tiny fp32 seed", seed)
    t, y, g = make_case(seed, 4, 4, 512, 8, 3.0)
    run(t, y, g, [0.7, 1.3, 0.0, 1.0], 4, "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_full_vocab(dtype):
    # 8 sequences, vocab 151936, budget 64, depth 15; odd temperatures (1/t not exact)
    say("sampled walk full vocab", dtype)
    t, y, g = make_case(11, 8, 15, 151936, 64, 14.0)  # e^14 outweighs the 151936 other tokens at t = 1
    alen = run(t, y, g, [0.3, 0.7, 1.0, 1.3, 2.9, 0.0, -1.0, 0.55], 15, dtype)
    assert alen.max() >= 2   # the plant makes deep acceptances happen


def test_ragged_vocab_scalar_path():
    # V not a multiple of the vector width: the element-wise loop
    say("sampled walk ragged vocab")
    t, y, g = make_case(5, 3, 5, 1001, 16, 4.0)
    run(t, y, g, [0.9, 0.25, 4.0], 5, "bf16")
    run(t, y, g, [0.9, 0.25, 4.0], 5, "f32")
