"""Seeded sweep over valid shapes: each entry point against the oracle at shapes drawn at
random within the built limits, beside the hand-picked cases of the other GPU files.

Every draw is fixed by its seed (printed before the case runs), so a failure names a
case that can be rerun alone.  The comparisons are those of the per-entry-point files:
attention elementwise (fp32 1e-5; bf16 atol 2e-2 / rtol 1e-2), the GDN step's o within
the activation tolerance with its fp32 state scratch within 1e-5 and the conv scratch
bit-exact, the tree build's topology bit-exact (drafter draws pass the oracle's score-gap
guard), and the walk and the commit bit-exact.
"""

import numpy as np
import pytest

from oracle import gaps
from tests import test_gpu_accept_commit as TC
from tests import test_gpu_attention as TA
from tests import test_gpu_build_tree as TB
from tests import test_gpu_gdn as TG
from tests import test_gpu_paged as TP
from tests import test_gpu_replay as TR
from tests import test_gpu_rope as TRo
from tests import test_gpu_sampled as TS
from tests.gpu_util import say
from tree_speculative_decoding_ddt_amd import synth

pytestmark = pytest.mark.gpu


def attention_shape(seed):
    r = np.random.default_rng(1000 + seed)
    dtype = "f32" if seed % 4 == 3 else "bf16"
    D = int(r.choice([64, 128, 256]))          # bf16 D = 64 runs the scalar kernel
    Hkv = int(r.integers(1, 5))
    G = int(r.choice([1, 2, 3, 6, 8]))
    n = int(r.integers(1, 4))
    B = int(r.integers(0, 65))
    L = int(r.integers(1, 16))
    Pmax = int(r.integers(1, 1300))
    prefix = [int(r.integers(0, Pmax + 1)) for _ in range(n)]
    return dict(n=n, B=B, L=L, Hq=G * Hkv, Hkv=Hkv, D=D, Pmax=Pmax, prefix=prefix, dtype=dtype)


@pytest.mark.parametrize("seed", range(30))
def test_attention_sweep(seed):
    c = attention_shape(seed)
    say("sweep tree_attn seed", seed, c)
    TA.run_case(2000 + seed, c["n"], c["B"], c["L"], c["Hq"], c["Hkv"], c["D"], c["Pmax"], c["prefix"], c["dtype"])


def gdn_shape(seed):
    r = np.random.default_rng(3000 + seed)
    B = int(r.integers(1, 65))
    return dict(n=int(r.integers(1, 4)), B=B, L=int(r.integers(1, min(B, 31) + 1)), H=int(r.integers(1, 5)),
                dk=int(r.choice([32, 64, 128])), W=int(r.integers(2, 9)), dtype="f32" if seed % 2 else "bf16")


@pytest.mark.parametrize("seed", range(20))
def test_gdn_sweep(seed):
    c = gdn_shape(seed)
    say("sweep gdn_tree_step seed", seed, c)
    TG.run_case(4000 + seed, c["n"], c["B"], c["L"], c["H"], c["dk"], c["W"], c["dtype"])


@pytest.mark.parametrize("seed", range(15))
def test_build_tree_sweep(seed):
    r = np.random.default_rng(5000 + seed)
    n, B, L, V = int(r.integers(1, 5)), int(r.integers(1, 65)), int(r.integers(1, 16)), int(r.integers(300, 6000))
    dtype = "f32" if seed % 3 == 0 else "bf16"
    # K < B only on continuous fp32 draws (bf16 rows tie often at the K-th value); vocabularies
    # of a few dozen bf16 tokens make near-tied path sums unavoidable (the gap guard refuses them)
    K = int(r.integers(1, B + 1)) if dtype == "f32" and seed % 2 else 0
    say("sweep build_tree seed", seed, dict(n=n, B=B, L=L, V=V, K=K, dtype=dtype))

    def make(t):
        z = synth.draft_logits(np.random.default_rng(t), n, L, V, 2.0)
        return (synth.quantize(z, "bf16")[1] if dtype == "bf16" else z), z

    _, _, z = gaps.first_gapped_seed(make, B, 6000 + 10 * seed)
    TB.run_and_compare(z, dtype, B, r.integers(0, V, size=n), K=K)


@pytest.mark.parametrize("seed", range(15))
def test_accept_sweep(seed):
    r = np.random.default_rng(7000 + seed)
    n, L, V, B = int(r.integers(1, 6)), int(r.integers(1, 16)), int(r.integers(50, 20000)), int(r.integers(1, 65))
    dtype = "f32" if seed % 2 else "bf16"
    say("sweep tree_accept seed", seed, dict(n=n, L=L, V=V, B=B, dtype=dtype))
    t, y = TC.tree_and_target(8000 + seed, n, L, V, B, dtype)
    TC.run_accept(t, y, L, dtype)


@pytest.mark.parametrize("seed", range(12))
def test_commit_sweep(seed):
    r = np.random.default_rng(9000 + seed)
    n, Pmax = int(r.integers(1, 5)), int(r.integers(8, 80))
    prefix = r.integers(0, Pmax + 1, size=n)
    c = dict(n=n, n_kv=int(r.integers(0, 4)), n_gdn=int(r.integers(0, 4)), Pmax=Pmax, prefix=prefix.tolist(),
             dtype="f32" if seed % 2 else "bf16")
    say("sweep commit seed", seed, c)
    TC.commit_case(9100 + seed, n, c["n_kv"], c["n_gdn"], c["dtype"], prefix, Pmax)


@pytest.mark.parametrize("seed", range(18))
def test_paged_attention_sweep(seed):
    c = attention_shape(100 + seed)
    r = np.random.default_rng(11000 + seed)
    ps = int(r.choice([1, 2, 4, 8, 16, 32, 64, 128]))
    maxb = (c["Pmax"] + ps - 1) // ps
    say("sweep tree_attn_paged seed", seed, dict(c, page_size=ps, max_blocks=maxb))
    TP.run_case(12000 + seed, c["n"], c["B"], c["L"], c["Hq"], c["Hkv"], c["D"], ps, maxb, c["prefix"], c["dtype"])


@pytest.mark.parametrize("seed", range(18))
def test_rope_attention_sweep(seed):
    c = attention_shape(200 + seed)
    r = np.random.default_rng(13000 + seed)
    rot = 16 * int(r.integers(1, c["D"] // 16 + 1))
    theta = float(r.choice([10000.0, 500000.0]))
    say("sweep tree_attn_rope seed", seed, dict(c, rot_dim=rot, theta=theta))
    TRo.run_case(14000 + seed, c["n"], c["B"], c["L"], c["Hq"], c["Hkv"], c["D"], c["Pmax"], c["prefix"], c["dtype"],
                 rot, theta)


@pytest.mark.parametrize("seed", range(15))
def test_replay_sweep(seed):
    c = gdn_shape(100 + seed)
    n_layers = int(np.random.default_rng(15000 + seed).integers(1, 21))  # past 16: two launches
    say("sweep gdn_replay seed", seed, dict(c, n_layers=n_layers))
    TR.run_case(16000 + seed, c["n"], c["B"], c["L"], c["H"], c["dk"], c["W"], c["dtype"], n_layers=n_layers)


@pytest.mark.parametrize("seed", range(15))
def test_sampled_walk_sweep(seed):
    r = np.random.default_rng(17000 + seed)
    n, L, V, B = int(r.integers(1, 6)), int(r.integers(1, 16)), int(r.integers(50, 20000)), int(r.integers(1, 65))
    temps = [float(t) for t in r.choice([0.0, -1.0, 0.3, 0.7, 1.0, 1.7, 4.0], size=n)]
    dtype = "f32" if seed % 2 else "bf16"
    say("sweep tree_accept_sampled seed", seed, dict(n=n, L=L, V=V, B=B, temps=temps, dtype=dtype))
    t, y, g = TS.make_case(18000 + seed, n, L, V, B, 4.0)
    TS.run(t, y, g, temps, L, dtype)
