"""GPU check of ddt_build_tree_noalloc (the tree build with the library's static
per-device scratch, for callers that cannot allocate) against ddt_build_tree with a
caller workspace: identical trees, bit for bit, on two calls in a row, the second
smaller than the first (the static array keeps the first call's contents)."""

import pytest
import torch

from tests.gpu_util import say
from tree_speculative_decoding_ddt_amd import ddt

pytestmark = pytest.mark.gpu

KEYS = ("tok", "parent", "depth", "score", "anc")


def draw(seed, n, L, V, dtype):
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(seed)
    z = 3.0 * torch.randn(n, L, V, generator=gen, device="cuda:0")
    # planted peaks at some depths: confident and uncertain depths mixed
    hit = torch.rand(n, L, generator=gen, device="cuda:0") < 0.6
    where = torch.randint(0, V, (n, L), generator=gen, device="cuda:0")
    peak = z.amax(dim=-1) + 8.0
    z.scatter_(2, where[..., None], torch.where(hit, peak, z.gather(2, where[..., None])[..., 0])[..., None])
    root = torch.randint(0, V, (n,), generator=gen, device="cuda:0", dtype=torch.int32)
    return z.to(dtype), root


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_call_twice(dtype):
    cases = [(16, 15, 151936, 64), (3, 6, 20000, 32)]  # second call smaller
    for i, (n, L, V, B) in enumerate(cases):
        say("noalloc build: call %d n=%d L=%d V=%d B=%d %s" % (i, n, L, V, B, dtype))
        z, root = draw(100 + i, n, L, V, dtype)
        ref = ddt.build_tree(z, B, root)
        got = ddt.build_tree_noalloc(z, B, root)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), (i, k)
        assert int((got["tok"] >= 0).sum()) == n * (B + 1)


def test_noalloc_after_a_larger_call_and_beside_workspace_calls():
    # a large call, then a small one with K < B, then the large one again
    for i, (n, L, V, B, K) in enumerate([(8, 15, 151936, 64, 0), (1, 4, 512, 8, 3), (8, 15, 151936, 64, 0)]):
        say("noalloc build: sequence call %d n=%d V=%d B=%d K=%d" % (i, n, V, B, K))
        z, root = draw(200 + (i % 2), n, L, V, torch.bfloat16)
        got = ddt.build_tree_noalloc(z, B, root, K=K)
        ref = ddt.build_tree(z, B, root, K=K)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), (i, k)
