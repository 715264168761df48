"""The C ABI without a GPU: the library loads, exports every function include/ddt.h
declares, sizes its workspaces, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from tree_speculative_decoding_ddt_amd import ddt

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ddt.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ddt_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported():
    L = ddt.lib()
    names = declared()
    assert len(names) == 24, names
    for name in names:
        assert hasattr(L, name), name
    assert sorted(ddt.EXPORTS) == names


def test_status_strings_and_version():
    L = ddt.lib()
    assert L.ddt_abi_version() == 1
    assert [L.ddt_status_string(i).decode() for i in range(5)] == [
        "DDT_OK", "DDT_ERR_ARG", "DDT_ERR_UNSUPPORTED", "DDT_ERR_WORKSPACE", "DDT_ERR_HIP"]


def test_workspace_queries():
    assert ddt.build_tree_workspace(16, 15, 151936, 64) > ddt.build_tree_workspace(1, 15, 151936, 64) > 0
    assert ddt.build_tree_workspace(1, 4, 512, 8) > 0
    assert ddt.build_tree_workspace(1, 4, 512, 65) == 0          # B > 64
    assert ddt.build_tree_workspace(1, 15, 2 ** 21, 64) == 0      # V > 2^20
    import torch
    assert ddt.tree_attn_workspace(1, 8, 2, 1, 64, 128, torch.float32) == 0   # scalar path: no workspace
    assert ddt.tree_attn_workspace(8, 64, 24, 4, 256, 32768, torch.bfloat16) > 0
    assert ddt.tree_attn_workspace(8, 64, 24, 4, 96, 32768, torch.bfloat16) == 0  # D not built
    assert ddt.tree_accept_workspace(8, 64, 151936) > 0


P = ctypes.c_void_p(256)  # a non-null placeholder: every call below fails validation before using it


def status(fn, *args):
    return getattr(ddt.lib(), fn)(*args)


def test_build_tree_noalloc_validation():
    # same checks as ddt_build_tree, plus the static scratch bound, all before any HIP call
    L = ddt.lib()
    assert L.ddt_build_tree_noalloc_max_scratch() == 8 << 20
    args = lambda **k: [k.get("z", P), 1, k.get("n", 1), k.get("L", 15), k.get("V", 1000), k.get("B", 64),
                        k.get("K", 0), P, P, P, P, P, P, None]
    assert status("ddt_build_tree_noalloc", *args(z=None)) == ddt.DDT_ERR_ARG
    assert status("ddt_build_tree_noalloc", *args(B=65)) == ddt.DDT_ERR_ARG
    assert status("ddt_build_tree_noalloc", *args(L=64)) == ddt.DDT_ERR_ARG
    assert ddt.build_tree_workspace(64, 15, 151936, 64) <= 8 << 20       # the stated fit
    big = dict(n=256, L=15, V=151936)
    assert ddt.build_tree_workspace(256, 15, 151936, 64) > 8 << 20
    assert status("ddt_build_tree_noalloc", *args(**big)) == ddt.DDT_ERR_WORKSPACE
    assert "static" in L.ddt_last_error().decode()


def test_build_tree_validation():
    args = lambda **k: [k.get("z", P), k.get("dt", 1), k.get("n", 1), k.get("L", 15), k.get("V", 1000),
                        k.get("B", 64), k.get("K", 0), P, P, P, P, P, P, P, k.get("ws", 1 << 30), None]
    assert status("ddt_build_tree", *args(z=None)) == ddt.DDT_ERR_ARG
    assert status("ddt_build_tree", *args(B=65)) == ddt.DDT_ERR_ARG
    assert status("ddt_build_tree", *args(L=0)) == ddt.DDT_ERR_ARG
    assert status("ddt_build_tree", *args(K=65)) == ddt.DDT_ERR_ARG
    assert status("ddt_build_tree", *args(dt=7)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_build_tree", *args(V=(1 << 20) + 1)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_build_tree", *args(ws=16)) == ddt.DDT_ERR_WORKSPACE
    assert "workspace" in ddt.lib().ddt_last_error().decode()


def test_tree_attn_validation():
    def args(**k):
        return [k.get("q", P), P, P, P, P, P, P, 1, k.get("B", 8), k.get("Hq", 2), k.get("Hkv", 1),
                k.get("D", 64), k.get("Pmax", 128), ctypes.c_float(0.0), k.get("dt", 0), P, k.get("ws", P), k.get("wsb", 1 << 30), None]
    assert status("ddt_tree_attn", *args(q=None)) == ddt.DDT_ERR_ARG
    assert status("ddt_tree_attn", *args(B=65)) == ddt.DDT_ERR_ARG
    assert status("ddt_tree_attn", *args(Hq=3, Hkv=2)) == ddt.DDT_ERR_ARG
    assert status("ddt_tree_attn", *args(D=96)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_tree_attn", *args(dt=3)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_tree_attn", *args(dt=1, D=256, Pmax=65536, wsb=8)) == ddt.DDT_ERR_WORKSPACE


def test_tree_attn_rope_validation():
    def args(**k):
        #       q             k_new v_new depth            rot                   theta
        return [k.get("q", P), P, P, k.get("depth", P), k.get("rot", 64), ctypes.c_float(k.get("theta", 1e4)),
                P, P, P, P, P, P, 1, k.get("B", 8), 2, 1, k.get("D", 64), 128, ctypes.c_float(0.0), k.get("dt", 0),
                P, P, k.get("wsb", 1 << 30), None]
    assert status("ddt_tree_attn_rope", *args(depth=None)) == ddt.DDT_ERR_ARG
    assert status("ddt_tree_attn_rope", *args(rot=24)) == ddt.DDT_ERR_UNSUPPORTED     # not a multiple of 16
    assert status("ddt_tree_attn_rope", *args(rot=128)) == ddt.DDT_ERR_UNSUPPORTED    # > D
    assert status("ddt_tree_attn_rope", *args(rot=0)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_tree_attn_rope", *args(theta=1.0)) == ddt.DDT_ERR_ARG
    assert status("ddt_tree_attn_rope", *args(theta=float("inf"))) == ddt.DDT_ERR_ARG
    assert status("ddt_tree_attn_rope", *args(D=96)) == ddt.DDT_ERR_UNSUPPORTED
    need = ddt.tree_attn_rope_workspace(1, 8, 2, 1, 64, 128, __import__("torch").float32)
    assert need >= 1 * 9 * 2 * 64 * 4 > 0                                              # room for the rotated queries
    assert status("ddt_tree_attn_rope", *args(wsb=need - 1)) == ddt.DDT_ERR_WORKSPACE
    r = [P, P, P, P, P, 64, ctypes.c_float(1e4), 1, 8, 2, 1, 64, 0, P, P, P, None]
    r2 = list(r); r2[3] = None
    assert status("ddt_tree_rope", *r2) == ddt.DDT_ERR_ARG
    r2 = list(r); r2[5] = 72
    assert status("ddt_tree_rope", *r2) == ddt.DDT_ERR_UNSUPPORTED
    r2 = list(r); r2[11] = 96
    assert status("ddt_tree_rope", *r2) == ddt.DDT_ERR_UNSUPPORTED


def test_paged_validation():
    def args(**k):
        #       q  kp vp  table                  maxb                 ps                    npages
        return [P, P, P, k.get("bt", P), k.get("maxb", 8), k.get("ps", 16), k.get("npages", 100), P, P, P, P,
                1, 8, 2, 1, k.get("D", 64), ctypes.c_float(0.0), 0, P, P, k.get("wsb", 1 << 30), None]
    assert status("ddt_tree_attn_paged", *args(bt=None)) == ddt.DDT_ERR_ARG
    assert status("ddt_tree_attn_paged", *args(ps=24)) == ddt.DDT_ERR_UNSUPPORTED      # not a power of two
    assert status("ddt_tree_attn_paged", *args(ps=0)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_tree_attn_paged", *args(npages=0)) == ddt.DDT_ERR_ARG
    assert status("ddt_tree_attn_paged", *args(maxb=1 << 20, ps=4096)) == ddt.DDT_ERR_ARG   # capacity > 2^30
    assert status("ddt_tree_attn_paged", *args(D=96)) == ddt.DDT_ERR_UNSUPPORTED
    assert ddt.tree_attn_paged_workspace(8, 64, 24, 4, 256, 2048, 16, __import__("torch").bfloat16) == \
        ddt.tree_attn_workspace(8, 64, 24, 4, 256, 32768, __import__("torch").bfloat16)
    kv = (ddt.KVLayer * 1)(ddt.KVLayer(256, 256, 256, 256))
    gd = (ddt.GDNLayer * 1)()
    c = [P, P, P, kv, 1, 2, 64, None, 8, 16, 100, 1, gd, 0, 1, 32, 32, 64, 4, 1, 1, 8, 4, None]
    assert status("ddt_commit_paged", *c) == ddt.DDT_ERR_ARG                             # null block table
    c[7] = P
    c[9] = 48
    assert status("ddt_commit_paged", *c) == ddt.DDT_ERR_UNSUPPORTED                     # page size


def test_gdn_validation():
    def args(**k):
        return [P] * 11 + [1, 8, k.get("L", 4), k.get("H", 1), k.get("dk", 32), k.get("dv", 32), k.get("C", 64),
                           k.get("W", 4), k.get("dt", 0), P, k.get("wsb", 1 << 30), None]
    assert status("ddt_gdn_tree_step", *args(C=63)) == ddt.DDT_ERR_ARG
    assert status("ddt_gdn_tree_step", *args(dk=48, dv=48, C=96)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_gdn_tree_step", *args(dv=64)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_gdn_tree_step", *args(W=9)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_gdn_tree_step", *args(L=64)) == ddt.DDT_ERR_ARG      # depth bound above 63
    assert status("ddt_gdn_tree_step", *args(L=-1)) == ddt.DDT_ERR_ARG
    assert status("ddt_gdn_tree_step", *args(wsb=64)) == ddt.DDT_ERR_WORKSPACE
    assert ddt.gdn_tree_step_workspace(8, 64, 32, 128) > ddt.gdn_tree_step_workspace(1, 64, 32, 128) > 0
    assert status("ddt_gdn_tree_step", *args(dt=2)) == ddt.DDT_ERR_UNSUPPORTED
    a = args()
    a[0] = None
    assert status("ddt_gdn_tree_step", *a) == ddt.DDT_ERR_ARG


def test_gdn_deferred_validation():
    def args(**k):
        a = [P] * 10 + [1, 8, k.get("L", 4), k.get("H", 1), k.get("dk", 32), k.get("dv", 32), k.get("C", 64),
                        k.get("W", 4), k.get("dt", ddt.DDT_BF16), P, k.get("wsb", 1 << 30), None]
        return a
    assert status("ddt_gdn_tree_step_deferred", *args(dt=ddt.DDT_F32)) == ddt.DDT_ERR_UNSUPPORTED  # bf16 only
    assert status("ddt_gdn_tree_step_deferred", *args(C=63)) == ddt.DDT_ERR_ARG
    assert status("ddt_gdn_tree_step_deferred", *args(dk=48, dv=48, C=96)) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_gdn_tree_step_deferred", *args(L=64)) == ddt.DDT_ERR_ARG
    assert status("ddt_gdn_tree_step_deferred", *args(wsb=64)) == ddt.DDT_ERR_WORKSPACE
    a = args()
    a[3] = None                                                       # conv scratch is required
    assert status("ddt_gdn_tree_step_deferred", *a) == ddt.DDT_ERR_ARG
    #     S  S_scratch n  B  H  dk  dv  ws ws_bytes stream
    st = [P, P, 1, 8, 1, 32, 32, P, 1 << 30, None]
    assert status("ddt_gdn_tree_states", *(st[:3] + [65] + st[4:])) == ddt.DDT_ERR_ARG       # B > 64
    assert status("ddt_gdn_tree_states", *(st[:5] + [48, 48] + st[7:])) == ddt.DDT_ERR_UNSUPPORTED
    assert status("ddt_gdn_tree_states", *(st[:8] + [64] + st[9:])) == ddt.DDT_ERR_WORKSPACE
    assert status("ddt_gdn_tree_states", *([None] + st[1:])) == ddt.DDT_ERR_ARG


def test_accept_and_commit_validation():
    a = [P, 0, P, P, 1, 8, 4, 512, P, P, P, P, 8, None]
    assert status("ddt_tree_accept", *a) == ddt.DDT_ERR_WORKSPACE
    a[5] = 65
    assert status("ddt_tree_accept", *a) == ddt.DDT_ERR_ARG
    kv = (ddt.KVLayer * 1)(ddt.KVLayer(256, 256, None, 256))
    gd = (ddt.GDNLayer * 1)()
    c = [P, P, P, kv, 1, 2, 64, 48, 1, gd, 0, 1, 32, 32, 64, 4, 1, 1, 8, 4, None]
    assert status("ddt_commit", *c) == ddt.DDT_ERR_ARG        # null cache pointer in layer 0
    kv[0] = ddt.KVLayer(256, 256, 256 + 8, 256)
    assert status("ddt_commit", *c) == ddt.DDT_ERR_ARG        # misaligned
    c[6] = 60
    kv[0] = ddt.KVLayer(256, 256, 256, 256)
    assert status("ddt_commit", *c) == ddt.DDT_ERR_ARG        # D*2 bytes not a multiple of 16


def test_gdn_replay_validation():
    lay = (ddt.GDNReplayLayer * 1)(ddt.GDNReplayLayer(256, 256, 256, 256, 256, 256, 256))
    #     rows acc  layers n_l H  dk  dv  C    W  dt n  B  L
    r = [P, P, lay, 1, 2, 32, 32, 128, 4, 1, 1, 8, 4, None]
    assert status("ddt_gdn_replay", *(r[:3] + [0] + r[4:])) == ddt.DDT_OK   # no layers: nothing to do
    r2 = list(r); r2[0] = None
    assert status("ddt_gdn_replay", *r2) == ddt.DDT_ERR_ARG                 # null acc_rows
    r2 = list(r); r2[7] = 96
    assert status("ddt_gdn_replay", *r2) == ddt.DDT_ERR_ARG                 # C != 2*H*dk
    r2 = list(r); r2[5] = r2[6] = 48; r2[7] = 192
    assert status("ddt_gdn_replay", *r2) == ddt.DDT_ERR_UNSUPPORTED         # dk not built
    r2 = list(r); r2[8] = 9
    assert status("ddt_gdn_replay", *r2) == ddt.DDT_ERR_UNSUPPORTED         # W > 8
    r2 = list(r); r2[12] = 64
    assert status("ddt_gdn_replay", *r2) == ddt.DDT_ERR_ARG                 # L > 63
    r2 = list(r); r2[9] = 2
    assert status("ddt_gdn_replay", *r2) == ddt.DDT_ERR_UNSUPPORTED         # dtype
    lay[0] = ddt.GDNReplayLayer(256, 256, 256, None, 256, 256, 256)
    assert status("ddt_gdn_replay", *r) == ddt.DDT_ERR_ARG                  # null beta
    lay[0] = ddt.GDNReplayLayer(256, 256, 256, 256, 256, 260, 256)
    assert status("ddt_gdn_replay", *r) == ddt.DDT_ERR_ARG                  # misaligned S


def test_accept_sampled_validation():
    a = [P, 0, P, P, P, P, 1, 8, 4, 512, P, P, P, P, 1 << 30, None]
    a2 = list(a); a2[2] = None
    assert status("ddt_tree_accept_sampled", *a2) == ddt.DDT_ERR_ARG       # no noise
    a2 = list(a); a2[3] = None
    assert status("ddt_tree_accept_sampled", *a2) == ddt.DDT_ERR_ARG       # no temperatures
    a2 = list(a); a2[14] = 8
    assert status("ddt_tree_accept_sampled", *a2) == ddt.DDT_ERR_WORKSPACE
    a2 = list(a); a2[1] = 5
    assert status("ddt_tree_accept_sampled", *a2) == ddt.DDT_ERR_UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        ddt.build_tree(torch.zeros(1, 4, 512), 8, torch.zeros(1, dtype=torch.int32))
