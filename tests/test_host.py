"""Host-side contracts that need no GPU: the bench's single-GPU guard, the product
package's independence from the oracle, the step's layer pattern, and the binding's
loud failure when the library is missing."""

import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "tree_speculative_decoding_ddt_amd")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_product_package_never_imports_the_oracle():
    for name in os.listdir(PKG):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        for node in ast.walk(tree):
            mods = []
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)


def test_layer_pattern_of_the_hybrid_stack():
    from tree_speculative_decoding_ddt_amd.step import HybridConfig
    p = HybridConfig().layer_pattern()
    assert len(p) == 64 and p.count("attn") == 16 and p.count("gdn") == 48
    assert p[:4] == ["gdn", "gdn", "gdn", "attn"] and p[-4:] == ["gdn", "gdn", "gdn", "attn"]
    assert HybridConfig(n_attn=1, n_gdn=2).layer_pattern() == ["gdn", "gdn", "attn"]
    assert HybridConfig(pattern=["attn", "gdn"]).layer_pattern() == ["attn", "gdn"]


def test_binding_fails_loudly_without_the_library(tmp_path):
    code = ("import tree_speculative_decoding_ddt_amd.ddt as d\n"
            "d.LIB_PATH = %r\n"
            "d._lib = None\n"
            "try:\n    d.lib()\nexcept RuntimeError as e:\n    print('refused:', e)\n" % str(tmp_path / "missing.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert "refused:" in r.stdout and "not built" in r.stdout
