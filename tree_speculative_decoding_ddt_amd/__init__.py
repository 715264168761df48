"""DDTree tree-verification step on MI355X (gfx950).

The step -- draft-tree build, tree-masked attention, branch-local Gated
DeltaNet + short conv, greedy tree walk, accepted-path commit -- runs in
hand-written HIP kernels behind the C ABI of ``libddt.so`` (declared in
``include/ddt.h``).  ``tree_speculative_decoding_ddt_amd.ddt`` is the thin
ctypes binding; ``synth`` draws seeded synthetic inputs.

Importing the package does not load the library; ``ddt.lib()`` does, and
raises if it has not been built.
"""
