"""CPU oracle for the DDTree verification step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy definition of what the step computes, written from
the source pages (cited per function by page title and section) and, where the
pages are silent, from the readings each module states in its own docstring.  It is independent of
the HIP library: the two share no code, and neither imports the other.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(``tree_speculative_decoding_ddt_amd``) never does, and fails loudly when its
HIP library is missing instead of falling back to this code.

Modules
  tree       -- per-depth log-softmax + top-K, best-first tree build, flatten
  attention  -- tree-masked attention as a dense masked softmax
  rope       -- rotary embedding of the tree rows at positions prefix + depth
  paged      -- the committed cache in pages: gather, paged attention, paged commit
  gdn        -- short causal conv + gated delta rule over the tree
  accept     -- target argmax + greedy tree walk
  sampled    -- the walk over sampled target tokens (Gumbel-max, noise as input)
  commit     -- copy of the accepted path into the committed buffers
  step       -- the whole verify step composed from the above

Every function takes and returns NumPy arrays; floating-point inputs are
promoted to float64 before any arithmetic.
"""

from . import tree, attention, rope, gdn, accept, commit, paged, sampled, step, gaps  # noqa: F401
