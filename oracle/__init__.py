"""CPU oracle for tree-based speculative verification — TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy/Python implementation of what the verification
step computes, written from the SpecInfer pages and shared with nothing on the
GPU side (no kernels, headers, helpers, tables or constants).  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
product path (the HIP library and its Python binding) never does.

Modules
  philox   Philox4x32-10 counter-based generator (Salmon et al., SC'11)
  tree     ancestor / child bitmasks and depths (TreeMask, section 4.2)
  attention  tree attention over the paged prefix + tree KV (Definition 4.1,
             TreeMask, Equations 1-4)
  verify   row statistics, VerifyGreedy, VerifyStochastic (multi-step
           speculative sampling), naive sampling verification
  commit   keep the accepted path's KV entries in contiguous slots
  exact    exact (rational) output distributions of MSS, used as pins

Parity notes: every function here is pinned by a CPU test against something
other than itself (worked values printed on the pages, textbook routines,
closed forms, brute force).  Functions without such a pin say so in their
docstring ("parity unpinned").
"""
from .status import *  # noqa: F401,F403
from . import philox, tree, attention, verify, commit, exact  # noqa: F401,E402
