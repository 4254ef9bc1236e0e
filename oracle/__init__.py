"""CPU oracle for support-aware paged alpha-entmax decode (TEST INFRASTRUCTURE).

This package is a plain, slow, fp64 restatement of what the decode path
computes, written from the EntmaxKV summary page (gist.science, paper
2605.21649: "EntmaxKV – Décodage Conscient du Support pour l'Attention
Entmax") and from the standard alpha-entmax mapping (Peters, Niculae &
Martins, 2019), which that page names but does not write out.

It is test infrastructure only.  Nothing but the test-suite, the smoke check
and the CPU-baseline leg of the benchmark may import or execute it; the
product path (the HIP library and its Python binding) never calls it, and it
shares no code, constants or helpers with that path.

Modules:
  entmax   -- the alpha-entmax threshold and weights (and a softmax branch
              used only to pin the alpha -> 1 limit)
  meta     -- per-page key metadata (bounding box, mean, variance)
  scores   -- box upper bound and Gaussian score moments per page
  select   -- top-k page selection and Gaussian-aware selection (tau-hat)
  softmax  -- softmax decode over a kept set and its dropped mass (the
              comparison side of the method)
  pipeline -- the per-(row, KV head) composition used by the tests

Every function is pinned by tests under tests/ (marked "not gpu") against
closed forms, invariants, special cases and brute force; see each module's
docstring.  The one approximation with no such pin is how well tau-hat - Delta
recovers the true support (the pages print no numbers for it): parity unpinned
for that property, only reported.
"""
from . import entmax, meta, scores, select, softmax, pipeline  # noqa: F401
