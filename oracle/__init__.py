"""Plain CPU oracle for SparVAR's block-sparse cross-scale attention.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The library (``block_sparse_cross_csla_amd``) never does, and this
package imports nothing from it: the two share no code.

It is written to be read against the pages ("SparVAR: Exploring Sparsity in
Visual AutoRegressive Modeling for Training-Free Acceleration", the ai.info
summary, sections "Key Contributions", "Main Findings" and "Methodology in
Plain English"), not to be fast: numpy, float64 for floating point, token-level
brute force wherever the method has a token-level definition.

Modules
-------
geometry   scale offsets, key tiles and query tiles of the multi-scale grid
csla       the CSLA token mask (sink + cross-scale locality window), its block
           aggregation, the per-row tile budget variant, and index lists
cs4a       decision-scale block scores, top-p selection, index mapping
attention  masked softmax attention (mask applied token-wise as -inf)
ocache     the decision-scale residual, upsampled onto a later scale's output
schedule   the per-scale loop with both modules and the window schedule

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself: library routines, closed forms, invariants, brute force on tiny
inputs and hand-derived fixtures under ``tests/golden/``.
"""
from . import geometry, csla, cs4a, attention, ocache, schedule  # noqa: F401
