"""Plain float64 CPU oracle for block-sparse and BLASST attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library (no
kernels, headers, helpers, tables or pre/post-processing); the only thing
both sides consume is the seeded input data from ``workloads``.

Every function states the passage of the source pages it follows:

* "Block-sparse attention in practice" (the multimodal DiT article):
  section 2.1 (mask families), section 2.3 (block grid, sparsity ratio),
  section 3.2 (multimodal mask recipe), section 3.3 (skip a masked block
  before loading K/V), section 5.2 (masked blocks take no part in the
  softmax statistics; padding blocks are never computed).
* "BLASST: Dynamic Blocked Attention Sparsity via Softmax Thresholding"
  (paper notes): section 3.1.1 (softmax and the pruning condition),
  Algorithm 1 (FlashAttention with BLASST), section 4 (tile-wide vote),
  section 4.2 (decode kernel skips the V load).
* "72 changes of attention" tutorial: section 4.2 (online softmax) and its
  GQA section (query heads grouped onto shared K/V heads).

Readings taken where the pages are silent or ambiguous are listed in the
module docstrings (threshold in the scaled-score domain, tile-uniform vote,
strict "<", ascending block order, empty rows give zero, decode tile = the
query heads sharing one K/V head, split-invariant decode).

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against library routines, closed forms, brute force or the pages' error
bound, except the synthetic-input generator readings (which live in
``workloads`` and are "parity unpinned": the pages print no values for
them).
"""

from . import masks, attention  # noqa: F401
