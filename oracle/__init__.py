"""Plain CPU oracle for the chunked tensor-parallel overlap GEMMs over a capacity UserBuffer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.  The
product path (``chunked_tp_overlap_amd``) never imports it and shares no code with it: no
kernels, helpers, tables or constants.  Both sides receive their inputs from the seeded
generators in ``chunked_tp_overlap_amd.workloads``, which hold none of the method's
arithmetic.

What the oracle computes, and where the pages define it
-------------------------------------------------------
Pages cited by title:

* [TE#3564] "[Feature Request] Support dynamic token counts in TP communication/GEMM
  overlap" (Transformer Engine issue 3564): sections "Problem", "Proposed API",
  "Implementation approach in the prototype".
* [TE#1344] "How to setup TP Overlap configs" (Transformer Engine issue 1344): the
  maintainer's option list ("method", "num_splits", "num_max_streams", "aggregate", ...).
* [MLM#1240] "[QUESTION] Do tp overlap support thd, whose sequence length is flexible?"
  (Megatron-LM discussion 1240): the QKV and MLP shape diagrams.

The method changes which bytes are read and where results go; it does not change the
arithmetic.  So the oracle is the plain definition written out, structured as an explicit
per-chunk loop over offsets into a capacity-sized buffer:

* all-gather side (column-parallel GEMM): each output element is the exact dot product
  of an active-prefix row of the UserBuffer with a weight column, rounded once to bf16;
* reduce-scatter side (row-parallel GEMM): each of the tp K-slice partial products is
  rounded to bf16, the tp partials are summed exactly and rounded once to bf16, and the
  result is cut into tp contiguous shards of T/tp rows.

Precision: fp64 products and sums (exact for the sizes used; see ``gemm``), bf16 encoded
with round-to-nearest-even from the exact value.

Pins (tests marked ``not gpu``): exact integer brute force on the tiny configuration,
exact integer-valued inputs at real shapes, closed forms (all-ones, identity, one-hot,
tp = 1), the invariants the method promises (chunked == unchunked, independence from
capacity and from the chunk/stream schedule, untouched bytes beyond the active prefix,
shard concatenation == full reduce, every row written once), the active-shape constraint
matrix of [TE#3564] and the option semantics of [TE#1344].  No function here is
"parity unpinned".
"""

from . import bf16, manager, plan, gemm  # noqa: F401

__all__ = ["bf16", "manager", "plan", "gemm"]
