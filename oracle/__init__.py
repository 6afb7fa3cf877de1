"""fp64 CPU oracle for the block-sparse attention backward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Parity status of each function (what pins it, in ``tests/test_oracle.py``):

* ``element_mask`` / ``block_lists``: hand-worked example (``tests/golden``),
  brute-force properties (ascending, row/column lists transpose each other,
  expansion reproduces the clipped mask).
* ``forward`` / ``backward`` (and the ``_dense`` twins): central finite
  differences of sum(dO*O) on tiny inputs (GQA, partial blocks, TND, padded
  BNSD), equality with torch fp64 autograd for the dense and the element-mask
  special cases, closed forms (Q = 0; one key per row; the worked sample of the
  aclnnBlockSparseAttentionGrad page), the dK / dV column-sum invariants, and
  the GQA / TND / padding identities.
* ``backward_dq_rows`` / ``backward_dkdv_rows``: equal to the matching rows of
  ``backward``.
* ``head_probs_and_ds`` (the P and dS the backward contracts, one head): every
  row of dS sums to zero with the exact forward's O and LSE, and every row of
  P sums to one within 4 * 2^-24 * max(1, |LSE|) with the LSE rounded to fp32
  (``tests/test_oracle.py``, with windows and attenMasks).
* the sliding window (``window=(pre, nxt)``, ``in_window``; in
  ``tests/test_oracle_window.py``): finite differences with windows that do and
  do not contain the diagonal, torch fp64 autograd on a hand-built element mask,
  the zero-width-window closed form, slab path == dense path (with rows the
  window leaves empty), the block lists against an interval formula, and the
  row-sampled helpers.
* the attenMask (``atten_mask``, ``allowed_pairs``; same file): torch fp64 autograd on
  a hand-built element mask (alone and with a window), finite differences (TND,
  with a window), slab path == dense path with a row the mask empties, and the
  row-sampled helpers.
* fp8 inputs (``oracle/fp8.py``: ``decode``, ``dequantize``, ``backward_fp8``,
  ``forward_fp8``; in ``tests/test_oracle_fp8.py``): hand-worked code values
  from the OCP format definitions (``tests/golden/fp8_values.json``), torch's
  float8 dtypes over all 256 codes, IEEE binary16 for E5M2, monotone positive
  codes, and the per-tensor factors against hand-scaled plain-oracle calls,
  scaling identities and a torch fp64 forward.

No function here is "parity unpinned".
"""
from .ref import *  # noqa: F401,F403
from .ref import __all__  # noqa: F401
