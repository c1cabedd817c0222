"""fp64 CPU oracle for 2D relative-position-encoded attention (forward).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never calls it, and this package
imports nothing from the product path.

What it computes, and the passages it follows:

* ``index``     - the per-axis index function g (iRPE summary page, "Rethinking
  and Improving Relative Position Encoding for Vision Transformer", Method,
  eq. 18), both readings of its rounding, and the Swin identity index with
  the shift by M-1 (Swin 2D RPE post, sections 3.1-3.2).
* ``buckets``   - token positions of one attention unit (a window or a whole
  grid) and the per-pair bucket id of the Product mapping (iRPE page, eq. 25;
  Swin post, section 3.2), or the two rows of the Cross mapping (eqs. 22-24),
  with no bucket for prefix (class) tokens.
* ``backward``  - gradients of the forward with respect to q, k, v and every
  table, from the same per-pair definition (softmax, scale, bucket sums).
* ``attention`` - the attention forward written as a per-pair definition:
  offset -> index -> table row -> logit term, softmax, value sum
  (iRPE page eqs. 1-3 and 13-17; Swin relative-bias record, "The claim").
  Two implementations: ``attention_literal`` (pure Python loops, tiny
  shapes) and ``attention`` (NumPy, per-pair gathers in query-row chunks).

Every function works in float64 on inputs upcast exactly from their dtype.

Parity status (pins live in tests/test_oracle_*.py):

* g for |x| <= alpha, oddness, monotonicity, saturation: pinned by invariants.
* g under the truncating reading at r = 1.9: pinned by the iRPE page's hand
  worked partition (Pitfalls, "Bucket edges are sharp").
* g under the capped reading beyond the last truncated step (offsets 11-13
  at r = 1.9, >= 29 at r = 3.8): parity unpinned beyond the invariants and
  the bucket counts; no page prints these values.
* Swin index: pinned by the Swin post's M = 3 worked example and table sizes.
* Attention: pinned by zero-table and constant-table reductions to a library
  softmax attention, by the Shaw-style page's printed weights (1D special
  case), by a large single-cell bias that pins the offset sign and axis
  order, and by literal-vs-vectorised agreement on tiny grids.
* The value term (r^V) is pinned only by closed forms (constant table,
  isolation); no page prints a value-term output.
* The undirected mappings (``undirected``; Euclidean eqs. 19-20 and
  Quantization eq. 21, each in the page's and the code's reading): pinned by
  the page's distance list and its adjacent-offsets example, a Fermat
  sum-of-two-squares count, Pythagorean offsets, symmetry and saturation
  invariants, the reduction to the directed index on an axis, and an
  attention-level reduction to a symmetric Product table on one row.
* The backward pass: pinned by central finite differences of the (pinned)
  forward for every input and table, in every mode and mapping, and by
  torch's autograd of a library softmax attention without position terms.
* The Cross mapping (iRPE page, Method, eqs. 22-24): pinned by the Shaw-style
  page's printed weights along a one-row and a one-column grid (which also
  fixes the row half [0, S) / column half [S, 2S) split of its table), by
  its identity with the Product mapping of the summed rows, and by
  literal-vs-vectorised agreement.
"""

from .index import (  # noqa: F401
    ROUND_CAPPED,
    ROUND_TRUNC,
    round_half_away,
    piecewise_index,
    half_width,
    axis_index_table,
)
from .buckets import Spec, unit_positions, bucket_map, num_buckets  # noqa: F401
from .undirected import UNDIRECTED_MAPS, undirected_index  # noqa: F401
from .attention import attention, attention_literal, unit_token_indices  # noqa: F401
