"""Float64 CPU oracle for paged split-KV decode attention and its LSE merge.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py``
may import or call anything in this package.  The GPU library never links,
imports or falls back to it, and this package imports nothing from the GPU
library: the two share only the seeded input generator, which holds none of
the method's arithmetic.

What it computes (KV-cache engineering page, section "Exact recent pages,
compact older pages"): single-token decode attention over a request's whole
key/value history, once in one pass, and once tile by tile where every tile
gives an output already divided by its own softmax sum plus the log-sum-exp
of its scores, and a merge reweights the tiles by exp(lse_t - max lse),
divides by the total weight and reports max + log(total) as the combined
log-sum-exp.  The merged result is softmax attention over every key.

The compact representation of older pages (same page and section: runs of
two representations, a page converted once fully written, with a CRC) is in
``compact``: E4M3 codes with one FP32 scale per block, dequantisation,
CRC-32 and an error bound for the log-sum-exp.

Every function here is pinned by ``tests/test_oracle.py`` against things
other than itself: brute force with exact summation, library routines
(torch's scaled-dot-product attention, scipy's logsumexp), closed forms,
hand-derived golden fixtures and planted mistakes; ``compact`` by
``tests/test_oracle_compact.py``.

``admission`` is a plain planner of which logical pages of which contexts
hold device pages each step (Staging without a stall, section "Admission
that does arithmetic"; GPU memory management, section "Pages held by right,
borrowed or free"), pinned by ``tests/test_oracle_admission.py``.
"""

from .attention import (  # noqa: F401
    widen_bf16,
    attend,
    tile_bounds,
    tile_partials,
    merge,
    decode_one_pass,
    decode_tiled,
    stress_partials,
    union_attention,
)
from . import admission, compact  # noqa: F401
