"""CPU oracle for block-sparse programmable attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute this package.  Its users are the test suite, the smoke check and the
CPU-baseline leg of the benchmark.  It shares no code with the GPU library: no
kernels, headers, helpers, constants or tables.

What it computes, in plain numpy float64:

* ``masks``     -- the element predicate M(b, i, j) of the mask menu (causal,
                   sliding window, document equality, prefix-LM, and/or trees),
                   evaluated directly on index arrays.
* ``blockmask`` -- the exact three-state block classification (empty, partial,
                   full) and the compacted row/column block tables derived from it.
* ``attention`` -- dense attention with a materialised score matrix:
                   scale, score modification, mask to -inf, softmax, weighted sum
                   of values, log-sum-exp; no online softmax, no tiling.
* ``merge``     -- the merge law of partial softmax states, used only to pin the
                   split-KV combination.
* ``paged``     -- the logical K/V of a paged cache (page-table gather), so that
                   paged attention is checked against dense attention on it.
* ``backward``  -- dQ, dK, dV of the dense definition by float64 autograd.
* ``selector``  -- block tables from selector candidate lists (range check, sort,
                   repeat removal, rule inside the chosen blocks, exact classes) and
                   the longest-row-first work order.

Parity status of every function is stated in its docstring; each is pinned by
the tests in ``tests/test_oracle_pins.py`` against values and identities that
the pages and elementary mathematics fix.
"""
from . import masks, blockmask, attention, merge, paged, backward, selector  # noqa: F401
