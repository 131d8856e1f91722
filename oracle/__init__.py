"""CPU oracle for the forward pass of dynamic block-sparse attention (BSA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call,
link or execute anything in this directory; only the test suite, the smoke
check and the CPU-baseline leg of the benchmark use it.  It shares no code
with the GPU path.

Source: "Decoupling Logical Masks from GPU Execution for Dynamic Block-Sparse
Attention" (Tessera).  The method reaches exactly (up to rounding order) the
result of dense attention restricted to the token pairs named by the logical
mask, E(M) (paper section 2.2 and section 4.2, "Coarsened": normalization and
the weighted value sum include only entries of E(M)).  The oracle is that
definition written out in float64:

* ``attention``   dense masked attention, every row (section 1, section 2.2)
* ``attention_rows``  the same definition for a chosen set of rows
* ``coverage``    enumeration of E(M) at token and at cell level
* ``stats``       density and active-block-run coverage (sections 4.3, 5.1)
* ``merge``       split-K partial states and their merge (section 4.3)
* ``brute``       pure-Python loops for tiny inputs (pins the vectorized code)

Readings of points the paper leaves open, used throughout: scores are scaled
by 1/sqrt(d); a query row with no active block outputs zeros; attention is
non-causal; the mask grid is ceil(N/B_Q) x ceil(N/B_KV), so the last block of
each dimension is ragged and keys j >= N never enter the softmax.

Parity pins (no function here is "parity unpinned"): tests/test_oracle_pins.py.
"""

from . import attention, brute, coverage, merge, stats  # noqa: F401
from .attention import attention as masked_attention  # noqa: F401
from .attention import attention_rows as masked_attention_rows  # noqa: F401
