"""CPU oracle for exact scaled-dot-product attention (float64, numpy).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it. It shares no code with the HIP kernels; the only common
module is the seeded input generator (`attn_inputs`), which holds no
attention arithmetic.

The oracle is the plain definition written out: it materialises the score
matrix S and the probability matrix P (row block by row block, to bound host
memory) and evaluates the textbook softmax backward. It does not tile over
keys and does not use the online-softmax recurrence; the method reaches the
same real-arithmetic result (page 1, key design 2, Theorem 1 statement), so
the definition is what the kernels are compared against.

Pins (tests/test_oracle_pins.py) tie it to what the pages and the
mathematics fix: the page-3 worked example, the two-block merge, row sums,
identical keys, the causal first row, finite differences, the D identity,
special cases, gradient invariants, mask reductions and permutation
equivariance. Packed variable-length batches are in oracle/varlen.py and
dropout in oracle/dropout.py (tests/test_oracle_varlen.py,
tests/test_oracle_dropout.py). The dropout generator (Philox4x32-10) is
pinned to rocRAND's implementation of the same function, run on the host, and
the GPU must reproduce it bit for bit. No function is left unpinned.
"""
from .attention import (  # noqa: F401
    kept_pairs,
    forward_head,
    backward_head,
    forward,
    backward,
    backward_head_sampled,
    merge_normalised,
    merge_softmax_blocks,
    softmax_block_state,
)
