"""CPU fp64 oracle for the FlashAttention backward pass.

TEST INFRASTRUCTURE ONLY.  This package is the independent checker of the
GPU library: it is imported only by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark.  The product path never imports it and it
never imports the product: the two share no code, constants or helpers.  The
only thing both sides consume is the seeded synthetic input data, produced
by a separate module that holds none of the method's arithmetic.

Contents
  attention  plain forward / backward with S, P, dS materialised (numpy fp64),
             for equal or different query/key lengths and packed varlen batches
  philox     Philox4x32-10 and the dropout keep mask (numpy uint64)

Parity pins (tests/test_oracle_*.py): finite differences, torch fp64 autograd
through scaled_dot_product_attention, invariants (sum_j dS_ij = 0,
sum_j dK_j = 0, sum_j dV_j = sum_i dO_i), special cases (N = 1, equal V
rows, causal row 0, the causal boundary, window support), the D identity,
the pages' memory table, and Philox outputs of two independent library
implementations compiled and run at test time.  No function here is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    Spec,
    backward,
    credited_flops,
    dropout_mask,
    forward,
    head_backward,
    head_columns_backward,
    head_forward,
    head_rows_backward,
    head_rows_forward,
    materialised_p_bytes,
    saved_state_bytes,
    valid_mask,
    varlen_backward,
)
from .philox import (  # noqa: F401
    dropout_keep,
    dropout_uniform_bits,
    keep_threshold,
    philox4x32_10,
)
