"""CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may
import this package.  The product (the HIP library and its Python binding) never does,
and the oracle never imports the product.  See ``oracle.attention`` (forward) and
``oracle.backward`` (gradients) for what is computed and which passages of the pages
each function follows.

Every function here is pinned by ``tests/test_oracle_pins.py`` to values printed on
the pages, closed forms, invariants and a 50-digit brute force on tiny inputs.
"""
from .attention import (  # noqa: F401
    visible_mask, scores, softmax_probs, attention, split_bounds, partial_state,
    split_states, merge_states, naive_average, attention_split, attention_varlen, flops,
)
from .backward import attention_bwd, row_dot  # noqa: F401
