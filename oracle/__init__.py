"""CPU fp64 oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the tests, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` use it. It shares no code, tables or
helpers with the HIP library; the only thing both sides share is the seeded
input generator, which holds none of the method's arithmetic.

What it computes follows the pages' central claim that the IO-aware tiled
method is exact, i.e. equal to standard attention up to numerical precision
(FlashAttention-2 review, "Введение" section; FlashAttention-1 news page,
"FlashAttention" section).  So the oracle is the textbook definition written
out: materialise the score matrix, apply a max-subtracted softmax, multiply by
V, and differentiate analytically.  ``tiled`` holds a separate fp64 model of
the block-wise online-softmax recurrence used only to pin that equivalence.

Pins (see tests/test_oracle.py): finite differences, PyTorch's CPU fp64
scaled_dot_product_attention and autograd, closed forms (scale = 0, identical
keys, causal row 0, N = 1, a hand-worked 2x2 example), invariants (softmax rows
sum to one, GQA equals MHA with repeated K/V heads, permutation invariance,
gradient identities) and the tiled model.  The block-sparse variant (an
optional block mask on the same functions) is pinned by PyTorch's fp64 masked
scaled_dot_product_attention, finite differences, closed forms and the tiled
model with block skipping (tests/test_oracle_sparse.py).
"""

from .attention import (  # noqa: F401
    attention_fwd,
    attention_bwd,
    attention_head_fwd,
    attention_head_bwd,
    attention_head_probs,
    kv_head_of,
)
from .tiled import tiled_attention_fwd  # noqa: F401
