"""CPU oracle for the RWKV-6 WKV forward operator -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import anything from this package.  The HIP library never
calls it, shares no code with it, and fails loudly when its own extension is
missing instead of falling back to it.

Contents (all arithmetic in float64 on the exact input values):

* ``wkv6_ref``         -- the recurrent definition, one token at a time;
* ``wkv6_bruteforce``  -- the explicit double sum over token pairs, with every
                          decay product formed term by term (tiny inputs only);
* ``decay``            -- w = exp(-exp(w_raw));
* ``wkv6_ref_backward`` -- gradients of sum(y * dy) w.r.t. every input, by the
                          adjoint of the recurrence;
* ``wkv5_ref``         -- RWKV-5: the same operator with one decay per channel
                          for every token;
* ``wkv4_ref``         -- RWKV-4: the normalised per-channel (vector-state)
                          operator, in its recurrent form;
* ``group_norm_heads``, ``wkv6_gn_ref`` -- the per-head group normalisation
                          and gate that follow the operator in a block.

Every function here is pinned by tests that do not rely on the oracle itself
(closed forms, a hand-worked example, invariants, brute force on tiny inputs);
there is no "parity unpinned" function in this package.
"""
from .wkv6_oracle import decay, wkv6_ref, wkv6_bruteforce, wkv6_ref_backward, split_heads, merge_heads
from .variants_oracle import wkv4_ref, wkv5_ref
from .epilogue_oracle import group_norm_heads, wkv6_gn_ref

__all__ = ["decay", "wkv6_ref", "wkv6_bruteforce", "wkv6_ref_backward", "split_heads", "merge_heads",
           "wkv4_ref", "wkv5_ref", "group_norm_heads", "wkv6_gn_ref"]
