"""CPU oracle -- TEST INFRASTRUCTURE ONLY.

A plain float64 NumPy definition of what the paged-attention library computes. Only the tests,
`__graft_entry__.smoke()` and the bench's CPU-baseline leg may import it; the library itself never
does, and the two share no code.
"""
from . import paged_attention  # noqa: F401
