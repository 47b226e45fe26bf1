"""fp64 CPU oracle for sink attention.  TEST INFRASTRUCTURE ONLY.

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg.  The HIP library never imports or calls anything here.
"""

from .attn import allowed_mask, ref_bwd, ref_decode, ref_fwd, unmasked_pairs
from .brute import brute_fwd

__all__ = ["allowed_mask", "ref_fwd", "ref_bwd", "ref_decode", "unmasked_pairs",
           "brute_fwd"]
