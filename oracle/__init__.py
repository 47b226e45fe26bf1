"""fp64 CPU oracle for sink attention.  TEST INFRASTRUCTURE ONLY.

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg.  The HIP library never imports or calls anything here.
"""

from .attn import (allowed_mask, gather_paged, ref_bwd, ref_bwd_varlen, ref_decode, ref_decode_paged, ref_fwd,
                   ref_fwd_varlen, unmasked_pairs)
from .brute import brute_fwd, brute_fwd_docs, brute_rope
from .rope import (apply_rope_adjoint, apply_rope_bf16, apply_rope_exact, ref_bwd_rope, ref_decode_rope, ref_fwd_rope,
                   rope_table, round_bf16, yarn_inv_freq, yarn_mscale)

__all__ = ["allowed_mask", "ref_fwd", "ref_bwd", "ref_decode", "ref_decode_paged", "gather_paged", "unmasked_pairs",
           "ref_fwd_varlen", "ref_bwd_varlen", "brute_fwd", "brute_fwd_docs", "brute_rope", "yarn_inv_freq",
           "yarn_mscale", "rope_table", "apply_rope_exact", "apply_rope_bf16", "round_bf16", "ref_fwd_rope", "ref_decode_rope",
           "apply_rope_adjoint", "ref_bwd_rope"]
