"""CPU oracle of the fused grouped-MLP MoE expert block.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import anything under oracle/.  The product
path (moe_grouped_mlp_amd) never imports, links or runs it, and the oracle
imports nothing from the product path: the two share no code.

It is a plain float64 NumPy implementation: `numerics` holds the bf16 and
MXFP8 (E4M3 + E8M0) storage formats, `moe` the expert block itself.
"""

from . import numerics, moe  # noqa: F401
