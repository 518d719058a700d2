"""fp64 CPU oracle for exact attention: test infrastructure, never the product path.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
"""
from .attention import (MASK_BLOCK, backward, backward_head, forward, forward_head, kv_head,
                        merge, probabilities_head, window_bounds)
from .fp8 import (e4m3_round, e4m3_values, forward_fp8_head, fp8_scores, hadamard, pow2_scale,
                  quantize_key_blocks, quantize_rows, quantize_tiles)

__all__ = ["MASK_BLOCK", "forward", "forward_head", "backward", "backward_head", "kv_head", "merge",
           "probabilities_head", "window_bounds", "e4m3_round", "e4m3_values", "forward_fp8_head",
           "fp8_scores", "hadamard", "pow2_scale", "quantize_key_blocks", "quantize_rows", "quantize_tiles"]
