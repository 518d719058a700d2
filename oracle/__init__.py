"""fp64 CPU oracle for exact attention: test infrastructure, never the product path.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
"""
from .attention import (backward, backward_head, forward, forward_head, kv_head, merge,
                        probabilities_head, window_bounds)

__all__ = ["forward", "forward_head", "backward", "backward_head", "kv_head", "merge",
           "probabilities_head", "window_bounds"]
