"""fp64 CPU oracle (test infrastructure only; see reference.py for the rules)."""
from .reference import *  # noqa: F401,F403
from .reference import (widen, kv_cache_write, gather_sequence, kv_head_of, is_visible,  # noqa: F401
                        visibility_matrix, attend, paged_attention, split_logical,
                        workload_attention, lse_merge, brute_force, fused_head_attention,
                        piecewise_segments, uniform_spans)
