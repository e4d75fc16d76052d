"""MI355X (gfx950) prioritized-replay sum tree: HIP kernels behind a C ABI.

The public ABI is include/per.h (libper.so); per.py is its Python binding.
"""
from .per import (PerBuffer, PerError, load, per_add, per_capacity, per_create, per_cursor,
                  per_destroy, per_flush, per_graph_mode, per_last_error, per_max_priority, per_min, per_sample,
                  per_rank_attach,
                  per_rank_ptrs, per_rank_refresh, per_rank_workspace_bytes,
                  per_sample_padded, per_sample_philox, per_sample_rank, per_sample_uniform,
                  per_set_sample_lanes, per_size,
                  per_state_dim, per_time_next, per_total, per_tree_ptrs, per_update, per_update_add,
                  per_update_static, per_workspace_bytes)

__all__ = ["PerBuffer", "PerError", "load", "per_add", "per_capacity", "per_create",
           "per_cursor", "per_destroy", "per_flush", "per_graph_mode", "per_last_error", "per_max_priority", "per_min",
           "per_rank_attach", "per_rank_ptrs", "per_rank_refresh",
           "per_rank_workspace_bytes", "per_sample", "per_sample_padded", "per_sample_philox",
           "per_sample_rank", "per_sample_uniform", "per_set_sample_lanes", "per_size", "per_state_dim", "per_time_next", "per_total", "per_tree_ptrs", "per_update",
           "per_update_add", "per_update_static",
           "per_workspace_bytes"]
