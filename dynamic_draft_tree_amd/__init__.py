"""libeagletree: EAGLE-2 dynamic draft trees on one MI355X (gfx950).

The product is the C-ABI library libeagletree.so (include/eagletree.h);
this package holds its HIP sources (csrc/), the build step and a thin
ctypes binding that passes torch device pointers and streams through.
"""
from .binding import (EXPORTS, EtError, Plan, et_accept,  # noqa: F401
                      et_accept_noalloc,
                      et_accept_sample, et_config, et_draft_step_hidden,
                      et_draft_step_static,
                      et_set_static_shape, et_static_tree,
                      et_draft_step, et_kv_commit, et_plan_create,
                      et_plan_destroy,
                      et_pool_capacity, et_pool_export, et_rerank,
                      et_rerank_mask, et_draft_step_last,
                      et_tree_attention, et_tree_mask, et_workspace_bytes,
                      et_workspace_init, lib, make_config)
