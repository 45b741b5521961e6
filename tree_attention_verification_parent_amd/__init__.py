"""MI355X-native tree-verification step of EAGLE-style speculative sampling.

The hot path (tree mask, tree attention, vocabulary statistics, acceptance
walk, KV compaction, feature gather) is hand-written HIP for gfx950 in csrc/, exported
through the C ABI declared in include/eagle_verify.h and bound here with
ctypes (binding.py).  Build with `python -m
tree_attention_verification_parent_amd.build`.
"""
from .binding import (EagleError, abi_version, alloc_workspace, attn_plan,  # noqa: F401
                      dtree_expand, testing_attn_plan, testing_read_floor,
                      dtree_rerank, dtree_select, feature_gather, kv_compact, lib,
                      tree_attn, tree_attn_parents, tree_attn_parents_noalloc,
                      tree_attn_workspace_bytes, tree_build,
                      validate_tree_host,
                      verify_accept, verify_accept_compact, verify_accept_workspace_bytes,
                      workspace_clear)
