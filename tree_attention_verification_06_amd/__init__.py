"""MI355X (gfx950) EAGLE tree verification: HIP kernels behind a C ABI, with a thin ctypes binding.

The C ABI (include/eagle.h) has four calls on the hot path: eagle_tree_build,
eagle_tree_verify, eagle_accept_commit and eagle_draft_expand; acceptance at temperature
T > 0 has eagle_tree_verify_sample and eagle_accept_commit_sample.  Besides them:
eagle_draft_pool (reads back the draft's candidate pool), eagle_pack_fragments (a
load-time weight layout), eagle_fuse_features (the EAGLE-3 draft input), and for a target of
several layers eagle_tree_verify_layers, eagle_accept_commit_layers and eagle_draft_kv_commit;
caches may be paged (PagedCache: a page pool addressed through a block table).  This package
re-exports them with the same names (argument marshalling only) and a small
convenience runner.  The library must be built first (__graft_entry__.build());
importing works without it, calling does not.
"""
from ._abi import (EAGLE_BF16, EAGLE_F32, EAGLE_OK, EagleError, Timer, eagle_accept_commit,
                   eagle_accept_commit_sample, eagle_draft_expand, eagle_draft_pool, eagle_fuse_features,
                   eagle_pack_fragments, eagle_tree_build, eagle_tree_verify, eagle_tree_verify_sample,
                   eagle_workspace_init, eagle_workspace_size, lib, status_str, EagleDraftParams, STAGES, LIB_PATH,
                   eagle_tree_verify_layers, eagle_accept_commit_layers, eagle_draft_kv_commit, PagedCache,
                   eagle_tree_verify_noalloc)

__all__ = ["EAGLE_BF16", "EAGLE_F32", "EAGLE_OK", "EagleError", "Timer", "eagle_accept_commit",
           "eagle_accept_commit_sample", "eagle_draft_expand", "eagle_draft_pool", "eagle_fuse_features",
           "eagle_pack_fragments", "eagle_tree_build", "eagle_tree_verify", "eagle_tree_verify_sample",
           "eagle_workspace_init", "eagle_workspace_size", "lib", "status_str", "EagleDraftParams", "STAGES",
           "LIB_PATH", "eagle_tree_verify_layers", "eagle_accept_commit_layers", "eagle_draft_kv_commit", "PagedCache",
           "eagle_tree_verify_noalloc"]
