"""fp64 CPU oracle of EAGLE tree verification.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy float64 implementation of what the
tree-verification path computes, written from the pages' statement of the
method:

* "Speculative decoding with EAGLE" (aiunderstanding.org), sections
  Deep dive and Technical insight: a cheap drafter proposes candidate tokens,
  the target checks all of them in one parallel pass and keeps the longest
  correct prefix; accepted tokens must equal the target's own (argmax) choice,
  so the output is identical to the target decoding alone; the drafter works
  on hidden features, is fed the true embedding of the previous token and
  reuses the target's LM head.
* "LLM parallel decoding EAGLE" (jisaku.com glossary), section on how EAGLE
  works: a one-layer decoder head predicts the next feature from the final
  hidden features; several token candidates per predicted feature are
  expanded into a tree; tree attention verifies every node in one forward
  pass and the longest valid path is accepted.  Its EAGLE vs EAGLE-2 table
  and FAQ Q3 give tree sizes (60 fixed; 40..120 adaptive) and the 0.3
  confidence threshold.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path;
the only shared module is ``workloads`` (seeded input draws and the bf16
storage format), which holds none of the method's arithmetic.

Parity unpinned: the static tree shapes and the dynamic-tree recipe are
readings (no shape is printed on the pages); accepted lengths of trained
models cannot be reproduced with random weights.  Everything else in this
package is pinned by the CPU tests (closed forms, brute force, chain and
single-node reductions, per-path sequential re-runs, lossless greedy
decoding).
"""
from .tree import tree_encode, pack_ancestors, encode_batch, TreeEncoding
from .layer import (as_f64, rms_norm, rope_rotate_half, attend, layer_rows, verify_forward,
                    lm_head_logits, lm_head_argmax, silu)
from .accept import (accept_sequence, accept_batch, commit_sequence, sample_accept_sequence, sample_summaries,
                     sample_accept_from_summaries)
from .draft import draft_expand, draft_select_level, draft_rerank, fuse_features
from .decode import (verify_forward_layers, commit_layers, draft_kv_rows, draft_kv_commit, eagle_decode,
                     greedy_decode)

__all__ = [
    "tree_encode", "pack_ancestors", "encode_batch", "TreeEncoding",
    "as_f64", "rms_norm", "rope_rotate_half", "attend", "layer_rows", "verify_forward",
    "lm_head_logits", "lm_head_argmax", "silu",
    "accept_sequence", "accept_batch", "commit_sequence", "sample_accept_sequence", "sample_summaries",
    "sample_accept_from_summaries",
    "draft_expand", "draft_select_level", "draft_rerank", "fuse_features",
    "verify_forward_layers", "commit_layers", "draft_kv_rows", "draft_kv_commit", "eagle_decode", "greedy_decode",
]
