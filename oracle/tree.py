"""Tree encode: parent array -> depth, ancestor sets, position ids.

TEST INFRASTRUCTURE (fp64 oracle; see the package docstring for who may import it).

Source: "LLM parallel decoding EAGLE" page, section on how EAGLE works (tree
expansion of candidates; tree attention lets every node be verified in one
forward pass).  Every node sees the committed prefix plus the nodes on its own
root path, itself included.  Readings where the pages are silent:
node 0 is the root (the last committed token, not yet in the KV cache), a
parent always precedes its child (0 <= parent[i] < i), and a node's position
id is prefix_len + depth.
"""
from dataclasses import dataclass

import numpy as np


class TreeError(ValueError):
    pass


@dataclass
class TreeEncoding:
    depth: np.ndarray   # [N] int64
    anc: np.ndarray     # [N][N] bool, anc[i, j] iff j is i or an ancestor of i
    pos: np.ndarray     # [N] int64


def validate_parent(parent):
    n = len(parent)
    if n < 1:
        raise TreeError("empty tree")
    if parent[0] != -1:
        raise TreeError("node 0 must be the root (parent -1)")
    for i in range(1, n):
        if not (0 <= parent[i] < i):
            raise TreeError(f"parent[{i}]={parent[i]} not in [0, {i})")


def tree_encode(parent, prefix_len):
    """depth(i) = depth(parent(i)) + 1; anc(i) = {i} U anc(parent(i)); pos(i) = prefix_len + depth(i)."""
    parent = [int(p) for p in parent]
    validate_parent(parent)
    n = len(parent)
    depth = np.zeros(n, dtype=np.int64)
    anc = np.zeros((n, n), dtype=bool)
    for i in range(n):
        if i > 0:
            depth[i] = depth[parent[i]] + 1
            anc[i] = anc[parent[i]]
        anc[i, i] = True
    return TreeEncoding(depth=depth, anc=anc, pos=prefix_len + depth)


def pack_ancestors(anc, mask_words):
    """Bit j of word w of row i is set iff anc[i, 64*w + j]."""
    n = anc.shape[0]
    if n > 64 * mask_words:
        raise TreeError("tree larger than the mask capacity")
    out = np.zeros((n, mask_words), dtype=np.uint64)
    for i in range(n):
        for j in np.nonzero(anc[i])[0]:
            out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


def encode_batch(parents, prefix_len, mask_words):
    """Concatenate the encodings of B trees: anc words [sum N][MW], depth [sum N], pos [sum N]."""
    encs = [tree_encode(p, int(prefix_len[b])) for b, p in enumerate(parents)]
    anc = np.concatenate([pack_ancestors(e.anc, mask_words) for e in encs])
    depth = np.concatenate([e.depth for e in encs])
    pos = np.concatenate([e.pos for e in encs])
    return encs, anc, depth, pos
