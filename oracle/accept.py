"""Acceptance of the longest target-consistent path, and the KV commit.

TEST INFRASTRUCTURE (fp64 oracle; see the package docstring for who may import it).

Sources: "Speculative decoding with EAGLE" page, Deep dive and FAQ (the target
checks the drafted tokens in one pass and keeps the longest correct prefix;
accepted tokens must equal the target's own choice, which makes the method
lossless); "LLM parallel decoding EAGLE" page, section on how EAGLE works
(the longest valid path of the tree is accepted).

Greedy rule, written out:
  match(j) = [tokens[j] == g[parent(j)]] for every non-root node j, where g is
  the target's argmax at each node; a node is consistent iff every non-root
  node on its root path (itself included) matches; the accepted leaf is the
  deepest consistent node (ties: lowest index); L = depth(leaf); the output is
  the L accepted tokens followed by the bonus token g[leaf].
Commit (reading): the root and the L accepted nodes get cache slots
prefix_len .. prefix_len + L; the new prefix length is prefix_len + L + 1; the
bonus token is not committed (it is the next step's root); the next draft
feature is the layer output h at the leaf.
"""
import numpy as np


def accept_sequence(parent, tokens, g, depth):
    """Returns (L, path [L+1] node ids root..leaf, out_tokens [L+1], next_token, leaf)."""
    n = len(parent)
    match = np.zeros(n, dtype=bool)
    match[0] = True  # the root is never checked
    for j in range(1, n):
        match[j] = int(tokens[j]) == int(g[parent[j]])
    ok = np.zeros(n, dtype=bool)
    for i in range(n):
        ok[i] = match[i] and (i == 0 or ok[parent[i]])
    leaf = 0
    for i in range(n):
        if ok[i] and depth[i] > depth[leaf]:
            leaf = i
    path = []
    j = leaf
    while j >= 0:
        path.append(j)
        j = parent[j] if j > 0 else -1
    path = path[::-1]
    L = int(depth[leaf])
    out = [int(tokens[p]) for p in path[1:]] + [int(g[leaf])]
    return L, path, out, int(g[leaf]), leaf


def accept_batch(parents, tokens, g, encs):
    """accept_sequence for each tree of a batch (node arrays concatenated)."""
    sizes = [len(p) for p in parents]
    off = np.concatenate([[0], np.cumsum(sizes)])
    res = []
    for b, par in enumerate(parents):
        r0, r1 = off[b], off[b + 1]
        res.append(accept_sequence(par, tokens[r0:r1], g[r0:r1], encs[b].depth))
    return res


def commit_sequence(k_cache_b, v_cache_b, k_tree_b, v_tree_b, path, prefix_len):
    """cache[:, prefix_len + d] <- tree KV of path[d], d = 0..L; returns the new prefix length.

    k_cache_b [Hkv][cap][D] (modified in place); k_tree_b [N][Hkv][D] (this tree's nodes).
    """
    cap = k_cache_b.shape[1]
    if prefix_len + len(path) > cap:
        raise ValueError("cache capacity exceeded")
    for d, node in enumerate(path):
        k_cache_b[:, prefix_len + d] = k_tree_b[node]
        v_cache_b[:, prefix_len + d] = v_tree_b[node]
    return prefix_len + len(path)
