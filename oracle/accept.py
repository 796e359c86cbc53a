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


def sample_accept_sequence(parent, tokens, logits, temperature, u, gumbel, trace=None):
    """Acceptance when the target samples at temperature T > 0 ("Speculative decoding with
    EAGLE", Deep dive and FAQ: accepted tokens must agree with the target's own choice, here
    its own sample, so the output distribution is unchanged).  The pages give no procedure;
    the reading is speculative sampling with deterministic candidates, walked from the root:
      at node n, p = softmax(logits[n] / T); its children c (in index order) are tried in
      turn: c is accepted iff u[c] * r < p(tokens[c]), where r is the probability mass left
      after removing the tokens of the children already rejected (r = 1 at first); accepted
      -> continue at c; all rejected (or a leaf) -> the bonus token is drawn from p with the
      rejected tokens removed, as argmax_v (log p(v) + gumbel[n][v]) over the tokens left.
    Each emitted token is then distributed exactly as the target's p at its position:
    P(accept the i-th child) = p(x_i) and P(bonus = y) = p(y) for y outside the children's
    tokens (sibling tokens are distinct).  u [n] uniforms in [0, 1) (u[c] decides node c),
    gumbel [n][V] standard Gumbel noise, logits [n][V]; all consumed as given (inputs).
    Only one bonus is drawn per call, at a node fixed by u alone, so every node may be given
    the same noise row.  trace (a list, optional) receives (c, u[c] * r, p(tokens[c])) for
    every child tried.  Returns (L, path root..leaf, out_tokens [L + 1], next_token, leaf)."""
    n = len(parent)
    children = [[] for _ in range(n)]
    for j in range(1, n):
        children[int(parent[j])].append(j)
    node, path = 0, [0]
    while True:
        z = np.asarray(logits[node], dtype=np.float64) / float(temperature)
        m = z.max()
        logp = z - (m + np.log(np.exp(z - m).sum()))
        rejected, r, nxt = [], 1.0, None
        for c in children[node]:
            x = int(tokens[c])
            px = float(np.exp(logp[x]))
            if trace is not None:
                trace.append((c, float(u[c]) * r, px))
            if float(u[c]) * r < px:
                nxt = c
                break
            rejected.append(x)
            r -= px
        if nxt is None:
            score = logp + np.asarray(gumbel[node], dtype=np.float64)
            score[rejected] = -np.inf
            bonus = int(np.argmax(score))
            break
        node = nxt
        path.append(node)
    out = [int(tokens[p]) for p in path[1:]] + [bonus]
    return len(path) - 1, path, out, bonus, node


def sample_summaries(parent, tokens, logits, temperature, gumbel_row):
    """Per-node summaries of the target's logits that the walk of sample_accept_sequence needs,
    with z = logits / T (fp64), for one tree sharing the noise row gumbel_row [V]:
      child_logit[c] = z[parent(c)][tokens[c]] for every non-root node c (NaN at the root);
      over the tokens that are not the token of a child of n ("the rest" of node n):
      rest_lse[n] = log sum exp z[n], rest_token[n] = argmax (z[n] + gumbel_row) (first
      index on ties).
    The vocabulary of node n splits into its child tokens and the rest, so its log-normaliser
    is the log-sum-exp of rest_lse[n] and its children's child_logit; a walk that stops at n
    has rejected every child, so its bonus argmax over the non-rejected tokens is
    rest_token[n].  Sibling tokens must be distinct (else ValueError)."""
    n = len(parent)
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    V = z.shape[1]
    g = np.asarray(gumbel_row, dtype=np.float64)
    child_logit = np.full(n, np.nan)
    kids = [[] for _ in range(n)]
    for c in range(1, n):
        kids[int(parent[c])].append(int(tokens[c]))
        child_logit[c] = z[int(parent[c]), int(tokens[c])]
    rest_lse = np.zeros(n)
    rest_token = np.zeros(n, dtype=np.int64)
    for node in range(n):
        if len(set(kids[node])) != len(kids[node]):
            raise ValueError(f"node {node}: two children with the same token")
        rest = np.ones(V, dtype=bool)
        rest[kids[node]] = False
        zr = z[node][rest]
        m = zr.max()
        rest_lse[node] = m + np.log(np.exp(zr - m).sum())
        score = z[node] + g
        score[~rest] = -np.inf
        rest_token[node] = int(np.argmax(score))
    return child_logit, rest_lse, rest_token


def sample_accept_from_summaries(parent, tokens, child_logit, rest_lse, rest_token, u, trace=None):
    """The walk of sample_accept_sequence on the summaries of sample_summaries (fp64): at node
    n the log-normaliser is logsumexp(rest_lse[n], child_logit of n's children); children are
    tried in index order, c accepted iff u[c] * r < exp(child_logit[c] - that), r -= that
    probability on rejection; the walk stops at the first node whose children are all
    rejected (or a leaf), with the bonus rest_token[n].  trace as in sample_accept_sequence.
    Returns (L, path, out_tokens, next_token, leaf)."""
    n = len(parent)
    children = [[] for _ in range(n)]
    for j in range(1, n):
        children[int(parent[j])].append(j)
    node, path = 0, [0]
    while True:
        terms = [float(rest_lse[node])] + [float(child_logit[c]) for c in children[node]]
        m = max(terms)
        lse = m + np.log(sum(np.exp(t - m) for t in terms))
        r, nxt = 1.0, None
        for c in children[node]:
            px = float(np.exp(float(child_logit[c]) - lse))
            if trace is not None:
                trace.append((c, float(u[c]) * r, px))
            if float(u[c]) * r < px:
                nxt = c
                break
            r -= px
        if nxt is None:
            bonus = int(rest_token[node])
            break
        node = nxt
        path.append(node)
    out = [int(tokens[p]) for p in path[1:]] + [bonus]
    return len(path) - 1, path, out, bonus, node


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
