"""Synthetic draft-tree topologies, given as parent arrays.

Convention for every tree produced here: node 0 is the root with parent -1 and
0 <= parent[i] < i for every other node (a topological order).

* ``rank_sum_tree`` - static sparse trees.  The pages say EAGLE-1 verifies a
  fixed topology of 60 nodes of depth 6 ("LLM parallel decoding EAGLE" page,
  EAGLE vs EAGLE-2 comparison table, and the operating-principle section) but
  print no shape.  Reading: from a full tree with the given per-level
  branching, keep the root plus the nodes whose sibling ranks along the path
  have the smallest sum (ties: shallower first, then breadth-first index of
  the full tree).  This keeps the most probable paths and is ancestor-closed.
* ``eagle2_style_tree`` - dynamic, context-dependent trees of 40..120 nodes
  (same page, comparison table: EAGLE-2 adapts the tree to confidence;
  FAQ Q3: confidence threshold 0.3).  Reading: every expanded node gets 10
  children whose probabilities are the 10-way softmax of N(0, 2) logits; a
  child is expanded iff its own probability is >= 0.3; depth <= 8; trees over
  120 nodes keep the root plus the 119 best by cumulative log-probability;
  trees under 40 nodes are redrawn from the next sub-seed.

These are test inputs only; the draft head's own expansion (which the method
computes) lives elsewhere and shares nothing with this module.
"""
import heapq
import numpy as np


def chain(n):
    return [-1] + list(range(n - 1))


def star(n):
    return [-1] + [0] * (n - 1)


def random_tree(rng, n):
    """Uniform random recursive tree: parent[i] ~ U{0..i-1}."""
    return [-1] + [int(rng.integers(0, i)) for i in range(1, n)]


def full_tree(branching):
    """Full tree with branching[l] children per node at level l, BFS order."""
    parent = [-1]
    level = [0]
    for b in branching:
        nxt = []
        for p in level:
            for _ in range(b):
                parent.append(p)
                nxt.append(len(parent) - 1)
        level = nxt
    return parent


def rank_sum_tree(branching, n_keep):
    """Root + (n_keep-1) nodes of the full tree with the smallest sibling-rank sums.

    Best-first search: a child's rank sum is >= its parent's, so popping a
    min-heap keyed by (rank_sum, depth, bfs_index) yields nodes in the final
    order, and every popped node's parent was popped earlier.
    """
    depth_max = len(branching)
    # bfs index of a node in the full tree = level offset + lexicographic rank within the level
    level_size = [1]
    for b in branching:
        level_size.append(level_size[-1] * b)
    level_off = np.cumsum([0] + level_size[:-1]).tolist()

    # heap entries: (rank_sum, depth, bfs_index, within_level_index, parent_bfs_index)
    heap = [(0, 0, 0, 0, -1)]
    kept = {}  # bfs index -> parent bfs index
    while heap and len(kept) < n_keep:
        rs, d, bfs, wl, par = heapq.heappop(heap)
        kept[bfs] = par
        if d < depth_max:
            b = branching[d]
            for r in range(b):
                cw = wl * b + r
                heapq.heappush(heap, (rs + r, d + 1, level_off[d + 1] + cw, cw, bfs))
    if len(kept) < n_keep:
        raise ValueError("full tree smaller than n_keep")
    # output in breadth-first order of the full tree (depth first, then position in level)
    order = sorted(kept)
    new = {b: i for i, b in enumerate(order)}
    return [-1 if kept[b] < 0 else new[kept[b]] for b in order]


# Static trees of the configurations (readings documented in the module docstring).
def static_tree_26():
    """26-node, depth-4 tree from branching [4,3,1,1] (a full tree of that branching has 41)."""
    return rank_sum_tree([4, 3, 1, 1], 26)


def static_tree_60():
    """60-node, depth-6 static EAGLE tree from a full 10-ary tree of depth 6."""
    return rank_sum_tree([10] * 6, 60)


def depths(parent):
    d = [0] * len(parent)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


def _softmax10(z):
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def eagle2_style_tree(seed, seq, *, branch=10, logit_std=2.0, thresh=0.3, max_depth=8,
                      n_min=40, n_max=120, tid=901):
    """Dynamic tree for sequence ``seq`` (see module docstring). Returns (parent, sub_seed_used)."""
    sub = 0
    while True:
        rng = np.random.default_rng([seed, tid, seq, sub])
        par, dep, cum = [-1], [0], [0.0]
        frontier = [0]
        for d in range(1, max_depth + 1):
            new = []
            for p in frontier:
                pr = _softmax10(rng.normal(0.0, logit_std, size=branch))
                for c in range(branch):
                    par.append(p)
                    dep.append(d)
                    cum.append(cum[p] + float(np.log(pr[c])))
                    if pr[c] >= thresh and d < max_depth:
                        new.append(len(par) - 1)
            frontier = new
            if not frontier:
                break
        n = len(par)
        keep = list(range(n))
        if n > n_max:
            rest = sorted(range(1, n), key=lambda i: (-cum[i], dep[i], i))[: n_max - 1]
            keep = [0] + sorted(rest)
        if len(keep) < n_min:
            sub += 1
            continue
        # cumulative log-prob never increases along a path, so the kept set is ancestor-closed
        kset = set(keep)
        assert all(par[i] in kset for i in keep if i != 0)
        # re-index: by depth, then new parent index, then cumulative log-prob (desc), then creation order
        new_idx = {0: 0}
        order = [0]
        maxd = max(dep[i] for i in keep)
        for d in range(1, maxd + 1):
            lvl = [i for i in keep if dep[i] == d]
            lvl.sort(key=lambda i: (new_idx[par[i]], -cum[i], i))
            for i in lvl:
                new_idx[i] = len(order)
                order.append(i)
        parent = [-1] + [new_idx[par[i]] for i in order[1:]]
        return parent, sub


def tree_tokens(rng, parent, vocab, root_token=None):
    """Token ids per node: uniform over [0, vocab), distinct within each sibling group."""
    n = len(parent)
    tok = np.zeros(n, dtype=np.int32)
    tok[0] = int(rng.integers(0, vocab)) if root_token is None else int(root_token)
    kids = {}
    for i in range(1, n):
        kids.setdefault(parent[i], []).append(i)
    for p in sorted(kids):
        ch = kids[p]
        draw = rng.choice(vocab, size=len(ch), replace=False)
        for i, t in zip(ch, draw):
            tok[i] = int(t)
    return tok


def planted_tree(rng, n, vocab, continuation, depth):
    """A random recursive tree of n nodes with random tokens whose first node at ``depth``
    carries ``continuation[0 .. depth-1]`` along its root path (siblings of a planted node
    get other tokens); depth 0 plants nothing.  Returns (parent, tokens); the root's token
    is left for the caller to set."""
    par = random_tree(rng, n)
    dep = depths(par)
    toks = tree_tokens(rng, par, vocab)
    cands = [i for i in range(n) if dep[i] == depth]
    if depth > 0 and cands:
        path = []
        j = cands[0]
        while j != -1:
            path.append(j)
            j = par[j]
        for d, node in enumerate(path[::-1][1:], start=1):
            toks[node] = int(continuation[d - 1])
            for s in range(n):
                if s != node and par[s] == par[node] and toks[s] == toks[node]:
                    toks[s] = (toks[s] + 1) % vocab
    return par, toks
