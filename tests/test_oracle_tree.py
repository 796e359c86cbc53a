"""Pins of the oracle's tree encode (parent array -> depth, ancestor masks, positions)."""
import numpy as np
import pytest

from oracle.tree import TreeError, encode_batch, pack_ancestors, tree_encode
from workloads import trees as T
from tests._golden import load


def brute_force_ancestors(parent):
    n = len(parent)
    anc = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        steps = 0
        while j != -1:
            anc[i, j] = True
            j = parent[j]
            steps += 1
            assert steps <= n
    return anc


def test_golden_7node():
    g = load("tree_7node.txt")
    e = tree_encode(g["parent"], g["prefix_len"][0])
    assert e.depth.tolist() == g["depth"]
    assert e.pos.tolist() == g["pos"]
    words = pack_ancestors(e.anc, 1)[:, 0]
    assert [int(w) for w in words] == g["anc_word0"]


@pytest.mark.parametrize("seed", range(20))
def test_random_trees_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 130))
    par = T.random_tree(rng, n)
    e = tree_encode(par, 7)
    assert (e.anc == brute_force_ancestors(par)).all()
    # popcount(anc i) = depth(i) + 1
    assert (e.anc.sum(1) == e.depth + 1).all()
    # anc(i) = anc(parent i) | {i}
    for i in range(1, n):
        want = e.anc[par[i]].copy()
        want[i] = True
        assert (e.anc[i] == want).all()
    mw = (n + 63) // 64
    words = pack_ancestors(e.anc, mw)
    for i in range(n):
        for j in range(n):
            bit = (int(words[i, j // 64]) >> (j % 64)) & 1
            assert bit == int(e.anc[i, j])
        assert all(int(words[i, w]) == 0 for w in range(mw) if 64 * w >= n)


def test_chain_is_lower_triangular():
    e = tree_encode(T.chain(70), 0)
    assert (e.anc == np.tril(np.ones((70, 70), dtype=bool))).all()
    assert e.depth.tolist() == list(range(70))


def test_star_is_identity_plus_root_column():
    e = tree_encode(T.star(9), 3)
    want = np.eye(9, dtype=bool)
    want[:, 0] = True
    assert (e.anc == want).all()
    assert e.pos.tolist() == [3] + [4] * 8


def test_single_node():
    e = tree_encode([-1], 5)
    assert e.anc.tolist() == [[True]] and e.pos.tolist() == [5]


@pytest.mark.parametrize("bad", [[], [0], [-1, 1], [-1, 0, 3], [-1, -1], [-1, 0, 2], [1, -1]])
def test_invalid_trees_rejected(bad):
    with pytest.raises(TreeError):
        tree_encode(bad, 0)


def test_mask_capacity():
    e = tree_encode(T.chain(65), 0)
    with pytest.raises(TreeError):
        pack_ancestors(e.anc, 1)
    assert pack_ancestors(e.anc, 2).shape == (65, 2)


def test_static_tree_fixtures():
    g = load("static_trees.txt")
    for name in ("static26", "static60"):
        par = g[name]
        d = T.depths(par)
        levels = np.bincount(d).tolist()
        assert levels == g[name + "_levels"]
    assert T.static_tree_26() == g["static26"]
    assert T.static_tree_60() == g["static60"]


def test_batch_concatenation():
    parents = [T.chain(3), T.star(4)]
    encs, anc, depth, pos = encode_batch(parents, [10, 20], 1)
    assert anc[:, 0].tolist() == [1, 3, 7, 1, 3, 5, 9]
    assert pos.tolist() == [10, 11, 12, 20, 21, 21, 21]
