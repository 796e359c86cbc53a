"""Pins of the oracle's acceptance rule and KV commit (hand-worked fixtures, brute force, lossless)."""
import numpy as np
import pytest

import oracle
from oracle.accept import accept_sequence, commit_sequence
from oracle.tree import tree_encode
from tests._golden import load
from tests._textbook import SequentialDecoder, greedy, logits_of, wf
from workloads import LayerDims, make_workload, trees as T


@pytest.mark.parametrize("name", ["accept_7node.txt", "accept_tie.txt"])
def test_golden(name):
    g = load(name)
    e = tree_encode(g["parent"], g["prefix_len"][0])
    L, path, out, nxt, leaf = accept_sequence(g["parent"], g["tokens"], g["g"], e.depth)
    assert L == g["accept_len"][0]
    assert path == g["path"]
    assert out == g["out_tokens"]
    assert nxt == g["next_token"][0]
    Hkv, D, cap = 2, 3, 32
    kc = np.zeros((Hkv, cap, D))
    vc = np.zeros((Hkv, cap, D))
    n = len(g["parent"])
    kt = np.arange(n * Hkv * D, dtype=float).reshape(n, Hkv, D) + 1
    vt = -kt
    P = g["prefix_len"][0]
    newP = commit_sequence(kc, vc, kt, vt, path, P)
    assert newP == g["new_prefix_len"][0]
    for slot, node in zip(g["commit_slots"], path):
        assert (kc[:, slot] == kt[node]).all() and (vc[:, slot] == vt[node]).all()
    untouched = [s for s in range(cap) if s not in g["commit_slots"]]
    assert (kc[:, untouched] == 0).all()


def brute_force_accept(parent, tokens, g, depth):
    n = len(parent)
    children = {i: [j for j in range(n) if parent[j] == i] for i in range(n)}
    leaves = [i for i in range(n) if not children[i]]
    ends = []
    for lf in leaves:
        path = []
        j = lf
        while j != -1:
            path.append(j)
            j = parent[j]
        path = path[::-1]
        end = path[0]
        for a, b in zip(path, path[1:]):
            if tokens[b] == g[a]:
                end = b
            else:
                break
        ends.append(end)
    best = min(ends, key=lambda e: (-depth[e], e))
    return best


@pytest.mark.parametrize("seed", range(40))
def test_accept_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    par = T.random_tree(rng, n)
    tokens = rng.integers(0, 3, size=n)  # tiny vocabulary: many matches, duplicate siblings, ties
    g = rng.integers(0, 3, size=n)
    e = tree_encode(par, 0)
    L, path, out, nxt, leaf = accept_sequence(par, tokens, g, e.depth)
    assert leaf == brute_force_accept(par, tokens, g, e.depth)
    assert L == e.depth[leaf] and len(path) == L + 1 and path[-1] == leaf and path[0] == 0
    assert out == [int(tokens[p]) for p in path[1:]] + [int(g[leaf])]


LOSSLESS_DIMS = LayerDims(64, 4, 2, 16, 96, 61, 1.0e4, 1e-5, "f32")


def _lm(seed):
    wl = make_workload(5, seed=seed, dims=LOSSLESS_DIMS, batch=1, prefix=0, parents=[[-1]])
    w = dict(wl.weights)
    # larger embeddings so the token identity drives the greedy choice
    w["embed"] = np.random.default_rng([seed, 77]).standard_normal(w["embed"].shape).astype(np.float32)
    return w


def _prefill(dims, w, prompt, cap):
    dec = SequentialDecoder(dims, w)
    for t in prompt:
        dec.step(wf(w["embed"][t]))
    Hkv, D = dims.n_kv_heads, dims.head_dim
    kc = np.zeros((1, Hkv, cap, D))
    vc = np.zeros((1, Hkv, cap, D))
    for s, (k, v) in enumerate(zip(dec.K, dec.V)):
        kc[0, :, s] = k
        vc[0, :, s] = v
    return dec, kc, vc


def _greedy_continuation(dims, w, prompt, root, n):
    dec = SequentialDecoder(dims, w)
    for t in prompt:
        dec.step(wf(w["embed"][t]))
    out = []
    t = root
    for _ in range(n):
        r = dec.step(wf(w["embed"][t]))
        t = greedy(logits_of(dims, w, r["h"]))
        out.append(t)
    return out


@pytest.mark.parametrize("seed,plant_depth", [(0, 3), (1, 4), (2, 0), (3, 2)])
def test_lossless_against_sequential_greedy(seed, plant_depth):
    dims = LOSSLESS_DIMS
    w = _lm(seed)
    rng = np.random.default_rng(seed + 100)
    prompt = rng.integers(0, dims.vocab, size=7).tolist()
    root = int(rng.integers(0, dims.vocab))
    greedy_toks = _greedy_continuation(dims, w, prompt, root, 8)
    # tree: random recursive tree; plant the greedy continuation along one root path
    par = T.random_tree(rng, 18)
    depth = T.depths(par)
    tokens = T.tree_tokens(rng, par, dims.vocab, root_token=root)
    cands = [i for i in range(len(par)) if depth[i] == plant_depth]
    if plant_depth > 0 and cands:
        leaf = cands[0]
        path = []
        j = leaf
        while j != -1:
            path.append(j)
            j = par[j]
        path = path[::-1]
        for d, node in enumerate(path[1:], start=1):
            tokens[node] = greedy_toks[d - 1]
            # keep sibling tokens distinct from the planted one
            for s in range(len(par)):
                if s != node and par[s] == par[node] and tokens[s] == tokens[node]:
                    tokens[s] = (tokens[s] + 1) % dims.vocab
    cap = 32
    _, kc, vc = _prefill(dims, w, prompt, cap)
    P = len(prompt)
    out = oracle.verify_forward(dims, w, None, [par], [P], kc, vc, embed_tokens=tokens)
    L, path, acc, nxt, leaf = accept_sequence(par, tokens, out["argmax"], out["encs"][0].depth)
    assert acc == greedy_toks[: L + 1]
    if plant_depth > 0 and cands:
        assert L >= plant_depth

    # compaction round-trip: decoding the bonus token from the committed cache equals
    # decoding the whole accepted sequence from scratch
    kc2, vc2 = kc.copy(), vc.copy()
    newP = commit_sequence(kc2[0], vc2[0], out["k_tree"], out["v_tree"], path, P)
    assert newP == P + L + 1
    dec = SequentialDecoder(dims, w, kc2[0, :, :newP], vc2[0, :, :newP])
    z1 = logits_of(dims, w, dec.step(wf(w["embed"][nxt]))["h"])
    seq = prompt + [root] + acc[:-1] + [nxt]
    dec2 = SequentialDecoder(dims, w)
    for t in seq:
        r = dec2.step(wf(w["embed"][t]))
    z2 = logits_of(dims, w, r["h"])
    assert np.abs(z1 - z2).max() < 1e-11
    assert greedy(z1) == greedy_toks[L + 1]
