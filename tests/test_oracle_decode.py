"""Pins of the layer-stack oracle (oracle/decode.py): tree verification through several
layers, the per-layer KV commit, the draft-KV update from true features and the EAGLE
decode loop, against a textbook left-to-right decoder (tests/_textbook.py, written
independently of oracle/) stacked layer on layer.

What the pages fix: the emitted text equals the target's own greedy decoding ("Speculative
decoding with EAGLE", Deep dive: lossless), every tree node sees exactly its prefix and
its root path, and the draft is fed the target's true features with the true next-token
embedding (Technical insight)."""
import numpy as np
import pytest

import oracle
from oracle.decode import draft_kv_commit, eagle_decode, greedy_decode, verify_forward_layers
from tests._textbook import SequentialDecoder, greedy, logits_of, wf
from workloads import LayerDims, stack_workload, trees as T

DIMS = LayerDims(64, 4, 2, 16, 96, 61, 1.0e4, 1e-5, "f32")
N_LAYERS = 3


class TextbookStack:
    """n textbook layers applied in order, each with its own growing cache."""

    def __init__(self, dims, layers, k_pre=None, v_pre=None):
        self.layers = [SequentialDecoder(dims, lw, None if k_pre is None else k_pre[l],
                                         None if v_pre is None else v_pre[l]) for l, lw in enumerate(layers)]

    def step(self, x):
        ks, vs = [], []
        for dec in self.layers:
            r = dec.step(x)
            ks.append(r["k"])
            vs.append(r["v"])
            x = r["h"]
        return dict(h=x, k=ks, v=vs)


def _prefixed(wl, b=0):
    P = int(wl.prefix_len[b])
    return ([wl.k_caches[l, b, :, :P] for l in range(wl.n_layers)],
            [wl.v_caches[l, b, :, :P] for l in range(wl.n_layers)])


def _wl(seed, prefix=9, n_layers=N_LAYERS):
    # embeddings N(0, 1) so that the token identity drives the greedy choice
    return stack_workload(seed, DIMS, n_layers, prefix=prefix, embed_std=1.0)


@pytest.mark.parametrize("seed", [0, 1])
def test_every_root_path_equals_sequential_stack(seed):
    """Each node's per-layer K/V and last-layer feature equal a left-to-right run of the
    textbook stack over the tokens of its root path, from the same prefix."""
    wl = _wl(seed)
    rng = np.random.default_rng(seed + 50)
    par = T.random_tree(rng, 14)
    toks = T.tree_tokens(rng, par, DIMS.vocab)
    P = int(wl.prefix_len[0])
    out = verify_forward_layers(DIMS, wl.weights, wl.layers, None, [par], [P], wl.k_caches, wl.v_caches,
                                embed_tokens=toks, want_logits=True)
    assert out["k_tree"].shape == (N_LAYERS, len(par), DIMS.n_kv_heads, DIMS.head_dim)
    kp, vp = _prefixed(wl)
    for i in range(len(par)):
        path = []
        j = i
        while j != -1:
            path.append(j)
            j = par[j]
        stack = TextbookStack(DIMS, wl.layers, kp, vp)
        for node in path[::-1]:
            r = stack.step(wf(wl.weights["embed"][toks[node]]))
        assert np.abs(r["h"] - out["h"][i]).max() < 1e-10
        for l in range(N_LAYERS):
            assert np.abs(r["k"][l] - out["k_tree"][l, i]).max() < 1e-10
            assert np.abs(r["v"][l] - out["v_tree"][l, i]).max() < 1e-10
        z = logits_of(DIMS, wl.weights, r["h"])
        assert np.abs(z - out["logits"][i]).max() < 1e-10
        assert greedy(z) == out["argmax"][i]


def test_stack_of_one_is_the_single_layer_pass():
    wl = _wl(3, n_layers=1)
    rng = np.random.default_rng(3)
    par = T.random_tree(rng, 9)
    toks = T.tree_tokens(rng, par, DIMS.vocab)
    P = int(wl.prefix_len[0])
    a = verify_forward_layers(DIMS, wl.weights, wl.layers, None, [par], [P], wl.k_caches, wl.v_caches,
                              embed_tokens=toks)
    w1 = dict(wl.layers[0], **wl.weights)
    b = oracle.verify_forward(DIMS, w1, None, [par], [P], wl.k_caches[0], wl.v_caches[0], embed_tokens=toks)
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["k_tree"][0], b["k_tree"])
    assert np.array_equal(a["argmax"], b["argmax"])


def _textbook_greedy(wl, n):
    """Greedy continuation of the root token by the textbook stack, with the feature of
    every consumed token and each step's K/V."""
    kp, vp = _prefixed(wl)
    stack = TextbookStack(DIMS, wl.layers, kp, vp)
    t = int(wl.root_token[0])
    toks, feats, kv = [], [], []
    for _ in range(n):
        r = stack.step(wf(wl.weights["embed"][t]))
        feats.append(r["h"])
        kv.append((r["k"], r["v"]))
        t = greedy(logits_of(DIMS, wl.weights, r["h"]))
        toks.append(t)
    return toks, feats, kv


def _planted_tree(rng, n, continuation, depth):
    return T.planted_tree(rng, n, DIMS.vocab, continuation, depth)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_eagle_loop_is_lossless_and_commits_every_layer(seed):
    """Several EAGLE steps with planted trees emit exactly the textbook greedy tokens; the
    committed slots of every layer's cache hold the textbook K/V of those positions; the
    draft cache slots hold the textbook draft layer's K/V of W_fc [f_(t-1) ; E[token_t]]
    with the textbook target features; the oracle's plain greedy loop agrees too."""
    wl = _wl(seed)
    P0 = int(wl.prefix_len[0])
    n_greedy = 24
    g_toks, g_feats, g_kv = _textbook_greedy(wl, n_greedy)
    rng = np.random.default_rng(seed + 7)
    plant = [3, 0, 2, 4, 1, 3]
    trees, emitted_so_far = [], 0
    # the tokens each step can plant: the greedy continuation after what has been emitted;
    # accept lengths are data-dependent, so trees are built step by step from the loop's state
    # float64 caches: a commit must not round what it stores
    kc, vc = wl.k_caches.astype(np.float64), wl.v_caches.astype(np.float64)
    dk, dv = wl.dk_cache.astype(np.float64), wl.dv_cache.astype(np.float64)
    P, root, feat = P0, int(wl.root_token[0]), wl.root_feature[0]
    emitted, lens = [], []
    for d in plant:
        cont = g_toks[emitted_so_far:]
        tree = _planted_tree(rng, 16, cont, d)
        trees.append(tree)
        e, P, root, feat, ls = eagle_decode(DIMS, wl.weights, wl.layers, kc, vc, P, root, feat, [tree],
                                            draft=(wl.draft_weights, dk, dv))
        emitted += e
        lens += ls
        emitted_so_far = len(emitted)
        assert ls[0] >= d
    assert emitted == g_toks[:len(emitted)]
    assert P == P0 + len(emitted)
    assert sum(lens) + len(lens) == len(emitted)
    # target caches: slot P0 + t holds the K/V of the t-th consumed token (root first)
    for t in range(P - P0):
        for l in range(N_LAYERS):
            assert np.abs(kc[l, 0, :, P0 + t] - g_kv[t][0][l]).max() < 1e-10
            assert np.abs(vc[l, 0, :, P0 + t] - g_kv[t][1][l]).max() < 1e-10
    assert (kc[:, 0, :, P:] == 0).all()
    # draft cache: textbook draft layer over rows W_fc [f_(t-1) ; E[token_t]]
    dkp = wl.dk_cache[0, :, :P0]
    dvp = wl.dv_cache[0, :, :P0]
    ddec = SequentialDecoder(DIMS, wl.draft_weights, dkp, dvp)
    consumed = [int(wl.root_token[0])] + g_toks
    prev = wf(wl.root_feature[0])
    wfc = wf(wl.draft_weights["w_fc"])
    for t in range(P - P0):
        row = wfc @ np.concatenate([prev, wf(wl.weights["embed"][consumed[t]])])
        r = ddec.step(row)
        assert np.abs(dk[0, :, P0 + t] - r["k"]).max() < 1e-10
        assert np.abs(dv[0, :, P0 + t] - r["v"]).max() < 1e-10
        prev = g_feats[t]
    assert (dk[0, :, P:] == 0).all()
    # the oracle's plain greedy loop (one-node trees through the stack)
    kc2, vc2 = wl.k_caches.astype(np.float64), wl.v_caches.astype(np.float64)
    toks, feats, gaps = greedy_decode(DIMS, wl.weights, wl.layers, kc2, vc2, P0, wl.root_token[0], 10)
    assert toks == g_toks[:10]
    assert all(np.abs(f - g).max() < 1e-10 for f, g in zip(feats, g_feats))


def test_draft_kv_commit_capacity_error():
    wl = _wl(4, prefix=9)
    dk = np.zeros((DIMS.n_kv_heads, 10, DIMS.head_dim))
    dv = dk.copy()
    h = np.zeros((3, DIMS.hidden))
    with pytest.raises(ValueError):
        draft_kv_commit(DIMS, wl.draft_weights, wl.weights["embed"], dk, dv, wl.root_feature[0], h, [1, 2, 3],
                        [0, 1, 2], 8)
