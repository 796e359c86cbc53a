"""Pins of the oracle's forward pass: tree attention, rotary, norms, the LM head and argmax."""
import math

import numpy as np
import pytest

import oracle
from oracle.layer import attend, layer_rows, linear, rope_rotate_half, rms_norm, lm_head_argmax
from oracle.tree import tree_encode
from tests._textbook import SequentialDecoder, greedy, logits_of, rope_complex
from workloads import LayerDims, make_workload, trees as T
from workloads.bf16 import f32_to_bf16_bits

TINY = LayerDims(64, 4, 2, 16, 96, 97, 1.0e4, 1e-5, "f32")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def causal_attention(q, k, v, n_past):
    """Explicit-loop causal attention: query t (absolute position n_past + t) sees keys 0..n_past+t."""
    n, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    out = np.zeros_like(q)
    for t in range(n):
        for h in range(Hq):
            sc = [float(np.dot(q[t, h], k[s, h // g])) / math.sqrt(D) for s in range(n_past + t + 1)]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            z = sum(w)
            for s in range(n_past + t + 1):
                out[t, h] += w[s] / z * v[s, h // g]
    return out


@pytest.mark.parametrize("P", [0, 5])
def test_chain_tree_equals_causal(P):
    N, Hq, Hkv, D = 6, 4, 2, 16
    q = rnd(1, N, Hq, D)
    k_all = rnd(2, P + N, Hkv, D)
    v_all = rnd(3, P + N, Hkv, D)
    e = tree_encode(T.chain(N), P)
    o = attend(q, k_all[:P].transpose(1, 0, 2), v_all[:P].transpose(1, 0, 2), k_all[P:], v_all[P:], e.anc)
    ref = causal_attention(q, k_all, v_all, P)
    assert np.abs(o - ref).max() < 1e-12


def test_single_node_equals_decode():
    P, Hq, Hkv, D = 9, 4, 2, 16
    q = rnd(4, 1, Hq, D)
    k_all = rnd(5, P + 1, Hkv, D)
    v_all = rnd(6, P + 1, Hkv, D)
    o = attend(q, k_all[:P].transpose(1, 0, 2), v_all[:P].transpose(1, 0, 2), k_all[P:], v_all[P:],
               np.ones((1, 1), dtype=bool))
    ref = causal_attention(q, k_all, v_all, P)
    assert np.abs(o - ref).max() < 1e-12


def test_zero_query_gives_mean_of_visible_values():
    # closed form: all scores 0 -> uniform weights over prefix + ancestors (self included)
    par = [-1, 0, 0, 1, 1, 2, 3]
    P, Hq, Hkv, D = 4, 2, 1, 8
    e = tree_encode(par, P)
    kp, vp = rnd(7, Hkv, P, D), rnd(8, Hkv, P, D)
    kt, vt = rnd(9, 7, Hkv, D), rnd(10, 7, Hkv, D)
    o = attend(np.zeros((7, Hq, D)), kp, vp, kt, vt, e.anc)
    for i in range(7):
        vis = [vp[0, s] for s in range(P)] + [vt[j, 0] for j in range(7) if e.anc[i, j]]
        want = np.mean(vis, axis=0)
        for h in range(Hq):
            assert np.abs(o[i, h] - want).max() < 1e-12


def test_constructed_weights_and_scale():
    # keys built so that q.k_j / sqrt(D) = log(w_j): output = sum w_j v_j / sum w_j
    D = 16
    q = rnd(11, D)
    wts = np.array([0.5, 2.0, 1.0, 3.0, 0.25])
    keys = np.stack([math.sqrt(D) * math.log(w) / np.dot(q, q) * q for w in wts])
    vals = rnd(12, 5, D)
    # prefix = first 3 keys; tree = chain of 2 (node 1 sees node 0)
    kp = keys[:3][None]
    vp = vals[:3][None]
    kt = keys[3:][:, None]
    vt = vals[3:][:, None]
    e = tree_encode([-1, 0], 3)
    o = attend(np.stack([q, q])[:, None], kp, vp, kt, vt, e.anc)
    want0 = (wts[:4, None] * vals[:4]).sum(0) / wts[:4].sum()
    want1 = (wts[:, None] * vals).sum(0) / wts.sum()
    assert np.abs(o[0, 0] - want0).max() < 1e-12
    assert np.abs(o[1, 0] - want1).max() < 1e-12


def test_gqa_equals_mha_with_repeated_kv():
    par = T.random_tree(np.random.default_rng(3), 15)
    P, Hq, Hkv, D = 6, 8, 2, 16
    e = tree_encode(par, P)
    q = rnd(13, 15, Hq, D)
    kp, vp = rnd(14, Hkv, P, D), rnd(15, Hkv, P, D)
    kt, vt = rnd(16, 15, Hkv, D), rnd(17, 15, Hkv, D)
    o = attend(q, kp, vp, kt, vt, e.anc)
    g = Hq // Hkv
    o2 = attend(q, np.repeat(kp, g, 0), np.repeat(vp, g, 0), np.repeat(kt, g, 1), np.repeat(vt, g, 1), e.anc)
    assert np.abs(o - o2).max() < 1e-12


def test_relabeling_invariance():
    rng = np.random.default_rng(5)
    par = T.random_tree(rng, 12)
    P, Hq, Hkv, D = 3, 4, 2, 16
    q = rnd(18, 12, Hq, D)
    kp, vp = rnd(19, Hkv, P, D), rnd(20, Hkv, P, D)
    kt, vt = rnd(21, 12, Hkv, D), rnd(22, 12, Hkv, D)
    o = attend(q, kp, vp, kt, vt, tree_encode(par, P).anc)
    # another topological order: sort by (depth, -index)
    d = T.depths(par)
    perm = sorted(range(12), key=lambda i: (d[i], -i))
    inv = {old: new for new, old in enumerate(perm)}
    par2 = [-1 if par[old] < 0 else inv[par[old]] for old in perm]
    o2 = attend(q[perm], kp, vp, kt[perm], vt[perm], tree_encode(par2, P).anc)
    assert np.abs(o2 - o[perm]).max() < 1e-12


def test_rope_matches_complex_form_and_properties():
    x = rnd(23, 5, 3, 16)
    pos = np.array([0, 1, 7, 100, 32775])
    r = rope_rotate_half(x, pos, 5.0e5)
    for t in range(5):
        assert np.abs(r[t] - rope_complex(x[t], int(pos[t]), 5.0e5)).max() < 1e-9
    assert np.abs(r[0] - x[0]).max() == 0.0
    assert np.abs(np.linalg.norm(r, axis=-1) - np.linalg.norm(x, axis=-1)).max() < 1e-12
    # relative-position property: <R(m)q, R(n)k> depends only on m - n
    q, k = rnd(24, 1, 1, 16), rnd(25, 1, 1, 16)
    a = np.sum(rope_rotate_half(q, [40], 1e4) * rope_rotate_half(k, [33], 1e4))
    b = np.sum(rope_rotate_half(q, [7], 1e4) * rope_rotate_half(k, [0], 1e4))
    assert abs(a - b) < 1e-12


def test_rms_norm_unit_rms():
    x = rnd(26, 4, 64) * 7.0
    y = rms_norm(x, np.ones(64), 0.0)
    assert np.abs(np.sqrt(np.mean(y * y, -1)) - 1).max() < 1e-14
    assert np.abs(rms_norm(3 * x, np.ones(64), 0.0) - y).max() < 1e-13


def test_linear_brute_force_bf16():
    w = f32_to_bf16_bits(rnd(27, 9, 5).astype(np.float32))
    x = rnd(28, 3, 5)
    y = linear(x, w)
    from workloads.bf16 import bf16_bits_to_f32
    wf = bf16_bits_to_f32(w)
    for i in range(3):
        for j in range(9):
            s = 0.0
            for k in range(5):
                s += x[i, k] * float(wf[j, k])
            assert abs(y[i, j] - s) < 1e-12


def test_argmax_first_index_of_max_and_gap():
    dims = LayerDims(4, 1, 1, 4, 0, 6, 0.0, 0.0, "f32")
    w = {"w_lm": np.array([[0, 0, 0, 0], [1, 0, 0, 0], [3, 0, 0, 0], [2, 0, 0, 0], [3, 0, 0, 0], [-5, 0, 0, 0]],
                          dtype=np.float32)}
    h = np.array([[1.0, 0, 0, 0], [-1.0, 0, 0, 0]])
    am, mx, gap, logits = lm_head_argmax(dims, w, h)
    assert am.tolist() == [2, 5]
    assert mx.tolist() == [3.0, 5.0]
    assert gap.tolist() == [0.0, 5.0]


def _tiny_workload(seed=0, n=14, P=5, dims=TINY):
    par = T.random_tree(np.random.default_rng(seed), n)
    return make_workload(2, seed=seed, dims=dims, batch=1, prefix=P, parents=[par])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_every_path_equals_sequential_decoding(seed):
    wl = _tiny_workload(seed)
    par = wl.parents[0]
    out = oracle.verify_forward(wl.dims, wl.weights, wl.x, wl.parents, wl.prefix_len, wl.k_cache, wl.v_cache)
    P = int(wl.prefix_len[0])
    leaves = [i for i in range(len(par)) if i not in par]
    for leaf in leaves:
        path = []
        j = leaf
        while j != -1:
            path.append(j)
            j = par[j]
        path = path[::-1]
        dec = SequentialDecoder(wl.dims, wl.weights, wl.k_cache[0, :, :P], wl.v_cache[0, :, :P])
        for node in path:
            r = dec.step(np.asarray(wl.x[node], dtype=np.float64))
            assert np.abs(r["h"] - out["h"][node]).max() < 1e-12
            assert np.abs(r["attn"] - out["attn"][node]).max() < 1e-12
            assert np.abs(r["k"] - out["k_tree"][node]).max() < 1e-12
            assert np.abs(r["q"] - out["q"][node]).max() < 1e-12
            z = logits_of(wl.dims, wl.weights, r["h"])
            assert np.abs(z - out["logits"][node]).max() < 1e-12
            assert greedy(z) == out["argmax"][node]


def test_attention_only_layer_path_equivalence():
    dims = LayerDims(32, 2, 2, 16, 0, 50, 0.0, 0.0, "f32")
    wl = _tiny_workload(4, n=10, P=3, dims=dims)
    par = wl.parents[0]
    out = oracle.verify_forward(dims, wl.weights, wl.x, wl.parents, wl.prefix_len, wl.k_cache, wl.v_cache)
    for leaf in [i for i in range(len(par)) if i not in par]:
        path = []
        j = leaf
        while j != -1:
            path.append(j)
            j = par[j]
        dec = SequentialDecoder(dims, wl.weights, wl.k_cache[0, :, :3], wl.v_cache[0, :, :3])
        for node in path[::-1]:
            r = dec.step(np.asarray(wl.x[node], dtype=np.float64))
            assert np.abs(r["h"] - out["h"][node]).max() < 1e-12


def test_bf16_inputs_widen_exactly():
    dims = LayerDims(64, 4, 2, 16, 96, 97, 1.0e4, 1e-5, "bf16")
    wl = _tiny_workload(6, dims=dims)
    a = oracle.verify_forward(dims, wl.weights, wl.x, wl.parents, wl.prefix_len, wl.k_cache, wl.v_cache)
    from workloads.bf16 import bf16_bits_to_f64
    w64 = {k: bf16_bits_to_f64(v) for k, v in wl.weights.items()}
    b = oracle.verify_forward(dims, w64, bf16_bits_to_f64(wl.x), wl.parents, wl.prefix_len,
                              bf16_bits_to_f64(wl.k_cache), bf16_bits_to_f64(wl.v_cache))
    assert np.abs(a["h"] - b["h"]).max() == 0.0
    assert (a["argmax"] == b["argmax"]).all()


def test_gain_is_applied():
    dims = TINY
    wl = make_workload(2, seed=9, dims=dims, batch=1, prefix=4, parents=[T.chain(3)], gamma_std=0.2)
    x = np.asarray(wl.x[0], dtype=np.float64)
    dec = SequentialDecoder(dims, wl.weights, wl.k_cache[0, :, :4], wl.v_cache[0, :, :4])
    r = dec.step(x)
    out = oracle.verify_forward(dims, wl.weights, wl.x, wl.parents, wl.prefix_len, wl.k_cache, wl.v_cache)
    assert np.abs(r["h"] - out["h"][0]).max() < 1e-12
    wl1 = make_workload(2, seed=9, dims=dims, batch=1, prefix=4, parents=[T.chain(3)], gamma_std=0.0)
    out1 = oracle.verify_forward(dims, wl1.weights, wl1.x, wl1.parents, wl1.prefix_len, wl1.k_cache, wl1.v_cache)
    assert np.abs(out1["h"][0] - out["h"][0]).max() > 1e-6
