"""Pins of the oracle's EAGLE-3 draft input (oracle.fuse_features): a hand-computed case
that fixes the feature order, identity blocks that select each feature exactly, linearity,
and the draft expansion taking the fused feature as its root feature."""
import numpy as np

import oracle
from workloads import DraftParams, make_workload
from workloads.configs import eagle3_inputs, mini_dims


def test_hand_computed_order_low_mid_high():
    # H = 1: W = [1 2 3] on (low, mid, high) = (1, 10, 100) is 1 + 20 + 300 = 321; a
    # reversed feature order would give 123, a dropped block 21 or 301
    w = np.array([[1.0, 2.0, 3.0]])
    out = oracle.fuse_features(w, np.array([[1.0]]), np.array([[10.0]]), np.array([[100.0]]))
    assert out.shape == (1, 1) and out[0, 0] == 321.0
    # H = 2, two sequences, integers: every product and sum is exact
    w = np.array([[1, 0, 0, 2, 0, 0], [0, -1, 3, 0, 0, 1]], dtype=float)
    low = np.array([[1, 2], [5, 6]], dtype=float)
    mid = np.array([[3, 4], [7, 8]], dtype=float)
    high = np.array([[9, 10], [11, 12]], dtype=float)
    # row 0: 1*low0 + 2*mid1; row 1: -low1 + 3*mid0 + high1
    expect = np.array([[1 + 8, -2 + 9 + 10], [5 + 16, -6 + 21 + 12]], dtype=float)
    assert np.array_equal(oracle.fuse_features(w, low, mid, high), expect)


def test_identity_blocks_select_each_feature():
    rng = np.random.default_rng(3)
    H, B = 8, 3
    f = [rng.standard_normal((B, H)) for _ in range(3)]
    eye, zero = np.eye(H), np.zeros((H, H))
    for i in range(3):
        blocks = [zero, zero, zero]
        blocks[i] = eye
        assert np.array_equal(oracle.fuse_features(np.concatenate(blocks, axis=1), *f), f[i])


def test_linear_in_features_and_zero_blocks_drop_a_feature():
    rng = np.random.default_rng(4)
    H, B = 16, 2
    w = rng.standard_normal((H, 3 * H))
    a = [rng.standard_normal((B, H)) for _ in range(3)]
    b = [rng.standard_normal((B, H)) for _ in range(3)]
    lhs = oracle.fuse_features(w, *[2.0 * x + y for x, y in zip(a, b)])
    rhs = 2.0 * oracle.fuse_features(w, *a) + oracle.fuse_features(w, *b)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    w0 = w.copy()
    w0[:, H:] = 0.0  # only the low block left: mid and high do not matter
    c = [a[0], b[1], b[2]]
    assert np.array_equal(oracle.fuse_features(w0, *a), oracle.fuse_features(w0, *c))


def test_draft_takes_the_fused_root_feature():
    """The EAGLE-3 draft is the ordinary draft expansion from the fused root feature."""
    params = DraftParams(depth=2, top_k=3, frontier=2, max_nodes=6)
    dims = mini_dims(hidden=128, n_q_heads=2, n_kv_heads=1, ffn=256, vocab=97)
    wl = make_workload(5, seed=21, dims=dims, batch=2, prefix=[5, 9], draft=params)
    w_fuse, feats = eagle3_inputs(wl)
    H = dims.hidden
    root = oracle.fuse_features(w_fuse, feats[:, :H], feats[:, H:2 * H], feats[:, 2 * H:])
    a = oracle.draft_expand(dims, params, wl.weights, wl.draft_weights, root, wl.root_token, wl.dk_cache,
                            wl.dv_cache, wl.prefix_len)
    b = oracle.draft_expand(dims, params, wl.weights, wl.draft_weights, wl.root_feature, wl.root_token,
                            wl.dk_cache, wl.dv_cache, wl.prefix_len)
    assert len(a) == 2 and len(b) == 2
    # a different root feature gives a different draft (the fusion is actually used)
    assert any(not np.array_equal(np.asarray(x["tokens"]), np.asarray(y["tokens"])) for x, y in zip(a, b))
