"""GPU parity of tree encode, tree verification and accept/commit against the fp64 oracle.

All calls go through the C ABI (ctypes binding).  Sizes span several GEMM tiles,
several KV chunks and ragged tails while the oracle still finishes in seconds.
"""
import numpy as np
import pytest

import oracle
from tests._gpu import HipPathRun, check_verify, oracle_verify
from workloads import make_workload, mini_dims, trees as T

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def bits(t):
    import torch
    t = t.contiguous().cpu()
    return (t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)).numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_build_bit_exact(seed):
    import torch
    import tree_attention_verification_06_amd as E
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    parents = [T.random_tree(rng, int(rng.integers(1, 129))) for _ in range(B)]
    parents[0] = T.chain(min(128, len(parents[0])))
    prefix = rng.integers(0, 5000, size=B).astype(np.int32)
    mw = 2
    _print("tree_build", seed, [len(p) for p in parents])
    off = np.concatenate([[0], np.cumsum([len(p) for p in parents])]).astype(np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    M = int(off[-1])
    anc = torch.zeros(M, mw, dtype=torch.int64, device="cuda")
    depth = torch.zeros(M, dtype=torch.int32, device="cuda")
    pos = torch.zeros(M, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    E.eagle_tree_build(dev(off), dev(np.concatenate(parents).astype(np.int32)), dev(prefix), mw, anc, depth, pos, st,
                       total_nodes=M, max_nodes=max(len(p) for p in parents))
    torch.cuda.synchronize()
    _, ref_anc, ref_depth, ref_pos = oracle.encode_batch(parents, prefix, mw)
    assert st.item() == 0
    assert (anc.cpu().numpy().view(np.uint64) == ref_anc).all()
    assert (depth.cpu().numpy() == ref_depth).all()
    assert (pos.cpu().numpy() == ref_pos).all()


def test_tree_build_rejects_malformed_tree():
    import torch
    import tree_attention_verification_06_amd as E
    parents = [[-1, 0, 1], [-1, 0, 2, 1], [0, 0]]  # second: parent[2] = 2 (not < 2); third: root not -1
    off = np.array([0, 3, 7, 9], dtype=np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    anc = torch.full((9, 1), -1, dtype=torch.int64, device="cuda")
    depth = torch.zeros(9, dtype=torch.int32, device="cuda")
    pos = torch.zeros(9, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    E.eagle_tree_build(dev(off), dev(np.concatenate(parents).astype(np.int32)), dev(np.zeros(3, np.int32)), 1, anc,
                       depth, pos, st, total_nodes=9, max_nodes=4)
    torch.cuda.synchronize()
    assert st.item() == E._abi.EAGLE_ERR_TREE
    a = anc.cpu().numpy().view(np.uint64)[:, 0]
    assert a[:3].tolist() == [1, 3, 7]          # the valid tree is encoded
    assert (a[3:] == 0).all()                    # malformed trees get empty masks


def test_verify_tiny_fp32_full_config():
    wl = make_workload(1)
    _print("verify cfg tiny fp32", wl.n_nodes)
    g = HipPathRun(wl).run().outputs()
    ref = oracle_verify(wl)
    errs = check_verify(g, ref, wl.dims, label="tiny-fp32")
    _print(errs)


@pytest.mark.parametrize("seed,prefix,tree", [(0, 300, "static60"), (1, 700, "random"), (2, 64, "chain")])
def test_verify_mini_bf16(seed, prefix, tree):
    dims = mini_dims()
    rng = np.random.default_rng(seed)
    par = {"static60": T.static_tree_60(), "random": T.random_tree(rng, 90), "chain": T.chain(64)}[tree]
    wl = make_workload(2, seed=seed, dims=dims, batch=1, prefix=prefix, parents=[par])
    _print("verify mini bf16", seed, prefix, tree, wl.n_nodes)
    g = HipPathRun(wl).run().outputs()
    ref = oracle_verify(wl)
    errs = check_verify(g, ref, dims, label=f"mini-{tree}")
    _print(errs)


def test_verify_mini_ragged_batch_dynamic_trees():
    dims = mini_dims()
    wl = make_workload(3, seed=5, dims=dims, prefix=[1000, 37, 513, 2048])
    _print("verify ragged", wl.tree_off, wl.mask_words)
    g = HipPathRun(wl).run().outputs()
    ref = oracle_verify(wl)
    errs = check_verify(g, ref, dims, label="ragged")
    _print(errs)


def test_verify_mini_small_trees_four_wave_attention():
    """Trees of at most 16 nodes: with 4 query heads per KV head a (sequence, KV head) pair
    has at most 64 query rows, so the attention runs its four-wave workgroups; a ragged
    batch with an empty prefix and prefixes over several key chunks."""
    dims = mini_dims()
    rng = np.random.default_rng(8)
    parents = [T.random_tree(rng, 16), T.chain(7), [-1], T.star(12)]
    wl = make_workload(2, seed=41, dims=dims, batch=4, prefix=[300, 1000, 0, 513], parents=parents)
    assert max(len(p) for p in parents) * dims.n_q_heads // dims.n_kv_heads <= 64
    _print("verify small trees", wl.tree_off)
    g = HipPathRun(wl).run().outputs()
    ref = oracle_verify(wl)
    errs = check_verify(g, ref, dims, label="small-trees")
    _print(errs)


def test_verify_few_rows_wider_layer_split_k_narrow_tiles():
    """Twelve rows through a layer of hidden 2048 (16 query heads, FFN 2816): every GEMM runs
    the 16-token tiles, and the down projection (K 2816 over 16 weight tiles) is split over
    K, so the narrow tiles' split-K hand-off and partial sums are compared with the oracle."""
    dims = mini_dims(hidden=2048, n_q_heads=16, n_kv_heads=4, ffn=2816)
    parents = [T.chain(5), T.star(6), [-1]]
    wl = make_workload(2, seed=44, dims=dims, batch=3, prefix=[300, 64, 0], parents=parents)
    _print("verify few rows, hidden 2048", wl.tree_off)
    g = HipPathRun(wl).run().outputs()
    ref = oracle_verify(wl)
    errs = check_verify(g, ref, dims, label="few-rows-2048")
    _print(errs)


def test_verify_mini_random_gains_and_embedding_input():
    dims = mini_dims()
    wl = make_workload(2, seed=11, dims=dims, batch=2, prefix=[129, 400], parents=[T.static_tree_60(),
                       T.random_tree(np.random.default_rng(3), 33)], gamma_std=0.2)
    wl.weights["embed"] = np.random.default_rng(4).standard_normal((dims.vocab, dims.hidden)).astype(np.float32)
    from workloads.bf16 import f32_to_bf16_bits
    wl.weights["embed"] = f32_to_bf16_bits(wl.weights["embed"])
    _print("verify embed-input", wl.tree_off)
    g = HipPathRun(wl, use_embed=True).run().outputs()
    ref = oracle_verify(wl, use_embed=True)
    errs = check_verify(g, ref, dims, label="embed")
    _print(errs)


@pytest.mark.parametrize("cfg", [1, 3])
def test_accept_commit_bit_exact(cfg):
    """Accept on the GPU's own argmax must equal the oracle's rule exactly; the commit must
    copy the GPU's own tree K/V rows bit for bit into the right slots."""
    dims = None if cfg == 1 else mini_dims()
    wl = make_workload(cfg, seed=21, dims=dims, prefix=None if cfg == 1 else [300, 77, 1024, 5])
    # plant paths: set tokens along one root path per tree to the GPU's argmax of the parent
    run0 = HipPathRun(wl, want_logits=False).run()
    g0 = run0.outputs()
    rng = np.random.default_rng(9)
    tokens = wl.tokens.copy()
    for b, par in enumerate(wl.parents):
        o = wl.tree_off[b]
        d = T.depths(par)
        leaf = max(range(len(par)), key=lambda i: (d[i], -i)) if b % 2 == 0 else int(rng.integers(0, len(par)))
        path = []
        j = leaf
        while j != -1:
            path.append(j)
            j = par[j]
        for node in path[::-1][1:]:
            tokens[o + node] = g0["argmax"][o + par[node]]
    wl.tokens = tokens
    run = HipPathRun(wl, want_logits=False)
    pre_k = run.t["k_cache"].clone()
    pre_v = run.t["v_cache"].clone()
    run.run(accept=True)
    g = run.outputs()
    v = run.v
    acc = v.accept_len.cpu().numpy()
    path = v.path.cpu().numpy()
    outt = v.out_tokens.cpu().numpy()
    nxt = v.next_token.cpu().numpy()
    newP = run.t["prefix_len"].cpu().numpy()
    kc = run.t["k_cache"]
    vc = run.t["v_cache"]
    assert g["status"] == 0
    for b, par in enumerate(wl.parents):
        o = wl.tree_off[b]
        n = len(par)
        L, pth, out, nt, leaf = oracle.accept_sequence(par, tokens[o:o + n], g["argmax"][o:o + n],
                                                      g["depth"][o:o + n])
        assert acc[b] == L and nxt[b] == nt
        assert path[b, :L + 1].tolist() == pth and (path[b, L + 1:] == -1).all()
        assert outt[b, :L + 1].tolist() == out and (outt[b, L + 1:] == -1).all()
        P = int(wl.prefix_len[b])
        assert newP[b] == P + L + 1
        if b % 2 == 0:
            assert L >= 1
        for dd, node in enumerate(pth):
            assert (bits(kc[b, :, P + dd]) == bits(v.k_tree[o + node])).all()
            assert (bits(vc[b, :, P + dd]) == bits(v.v_tree[o + node])).all()
        # untouched slots stay as they were
        cap = kc.shape[2]
        others = [s for s in range(cap) if not (P <= s <= P + L)]
        assert (bits(kc[b][:, others]) == bits(pre_k[b][:, others])).all()
        assert (bits(vc[b][:, others]) == bits(pre_v[b][:, others])).all()
        nf = v.next_feature[b].cpu().numpy()
        assert (nf == g["h"][o + leaf]).all()


def test_verify_and_accept_degenerate_trees():
    """Root-only trees (with and without a prefix), a 128-node chain (two mask words, the
    deepest path the library accepts) and a star, in one ragged batch; then acceptance with
    the chain planted along its whole length."""
    dims = mini_dims()
    parents = [[-1], [-1], T.chain(128), T.star(40)]
    wl = make_workload(2, seed=31, dims=dims, batch=4, prefix=[0, 17, 0, 1000], parents=parents)
    assert wl.mask_words == 2
    _print("verify degenerate", wl.tree_off)
    run0 = HipPathRun(wl)
    g0 = run0.run().outputs()
    ref = oracle_verify(wl)
    _print(check_verify(g0, ref, dims, label="degenerate"))
    # plant the whole chain: every node's token is the GPU's argmax at its parent
    tokens = wl.tokens.copy()
    o = wl.tree_off[2]
    for i in range(1, 128):
        tokens[o + i] = g0["argmax"][o + i - 1]
    wl.tokens = tokens
    run = HipPathRun(wl, want_logits=False)
    run.run(accept=True)
    g = run.outputs()
    v = run.v
    acc = v.accept_len.cpu().numpy()
    nxt = v.next_token.cpu().numpy()
    newP = run.t["prefix_len"].cpu().numpy()
    assert g["status"] == 0
    for b, par in enumerate(parents):
        ob = wl.tree_off[b]
        n = len(par)
        L, pth, out, nt, leaf = oracle.accept_sequence(par, tokens[ob:ob + n], g["argmax"][ob:ob + n],
                                                      g["depth"][ob:ob + n])
        assert acc[b] == L and nxt[b] == nt and newP[b] == int(wl.prefix_len[b]) + L + 1
    assert acc[0] == 0 and acc[1] == 0 and acc[2] == 127   # root-only trees accept only the bonus


def test_accept_reports_cache_overflow():
    """A sequence whose accepted path would run past the cache capacity gets accept_len -1,
    no commit and EAGLE_ERR_CAPACITY in the device status; the other sequences commit."""
    import tree_attention_verification_06_amd as E
    dims = mini_dims()
    parents = [T.chain(6), T.chain(6)]
    wl = make_workload(2, seed=33, dims=dims, batch=2, prefix=[10, 10], parents=parents, cache_slack=0)
    cap = wl.cache_cap
    # sequence 1 starts 3 slots short of the end: committing its 6-node path cannot fit
    wl.prefix_len = np.array([10, cap - 3], dtype=np.int32)
    run0 = HipPathRun(wl, want_logits=False, max_prefix=cap)
    g0 = run0.run().outputs()
    tokens = wl.tokens.copy()
    for b in range(2):
        o = wl.tree_off[b]
        for i in range(1, 6):
            tokens[o + i] = g0["argmax"][o + i - 1]
    wl.tokens = tokens
    run = HipPathRun(wl, want_logits=False, max_prefix=cap)
    pre_k = run.t["k_cache"].clone()
    t, v = run.t, run.v
    v.encode(t["tree_off"], t["parent"], t["prefix_len"], run.M)
    v.verify(t["tree_off"], t["tokens"], t["prefix_len"], run.M, x=t["x"])
    v.accept(t["tree_off"], t["parent"], t["tokens"], t["prefix_len"])
    import torch
    torch.cuda.synchronize()
    assert int(v.status.item()) == E._abi.EAGLE_ERR_CAPACITY
    acc = v.accept_len.cpu().numpy()
    newP = t["prefix_len"].cpu().numpy()
    assert acc[0] == 5 and newP[0] == 10 + 6
    assert acc[1] == -1 and newP[1] == cap - 3
    assert (bits(t["k_cache"][1]) == bits(pre_k[1])).all()


def test_accept_refuses_malformed_or_stale_trees():
    """Acceptance must not commit a tree whose encoding it cannot trust: (a) a malformed
    parent array, after a tree encode that zeroed its masks while the depth buffer still
    holds an earlier tree's depths; (b) a well-formed parent array whose depth and masks
    are those of another tree (encode not rerun).  Either sequence gets accept_len -1,
    path -1, no commit and no prefix advance, with EAGLE_ERR_TREE; the other sequence of
    the batch is accepted and committed as usual."""
    import torch
    import tree_attention_verification_06_amd as E
    dims = mini_dims()
    parents = [T.chain(6), T.chain(6)]
    wl = make_workload(2, seed=35, dims=dims, batch=2, prefix=[40, 40], parents=parents)
    run0 = HipPathRun(wl, want_logits=False)
    g0 = run0.run().outputs()
    tokens = wl.tokens.copy()
    for b in range(2):          # plant both chains in full: a trusted tree accepts depth 5
        o = wl.tree_off[b]
        for i in range(1, 6):
            tokens[o + i] = g0["argmax"][o + i - 1]
    for case in ("malformed", "stale"):
        wl.tokens = tokens
        run = HipPathRun(wl, want_logits=False)
        t, v = run.t, run.v
        v.encode(t["tree_off"], t["parent"], t["prefix_len"], run.M)
        v.verify(t["tree_off"], t["tokens"], t["prefix_len"], run.M, x=t["x"])
        torch.cuda.synchronize()
        assert int(v.status.item()) == 0 and v.depth[6:12].cpu().tolist() == [0, 1, 2, 3, 4, 5]
        bad = np.concatenate([T.chain(6), T.chain(6)]).astype(np.int32)
        if case == "malformed":
            bad[6 + 3] = 3                   # parent[3] = 3: not below its own index
            t["parent"].copy_(torch.from_numpy(bad))
            v.encode(t["tree_off"], t["parent"], t["prefix_len"], run.M)   # zeroes tree 1's masks
            torch.cuda.synchronize()
            assert int(v.status.item()) == E._abi.EAGLE_ERR_TREE
            v.status.zero_()
        else:
            bad[6:12] = [-1, 0, 0, 0, 0, 0]  # a star given to accept with the chain's encoding
            t["parent"].copy_(torch.from_numpy(bad))
        pre_k = t["k_cache"].clone()
        v.accept(t["tree_off"], t["parent"], t["tokens"], t["prefix_len"])
        torch.cuda.synchronize()
        _print("accept refuses", case)
        assert int(v.status.item()) == E._abi.EAGLE_ERR_TREE
        acc = v.accept_len.cpu().numpy()
        newP = t["prefix_len"].cpu().numpy()
        assert acc[0] == 5 and newP[0] == 40 + 6
        assert acc[1] == -1 and newP[1] == 40 and int(v.next_token[1].item()) == -1
        assert (v.path[1].cpu().numpy() == -1).all() and (v.out_tokens[1].cpu().numpy() == -1).all()
        assert (bits(t["k_cache"][1]) == bits(pre_k[1])).all()


@pytest.mark.parametrize("cfg", [1, 2])
def test_verify_prefix_longer_than_planned(cfg):
    """max_prefix only sizes the split of the prefix over workgroups: a device prefix_len
    beyond it (a decode loop whose plan was made at its first step) is still attended in
    full, and the outputs match the oracle.  The fp32 case spans several of its 512-key
    blocks."""
    dims = None if cfg == 1 else mini_dims()
    prefix = [1300] if cfg == 1 else [900, 260]
    parents = None if cfg == 1 else [T.static_tree_60(), T.random_tree(np.random.default_rng(8), 30)]
    wl = make_workload(cfg, seed=37, dims=dims, batch=len(prefix), prefix=prefix, parents=parents)
    _print("verify prefix beyond plan", cfg, prefix)
    g = HipPathRun(wl, max_prefix=128).run().outputs()
    ref = oracle_verify(wl)
    assert g["status"] == 0
    _print(check_verify(g, ref, wl.dims, label=f"prefix-beyond-plan-{cfg}"))


def test_tree_build_refuses_tree_beyond_max_nodes():
    import torch
    import tree_attention_verification_06_amd as E
    parents = [T.chain(5), T.chain(9)]
    off = np.array([0, 5, 14], dtype=np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    anc = torch.full((14, 1), -1, dtype=torch.int64, device="cuda")
    depth = torch.zeros(14, dtype=torch.int32, device="cuda")
    pos = torch.zeros(14, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    E.eagle_tree_build(dev(off), dev(np.concatenate(parents).astype(np.int32)), dev(np.zeros(2, np.int32)), 1, anc,
                       depth, pos, st, total_nodes=14, max_nodes=8)
    torch.cuda.synchronize()
    assert st.item() == E._abi.EAGLE_ERR_CAPACITY
    a = anc.cpu().numpy().view(np.uint64)[:, 0]
    assert a[:5].tolist() == [1, 3, 7, 15, 31]       # the tree within max_nodes is encoded
    assert (a[5:] == np.uint64(0xFFFFFFFFFFFFFFFF)).all()  # the other is not written


def test_verify_fp32_ragged_batch_several_key_blocks():
    """The fp32 layer on a ragged batch: three trees (one past the 64-node single mask word,
    so two mask words) with prefixes that span one, two and three 128-key blocks of the
    fp32 attention, against the oracle; then acceptance with a planted path, bit-exact on
    the GPU's own argmax."""
    from workloads.configs import TINY
    rng = np.random.default_rng(12)
    parents = [T.random_tree(rng, 70), T.chain(9), T.static_tree_26()]
    wl = make_workload(1, seed=47, dims=TINY, batch=3, prefix=[100, 250, 300], parents=parents)
    assert wl.mask_words == 2
    _print("verify fp32 ragged", wl.tree_off.tolist(), wl.prefix_len.tolist())
    g = HipPathRun(wl).run().outputs()
    ref = oracle_verify(wl)
    _print(check_verify(g, ref, wl.dims, label="fp32-ragged"))
    tokens = wl.tokens.copy()
    o = wl.tree_off[1]
    for i in range(1, 9):
        tokens[o + i] = g["argmax"][o + i - 1]
    wl.tokens = tokens
    run = HipPathRun(wl, want_logits=False)
    run.run(accept=True)
    g2 = run.outputs()
    acc = run.v.accept_len.cpu().numpy()
    assert g2["status"] == 0
    for b, par in enumerate(parents):
        ob = wl.tree_off[b]
        n = len(par)
        L, pth, out, nt, leaf = oracle.accept_sequence(par, tokens[ob:ob + n], g2["argmax"][ob:ob + n],
                                                      g2["depth"][ob:ob + n])
        assert acc[b] == L
    assert acc[1] == 8
