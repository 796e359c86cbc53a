"""Pins of the oracle's draft-head tree expansion."""
import itertools

import numpy as np
import pytest

from oracle.draft import draft_expand, draft_rerank, log_softmax, topk_stable
from tests._textbook import SequentialDecoder, greedy, logits_of, wf
from workloads import DraftParams, LayerDims, make_workload

DD = LayerDims(32, 2, 1, 16, 48, 13, 1.0e4, 1e-5, "f32")


def _wl(seed=0, B=2, P=4, vocab=13, draft=None):
    dims = LayerDims(32, 2, 1, 16, 48, vocab, 1.0e4, 1e-5, "f32")
    wl = make_workload(5, seed=seed, dims=dims, batch=B, prefix=P, draft=draft)
    # stronger LM-head weights so draft probabilities are far from uniform
    wl.weights["w_lm"] = (wl.weights["w_lm"] * 40).astype(np.float32)
    return wl


def _run(wl, params, trace=False):
    return draft_expand(wl.dims, params, wl.weights, wl.draft_weights, wl.root_feature, wl.root_token,
                        wl.dk_cache, wl.dv_cache, wl.prefix_len, trace=trace)


def test_topk_is_stable_selection():
    rng = np.random.default_rng(1)
    for _ in range(50):
        row = rng.integers(0, 5, size=20).astype(float)  # many ties
        k = int(rng.integers(1, 20))
        got = topk_stable(row, k).tolist()
        left = list(range(20))
        want = []
        for _ in range(k):
            best = left[0]
            for i in left:
                if row[i] > row[best]:
                    best = i
            want.append(best)
            left.remove(best)
        assert got == want


def test_log_softmax_normalised():
    z = np.random.default_rng(2).standard_normal((4, 1000)) * 30
    assert np.abs(np.exp(log_softmax(z)).sum(1) - 1).max() < 1e-12


@pytest.mark.parametrize("seed", [0, 1])
def test_k1_f1_is_sequential_greedy_drafting(seed):
    wl = _wl(seed)
    D = 5
    res = _run(wl, DraftParams(depth=D, top_k=1, frontier=1, max_nodes=D + 1, conf_threshold=0.0))
    for b in range(wl.batch):
        P = int(wl.prefix_len[b])
        dec = SequentialDecoder(wl.dims, wl.draft_weights, wl.dk_cache[b, :, :P], wl.dv_cache[b, :, :P])
        f = wf(wl.root_feature[b])
        t = int(wl.root_token[b])
        toks = [t]
        cum = [0.0]
        for _ in range(D):
            row = wf(wl.draft_weights["w_fc"]) @ np.concatenate([f, wf(wl.weights["embed"][t])])
            f = dec.step(row)["h"]
            z = logits_of(wl.dims, wl.weights, f)
            t = greedy(z)
            lse = np.log(np.sum(np.exp(z - z.max()))) + z.max()
            cum.append(cum[-1] + min(0.0, z[t] - lse))
            toks.append(t)
        assert res[b]["tokens"] == toks
        assert res[b]["parent"] == [-1] + list(range(D))
        assert np.abs(np.array(res[b]["cum"]) - np.array(cum)).max() < 1e-10


@pytest.mark.parametrize("seed", [0, 3])
def test_tree_invariants(seed):
    wl = _wl(seed)
    params = DraftParams(depth=4, top_k=3, frontier=3, max_nodes=12, conf_threshold=0.0)
    res = _run(wl, params, trace=True)
    for r in res:
        par, cum = r["parent"], r["cum"]
        assert len(par) == 12 and par[0] == -1
        assert all(0 <= par[i] < i for i in range(1, len(par)))
        depth = [0] * len(par)
        for i in range(1, len(par)):
            depth[i] = depth[par[i]] + 1
            assert cum[i] <= cum[par[i]]
        assert depth == sorted(depth)
        # root + the best 11 generated nodes by (cum desc, depth, generation order)
        pool = r["pool"]
        best = sorted(range(1, len(pool)), key=lambda i: (-pool[i]["cum"], pool[i]["depth"], pool[i]["gen"]))[:11]
        assert sorted(r["order"][1:]) == sorted(best)
        # level structure: level 1 expands the root; later levels expand <= frontier nodes
        assert [len(lv["frontier"]) for lv in r["levels"]] == [1, 3, 3, 3]
        for lv in r["levels"]:
            assert len(lv["children"]) == 3 * len(lv["frontier"])
            nxt = lv["next"]
            kids = lv["children"]
            keyed = sorted(kids, key=lambda i: (-pool[i]["cum"], pool[i]["depth"], pool[i]["gen"]))
            assert nxt == keyed[:3]


def _pool_paths(r):
    pool = r["pool"]
    paths = set()
    for i in range(len(pool)):
        p = []
        j = i
        while j >= 0:
            p.append(pool[j]["token"])
            j = pool[j]["parent"]
        paths.add(tuple(p[::-1]))
    return paths


def test_lower_threshold_widens_search():
    wl = _wl(5, B=1)
    sizes = []
    pools = []
    for tau in [0.5, 0.3, 0.2, 0.1, 0.0]:
        params = DraftParams(depth=4, top_k=3, frontier=0, max_nodes=10 ** 6, conf_threshold=tau)
        r = _run(wl, params, trace=True)[0]
        sizes.append(len(r["parent"]))
        pools.append(_pool_paths(r))
    assert sizes == sorted(sizes)
    assert sizes[0] < sizes[-1]
    for a, b in zip(pools, pools[1:]):
        assert a <= b


def test_rerank_brute_force():
    rng = np.random.default_rng(7)
    pool = [dict(token=0, parent=-1, depth=0, cum=0.0, gen=(0, 0, 0))]
    for lvl in range(1, 4):
        parents = [i for i in range(len(pool)) if pool[i]["depth"] == lvl - 1][:3]
        for r, p in enumerate(parents):
            for c in range(3):
                pool.append(dict(token=int(rng.integers(0, 50)), parent=p, depth=lvl,
                                 cum=pool[p]["cum"] - float(rng.choice([0.5, 1.0, 1.5])), gen=(lvl, r, c)))
    par, tok, cum, order = draft_rerank(pool, 8)
    # brute force: among ancestor-closed subsets of size 8 containing the root, the chosen one
    # holds the 7 best keys
    keys = sorted(range(1, len(pool)), key=lambda i: (-pool[i]["cum"], pool[i]["depth"], pool[i]["gen"]))
    assert set(order[1:]) == set(keys[:7])
    for i in range(1, 8):
        assert 0 <= par[i] < i
        assert order[par[i]] == pool[order[i]]["parent"]
        assert tok[i] == pool[order[i]]["token"]
    # depth-major ordering, cum descending within a depth
    for a, b in itertools.combinations(range(1, 8), 2):
        da, db = pool[order[a]]["depth"], pool[order[b]]["depth"]
        assert da < db or (da == db and cum[a] >= cum[b])


@pytest.mark.parametrize("tau", [0.0, 0.2])
def test_forcing_own_decisions_reproduces_free_run(tau):
    """Teacher forcing with the oracle's own top-k and frontier choices changes nothing."""
    wl = _wl(4)
    params = DraftParams(depth=4, top_k=3, frontier=2, max_nodes=9, conf_threshold=tau)
    free = _run(wl, params, trace=True)
    force = []
    for r in free:
        pool = r["pool"]
        f = dict(tokens={}, frontier={})
        for lvl, lv in enumerate(r["levels"], start=1):
            f["tokens"][lvl] = [[pool[c]["token"] for c in lv["children"] if pool[c]["parent"] == n]
                                for n in lv["frontier"]]
            if lvl >= 2:
                f["frontier"][lvl] = list(lv["frontier"])
        force.append(f)
    forced = draft_expand(wl.dims, params, wl.weights, wl.draft_weights, wl.root_feature, wl.root_token,
                          wl.dk_cache, wl.dv_cache, wl.prefix_len, trace=True, force=force)
    for a, b in zip(free, forced):
        assert a["parent"] == b["parent"] and a["tokens"] == b["tokens"] and a["cum"] == b["cum"]
        assert [c["token"] for c in a["pool"]] == [c["token"] for c in b["pool"]]


@pytest.mark.parametrize("seed,tau", [(0, 0.0), (3, 0.0), (6, 0.2)])
def test_branching_tree_equals_sequential_run_along_each_root_path(seed, tau):
    """Every expanded node of a branching draft (top-3, frontier 3, depth 4) must carry
    exactly what the one-layer draft head computes when it is run left to right over that
    node's root path alone ("LLM parallel decoding EAGLE" page, how EAGLE works: the head
    predicts the next feature from the feature and token before it, and its candidates are
    expanded into a tree; "Speculative decoding with EAGLE" page, technical insight: the
    row for a token is formed from the feature before it and that token's true embedding).
    A draft row that also saw nodes off its own root path, or took a sibling's feature,
    gives a different f_hat and different child log-probabilities."""
    wl = _wl(seed, B=2)
    params = DraftParams(depth=4, top_k=3, frontier=3, max_nodes=40, conf_threshold=tau)
    res = _run(wl, params, trace=True)
    W_fc, E = wf(wl.draft_weights["w_fc"]), wl.weights["embed"]
    checked = 0
    for b, r in enumerate(res):
        pool = r["pool"]
        P = int(wl.prefix_len[b])
        expanded = [(lvl, row, n) for lvl, lv in enumerate(r["levels"]) for row, n in enumerate(lv["frontier"])]
        assert len(expanded) > 4 and any(pool[n]["depth"] >= 2 for _, _, n in expanded)
        for lvl, row, n in expanded:
            path = []
            j = n
            while j >= 0:
                path.append(j)
                j = pool[j]["parent"]
            path.reverse()
            dec = SequentialDecoder(wl.dims, wl.draft_weights, wl.dk_cache[b, :, :P], wl.dv_cache[b, :, :P])
            f = wf(wl.root_feature[b])
            cum = 0.0
            for j in path:
                f = dec.step(W_fc @ np.concatenate([f, wf(E[pool[j]["token"]])]))["h"]
                if j != n:
                    z = logits_of(wl.dims, wl.weights, f)
                    lse = z.max() + np.log(np.sum(np.exp(z - z.max())))
                    nxt = path[path.index(j) + 1]
                    cum += min(0.0, z[pool[nxt]["token"]] - lse)
            assert dec.pos == P + pool[n]["depth"] + 1
            assert np.abs(r["levels"][lvl]["fhat"][row] - f).max() < 1e-10 * max(1.0, np.abs(f).max())
            assert abs(pool[n]["cum"] - cum) < 1e-10
            z = logits_of(wl.dims, wl.weights, f)
            lse = z.max() + np.log(np.sum(np.exp(z - z.max())))
            kids = [c for c in r["levels"][lvl]["children"] if pool[c]["parent"] == n]
            left = list(range(len(z)))
            for c in kids:                      # children = the top_k tokens by an explicit scan
                best = left[0]
                for t in left:
                    if z[t] > z[best]:
                        best = t
                left.remove(best)
                assert pool[c]["token"] == best
                assert abs(pool[c]["logp"] - (z[best] - lse)) < 1e-10
                assert abs(pool[c]["cum"] - (cum + min(0.0, z[best] - lse))) < 1e-10
            checked += 1
    assert checked >= 10
