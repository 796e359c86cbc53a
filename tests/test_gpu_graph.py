"""The verification step (tree encode -> verify -> accept + commit) captured once into a HIP
graph and replayed, as the benchmark runs it, must give exactly what the same steps give
when launched one by one: every replay is compared bit for bit with an eager step from the
same state (each step commits into the cache and advances the prefix, so consecutive steps
differ), with eager work and synchronisations of the program between the replays.  The
step launches kernels only (no memset nodes, no host synchronisation)."""
import numpy as np
import pytest

from workloads import make_workload, mini_dims, trees as T
from workloads.device import upload

pytestmark = pytest.mark.gpu


def _state(v, t):
    import torch
    keys = ("anc", "depth", "pos", "k_tree", "v_tree", "h", "argmax", "maxlogit", "accept_len", "path",
            "out_tokens", "next_token", "next_feature", "status")
    out = {k: getattr(v, k).clone() for k in keys}
    out.update(prefix=t["prefix_len"].clone(), k_cache=t["k_cache"].clone(), v_cache=t["v_cache"].clone())
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("layout", [0, 1])
def test_graph_replays_equal_eager_steps(layout):
    import torch
    from tree_attention_verification_06_amd.runner import TreeVerifier, with_packed_weights
    dims = mini_dims()
    parents = [T.static_tree_60(), T.random_tree(np.random.default_rng(6), 33), T.chain(12)]
    wl = make_workload(2, seed=45, dims=dims, batch=3, prefix=[300, 64, 1000], parents=parents, cache_slack=64)
    t = upload(wl)
    M = wl.n_nodes
    w = with_packed_weights(t["weights"]) if layout else t["weights"]
    v = TreeVerifier(dims, w, t["k_cache"], t["v_cache"], batch=3, max_total_nodes=M, max_nodes=60,
                     max_prefix=wl.cache_cap, lm_layout=layout, weight_layout=layout)
    # plant a depth-2 path in tree 2 from a first eager step, so commits of several slots occur
    v.step(t["tree_off"], t["parent"], t["tokens"], t["prefix_len"].clone(), M, x=t["x"])
    torch.cuda.synchronize()
    g = v.argmax.cpu().numpy()
    tok = wl.tokens.copy()
    o = int(wl.tree_off[2])
    tok[o + 1], tok[o + 2] = g[o], g[o + 1]
    t["tokens"].copy_(torch.from_numpy(tok))
    k0, v0, p0 = t["k_cache"].clone(), t["v_cache"].clone(), t["prefix_len"].clone()

    def step():
        v.step(t["tree_off"], t["parent"], t["tokens"], t["prefix_len"], M, x=t["x"])

    n = 4
    eager = []
    for _ in range(n):
        step()
        eager.append(_state(v, t))
    assert int(eager[0]["accept_len"][2]) >= 2
    assert not torch.equal(eager[0]["h"], eager[1]["h"])   # the prefix grew: the steps differ
    t["k_cache"].copy_(k0)
    t["v_cache"].copy_(v0)
    t["prefix_len"].copy_(p0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.synchronize()
    # capture enqueues nothing: the state is still the initial one
    assert torch.equal(t["prefix_len"], p0) and torch.equal(t["k_cache"], k0)
    for i in range(n):
        graph.replay()
        torch.cuda.synchronize()
        got = _state(v, t)
        for k, ref in eager[i].items():
            assert torch.equal(got[k], ref), (i, k)
        junk = torch.randn(1 << 20, device="cuda")   # eager work of the program between replays
        (junk * 2).sum().item()
        print("graph replay", layout, i, "equals eager", flush=True)
